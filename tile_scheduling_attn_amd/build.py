"""Build libattn_bwd.so (HIP kernels for gfx950 + host schedule/simulator +
C ABI) in-tree with hipcc.  `python tile_scheduling_attn_amd/build.py` (run as a
file: importing the package loads the library this builds)."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libattn_bwd.so")

SOURCES = ["api.cpp", "schedule.cpp", "bwd_kernels.hip", "bwd_kernels_d64.hip", "bwd_pair.hip", "fwd_kernels.hip", "noalloc.hip",
           "measure_kernels.hip"]
# per-source extra flags: the bf16 d = 64 kernels keep MFMA results in
# architectural registers (see the comment at the top of that file)
SOURCE_FLAGS = {"bwd_kernels_d64.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}
# Packed fp32 VALU forms are switched off for every HIP source.
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-munsafe-fp-atomics", "-Wall", "-Wno-unused-function"]


def build(verbose: bool = False, extra_flags=None) -> str:
    """Compile every source and link the shared library; always rebuilds."""
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src + ".o")
        cmd = ["hipcc", *HIP_FLAGS, *SOURCE_FLAGS.get(src, []), *(extra_flags or []), "-I", INCLUDE, "-I", CSRC,
               "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{err}")
        if verbose and err.strip():
            print(err, file=sys.stderr)
        objs.append(obj)
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = ["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, LIB)
    return LIB


def resource_usage() -> str:
    """Per-kernel register, scratch and occupancy figures of the HIP sources,
    from the compiler's kernel-resource-usage remarks, as a markdown table
    (compiles the device code again, with the build's flags)."""
    import re
    rows = []
    for src in SOURCES:
        if not src.endswith(".hip"):
            continue
        cmd = ["hipcc", *HIP_FLAGS, *SOURCE_FLAGS.get(src, []), "-I", INCLUDE, "-I", CSRC, "--cuda-device-only",
               "-c", os.path.join(CSRC, src), "-o", os.devnull, "-Rpass-analysis=kernel-resource-usage"]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
        cur = None
        for line in r.stderr.splitlines():
            m = re.search(r"remark: Function Name: (\S+)", line)
            if m:
                cur = {"source": src, "kernel": m.group(1)}
                rows.append(cur)
                continue
            m = re.search(r"remark:\s+([A-Za-z ]+?)(?: \[[^\]]*\])?:\s+(-?\d+)", line)
            if m and cur is not None:
                cur[m.group(1).strip()] = int(m.group(2))
    cols = ["VGPRs", "AGPRs", "TotalSGPRs", "ScratchSize", "VGPRs Spill", "SGPRs Spill", "Occupancy", "LDS Size"]
    out = ["| source | kernel | " + " | ".join(cols) + " |", "|" + "---|" * (len(cols) + 2)]
    for r in rows:
        out.append(f"| {r['source']} | `{r['kernel']}` | " + " | ".join(str(r.get(c, "")) for c in cols) + " |")
    return "\n".join(out)


if __name__ == "__main__":
    if "--resource-usage" in sys.argv:
        print(resource_usage())
    else:
        print(build(verbose="-v" in sys.argv))
