"""Seeded synthetic inputs for the attention backward workloads.

This module holds the workload table and the random-number recipe only; it
contains none of the attention arithmetic.  Both the CPU oracle side (tests)
and the GPU side (tests, bench, smoke) draw their Q, K, V and dO from here so
that the two see the same values.

Recipe (the pages measure on "BF16 random inputs", DASH paper, Experimental
setup): Q, K, V, dO are i.i.d. N(0, 1) drawn in float32 from NumPy's PCG64
generator, seed = base seed of the workload, +1 for dO; for bf16 workloads
the float32 values are rounded to nearest-even bf16.  O and lse are not drawn:
they come from a forward pass over these Q, K, V (outside this module).
"""
from __future__ import annotations

from dataclasses import dataclass, field
import numpy as np

__all__ = ["Workload", "WORKLOADS", "draw_qkv_do", "round_bf16_np"]


@dataclass(frozen=True)
class Workload:
    name: str
    b: int
    h: int
    s: int
    d: int
    dtype: str            # "bf16" or "fp32"
    masks: tuple          # subset of ("full", "causal")
    schedules: tuple      # schedule names compared on this workload
    seed: int
    description: str = ""

    @property
    def heads(self) -> int:
        return self.b * self.h

    def flops(self, causal: bool) -> float:
        """Algorithmic FLOP of one backward: 5 contractions of 2*s*s*d each per
        head (FlashAttention convention), halved under the causal mask."""
        f = 10.0 * self.b * self.h * self.s * self.s * self.d
        return f / 2 if causal else f


WORKLOADS = {
    "tiny": Workload("tiny", 1, 1, 128, 64, "fp32", ("full", "causal"),
                     ("naive", "descending", "shift", "symmetric_shift", "atomic"), 20261,
                     "b1 h1 s128 d64 fp32, tile 64x64, all schedules"),
    "s2k_d64_causal": Workload("s2k_d64_causal", 4, 16, 2048, 64, "bf16", ("causal",),
                               ("descending", "symmetric_shift", "naive", "atomic"), 20262,
                               "b4 h16 s2048 d64 bf16 causal"),
    "s8k_d128_full": Workload("s8k_d128_full", 2, 16, 8192, 128, "bf16", ("full",),
                              ("shift", "naive", "atomic"), 20263,
                              "b2 h16 s8192 d128 bf16 full mask"),
    "s8k_d128_causal": Workload("s8k_d128_causal", 2, 16, 8192, 128, "bf16", ("causal",),
                                ("descending", "symmetric_shift", "atomic"), 20264,
                                "b2 h16 s8192 d128 bf16 causal"),
    "s16k_d128": Workload("s16k_d128", 1, 32, 16384, 128, "bf16", ("full", "causal"),
                          ("shift", "naive", "descending", "symmetric_shift", "atomic"), 20265,
                          "b1 h32 s16384 d128 bf16 full and causal"),
}


def round_bf16_np(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even), returned as
    float32 holding exactly representable bf16 values.  NaN/Inf are not
    produced by N(0,1) draws and are not handled."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    u = (u + 0x7FFF + lsb) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def draw_qkv_do(b: int, h: int, s: int, d: int, seed: int, dtype: str = "bf16"):
    """Return (q, k, v, do) as float32 NumPy arrays of shape [b, h, s, d].

    Values are N(0,1) from PCG64(seed) (q, k, v drawn in that order) and
    PCG64(seed + 1) (do); bf16 workloads round them to bf16."""
    rng = np.random.Generator(np.random.PCG64(seed))
    shape = (b, h, s, d)
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    rng2 = np.random.Generator(np.random.PCG64(seed + 1))
    do = rng2.standard_normal(shape, dtype=np.float32)
    if dtype == "bf16":
        q, k, v, do = (round_bf16_np(t) for t in (q, k, v, do))
    elif dtype != "fp32":
        raise ValueError(f"unknown dtype {dtype!r}")
    return q, k, v, do
