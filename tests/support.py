"""Helpers shared by the GPU tests: seeded inputs on the device, the forward
pass that produces O and lse, and the oracle comparison."""
from __future__ import annotations

import math

import numpy as np

import workloads


def device():
    import torch
    return torch.device("cuda:0")


def torch_dtype(name):
    import torch
    return {"bf16": torch.bfloat16, "fp32": torch.float32}[name]


def forward_fp32(q, k, v, causal: bool, scale: float, out_dtype):
    """Softmax attention forward in float32 on the device with plain PyTorch
    ops, producing the O (in `out_dtype`) and lse (float32, natural log of the
    scaled logits) that the backward consumes.  Input preparation only; the
    tests judge the backward against the fp64 oracle, which recomputes its own
    forward from Q, K, V."""
    import torch
    b, h, s, d = q.shape
    o = torch.empty((b, h, s, d), dtype=out_dtype, device=q.device)
    lse = torch.empty((b, h, s), dtype=torch.float32, device=q.device)
    per = max(1, int(2 ** 30 // (s * s * 4)))  # heads per chunk: ~1 GiB of scores
    qf, kf, vf = (t.reshape(b * h, s, d) for t in (q, k, v))
    of, lf = o.view(b * h, s, d), lse.view(b * h, s)
    mask = None
    if causal:
        mask = torch.ones((s, s), dtype=torch.bool, device=q.device).triu(1)
    for i in range(0, b * h, per):
        qi = qf[i:i + per].float()
        kt = kf[i:i + per].float().transpose(1, 2).contiguous()
        sc = torch.matmul(qi, kt) * scale
        if mask is not None:
            sc.masked_fill_(mask, float("-inf"))
        l = torch.logsumexp(sc, dim=-1)
        p = torch.exp(sc - l[..., None])
        of[i:i + per] = torch.matmul(p, vf[i:i + per].float()).to(out_dtype)
        lf[i:i + per] = l
        del sc, p
    return o, lse


class Problem:
    """Seeded inputs of one workload shape on the host (float32 NumPy, values
    exactly representable in the element type) and on the device."""

    def __init__(self, b, h, s, d, dtype, seed, causal):
        import torch
        self.b, self.h, self.s, self.d, self.dtype, self.causal = b, h, s, d, dtype, causal
        self.scale = 1.0 / math.sqrt(d)
        self.qn, self.kn, self.vn, self.don = workloads.draw_qkv_do(b, h, s, d, seed, dtype)
        td = torch_dtype(dtype)
        dev = device()
        self.q, self.k, self.v, self.do = (torch.from_numpy(x).to(dev).to(td)
                                           for x in (self.qn, self.kn, self.vn, self.don))
        self.o, self.lse = forward_fp32(self.q, self.k, self.v, causal, self.scale, td)

    def run(self, schedule, out=None):
        import tile_scheduling_attn_amd as tsa
        return tsa.backward(self.q, self.k, self.v, self.o, self.do, self.lse, self.causal,
                            schedule, self.scale, out=out)

    def oracle(self, heads=None):
        """fp64 truth for the selected flat head indices (all by default):
        dict name -> array [len(heads), s, d]."""
        import oracle
        H = self.b * self.h
        heads = list(range(H)) if heads is None else list(heads)
        sel = lambda x: x.reshape(H, self.s, self.d)[heads]
        return oracle.attn_fwd_bwd(sel(self.qn), sel(self.kn), sel(self.vn), sel(self.don),
                                   self.causal, self.scale)


def rel_err(gpu, ref):
    """max |gpu - ref| / max |ref| over one tensor."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(gpu - ref)) / (den if den > 0 else 1.0))


def to_np_heads(t, heads):
    b, h, s, d = t.shape
    return t.reshape(b * h, s, d)[list(heads)].float().cpu().numpy()


TOL = {"bf16": 2e-2, "fp32": 1e-4}

# Measured parity errors of this test session, (case, tensor) -> error; the
# conftest writes them to the file named by ATTN_PARITY_RECORD, if set.
# A measurement record only: no test reads it back as an expected value.
ERRORS = {}


def record_error(case, tensor, err, tol):
    ERRORS[f"{case} | {tensor}"] = {"rel_err": float(err), "tol": None if tol is None else float(tol)}
