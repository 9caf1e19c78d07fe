"""GPU parity of the HIP attention forward (O and lse) with the fp64 oracle,
bitwise reproducibility, and the backward fed with it, through the C ABI.

Tolerance: O per tensor as for the backward (max|o_gpu - o_oracle| /
max|o_oracle| <= 2e-2 for bf16 inputs, 1e-4 for fp32); lse (fp32 output,
exact bf16 products accumulated in fp32) to 1e-3 absolute."""
import math

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import tile_scheduling_attn_amd as tsa  # noqa: E402
import workloads  # noqa: E402
from support import TOL, rel_err  # noqa: E402


def _say(msg):
    print(msg, flush=True)


def _inputs(b, h, s, d, dt, seed):
    qn, kn, vn, don = workloads.draw_qkv_do(b, h, s, d, seed, dt)
    td = torch.float32 if dt == "fp32" else torch.bfloat16
    q, k, v, do = (torch.from_numpy(x).cuda().to(td) for x in (qn, kn, vn, don))
    return (qn, kn, vn, don), (q, k, v, do)


def _oracle_fwd(arrs, heads, causal, scale):
    import oracle
    qn, kn, vn, _ = arrs
    b, h, s, d = qn.shape
    H = b * h
    sel = lambda x: np.ascontiguousarray(x.reshape(H, s, d)[list(heads)])
    return oracle.attn_fwd(sel(qn), sel(kn), sel(vn), causal, scale)


def _check(o, lse, arrs, heads, causal, scale, dt, tag):
    b, h, s, d = arrs[0].shape
    ref_o, ref_lse = _oracle_fwd(arrs, heads, causal, scale)
    got_o = o.float().cpu().numpy().reshape(b * h, s, d)[list(heads)]
    got_l = lse.cpu().numpy().reshape(b * h, s)[list(heads)]
    eo = rel_err(got_o, ref_o)
    el = float(np.abs(got_l - ref_lse).max())
    _say(f"{tag}: O rel err {eo:.3e}, lse abs err {el:.3e}")
    assert eo <= TOL[dt], tag
    assert el <= 1e-3, tag


SHAPES = [
    (1, 1, 128, 64, "fp32"),
    (2, 2, 256, 128, "fp32"),
    (1, 2, 130, 64, "fp32"),       # ragged: 2 rows past the last full tile
    (1, 2, 512, 64, "bf16"),
    (2, 1, 384, 128, "bf16"),
    (1, 3, 200, 64, "bf16"),       # ragged
    (1, 2, 300, 128, "bf16"),      # ragged
    (1, 1, 1, 64, "bf16"),         # a single row
    (1, 1, 64, 128, "bf16"),       # one partial tile
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda x: "-".join(map(str, x)))
@pytest.mark.parametrize("causal", [False, True])
def test_forward_parity_small(shape, causal):
    b, h, s, d, dt = shape
    arrs, (q, k, v, _) = _inputs(b, h, s, d, dt, 3000 + s + d + h)
    scale = 1.0 / math.sqrt(d)
    o, lse = tsa.forward(q, k, v, causal, scale)
    torch.cuda.synchronize()
    _check(o, lse, arrs, range(b * h), causal, scale, dt, f"fwd {shape} causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
def test_forward_parity_s8k_d128_sampled_heads(causal):
    wl = workloads.WORKLOADS["s8k_d128_full"]
    arrs, (q, k, v, _) = _inputs(wl.b, wl.h, wl.s, wl.d, wl.dtype, wl.seed)
    scale = 1.0 / math.sqrt(wl.d)
    o, lse = tsa.forward(q, k, v, causal, scale)
    torch.cuda.synchronize()
    H = wl.b * wl.h
    _check(o, lse, arrs, [0, H - 1], causal, scale, wl.dtype, f"fwd s8k d128 causal={causal}")


def test_forward_is_bitwise_reproducible():
    arrs, (q, k, v, _) = _inputs(1, 8, 2048, 128, "bf16", 17)
    o0, l0 = tsa.forward(q, k, v, True)
    for _ in range(5):
        o1, l1 = tsa.forward(q, k, v, True)
        torch.cuda.synchronize()
        assert torch.equal(o0.view(torch.int16), o1.view(torch.int16))
        assert torch.equal(l0, l1)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_fed_by_the_forward(causal):
    """End to end: this forward's O and lse into the deterministic backward;
    gradients against the oracle's (which recomputes its own forward)."""
    import oracle
    b, h, s, d = 1, 2, 640, 128
    arrs, (q, k, v, do) = _inputs(b, h, s, d, "bf16", 29)
    scale = 1.0 / math.sqrt(d)
    o, lse = tsa.forward(q, k, v, causal, scale)
    dq, dk, dv = tsa.backward(q, k, v, o, do, lse, causal, "descending", scale)
    torch.cuda.synchronize()
    assert tsa.attn_bwd_query_status() == 0, tsa.last_error()
    qn, kn, vn, don = (x.reshape(b * h, s, d) for x in arrs)
    ref = oracle.attn_fwd_bwd(qn, kn, vn, don, causal, scale)
    for name, g in zip(("dq", "dk", "dv"), (dq, dk, dv)):
        e = rel_err(g.float().cpu().numpy().reshape(b * h, s, d), ref[name])
        _say(f"fwd->bwd causal={causal} {name}: {e:.3e}")
        assert e <= TOL["bf16"]
