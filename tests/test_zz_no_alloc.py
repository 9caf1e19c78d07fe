"""The allocation-free entry point, through the C ABI: two calls in a row
(the second one smaller, so it reuses the device array the first one
filled) give the bits of attn_bwd_deterministic_ex with the same schedule,
and a problem too large for the array is refused before any launch."""
import math
import sys

import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import tile_scheduling_attn_amd as tsa  # noqa: E402
from support import Problem  # noqa: E402


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _noalloc(pb, sched, out):
    dq, dk, dv = out
    b, h, s, d = pb.q.shape
    stream = torch.cuda.current_stream().cuda_stream
    return tsa.attn_bwd_deterministic_noalloc(pb.q, pb.k, pb.v, pb.o, pb.do, pb.lse, dq, dk, dv, b, h, s, d,
                                              pb.causal, sched, pb.dtype, pb.scale, stream)


CASES = [  # (b, h, s, d, dtype, causal, schedule), second smaller than the first
    (2, 4, 1536, 128, "bf16", True, "symmetric_shift"),
    (1, 3, 300, 64, "bf16", False, "shift"),
    (1, 2, 200, 64, "fp32", True, "descending"),
]


def test_noalloc_matches_the_allocating_entry_point():
    assert tsa.attn_bwd_noalloc_capacity() == 64 << 20
    view = {"bf16": torch.int16, "fp32": torch.int32}
    for i, (b, h, s, d, dt, causal, sched) in enumerate(CASES):
        _say(f"noalloc call {i}: b{b} h{h} s{s} d{d} {dt} causal={causal} {sched}")
        pb = Problem(b, h, s, d, dt, 6060 + i, causal)
        ref = [t.clone() for t in pb.run(sched)]
        out = [torch.full_like(pb.q, float("nan")) for _ in range(3)]
        rc = _noalloc(pb, sched, out)
        assert rc == 0, tsa.last_error()
        torch.cuda.synchronize()
        assert tsa.attn_bwd_query_status() == 0, tsa.last_error()
        for a, g in zip(ref, out):
            assert torch.equal(a.view(view[dt]), g.view(view[dt])), f"case {i}"


def test_noalloc_refuses_a_problem_larger_than_its_array():
    # b2 h16 s8192 d128 needs a 134 MB accumulator: refused before any launch
    pb = Problem(1, 1, 128, 128, "bf16", 1, False)
    stream = torch.cuda.current_stream().cuda_stream
    rc = tsa.attn_bwd_deterministic_noalloc(pb.q, pb.k, pb.v, pb.o, pb.do, pb.lse, pb.q, pb.k, pb.v,
                                            2, 16, 8192, 128, 0, "shift", "bf16", 1 / math.sqrt(128), stream)
    assert rc == -6, (rc, tsa.last_error())
    assert "no-allocation" in tsa.last_error()
    # and the next call is unaffected
    out = [torch.empty_like(pb.q) for _ in range(3)]
    assert _noalloc(pb, "naive", out) == 0
    torch.cuda.synchronize()
    ref = pb.run("naive")
    for a, g in zip(ref, out):
        assert torch.equal(a.view(torch.int16), g.view(torch.int16))
