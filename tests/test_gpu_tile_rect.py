"""Rectangular bf16 tiles (attn_bwd_set_tile_shape: 64-row Q tiles against
128-row KV tiles, Br != Bc): parity with the fp64 oracle on ragged shapes
under every schedule (the rectangular Shift and Symmetric Shift rank tables
among them), bitwise determinism, the same bits under both work placements,
NAIVE and DESCENDING sharing dQ bits, and sampled parity at the full
s = 8192, d = 128 causal size."""
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import tile_scheduling_attn_amd as tsa  # noqa: E402
from support import Problem, TOL, rel_err, record_error, to_np_heads  # noqa: E402

SCHEDS = ("naive", "descending", "shift", "symmetric_shift", "atomic", "auto")


@pytest.fixture
def rect():
    tsa.attn_bwd_set_tile_shape("bf16", 64, 128)
    yield
    tsa.attn_bwd_set_tile_shape("bf16", 0, 0)


@pytest.mark.parametrize("shape", [(1, 2, 512, 128), (2, 2, 200, 64), (1, 3, 1000, 128), (1, 1, 64, 64),
                                   (1, 2, 1100, 64)],
                         ids=lambda x: "-".join(map(str, x)))
@pytest.mark.parametrize("causal", [False, True])
def test_rect_parity_and_determinism(shape, causal, rect):
    b, h, s, d = shape
    assert tsa.attn_bwd_tile_shape("bf16") == (64, 128)
    pb = Problem(b, h, s, d, "bf16", 5500 + s + d, causal)
    n = -(-s // 128)  # KV tiles; Q tiles 2n
    ref = pb.oracle()
    outs = {}
    for sched in SCHEDS:
        if sched == "symmetric_shift" and causal and n % 2:
            continue
        print(f"rect 64x128 {shape} causal={causal} {sched}", flush=True)
        g = [t.clone() for t in pb.run(sched)]
        torch.cuda.synchronize()
        assert tsa.attn_bwd_query_status() == 0, tsa.last_error()
        for name, t in zip(("dq", "dk", "dv"), g):
            e = rel_err(to_np_heads(t, range(b * h)), ref[name])
            record_error(f"rect64x128 {shape} causal={causal} {sched}", name, e, TOL["bf16"])
            assert e <= TOL["bf16"], (sched, name, e)
        if sched != "atomic":
            for _ in range(2):
                again = pb.run(sched)
                for x, y in zip(g, again):
                    assert torch.equal(x.view(torch.int16), y.view(torch.int16)), sched
        outs[sched] = g
    assert torch.equal(outs["naive"][0].view(torch.int16), outs["descending"][0].view(torch.int16))


@pytest.mark.parametrize("causal", [False, True])
def test_rect_placements_give_the_same_bits(causal, rect):
    pb = Problem(1, 8, 4096, 128, "bf16", 778, causal)
    for sched in ("shift", "naive", "symmetric_shift") if causal else ("shift", "naive"):
        res = {}
        for place in ("xcd", "global"):
            tsa.attn_bwd_set_placement(place)
            try:
                res[place] = [t.clone() for t in pb.run(sched)]
            finally:
                tsa.attn_bwd_set_placement("xcd")
            assert tsa.attn_bwd_query_status() == 0, tsa.last_error()
        for x, y in zip(res["xcd"], res["global"]):
            assert torch.equal(x.view(torch.int16), y.view(torch.int16)), sched


def test_rect_full_size_sampled_parity(rect):
    """s8k d128 causal (b2 h16) with rectangular Symmetric Shift: sampled heads
    against the oracle, and two runs bitwise equal."""
    pb = Problem(2, 16, 8192, 128, "bf16", 31337, True)
    g = [t.clone() for t in pb.run("symmetric_shift")]
    again = pb.run("symmetric_shift")
    torch.cuda.synchronize()
    assert tsa.attn_bwd_query_status() == 0, tsa.last_error()
    for x, y in zip(g, again):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))
    heads = [0, 31]
    ref = pb.oracle(heads=heads)
    for name, t in zip(("dq", "dk", "dv"), g):
        e = rel_err(to_np_heads(t, heads), ref[name])
        record_error("rect64x128 s8k d128 causal symmetric_shift heads 0,31", name, e, TOL["bf16"])
        assert e <= TOL["bf16"], (name, e)


@pytest.mark.parametrize("causal", [False, True])
def test_rect_injected_delays_keep_the_bits(causal, rect):
    """Random sleeps before every reduction phase (attn_bwd_set_debug) move the
    hand-offs of the rectangular rank tables in time; the bits must not move."""
    pb = Problem(1, 8, 2048, 128, "bf16", 9191, causal)
    scheds = ("shift", "symmetric_shift", "descending") if causal else ("shift", "naive")
    try:
        for sched in scheds:
            tsa.attn_bwd_set_debug(0, 0, 0)
            ref = [t.clone() for t in pb.run(sched)]
            for seed in (3, 0xabcdef):
                tsa.attn_bwd_set_debug(0, 0, seed)
                got = pb.run(sched)
                torch.cuda.synchronize()
                assert tsa.attn_bwd_query_status() == 0, tsa.last_error()
                for x, y in zip(ref, got):
                    assert torch.equal(x.view(torch.int16), y.view(torch.int16)), (sched, seed)
    finally:
        tsa.attn_bwd_set_debug(0, 0, 0)
