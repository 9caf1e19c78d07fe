"""The eight-wave pair kernel (attn_bwd_set_main_kernel("pair"): bf16,
d = 64 and 128, 128 x 128 tiles, deterministic schedules): parity with the fp64
oracle on ragged shapes under every deterministic schedule, the bits of the
four-wave kernel (both perform every addition in the same order), bitwise
determinism, both work placements, injected reduction-phase delays, and
sampled parity at the full s = 8192 size."""
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import tile_scheduling_attn_amd as tsa  # noqa: E402
from support import Problem, TOL, rel_err, record_error, to_np_heads  # noqa: E402

DET = ("naive", "descending", "shift", "symmetric_shift", "auto")


@pytest.fixture
def pair():
    tsa.attn_bwd_set_main_kernel("pair")
    yield
    tsa.attn_bwd_set_main_kernel("auto")


def bits(ts):
    return [t.view(torch.int16).clone() for t in ts]


def same_bits(a, b):
    return all(torch.equal(x, y) for x, y in zip(a, b))


@pytest.mark.parametrize("shape", [(1, 2, 512, 128), (1, 3, 1000, 128), (2, 2, 200, 128), (1, 1, 128, 128),
                                   (1, 2, 1100, 128), (1, 2, 512, 64), (2, 2, 200, 64), (1, 3, 1100, 64)],
                         ids=lambda x: "-".join(map(str, x)))
@pytest.mark.parametrize("causal", [False, True])
def test_pair_parity_and_four_wave_bits(shape, causal, pair):
    b, h, s, d = shape
    assert tsa.attn_bwd_main_kernel() == "pair"
    pb = Problem(b, h, s, d, "bf16", 7700 + s, causal)
    n = -(-s // 128)
    ref = pb.oracle()
    for sched in DET:
        if sched == "symmetric_shift" and causal and n % 2:
            continue
        print(f"pair {shape} causal={causal} {sched}", flush=True)
        got = bits(pb.run(sched))
        torch.cuda.synchronize()
        assert tsa.attn_bwd_query_status() == 0, tsa.last_error()
        for name, t in zip(("dq", "dk", "dv"), got):
            e = rel_err(to_np_heads(t.view(torch.bfloat16), range(b * h)), ref[name])
            record_error(f"pair {shape} causal={causal} {sched}", name, e, TOL["bf16"])
            assert e <= TOL["bf16"], (sched, name, e)
        assert same_bits(got, bits(pb.run(sched))), sched
        tsa.attn_bwd_set_main_kernel("four_wave")
        try:
            four = bits(pb.run(sched))
        finally:
            tsa.attn_bwd_set_main_kernel("pair")
        assert same_bits(got, four), sched


def test_pair_atomic_uses_the_four_wave_kernel(pair):
    """ATOMIC has no pair form: it runs as before, and its dK and dV keep the
    deterministic schedules' bits."""
    pb = Problem(1, 2, 640, 128, "bf16", 7799, True)
    a = bits(pb.run("atomic"))
    n = bits(pb.run("naive"))
    assert tsa.attn_bwd_query_status() == 0, tsa.last_error()
    assert same_bits(a[1:], n[1:])


def test_pair_twenty_runs_and_placements(pair):
    pb = Problem(1, 8, 4096, 128, "bf16", 7801, True)
    for sched in ("symmetric_shift", "descending", "shift"):
        ref = bits(pb.run(sched))
        for _ in range(19):
            assert same_bits(ref, bits(pb.run(sched))), sched
        tsa.attn_bwd_set_placement("global")
        try:
            glob = bits(pb.run(sched))
        finally:
            tsa.attn_bwd_set_placement("xcd")
        assert tsa.attn_bwd_query_status() == 0, tsa.last_error()
        assert same_bits(ref, glob), sched


@pytest.mark.parametrize("causal", [False, True])
def test_pair_injected_delays_keep_the_bits(causal, pair):
    pb = Problem(1, 8, 2048, 128, "bf16", 7802, causal)
    scheds = ("symmetric_shift", "descending") if causal else ("shift", "naive")
    try:
        for sched in scheds:
            tsa.attn_bwd_set_debug(0, 0, 0)
            ref = bits(pb.run(sched))
            for seed in (5, 0x5eed):
                tsa.attn_bwd_set_debug(0, 0, seed)
                got = bits(pb.run(sched))
                torch.cuda.synchronize()
                assert tsa.attn_bwd_query_status() == 0, tsa.last_error()
                assert same_bits(ref, got), (sched, seed)
    finally:
        tsa.attn_bwd_set_debug(0, 0, 0)


def test_pair_timeout_is_reported_and_the_next_call_is_correct(pair):
    """A wait that can never be satisfied ends through the kernel's own bounded
    poll; the next call runs normally."""
    pb = Problem(1, 2, 1024, 128, "bf16", 7803, False)
    ref = bits(pb.run("shift"))
    try:
        # every wait looks for a flag value nobody publishes; 64 polls each
        tsa.attn_bwd_set_debug(64, 1000, 0)
        pb.run("shift")
        rc = tsa.attn_bwd_query_status()
        assert rc == -5, (rc, tsa.last_error())
    finally:
        tsa.attn_bwd_set_debug(0, 0, 0)
    assert same_bits(ref, bits(pb.run("shift")))
    assert tsa.attn_bwd_query_status() == 0


@pytest.mark.parametrize("causal,sched", [(False, "shift"), (True, "symmetric_shift")])
def test_pair_full_size_sampled_parity(causal, sched, pair):
    pb = Problem(2, 16, 8192, 128, "bf16", 7804, causal)
    got = bits(pb.run(sched))
    torch.cuda.synchronize()
    assert tsa.attn_bwd_query_status() == 0, tsa.last_error()
    heads = [0, 17, 31]
    ref = pb.oracle(heads=heads)
    for name, t in zip(("dq", "dk", "dv"), got):
        e = rel_err(to_np_heads(t.view(torch.bfloat16), heads), ref[name])
        record_error(f"pair s8k d128 causal={causal} {sched} heads 0,17,31", name, e, TOL["bf16"])
        assert e <= TOL["bf16"], (name, e)
    tsa.attn_bwd_set_main_kernel("four_wave")
    try:
        four = bits(pb.run(sched))
    finally:
        tsa.attn_bwd_set_main_kernel("pair")
    assert same_bits(got, four)


def test_pair_d64_s2k_causal_sampled_parity(pair):
    """b4 h16 s2048 d64 causal, Symmetric Shift: sampled heads against the
    oracle and the four-wave kernel's bits."""
    pb = Problem(4, 16, 2048, 64, "bf16", 7805, True)
    got = bits(pb.run("symmetric_shift"))
    torch.cuda.synchronize()
    assert tsa.attn_bwd_query_status() == 0, tsa.last_error()
    heads = [0, 33, 63]
    ref = pb.oracle(heads=heads)
    for name, t in zip(("dq", "dk", "dv"), got):
        e = rel_err(to_np_heads(t.view(torch.bfloat16), heads), ref[name])
        record_error("pair s2k d64 causal symmetric_shift heads 0,33,63", name, e, TOL["bf16"])
        assert e <= TOL["bf16"], (name, e)
    tsa.attn_bwd_set_main_kernel("four_wave")
    try:
        four = bits(pb.run("symmetric_shift"))
    finally:
        tsa.attn_bwd_set_main_kernel("pair")
    assert same_bits(got, four)
