"""Failure and race paths of the deterministic backward, forced from the host
through the library's test hooks (attn_bwd_set_debug); every kernel still
runs to its end.

* Race detection: bitwise determinism is the race detector.  With random
  delays injected before every reduction phase (seeded from the host), the
  hand-offs of the dQ reduction happen at other times and in other relative
  orders than in an undisturbed run; a flag-protocol bug (a contributor
  reading the accumulator before its predecessor's release) would change
  bits.  The results must stay bitwise identical.
* Failure detection: with a tiny poll limit and a flag value that is never
  published, every bounded wait gives up; the call still ends, the device
  status reports ATTN_ERR_TIMEOUT, and the next normal call is clean."""
import sys

import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import tile_scheduling_attn_amd as tsa  # noqa: E402
from support import Problem, TOL, rel_err, to_np_heads  # noqa: E402


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture
def debug_hooks():
    yield tsa.attn_bwd_set_debug
    tsa.attn_bwd_set_debug(0, 0, 0)


# (b, h, s, d, causal, schedules): waits on every schedule kind, both head
# dimensions, XCD placement with several chunks and the global queue
RACE_CASES = [
    (1, 8, 2048, 128, False, ("shift", "naive")),
    (1, 8, 2048, 128, True, ("descending", "symmetric_shift", "shift")),
    (2, 8, 1024, 64, True, ("symmetric_shift", "naive")),
]


@pytest.mark.parametrize("case", RACE_CASES, ids=lambda c: f"s{c[2]}-d{c[3]}-{'causal' if c[4] else 'full'}")
def test_injected_delays_keep_results_bitwise(case, debug_hooks):
    b, h, s, d, causal, scheds = case
    pb = Problem(b, h, s, d, "bf16", 9090 + s + d, causal)
    for sched in scheds:
        debug_hooks(0, 0, 0)
        ref = [t.clone() for t in pb.run(sched)]
        torch.cuda.synchronize()
        for seed in (1, 2, 0xdeadbeef):
            _say(f"race {case[:5]} {sched} seed {seed:#x}")
            debug_hooks(0, 0, seed)
            for place in ("xcd", "global"):
                tsa.attn_bwd_set_placement(place)
                try:
                    out = pb.run(sched)
                    torch.cuda.synchronize()
                finally:
                    tsa.attn_bwd_set_placement("xcd")
                assert tsa.attn_bwd_query_status() == 0, tsa.last_error()
                for a, b_ in zip(ref, out):
                    assert torch.equal(a.view(torch.int16), b_.view(torch.int16)), f"{sched} seed {seed} {place}"


@pytest.mark.parametrize("sched", ["naive", "shift"])
def test_expired_waits_report_timeout_and_next_call_is_clean(sched, debug_hooks):
    pb = Problem(1, 4, 1024, 128, "bf16", 31337, False)
    assert tsa.attn_bwd_query_status() == 0
    # every wait looks for a flag value nobody publishes; 64 polls each
    debug_hooks(64, 1000, 0)
    _say(f"timeout path {sched}")
    pb.run(sched)
    rc = tsa.attn_bwd_query_status()
    assert rc == -5, (rc, tsa.last_error())
    assert "expired" in tsa.last_error()
    # the status word was cleared by the query; a normal call is clean and right
    debug_hooks(0, 0, 0)
    g = pb.run(sched)
    torch.cuda.synchronize()
    assert tsa.attn_bwd_query_status() == 0, tsa.last_error()
    ref = pb.oracle([0, 3])
    for name, t in zip(("dq", "dk", "dv"), g):
        assert rel_err(to_np_heads(t, [0, 3]), ref[name]) <= TOL["bf16"], name




def test_wait_histogram_accounts_for_every_wait_cycle():
    """The per-(item, step) wait histogram sums exactly to the wait-cycle
    total of the same call, puts nothing on a rank-0 task (Shift's first
    task of every item is its Q tile's first contribution), and is cleared
    between calls."""
    pb = Problem(1, 8, 2048, 128, "bf16", 4242, False)
    tsa.attn_bwd_set_wait_stats(True)
    try:
        for _ in range(2):
            pb.run("shift")
            wait, item, polls = tsa.attn_bwd_get_wait_stats()
            hist = tsa.attn_bwd_get_wait_hist()
            assert tsa.attn_bwd_query_status() == 0, tsa.last_error()
            _say(f"wait {wait} of {item} cycles, {polls} polls")
            assert sum(map(sum, hist)) == wait
            assert all(row[0] == 0 for row in hist)
            assert all(v == 0 for row in hist[16:] for v in row)  # 16 items per head
    finally:
        tsa.attn_bwd_set_wait_stats(False)


def test_handoff_latency_measures_every_xcd_distance():
    """The hand-off probe runs its bounded ping-pong to the end between work
    group 0 and work groups 1..8 (every XCD distance, the last one on work
    group 0's XCD when the device deals groups to its XCDs in turn), and a
    64 KiB tile written through to memory costs more per turn than the flag
    alone."""
    seen = set()
    for pong in range(1, 9):
        flag_ns, a, b = tsa.attn_bwd_handoff_latency(pong, iters=200, mode=0)
        tile_ns, a2, b2 = tsa.attn_bwd_handoff_latency(pong, iters=200, mode=2)
        _say(f"pong {pong}: XCD {a} -> {b}: flag {flag_ns:.0f} ns, tile {tile_ns:.0f} ns")
        assert 0 <= a < 8 and 0 <= b < 8 and 0 < flag_ns < tile_ns < 1e6
        seen.add((b - a) % 8)
    assert len(seen) == 8
