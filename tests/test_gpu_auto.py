"""ATTN_SCHED_AUTO on the call path: on every workload it resolves to a
deterministic schedule, gives exactly that schedule's bits, and is (within
timing noise) the fastest of the deterministic schedules measured on the
device.  The review page ("If this is right") calls the schedules
complementary and has an implementation select one per configuration."""
import statistics
import sys

import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import tile_scheduling_attn_amd as tsa  # noqa: E402
import workloads  # noqa: E402
from support import Problem  # noqa: E402

DET = ("naive", "descending", "shift", "symmetric_shift")
# timing noise between back-to-back runs on one box stays within a few percent
MARGIN = 1.07


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _median_ms(pb, sched, calls=5):
    out = [torch.empty_like(pb.q) for _ in range(3)]
    for _ in range(2):
        pb.run(sched, out=out)
    times = []
    for _ in range(calls):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        pb.run(sched, out=out)
        b.record()
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    return statistics.median(times)


@pytest.mark.parametrize("name,causal", [("tiny", False), ("tiny", True), ("s2k_d64_causal", True),
                                         ("s8k_d128_full", False), ("s8k_d128_causal", True),
                                         ("s16k_d128", False), ("s16k_d128", True)])
def test_auto_resolves_to_the_fastest_schedule(name, causal):
    wl = workloads.WORKLOADS[name]
    pb = Problem(wl.b, wl.h, wl.s, wl.d, wl.dtype, wl.seed, causal)
    pick = tsa.attn_bwd_resolve_schedule(wl.b, wl.h, wl.s, wl.d, causal, wl.dtype)
    assert pick in DET
    # AUTO gives exactly the bits of the schedule it resolves to
    view = torch.int32 if wl.dtype == "fp32" else torch.int16
    a = pb.run("auto")
    b = pb.run(pick)
    torch.cuda.synchronize()
    assert tsa.attn_bwd_query_status() == 0, tsa.last_error()
    for x, y in zip(a, b):
        assert torch.equal(x.view(view), y.view(view))
    if name == "tiny":
        return  # microseconds: launch overhead, not the schedule, decides
    n = -(-wl.s // tsa.attn_bwd_tile_size(wl.dtype))
    times = {}
    for sched in DET:
        if sched == "symmetric_shift" and causal and n % 2:
            continue
        if sched == "symmetric_shift" and not causal:
            continue  # the same schedule as shift under the full mask
        times[sched] = _median_ms(pb, sched)
    best = min(times, key=times.get)
    _say(f"{name} causal={causal}: auto -> {pick}; measured ms {times}; fastest {best}")
    assert times[pick] <= MARGIN * times[best], (pick, times)
