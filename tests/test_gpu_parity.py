"""GPU parity of the HIP backward with the fp64 oracle, bitwise determinism,
and schedule invariance, through the C ABI.

Tolerance: per tensor, max|g_gpu - g_oracle| / max|g_oracle| <= 2e-2 for
bf16 inputs and 1e-4 for fp32 inputs.  The deterministic schedules must give
bitwise identical dQ, dK, dV over repeated runs (the pages report a maximum
run-to-run deviation of exactly 0 for deterministic kernels)."""
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import tile_scheduling_attn_amd as tsa  # noqa: E402
import workloads  # noqa: E402
from support import Problem, TOL, rel_err, record_error, to_np_heads  # noqa: E402

DET = ("naive", "descending", "shift", "symmetric_shift")


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _check_parity(pb, grads, heads, tag):
    # the oracle of one problem is the same for every schedule: computed once
    cache = pb.__dict__.setdefault("_oracle_cache", {})
    key = tuple(heads)
    if key not in cache:
        cache[key] = pb.oracle(heads)
    ref = cache[key]
    tol = TOL[pb.dtype]
    errs = {}
    for name, g in zip(("dq", "dk", "dv"), grads):
        errs[name] = rel_err(to_np_heads(g, heads), ref[name])
        record_error(tag, name, errs[name], tol)
    _say(f"{tag}: rel errs {errs}")
    for name, e in errs.items():
        assert e <= tol, f"{tag} {name}: {e} > {tol}"
    assert tsa.attn_bwd_query_status() == 0, tsa.last_error()


def _schedules_for(pb, names):
    out = []
    n = -(-pb.s // tsa.attn_bwd_tile_size(pb.dtype))
    for name in names:
        if name == "symmetric_shift" and pb.causal and n % 2:
            continue
        out.append(name)
    return out


# ---------------------------------------------------------------- small shapes
@pytest.mark.parametrize("causal", [False, True])
def test_tiny_fp32_all_schedules(causal):
    """b1 h1 s128 d64 fp32, 64x64 tiles (two tiles per side)."""
    wl = workloads.WORKLOADS["tiny"]
    pb = Problem(wl.b, wl.h, wl.s, wl.d, "fp32", wl.seed, causal)
    for sched in DET + ("atomic",):
        _say(f"tiny fp32 causal={causal} schedule={sched}")
        torch.cuda.synchronize()
        g = pb.run(sched)
        torch.cuda.synchronize()
        _check_parity(pb, g, range(pb.b * pb.h), f"tiny causal={causal} {sched}")


SMALL = [
    # b, h, s, d, dtype   (several tiles, ragged tails, both head dims)
    (1, 2, 512, 64, "bf16"),
    (2, 1, 384, 128, "bf16"),
    (1, 3, 200, 64, "bf16"),      # ragged: 200 = 128 + 72
    (1, 2, 300, 128, "bf16"),     # ragged: 3 tiles, last one 44 rows
    (1, 2, 500, 128, "bf16"),     # ragged, even tile count (causal Symmetric Shift at d=128)
    (1, 2, 130, 64, "fp32"),      # ragged fp32: 64 + 64 + 2
    (2, 2, 256, 128, "fp32"),
    (1, 1, 1, 64, "bf16"),        # a single row
    (1, 1, 64, 128, "bf16"),      # one partial tile
]


@pytest.mark.parametrize("shape", SMALL, ids=lambda x: "-".join(map(str, x)))
@pytest.mark.parametrize("causal", [False, True])
def test_small_shapes_all_schedules(shape, causal):
    b, h, s, d, dt = shape
    pb = Problem(b, h, s, d, dt, 1000 + s + d + b * 7 + h, causal)
    for sched in _schedules_for(pb, DET + ("atomic",)):
        _say(f"small {shape} causal={causal} schedule={sched}")
        g = pb.run(sched)
        torch.cuda.synchronize()
        _check_parity(pb, g, range(b * h), f"{shape} causal={causal} {sched}")


def test_symmetric_shift_odd_tile_count_is_rejected():
    pb = Problem(1, 1, 384, 64, "bf16", 5, True)  # 3 tiles
    with pytest.raises(tsa.AttnError) as e:
        pb.run("symmetric_shift")
    assert e.value.code == -2


# ---------------------------------------------------------------- configs
def _run_config(name, causal, schedules, heads=None, tag=""):
    wl = workloads.WORKLOADS[name]
    _say(f"config {name} causal={causal}: generating inputs")
    pb = Problem(wl.b, wl.h, wl.s, wl.d, wl.dtype, wl.seed, causal)
    H = wl.b * wl.h
    heads = sorted({0, H // 2, H - 1}) if heads == "sample" else (heads or range(H))
    results = {}
    for sched in _schedules_for(pb, schedules):
        _say(f"config {name} causal={causal} schedule={sched}")
        g = pb.run(sched)
        torch.cuda.synchronize()
        _check_parity(pb, g, heads, f"{name} causal={causal} {sched}")
        results[sched] = [t.clone() for t in g]
    return pb, results


def test_config_s2k_d64_causal():
    pb, res = _run_config("s2k_d64_causal", True, ("descending", "symmetric_shift", "naive", "atomic", "auto"))
    # NAIVE and DESCENDING share the dQ order: dQ is bitwise equal
    assert torch.equal(res["naive"][0].view(torch.int16), res["descending"][0].view(torch.int16))


def test_config_s8k_d128_full():
    pb, res = _run_config("s8k_d128_full", False, ("shift", "naive", "atomic", "auto"), heads="sample")


def test_config_s8k_d128_causal():
    _run_config("s8k_d128_causal", True, ("descending", "symmetric_shift", "atomic"), heads="sample")


@pytest.mark.parametrize("causal", [False, True])
def test_config_s16k_d128(causal):
    scheds = (("shift", "naive", "descending", "atomic") if not causal
              else ("descending", "symmetric_shift", "shift", "naive", "atomic"))
    pb, res = _run_config("s16k_d128", causal, scheds, heads="sample")
    # NAIVE and DESCENDING share the dQ order: dQ is bitwise equal
    assert torch.equal(res["naive"][0].view(torch.int16), res["descending"][0].view(torch.int16))


# ---------------------------------------------------------------- determinism
@pytest.mark.parametrize("name,causal,scheds", [
    ("tiny", False, DET),
    ("tiny", True, DET),
    ("s2k_d64_causal", True, ("descending", "symmetric_shift", "naive", "shift")),
    ("s8k_d128_full", False, ("shift", "naive")),
    ("s8k_d128_causal", True, ("symmetric_shift", "descending")),
    ("s16k_d128", False, ("shift", "naive")),
    ("s16k_d128", True, ("descending", "symmetric_shift")),
])
def test_bitwise_determinism_20_runs(name, causal, scheds):
    wl = workloads.WORKLOADS[name]
    pb = Problem(wl.b, wl.h, wl.s, wl.d, wl.dtype, wl.seed, causal)
    view = torch.int32 if wl.dtype == "fp32" else torch.int16
    for sched in scheds:
        _say(f"determinism {name} causal={causal} {sched}")
        ref = [t.clone() for t in pb.run(sched)]
        out = [torch.empty_like(t) for t in ref]
        for it in range(19):
            for t in out:
                t.fill_(float("nan"))
            pb.run(sched, out=out)
            torch.cuda.synchronize()
            for a, b_ in zip(ref, out):
                assert torch.equal(a.view(view), b_.view(view)), f"{sched} run {it + 1}"
        assert tsa.attn_bwd_query_status() == 0


@pytest.mark.parametrize("name,causal", [("s8k_d128_full", False), ("s8k_d128_causal", True)])
def test_atomic_run_to_run_deviation_is_reported(name, causal):
    """The non-deterministic variant may differ between runs (the summary
    page's Key results give ~2.4e-4 full / 4.9e-4 causal on unstated shapes);
    it must still meet the parity bar, which the config tests check.  Here
    the maximum deviation of dQ, dK and dV over 5 extra runs is recorded,
    raw and relative to max|g|; the deterministic schedules' is exactly 0
    (the 20-run tests)."""
    wl = workloads.WORKLOADS[name]
    pb = Problem(wl.b, wl.h, wl.s, wl.d, wl.dtype, wl.seed, causal)
    ref = [t.float() for t in pb.run("atomic")]
    dev = [0.0, 0.0, 0.0]
    for _ in range(5):
        out = pb.run("atomic")
        for i, (a, b_) in enumerate(zip(ref, out)):
            dev[i] = max(dev[i], float((a - b_.float()).abs().max()))
    for i, tname in enumerate(("dq", "dk", "dv")):
        rel = dev[i] / float(ref[i].abs().max())
        record_error(f"{name} causal={causal} atomic run-to-run max deviation (raw {dev[i]:.3e})", tname, rel, None)
        _say(f"atomic {tname} run-to-run max deviation: {dev[i]:.3e} (relative {rel:.3e})")
    assert dev[1] == 0.0 and dev[2] == 0.0  # dK, dV never go through the atomics


# ---------------------------------------------------------------- misc
def test_caller_workspace_and_stream_match_library_workspace():
    pb = Problem(1, 4, 640, 128, "bf16", 77, True)
    ref = [t.clone() for t in pb.run("descending")]
    nbytes = tsa.attn_bwd_workspace_bytes(1, 4, 640, 128, 1, "descending")
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        out = tsa.backward(pb.q, pb.k, pb.v, pb.o, pb.do, pb.lse, True, "descending", workspace=ws)
    st.synchronize()
    for a, b_ in zip(ref, out):
        assert torch.equal(a.view(torch.int16), b_.view(torch.int16))
    # the size the single global queue needs (no per-XCD accumulator copies)
    tsa.attn_bwd_set_placement("global")
    try:
        nglobal = tsa.attn_bwd_workspace_bytes(1, 4, 640, 128, 1, "descending")
    finally:
        tsa.attn_bwd_set_placement("xcd")
    assert nglobal <= nbytes
    # between the two: runs with the global queue, same bits
    mid = torch.empty(nglobal, dtype=torch.uint8, device="cuda")
    out = tsa.backward(pb.q, pb.k, pb.v, pb.o, pb.do, pb.lse, True, "descending", workspace=mid)
    for a, b_ in zip(ref, out):
        assert torch.equal(a.view(torch.int16), b_.view(torch.int16))
    small = torch.empty(nglobal - 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(tsa.AttnError) as e:
        tsa.backward(pb.q, pb.k, pb.v, pb.o, pb.do, pb.lse, True, "descending", workspace=small)
    assert e.value.code == -6


# (b, h, s, d, causal): shapes whose launches use XCD placement with 1, 2
# and 4 chunks per head and the global fallback (fewer than 8 items)
PLACEMENT_SHAPES = [(2, 8, 2048, 128, False), (1, 16, 4096, 64, True), (1, 4, 8192, 128, False),
                    (1, 2, 16384, 128, True), (2, 16, 1024, 64, True), (1, 1, 512, 64, False)]


@pytest.mark.parametrize("shape", PLACEMENT_SHAPES, ids=lambda x: "-".join(map(str, x)))
def test_xcd_and_global_placement_give_the_same_bits(shape):
    """The reduction order comes from the schedule alone: per-XCD queues with
    per-XCD accumulator copies (hand-offs within an XCD through its L2) and
    the single global queue give bitwise identical gradients, and no call
    reports a placement error."""
    b, h, s, d, causal = shape
    pb = Problem(b, h, s, d, "bf16", 4242, causal)
    for sched in _schedules_for(pb, DET):
        _say(f"placement {shape} {sched}")
        outs = {}
        for place in ("global", "xcd"):
            tsa.attn_bwd_set_placement(place)
            try:
                outs[place] = [t.clone() for t in pb.run(sched)]
            finally:
                tsa.attn_bwd_set_placement("xcd")
            assert tsa.attn_bwd_query_status() == 0, tsa.last_error()
        for a, b_ in zip(outs["global"], outs["xcd"]):
            assert torch.equal(a.view(torch.int16), b_.view(torch.int16)), f"{shape} {sched}"
    if s <= 8192:  # the oracle's s x s matrices stay small enough
        _check_parity(pb, outs["xcd"], [0, b * h - 1], f"placement {shape}")


@pytest.mark.parametrize("shape", [PLACEMENT_SHAPES[0], PLACEMENT_SHAPES[2], PLACEMENT_SHAPES[3]],
                         ids=lambda x: "-".join(map(str, x)))
def test_atomic_variant_matches_ordered_sum_within_one_rounding(shape):
    """The atomic variant adds the same fp32 partials as the naive order,
    only in an unordered sequence, so its dQ may differ from the naive
    schedule's by the reassociation error of the fp32 sum (tiny) plus one
    bf16 rounding step of the element: |a - n| <= 2^-7 max(|a|, |n|) +
    1e-5 max|n|.  A lost or doubled partial (an atomic that did not see
    another's update) moves an element by a whole partial, far beyond that.
    Its dK and dV come from the same per-tile accumulation in the same order
    as the naive schedule's: bitwise equal.  The placement switch only
    changes the deterministic schedules' queues; both settings are run."""
    b, h, s, d, causal = shape
    pb = Problem(b, h, s, d, "bf16", 5151, causal)
    ref = [t.clone() for t in pb.run("naive")]
    for place in ("xcd", "global"):
        _say(f"atomic vs naive {shape} placement {place}")
        tsa.attn_bwd_set_placement(place)
        try:
            out = [t.clone() for t in pb.run("atomic")]
        finally:
            tsa.attn_bwd_set_placement("xcd")
        assert tsa.attn_bwd_query_status() == 0, tsa.last_error()
        a, n_ = out[0].float(), ref[0].float()
        bound = 2.0 ** -7 * torch.maximum(a.abs(), n_.abs()) + 1e-5 * float(n_.abs().max())
        excess = float(((a - n_).abs() - bound).max())
        assert excess <= 0, f"{shape} {place}: atomic dQ off by more than one rounding ({excess})"
        for x, y in zip(out[1:], ref[1:]):
            assert torch.equal(x.view(torch.int16), y.view(torch.int16)), f"{shape} {place}"


def test_default_entry_point_bf16():
    pb = Problem(1, 2, 256, 64, "bf16", 91, False)
    dq, dk, dv = (torch.empty_like(pb.q) for _ in range(3))
    rc = tsa.attn_bwd_deterministic(pb.q, pb.k, pb.v, pb.o, pb.do, pb.lse, dq, dk, dv,
                                    1, 2, 256, 64, 0, "shift")
    assert rc == 0, tsa.last_error()
    torch.cuda.synchronize()
    _check_parity(pb, (dq, dk, dv), range(2), "default entry")


def test_kernel_timing_and_wait_stats():
    pb = Problem(1, 8, 2048, 128, "bf16", 3, False)
    tsa.attn_bwd_set_timing(True)
    tsa.attn_bwd_set_wait_stats(True)
    try:
        pb.run("naive")
        pre, main, fin = tsa.attn_bwd_get_kernel_times()
        wait, item, polls = tsa.attn_bwd_get_wait_stats()
    finally:
        tsa.attn_bwd_set_timing(False)
        tsa.attn_bwd_set_wait_stats(False)
    _say(f"timing pre={pre:.4f} main={main:.4f} fin={fin:.4f} ms; wait={wait} item={item} polls={polls}")
    assert main > 0 and pre > 0 and fin == 0
    assert item > 0 and polls > 0 and wait <= item


def test_gradient_identities_full_size():
    """sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i hold for the exact gradient
    (rows of P sum to one); on the bf16 outputs they hold to rounding."""
    wl = workloads.WORKLOADS["s8k_d128_full"]
    pb = Problem(1, 4, wl.s, wl.d, "bf16", 55, False)
    dq, dk, dv = pb.run("shift")
    torch.cuda.synchronize()
    sdk = dk.float().sum(dim=2)
    sdv = dv.float().sum(dim=2)
    sdo = pb.do.float().sum(dim=2)
    scale_dk = dk.float().abs().sum(dim=2).max()
    assert float(sdk.abs().max()) <= 2e-2 * float(scale_dk)
    assert float((sdv - sdo).abs().max()) <= 2e-2 * float(dv.float().abs().sum(dim=2).max())


def test_items_longer_than_one_record_block():
    """An item with more tasks than the kernel keeps in LDS at once (257 Q
    tiles of 64 rows, fp32, ragged tail): the records are reloaded mid-item.
    Shift with 257 KV tiles runs in two rounds of 129 (more KV tiles than the
    256 resident work groups)."""
    s = 257 * 64 - 40
    pb = Problem(1, 1, s, 64, "fp32", 4242, False)
    for sched in ("naive", "shift"):
        _say(f"long item fp32 s={s} {sched}")
        g = pb.run(sched)
        torch.cuda.synchronize()
        _check_parity(pb, g, [0], f"long item s={s} {sched}")
    assert tsa.attn_sched_min_workers(257, False, "shift") == 129


@pytest.mark.parametrize("causal", [False, True])
def test_shift_rounds_with_more_tiles_than_work_groups(causal):
    """bf16 with 257 KV tiles of 128 rows (s = 32896, more KV tiles than the
    256 resident work groups): Shift runs in two rounds; parity with the
    oracle, bitwise repeatable, and the same bits under both placements."""
    s = 257 * 128
    pb = Problem(1, 1, s, 64, "bf16", 2570 + causal, causal)
    _say(f"shift rounds s={s} causal={causal}")
    ref = [t.clone() for t in pb.run("shift")]
    torch.cuda.synchronize()
    assert tsa.attn_bwd_query_status() == 0, tsa.last_error()
    _check_parity(pb, ref, [0], f"shift rounds s={s} causal={causal}")
    for place in ("global", "xcd"):
        tsa.attn_bwd_set_placement(place)
        try:
            out = pb.run("shift")
            torch.cuda.synchronize()
        finally:
            tsa.attn_bwd_set_placement("xcd")
        for a, b_ in zip(ref, out):
            assert torch.equal(a.view(torch.int16), b_.view(torch.int16)), place
