#!/usr/bin/env python3
"""Benchmark of the deterministic attention backward on one MI355X.

A step is one call of the backward (preprocess D = rowsum(dO*O), the main
kernel with the ordered dQ reduction, and for the atomic variant the dQ
finalize) over the workload's synthetic inputs, which are resident in HBM
before timing starts.  The forward pass that produces O and lse runs once,
untimed.  Throughput uses the FlashAttention FLOP convention
(5 contractions x 2*s*s*d per head, halved under the causal mask).

Besides the headline workload (b2 h16 s8192 d128, full mask, the schedule
ATTN_SCHED_AUTO resolves to), every workload of the task's list is timed per
schedule: median, min and max over the timed calls of each (config,
schedule), % of the bf16 MFMA peak at the nominal 2.4 GHz and at the clock
the kernel actually ran at, and the ratio to the non-deterministic atomic
variant.  Those records go to stderr, one JSON object per line, and into the
headline line under "per_config".

Prints ONE JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA (2.4 GHz)
PEAK_FP32_MFMA_TFLOPS = 157.3
NOMINAL_MHZ = 2400.0
METRIC = "deterministic attn-bwd TFLOPS (bf16, 1 GPU) & % of MFMA peak; vs non-det"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_bwd_main_s8k_d128_full_shift.json")
# the backward kernel's source: its own file and the device helpers it includes
KERNEL_SOURCES = [os.path.join(ROOT, "tile_scheduling_attn_amd", "csrc", f)
                  for f in ("bwd_main.h", "bwd_kernels.hip", "attn_device.h")]
# (workload, mask) -> schedules timed for the per-config records
PER_CONFIG = [
    ("tiny", False, ("naive", "descending", "shift", "atomic")),
    ("tiny", True, ("naive", "descending", "shift", "symmetric_shift", "atomic")),
    ("s2k_d64_causal", True, ("descending", "symmetric_shift", "naive", "atomic")),
    ("s8k_d128_full", False, ("shift", "naive", "descending", "atomic")),
    ("s8k_d128_causal", True, ("descending", "symmetric_shift", "shift", "naive", "atomic")),
    ("s16k_d128", False, ("shift", "naive", "atomic")),
    ("s16k_d128", True, ("descending", "symmetric_shift", "atomic")),
]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_sha():
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def main_kernel_name(tsa, wl, causal, schedule):
    """The main kernel a call of this workload and schedule runs under the
    library's current settings (the library's own rule)."""
    k = tsa.attn_bwd_resolve_main_kernel(wl.d, causal, wl.dtype, schedule)
    return "bwd_pair_kernel" if k == "pair" else "bwd_main_kernel"


def traffic_per_launch(workload, schedule):
    """HBM bytes per launch of the main kernel from the committed rocprofv3
    PMC summary, if it was taken on the current kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != kernel_source_sha():
        return None
    if t.get("workload") != workload or t.get("schedule") != schedule:
        return None
    return t.get("hbm_bytes_per_launch")


def time_calls(tsa, pb, schedule, steps, warmup, torch):
    """`steps` timed calls after `warmup` untimed ones.  ms_per_step: events
    around all timed calls on the launch stream; per-call times (preprocess
    to the last kernel, and the main kernel alone) from the library's own
    HIP events on that stream."""
    out = [torch.empty_like(pb.q) for _ in range(3)]
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        pb.run(schedule, out=out)
    torch.cuda.synchronize()
    tsa.attn_bwd_set_timing(True)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record(stream)
    for _ in range(steps):
        pb.run(schedule, out=out)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    tsa.attn_bwd_set_timing(False)
    pre, main, fin = tsa.attn_bwd_get_kernel_times()
    totals, mains = tsa.attn_bwd_get_call_times(steps)
    rc = tsa.attn_bwd_query_status()
    if rc != 0:
        raise RuntimeError(f"device status {rc}: {tsa.last_error()}")
    return {"ms_per_step": start.elapsed_time(end) / steps, "wall_s": wall,
            "ms_preprocess": pre, "ms_main": main, "ms_finalize": fin,
            "call_ms": totals, "main_ms": mains}


def time_forward(tsa, pb, steps, torch):
    """The library's attention forward on the same inputs (context only: the
    forward is not part of the timed backward).  FLOP convention: 2
    contractions x 2*s*s*d per head, halved under the causal mask."""
    o, lse = torch.empty_like(pb.q), torch.empty_like(pb.lse)
    for _ in range(2):
        tsa.forward(pb.q, pb.k, pb.v, pb.causal, pb.scale, out=(o, lse))
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(steps):
        tsa.forward(pb.q, pb.k, pb.v, pb.causal, pb.scale, out=(o, lse))
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    flops = 4.0 * pb.b * pb.h * pb.s * pb.s * pb.d / (2 if pb.causal else 1)
    return {"ms": round(ms, 4), "tflops": round(flops / (ms * 1e-3) / 1e12, 2)}


def flag_wait_stats(tsa, pb, schedule, torch, hist_file=None):
    """One extra, untimed call with the kernel's wait counters on: the share of
    work-item cycles that work groups spent polling dQ flags for their turn,
    the task positions (steps of an item) where most of that waiting
    happened, and the shader clock the main kernel ran at.  hist_file: also
    write the whole (item mod 64, step) histogram there as JSON."""
    out = [torch.empty_like(pb.q) for _ in range(3)]
    tsa.attn_bwd_set_wait_stats(True)
    try:
        pb.run(schedule, out=out)
        wait, item, polls = tsa.attn_bwd_get_wait_stats()
        mhz = tsa.attn_bwd_get_clock()
        hist = tsa.attn_bwd_get_wait_hist()
    finally:
        tsa.attn_bwd_set_wait_stats(False)
    by_step = [sum(row[j] for row in hist) for j in range(len(hist[0]))]
    total = sum(by_step)
    top = sorted(range(len(by_step)), key=lambda j: -by_step[j])[:4]
    if hist_file:
        with open(hist_file, "w") as f:
            json.dump({"workload": f"b={pb.b} h={pb.h} s={pb.s} d={pb.d} causal={pb.causal}",
                       "schedule": schedule, "wait_cycles": wait, "item_cycles": item,
                       "rows": "work item of the head mod 64", "columns": "task position in the item (last: 127 or more)",
                       "cycles": hist}, f)
    return {"wait_cycles": wait, "item_cycles": item, "polls": polls,
            "fraction": round(wait / item, 5) if item else None, "clock_mhz": round(mhz, 1),
            "top_steps": {str(j): round(by_step[j] / total, 4) for j in top} if total else {}}


def cpu_baseline(pb, heads, flops_per_head):
    """The fp64 oracle backward (as it stands) on `heads` heads of the same
    workload, using the O and lse of the forward pass; backward stage only."""
    import oracle
    oracle.build(force=False)
    H = pb.b * pb.h
    sel = list(range(min(heads, H)))
    g = lambda x: x.reshape(H, pb.s, pb.d)[sel]
    o = pb.o.float().cpu().numpy().reshape(H, pb.s, pb.d)[sel]
    lse = pb.lse.cpu().numpy().reshape(H, pb.s)[sel]
    t0 = time.perf_counter()
    oracle.attn_bwd(g(pb.qn), g(pb.kn), g(pb.vn), o, g(pb.don), lse, pb.causal, pb.scale)
    dt = time.perf_counter() - t0
    return {"value": round(flops_per_head * len(sel) / dt / 1e12, 6), "unit": "TFLOPS",
            "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{len(sel)} of {H} heads (s={pb.s}, d={pb.d}, "
                      f"{'causal' if pb.causal else 'full'} mask), fp64 backward stage only, "
                      f"{dt:.1f} s; same FLOP convention"}


def config_records(tsa, torch, steps, warmup):
    """One record per (workload, mask, schedule) of the task's list."""
    import workloads
    from tests.support import Problem
    records = []
    for name, causal, scheds in PER_CONFIG:
        wl = workloads.WORKLOADS[name]
        pb = Problem(wl.b, wl.h, wl.s, wl.d, wl.dtype, wl.seed, causal)
        torch.cuda.synchronize()
        flops = wl.flops(causal)
        peak = PEAK_BF16_TFLOPS if wl.dtype == "bf16" else PEAK_FP32_MFMA_TFLOPS
        auto = tsa.attn_bwd_resolve_schedule(wl.b, wl.h, wl.s, wl.d, causal, wl.dtype)
        atomic_ms = None
        rows = []
        for sched in scheds:
            r = time_calls(tsa, pb, sched, steps, warmup, torch)
            waits = flag_wait_stats(tsa, pb, sched, torch)
            med = statistics.median(r["call_ms"])
            tfl = flops / (med * 1e-3) / 1e12
            clock = waits["clock_mhz"]
            rec = {"workload": name, "b": wl.b, "h": wl.h, "s": wl.s, "d": wl.d, "dtype": wl.dtype,
                   "causal": causal, "schedule": sched, "auto_pick": sched == auto, "calls": len(r["call_ms"]),
                   "ms_median": round(med, 4), "ms_min": round(min(r["call_ms"]), 4),
                   "ms_max": round(max(r["call_ms"]), 4),
                   "main_ms_median": round(statistics.median(r["main_ms"]), 4),
                   "tflops": round(tfl, 2), "pct_of_peak": round(100 * tfl / peak, 2),
                   "clock_mhz": clock,
                   "pct_of_peak_at_clock": round(100 * tfl / (peak * clock / NOMINAL_MHZ), 2) if clock else None,
                   "flag_wait_fraction": waits["fraction"],
                   "main_kernel": main_kernel_name(tsa, wl, causal, sched)}
            if sched == "atomic":
                atomic_ms = med
            rows.append(rec)
        for rec in rows:
            if atomic_ms and rec["schedule"] != "atomic":
                rec["det_over_nondet"] = round(atomic_ms / rec["ms_median"], 4)
            log(json.dumps(rec))
        records.extend(rows)
        del pb
        torch.cuda.empty_cache()
    return records


def atomic_roofline(tsa, torch, wl, causal, ms_main):
    """The ATOMIC variant's main kernel against the device's fp32 atomic-add
    throughput: the library's rate kernel makes as many adds, in the same
    pattern, into an accumulator of the same size."""
    tile = tsa.attn_bwd_tile_size(wl.dtype)
    n = -(-wl.s // tile)
    heads = wl.b * wl.h
    tasks = heads * (n * (n + 1) // 2 if causal else n * n)
    adds = tasks * tile * wl.d                     # one fp32 add per dQ element of each task
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    acc = torch.empty(heads * n * tile * wl.d, dtype=torch.float32, device="cuda")
    per_group = max(1, round(adds / (cus * 128 * 128)))
    ms, made = tsa.attn_bwd_atomic_rate(acc, per_group)
    del acc
    rate = made / (ms * 1e-3)
    achieved = adds / (ms_main * 1e-3)
    return {"bound": "fp32 atomic adds", "achieved_adds_per_s": float(f"{achieved:.4g}"),
            "peak_adds_per_s": float(f"{rate:.4g}"), "frac": round(achieved / rate, 4),
            "variant_adds": adds, "rate_kernel_adds": int(made), "rate_kernel_ms": round(ms, 4)}


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="s8k_d128_full")
    ap.add_argument("--causal", type=int, default=None, help="override the workload's mask")
    ap.add_argument("--schedule", default="auto", help="schedule of the headline (default: auto)")
    ap.add_argument("--compare", default="naive,atomic",
                    help="comma list of schedules also timed for context ('none' for none)")
    ap.add_argument("--per-config", type=int, default=1, help="time every workload and schedule (0: skip)")
    ap.add_argument("--cpu-heads", type=int, default=16, help="heads in the CPU oracle sample (0: skip)")
    ap.add_argument("--placement", default="xcd", choices=("xcd", "global"),
                    help="work placement of the deterministic kernel (per-XCD queues or one global queue)")
    ap.add_argument("--main-kernel", default="auto", choices=("auto", "four_wave", "pair"),
                    help="main kernel of deterministic bf16 128 x 128 calls (auto: pair under the causal mask at d = 128)")
    ap.add_argument("--wait-hist", metavar="FILE", default=None,
                    help="write the headline schedule's flag-wait histogram (item mod 64 x step) to FILE")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB five times (scales the HBM "
                         "traffic counters of a profiler run) and exit")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: heads are independent, so the path would shard "
              "by heads across GPUs without communication; the benchmark is a one-GPU measurement.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n * 4, "copy_calibration_bytes_written": n * 4,
                          "launches": 5}))
        return
    import tile_scheduling_attn_amd as tsa
    import workloads
    from tests.support import Problem

    tsa.attn_bwd_set_placement(args.placement)
    tsa.attn_bwd_set_main_kernel(args.main_kernel)
    wl = workloads.WORKLOADS[args.workload]
    causal = (wl.masks[0] == "causal") if args.causal is None else bool(args.causal)
    schedule = args.schedule
    if schedule == "auto":
        schedule = tsa.attn_bwd_resolve_schedule(wl.b, wl.h, wl.s, wl.d, causal, wl.dtype)
    log(f"workload {wl.name}: b={wl.b} h={wl.h} s={wl.s} d={wl.d} {wl.dtype} "
        f"{'causal' if causal else 'full'}; schedule {args.schedule} -> {schedule}")
    pb = Problem(wl.b, wl.h, wl.s, wl.d, wl.dtype, wl.seed, causal)
    torch.cuda.synchronize()
    flops = wl.flops(causal)

    res = time_calls(tsa, pb, args.schedule, args.steps, args.warmup, torch)
    tflops = flops / (res["ms_per_step"] * 1e-3) / 1e12
    main_tflops = flops / (res["ms_main"] * 1e-3) / 1e12
    log(f"{schedule}: {res['ms_per_step']:.3f} ms/step, {tflops:.1f} TFLOPS "
        f"(main kernel {res['ms_main']:.3f} ms, {main_tflops:.1f} TFLOPS)")

    extra = {}
    for other in [x for x in args.compare.split(",") if x and x not in (schedule, "none")]:
        if other == "symmetric_shift" and causal and (wl.s // 128) % 2:
            continue
        r2 = time_calls(tsa, pb, other, max(5, args.steps // 2), 2, torch)
        t2 = flops / (r2["ms_per_step"] * 1e-3) / 1e12
        extra[other] = {"ms_per_step": round(r2["ms_per_step"], 4), "tflops": round(t2, 2),
                        "ms_main": round(r2["ms_main"], 4)}
        log(f"{other}: {r2['ms_per_step']:.3f} ms/step, {t2:.1f} TFLOPS")

    if "atomic" in extra:
        extra["atomic"]["atomic_roofline"] = atomic_roofline(tsa, torch, wl, causal, extra["atomic"]["ms_main"])
        log(f"atomic variant: {extra['atomic']['atomic_roofline']}")

    peak = PEAK_BF16_TFLOPS if wl.dtype == "bf16" else PEAK_FP32_MFMA_TFLOPS
    roofline = {"bound": "mfma", "achieved": round(main_tflops, 2), "peak": peak,
                "unit": "TFLOP/s", "frac": round(main_tflops / peak, 4),
                "traffic": traffic_per_launch(wl.name, schedule),
                "kernel": main_kernel_name(tsa, wl, causal, schedule),
                "algorithmic_flop_per_launch": flops}

    fwd = time_forward(tsa, pb, max(5, args.steps // 2), torch)
    log(f"forward (context): {fwd['ms']:.3f} ms, {fwd['tflops']:.1f} TFLOPS")

    waits = flag_wait_stats(tsa, pb, schedule, torch, args.wait_hist)
    log(f"dQ flag waits: {waits['fraction']} of work-item cycles ({waits['polls']} polls); "
        f"clock {waits['clock_mhz']} MHz")

    cpu = None
    if args.cpu_heads > 0:
        log(f"timing the CPU oracle on {args.cpu_heads} head(s)")
        cpu = cpu_baseline(pb, args.cpu_heads, flops / (wl.b * wl.h))
        log(f"cpu oracle: {cpu['value']} TFLOPS on {cpu['cores']} threads")
    headline_ms = statistics.median(res["call_ms"])
    del pb
    torch.cuda.empty_cache()

    per_config = config_records(tsa, torch, args.steps, args.warmup) if args.per_config else []

    clock = waits["clock_mhz"]
    line = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic: Q,K,V,dO ~ N(0,1) (PCG64, seeded), O and lse from an fp32 forward",
        "config": {"workload": f"{wl.name}: b={wl.b} h={wl.h} s={wl.s} d={wl.d} "
                               f"{'causal' if causal else 'full'} mask, schedule {args.schedule} -> {schedule}",
                   "b": wl.b, "h": wl.h, "s": wl.s, "d": wl.d, "causal": causal,
                   "schedule": schedule, "schedule_requested": args.schedule,
                   "tile": tsa.attn_bwd_tile_size(wl.dtype), "placement": args.placement,
                   "main_kernel": roofline["kernel"]},
        "pct_of_peak": round(100 * tflops / peak, 2),
        "pct_of_peak_at_clock": round(100 * tflops / (peak * clock / NOMINAL_MHZ), 2) if clock else None,
        "clock_mhz": clock,
        "call_ms": {"median": round(headline_ms, 4), "min": round(min(res["call_ms"]), 4),
                    "max": round(max(res["call_ms"]), 4)},
        "kernel_ms": {"preprocess": round(res["ms_preprocess"], 4), "main": round(res["ms_main"], 4),
                      "finalize": round(res["ms_finalize"], 4)},
        "compare": extra,
        "roofline": roofline,
        "flag_wait": waits,
        "forward": fwd,
        "cpu_baseline": cpu,
        "per_config": per_config,
    }
    if "atomic" in extra:
        line["det_over_nondet"] = round(tflops / extra["atomic"]["tflops"], 4)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
