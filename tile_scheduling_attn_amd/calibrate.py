"""Calibrate the DAG model's task costs on this GPU, then pick schedules.

    python tile_scheduling_attn_amd/calibrate.py [--steps K] [--tiles 128,64]
                                                 [--measure-only | --samples FILE | --handoff]

Times the main kernel of the backward for every (workload, mask, schedule)
below with the library's own launch-stream events (under the library's
default XCD placement), fits the model's compute and reduction costs c and r
and the edge cost e (a release reaching the next contributor on another XCD)
per head dimension with `attn_sched_fit` (the DAG of the review page's "What
carries the argument", with the kernel's XCD placement, simulator placement
2), fits the pages' model (e = 0) too, and prints one JSON document:
the fitted costs, measured against simulated makespan for every sample, and
the schedule
`attn_sched_select` picks for each shape.  `--measure-only` prints the
timings as JSON and stops (the fit is host work of a minute or two);
`--samples FILE` fits timings saved that way.  `--tiles 128,64` also times
every launch with 64-row tiles (attn_bwd_set_tile) and adds the tile
granularity check the review page asks for ("What would settle it"): the
costs fitted at 128 rows, scaled to 64 (a compute phase by its T^2 d MFMA
work, a reduction by its T d accumulator bytes), predict the 64-row
makespans, next to the measurements, a fit of their own, and the pages'
closed form m*n*(c+r) for the full-mask Shift launches.  `--handoff` measures
what the fit only infers: the latency of one dQ hand-off (flag, and flag
plus a 64 KiB tile) between work groups at every XCD distance.  Inputs are
seeded N(0, 1) Q, K, V,
dO with O and lse of the right scale; the kernel's running time does not
depend on the values.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))

# the simulator's model of the kernel's default work placement (per-XCD queues)
PLACEMENT = 2

# (workload name, causal, schedules timed)
PLAN = [
    ("s2k_d64_causal", True, ("naive", "descending", "shift", "symmetric_shift")),
    ("s8k_d128_full", False, ("naive", "descending", "shift")),
    ("s8k_d128_causal", True, ("naive", "descending", "shift", "symmetric_shift")),
    ("s16k_d128", False, ("naive", "shift")),
    ("s16k_d128", True, ("descending", "symmetric_shift")),
]


def inputs(wl, torch):
    g = torch.Generator(device="cuda").manual_seed(wl.seed)
    shape = (wl.b, wl.h, wl.s, wl.d)
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    q, k, v, o, do = (torch.randn(shape, generator=g, device="cuda", dtype=torch.float32).to(dt) for _ in range(5))
    # lse of the scale a softmax over s keys has: log(s) plus a small spread
    lse = (math.log(wl.s) + 0.1 * torch.randn(shape[:3], generator=g, device="cuda")).contiguous()
    return q, k, v, o, do, lse


def time_main(tsa, args, schedule, causal, steps, torch):
    q, k, v, o, do, lse = args
    out = [torch.empty_like(q) for _ in range(3)]
    for _ in range(2):
        tsa.backward(q, k, v, o, do, lse, causal, schedule, out=out)
    torch.cuda.synchronize()
    tsa.attn_bwd_set_timing(True)
    for _ in range(steps):
        tsa.backward(q, k, v, o, do, lse, causal, schedule, out=out)
    torch.cuda.synchronize()
    tsa.attn_bwd_set_timing(False)
    if tsa.attn_bwd_query_status() != 0:
        raise RuntimeError(tsa.last_error())
    return tsa.attn_bwd_get_kernel_times()[1]


def zero_edge_fit(tsa, ss):
    """The pages' model (e = 0): the best r/c on a log grid, c in closed form."""
    best = None
    for i in range(121):
        rho = 10 ** (-4 + 6 * i / 120)
        x = [tsa.attn_dagsim(n, causal, sched, heads, w, PLACEMENT, 1.0, rho)[0] / ms
             for n, causal, sched, heads, w, ms, _ in ss]
        c = sum(x) / sum(v * v for v in x)
        err = math.sqrt(sum((c * v - 1) ** 2 for v in x) / len(x))
        if best is None or err < best[3]:
            best = (c, c * rho, 0.0, err)
    return best


def parse_shapes(text):
    """'128,64,64x128' -> [(128, 128), (64, 64), (64, 128)] as (Br, Bc)."""
    out = []
    for tok in text.split(","):
        br, _, bc = tok.partition("x")
        out.append((int(br), int(bc or br)))
    return out


def measure(steps, shapes=((128, 128),)):
    import torch
    import tile_scheduling_attn_amd as tsa
    import workloads

    workers = torch.cuda.get_device_properties(0).multi_processor_count  # one work group per CU
    samples = []  # (n KV tiles, causal, schedule, heads, workers, ms, workload, d, Bc, Br)
    for name, causal, scheds in PLAN:
        wl = workloads.WORKLOADS[name]
        args = inputs(wl, torch)
        for br, bc in shapes:
            tsa.attn_bwd_set_tile_shape(wl.dtype, br, bc)
            try:
                n = -(-wl.s // bc)
                for sched in scheds:
                    ms = time_main(tsa, args, sched, causal, steps, torch)
                    print(f"{name} causal={causal} tile={br}x{bc} {sched}: {ms:.4f} ms", file=sys.stderr, flush=True)
                    samples.append((n, causal, sched, wl.b * wl.h, workers, ms, name, wl.d, bc, br))
            finally:
                tsa.attn_bwd_set_tile_shape(wl.dtype, 0, 0)
        del args
        torch.cuda.empty_cache()
    return samples


def granularity(tsa, samples, fits):
    """Tile granularity check: 64-row launches against the 128-row costs
    scaled to 64 rows, a fit of their own, and the closed form m*n*(c+r);
    64 x 128 launches (Br != Bc) against the 128-row costs scaled to them."""
    out = {}
    for d in sorted({s[7] for s in samples}):
        f = fits.get(f"d{d}")
        rect = [s for s in samples if s[7] == d and s[8] == 128 and s[9] == 64]
        if f and rect:
            c, r, e = f["c_us"] * 1e-3, f["r_us"] * 1e-3, f["e_us"] * 1e-3
            # a 64 x 128 task: half the matrix work and half the accumulator
            # bytes of a 128 x 128 one
            cr, rr = c / 2, r / 2
            rows = []
            for n, causal, sched, heads, w, ms, name, _, _, _ in rect:
                pred = tsa.attn_dagsim_rect(n, 2, causal, sched, heads, w, PLACEMENT, cr, rr, e)[0]
                row = {"workload": name, "causal": causal, "schedule": sched, "kv_tiles": n, "q_tiles": 2 * n,
                       "measured_ms": round(ms, 4), "scaled_model_ms": round(pred, 4)}
                sq = [x for x in samples if x[6] == name and x[1] == causal and x[2] == sched and x[8] == 128
                      and x[9] == 128]
                if sq:
                    row["measured_ms_128x128"] = round(sq[0][5], 4)
                if not causal and sched == "shift":
                    # total work per worker: heads * 2n^2 tasks of c/2 + r/2 over w workers
                    row["closed_form_ms"] = round(heads * 2 * n * n * (cr + rr) / w, 4)
                rows.append(row)
            rel = [abs(x["scaled_model_ms"] / x["measured_ms"] - 1) for x in rows]
            out[f"d{d}_64x128"] = {"scaled_costs_us": {"c": round(cr * 1e3, 4), "r": round(rr * 1e3, 4),
                                                       "e": round(e * 1e3, 4)},
                                   "scaled_model_rms_rel_err": round(math.sqrt(sum(x * x for x in rel) / len(rel)), 4),
                                   "samples": rows}
        s64 = [s for s in samples if s[7] == d and s[8] == 64]
        if not f or not s64:
            continue
        c, r, e = f["c_us"] * 1e-3, f["r_us"] * 1e-3, f["e_us"] * 1e-3
        c64, r64 = c * 0.25, r * 0.5
        cf, rf, ef, rms = tsa.attn_sched_fit([s[:6] for s in s64], placement=PLACEMENT)
        rows = []
        for n, causal, sched, heads, w, ms, name, _, _, _ in s64:
            pred = tsa.attn_dagsim_edge(n, causal, sched, heads, w, PLACEMENT, c64, r64, e)[0]
            row = {"workload": name, "causal": causal, "schedule": sched, "n": n, "measured_ms": round(ms, 4),
                   "scaled_model_ms": round(pred, 4)}
            t128 = [x for x in samples if x[6] == name and x[1] == causal and x[2] == sched and x[8] == 128]
            if t128:
                row["measured_ms_tile128"] = round(t128[0][5], 4)
            if not causal and sched == "shift":
                # the pages' closed form for n workers per head, m heads in turn,
                # spread over the resident work groups: m*n*(c+r) * n / workers
                row["closed_form_ms_tile64"] = round(heads * n * (c64 + r64) * n / w, 4)
                row["closed_form_ms_tile128"] = round(heads * (n // 2) * (c + r) * (n // 2) / w, 4)
            rows.append(row)
        rel = [abs(x["scaled_model_ms"] / x["measured_ms"] - 1) for x in rows]
        out[f"d{d}"] = {"scaled_costs_us": {"c": round(c64 * 1e3, 4), "r": round(r64 * 1e3, 4), "e": round(e * 1e3, 4)},
                        "scaled_model_rms_rel_err": round(math.sqrt(sum(x * x for x in rel) / len(rel)), 4),
                        "own_fit_us": {"c": round(cf * 1e3, 4), "r": round(rf * 1e3, 4), "e": round(ef * 1e3, 4),
                                       "rms_rel_err": round(rms, 4)},
                        "samples": rows}
    return out


def fit(samples):
    import tile_scheduling_attn_amd as tsa

    # older samples: no tile (128), or no Q tile (square)
    samples = [tuple(s) + ((128,) if len(s) < 9 else ()) for s in samples]
    samples = [tuple(s) + ((s[8],) if len(s) < 10 else ()) for s in samples]
    report = {"fits": {}}
    for d in sorted({s[7] for s in samples}):
        ss = [tuple(s[:7]) for s in samples if s[7] == d and s[8] == 128 and s[9] == 128]
        print(f"fitting d={d} ({len(ss)} samples)", file=sys.stderr, flush=True)
        c, r, e, rms = tsa.attn_sched_fit([s[:6] for s in ss], placement=PLACEMENT)
        c0, r0, _, rms0 = zero_edge_fit(tsa, ss)
        rows = []
        for n, causal, sched, heads, w, ms, name in ss:
            pred = tsa.attn_dagsim_edge(n, causal, sched, heads, w, PLACEMENT, c, r, e)[0]
            pred0 = tsa.attn_dagsim(n, causal, sched, heads, w, PLACEMENT, c0, r0)[0]
            rows.append({"workload": name, "causal": causal, "schedule": sched, "measured_ms": round(ms, 4),
                         "model_ms": round(pred, 4), "model_e0_ms": round(pred0, 4)})
        picks = {}
        for n, causal, _, heads, w, _, name in ss:
            key = f"{name} {'causal' if causal else 'full'}"
            if key not in picks:
                sel, t = tsa.attn_sched_select(n, causal, heads, w, c, r, e, placement=PLACEMENT)
                picks[key] = {"schedule": sel, "model_ms": round(t, 4)}
        report["fits"][f"d{d}"] = {"c_us": round(c * 1e3, 4), "r_us": round(r * 1e3, 4), "e_us": round(e * 1e3, 4),
                                   "rms_rel_err": round(rms, 4),
                                   "e0": {"c_us": round(c0 * 1e3, 4), "r_us": round(r0 * 1e3, 4),
                                          "rms_rel_err": round(rms0, 4)},
                                   "samples": rows, "selected": picks}
    if any(s[8] == 64 or s[9] != s[8] for s in samples):
        report["granularity"] = granularity(tsa, samples, report["fits"])
    return report


def handoff(iters=2000, reps=3):
    """Measured hand-off latency per XCD distance (attn_bwd_handoff_latency):
    for work group 0 and work groups 1..8, the nanoseconds per turn of the
    flag alone, of a 64 KiB tile written through to memory (the main
    kernel's hand-off between XCDs), and, when both groups share an XCD, of
    the tile through that XCD's L2 (its hand-off within an XCD); median of
    `reps` runs of `iters` turns."""
    import statistics
    import torch
    import tile_scheduling_attn_amd as tsa

    buf = torch.empty(int(tsa.lib.attn_bwd_handoff_bytes()) // 4, dtype=torch.float32, device="cuda")
    rows = []
    for pong in range(1, 9):
        row = {"pong": pong}
        for mode, key in ((0, "flag_ns"), (2, "tile_through_memory_ns"), (1, "tile_through_l2_ns")):
            runs = [tsa.attn_bwd_handoff_latency(pong, iters, mode, buf) for _ in range(reps)]
            row["xcd_ping"], row["xcd_pong"] = runs[0][1], runs[0][2]
            if mode == 1 and row["xcd_ping"] != row["xcd_pong"]:
                continue  # L2-scope hand-offs are only coherent within one XCD
            row[key] = round(statistics.median(r[0] for r in runs), 1)
        row["xcd_distance"] = (row["xcd_pong"] - row["xcd_ping"]) % 8
        print(json.dumps(row), file=sys.stderr, flush=True)
        rows.append(row)
    return {"iters": iters, "reps": reps, "rows": rows}


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--tiles", default="128",
                    help="comma list of bf16 tile shapes to time: 128, 64 (square) or 64x128 (Br x Bc)")
    g = ap.add_mutually_exclusive_group()
    g.add_argument("--measure-only", action="store_true")
    g.add_argument("--samples", metavar="FILE")
    g.add_argument("--handoff", action="store_true", help="measure the hand-off latency per XCD distance and stop")
    a = ap.parse_args()
    if a.handoff:
        print(json.dumps(handoff(), indent=1))
        return
    if a.samples:
        with open(a.samples) as f:
            samples = json.load(f)["samples"]
    else:
        samples = measure(a.steps, parse_shapes(a.tiles))
        if a.measure_only:
            print(json.dumps({"samples": samples}))
            return
    print(json.dumps(fit(samples), indent=1))


if __name__ == "__main__":
    main()
