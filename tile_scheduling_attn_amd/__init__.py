"""Deterministic attention backward for MI355X (gfx950), scheduled with DASH.

Thin ctypes binding over libattn_bwd.so (C ABI in include/attn_bwd.h).  The
binding only marshals arguments: every step of the backward runs in the HIP
kernels of the library, and importing this package fails loudly if the
library is missing.  PyTorch is used only for device memory and streams.
"""
from __future__ import annotations

import ctypes
import math
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libattn_bwd.so")

SCHEDULES = {"naive": 0, "descending": 1, "shift": 2, "symmetric_shift": 3, "atomic": 4, "auto": 5}
DTYPES = {"bf16": 0, "fp32": 1}
STATUS = {0: "ATTN_OK", -1: "ATTN_ERR_INVALID_ARG", -2: "ATTN_ERR_UNSUPPORTED",
          -3: "ATTN_ERR_COSCHEDULE", -4: "ATTN_ERR_HIP", -5: "ATTN_ERR_TIMEOUT",
          -6: "ATTN_ERR_WORKSPACE", -7: "ATTN_ERR_DEADLOCK", -8: "ATTN_ERR_PLACEMENT",
          -9: "ATTN_ERR_INTERNAL"}

# every function declared in include/attn_bwd.h
EXPORTS = ("attn_fwd", "attn_bwd_deterministic", "attn_bwd_deterministic_ex", "attn_bwd_workspace_bytes",
           "attn_bwd_query_status", "attn_bwd_last_error", "attn_bwd_tile_size",
           "attn_bwd_set_timing", "attn_bwd_get_kernel_times", "attn_bwd_set_placement", "attn_bwd_set_wait_stats",
           "attn_bwd_get_wait_stats", "attn_sched_size", "attn_sched_get",
           "attn_sched_min_workers", "attn_dagsim", "attn_dagsim_edge", "attn_sched_select",
           "attn_sched_fit", "attn_bwd_get_call_times", "attn_bwd_get_clock", "attn_bwd_set_debug",
           "attn_bwd_resolve_schedule", "attn_bwd_deterministic_noalloc", "attn_bwd_noalloc_capacity",
           "attn_bwd_set_tile", "attn_bwd_atomic_rate", "attn_bwd_get_wait_hist",
           "attn_bwd_handoff_latency", "attn_bwd_handoff_bytes", "attn_sched_size_rect", "attn_sched_get_rect",
           "attn_sched_min_workers_rect", "attn_dagsim_rect", "attn_bwd_set_tile_shape", "attn_bwd_tile_shape",
           "attn_bwd_set_main_kernel", "attn_bwd_main_kernel", "attn_bwd_resolve_main_kernel")


class AttnError(RuntimeError):
    def __init__(self, code: int, where: str, msg: str):
        self.code = code
        super().__init__(f"{where}: {STATUS.get(code, code)}: {msg}")


def _load():
    # PyTorch ships its own HIP runtime (same soname as the system one).  Load
    # it first so that the library binds to the runtime that owns the
    # caller's tensors and streams instead of bringing up a second one.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python tile_scheduling_attn_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i, f, d, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_double, ctypes.c_size_t
    ip, dp = ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_double)
    ull = ctypes.POINTER(ctypes.c_ulonglong)
    fp = ctypes.POINTER(ctypes.c_float)
    lib.attn_fwd.argtypes = [vp] * 5 + [i] * 6 + [f, vp]
    lib.attn_fwd.restype = i
    lib.attn_bwd_deterministic.argtypes = [vp] * 9 + [i] * 6
    lib.attn_bwd_deterministic.restype = i
    lib.attn_bwd_deterministic_ex.argtypes = [vp] * 9 + [i] * 7 + [f, vp, sz, vp]
    lib.attn_bwd_deterministic_ex.restype = i
    lib.attn_bwd_workspace_bytes.argtypes = [i] * 6
    lib.attn_bwd_workspace_bytes.restype = sz
    lib.attn_bwd_query_status.argtypes = [vp]
    lib.attn_bwd_query_status.restype = i
    lib.attn_bwd_last_error.argtypes = []
    lib.attn_bwd_last_error.restype = ctypes.c_char_p
    lib.attn_bwd_tile_size.argtypes = [i]
    lib.attn_bwd_tile_size.restype = i
    lib.attn_bwd_set_timing.argtypes = [i]
    lib.attn_bwd_set_timing.restype = i
    lib.attn_bwd_get_kernel_times.argtypes = [fp, fp, fp]
    lib.attn_bwd_get_kernel_times.restype = i
    lib.attn_bwd_set_placement.argtypes = [i]
    lib.attn_bwd_set_placement.restype = i
    lib.attn_bwd_set_main_kernel.argtypes = [i]
    lib.attn_bwd_set_main_kernel.restype = i
    lib.attn_bwd_main_kernel.argtypes = []
    lib.attn_bwd_main_kernel.restype = i
    lib.attn_bwd_resolve_main_kernel.argtypes = [i, i, i, i]
    lib.attn_bwd_resolve_main_kernel.restype = i
    lib.attn_bwd_set_wait_stats.argtypes = [i]
    lib.attn_bwd_set_wait_stats.restype = i
    lib.attn_bwd_get_wait_stats.argtypes = [ull, ull, ull]
    lib.attn_bwd_get_wait_stats.restype = i
    lib.attn_sched_size.argtypes = [i, i, i, ip, ip]
    lib.attn_sched_size.restype = i
    lib.attn_sched_get.argtypes = [i, i, i, ip, ip, ip, ip, ip]
    lib.attn_sched_get.restype = i
    lib.attn_sched_min_workers.argtypes = [i, i, i]
    lib.attn_sched_min_workers.restype = i
    lib.attn_dagsim.argtypes = [i, i, i, i, i, i, d, d, dp, dp, dp]
    lib.attn_dagsim.restype = i
    lib.attn_dagsim_edge.argtypes = [i, i, i, i, i, i, d, d, d, dp, dp, dp]
    lib.attn_dagsim_edge.restype = i
    lib.attn_sched_select.argtypes = [i, i, i, i, i, d, d, d, ip, dp]
    lib.attn_sched_select.restype = i
    lib.attn_sched_fit.argtypes = [i, ip, ip, ip, ip, ip, i, dp, dp, dp, dp, dp]
    lib.attn_sched_fit.restype = i
    lib.attn_bwd_get_call_times.argtypes = [fp, fp, i, ip]
    lib.attn_bwd_get_call_times.restype = i
    lib.attn_bwd_get_clock.argtypes = [dp]
    lib.attn_bwd_get_clock.restype = i
    lib.attn_bwd_set_debug.argtypes = [ctypes.c_uint, i, ctypes.c_uint]
    lib.attn_bwd_set_debug.restype = i
    lib.attn_bwd_atomic_rate.argtypes = [vp, ctypes.c_size_t, i, vp, ctypes.POINTER(ctypes.c_float), dp]
    lib.attn_bwd_atomic_rate.restype = i
    lib.attn_bwd_get_wait_hist.argtypes = [ull]
    lib.attn_bwd_get_wait_hist.restype = i
    lib.attn_bwd_handoff_latency.argtypes = [vp, sz, i, i, i, vp, dp, ip, ip]
    lib.attn_bwd_handoff_latency.restype = i
    lib.attn_bwd_handoff_bytes.argtypes = []
    lib.attn_bwd_handoff_bytes.restype = sz
    lib.attn_sched_size_rect.argtypes = [i, i, i, i, ip, ip]
    lib.attn_sched_size_rect.restype = i
    lib.attn_sched_get_rect.argtypes = [i, i, i, i, ip, ip, ip, ip, ip]
    lib.attn_sched_get_rect.restype = i
    lib.attn_sched_min_workers_rect.argtypes = [i, i, i, i]
    lib.attn_sched_min_workers_rect.restype = i
    lib.attn_dagsim_rect.argtypes = [i, i, i, i, i, i, i, d, d, d, dp, dp, dp]
    lib.attn_dagsim_rect.restype = i
    lib.attn_bwd_set_tile_shape.argtypes = [i, i, i]
    lib.attn_bwd_set_tile_shape.restype = i
    lib.attn_bwd_tile_shape.argtypes = [i, ip, ip]
    lib.attn_bwd_tile_shape.restype = i
    lib.attn_bwd_resolve_schedule.argtypes = [i] * 6
    lib.attn_bwd_resolve_schedule.restype = i
    lib.attn_bwd_deterministic_noalloc.argtypes = [vp] * 9 + [i] * 7 + [f, vp]
    lib.attn_bwd_deterministic_noalloc.restype = i
    lib.attn_bwd_noalloc_capacity.argtypes = []
    lib.attn_bwd_noalloc_capacity.restype = sz
    lib.attn_bwd_set_tile.argtypes = [i, i]
    lib.attn_bwd_set_tile.restype = i
    return lib


lib = _load()


def last_error() -> str:
    return lib.attn_bwd_last_error().decode()


def _check(rc: int, where: str) -> int:
    if rc < 0:
        raise AttnError(rc, where, last_error())
    return rc


def _sched_id(schedule) -> int:
    if isinstance(schedule, str):
        return SCHEDULES[schedule]
    return int(schedule)


def _ptr(x) -> int:
    if x is None:
        return 0
    if isinstance(x, int):
        return x
    return int(x.data_ptr())


# ---------------------------------------------------------------------------
# C ABI, same names and arguments (pointers may be ints or tensors)
# ---------------------------------------------------------------------------
def attn_fwd(q, k, v, o, lse, b, h, s, d, causal, dtype, scale, stream) -> int:
    dt = DTYPES[dtype] if isinstance(dtype, str) else int(dtype)
    return lib.attn_fwd(*(_ptr(t) for t in (q, k, v, o, lse)), b, h, s, d, int(causal), dt, float(scale),
                        int(stream or 0))


def attn_bwd_deterministic(q, k, v, o, dO, lse, dq, dk, dv, b, h, s, d, causal, schedule) -> int:
    return lib.attn_bwd_deterministic(*(_ptr(t) for t in (q, k, v, o, dO, lse, dq, dk, dv)),
                                      b, h, s, d, int(causal), _sched_id(schedule))


def attn_bwd_deterministic_ex(q, k, v, o, dO, lse, dq, dk, dv, b, h, s, d, causal, schedule,
                              dtype, scale, workspace, workspace_bytes, stream) -> int:
    dt = DTYPES[dtype] if isinstance(dtype, str) else int(dtype)
    return lib.attn_bwd_deterministic_ex(*(_ptr(t) for t in (q, k, v, o, dO, lse, dq, dk, dv)),
                                         b, h, s, d, int(causal), _sched_id(schedule), dt,
                                         float(scale), _ptr(workspace), int(workspace_bytes),
                                         int(stream or 0))


def attn_bwd_deterministic_noalloc(q, k, v, o, dO, lse, dq, dk, dv, b, h, s, d, causal, schedule,
                                   dtype, scale, stream) -> int:
    dt = DTYPES[dtype] if isinstance(dtype, str) else int(dtype)
    return lib.attn_bwd_deterministic_noalloc(*(_ptr(t) for t in (q, k, v, o, dO, lse, dq, dk, dv)),
                                              b, h, s, d, int(causal), _sched_id(schedule), dt,
                                              float(scale), int(stream or 0))


def attn_bwd_noalloc_capacity() -> int:
    return lib.attn_bwd_noalloc_capacity()


def attn_bwd_workspace_bytes(b, h, s, d, causal, schedule) -> int:
    return lib.attn_bwd_workspace_bytes(b, h, s, d, int(causal), _sched_id(schedule))


def attn_bwd_query_status(stream=None) -> int:
    return lib.attn_bwd_query_status(int(stream or 0))


def attn_bwd_last_error() -> str:
    return last_error()


def attn_bwd_tile_size(dtype) -> int:
    return lib.attn_bwd_tile_size(DTYPES[dtype] if isinstance(dtype, str) else int(dtype))


def attn_bwd_set_tile(dtype, tile) -> None:
    """Tile edge of later bf16 calls: 128 (default, or 0) or 64."""
    dt = DTYPES[dtype] if isinstance(dtype, str) else int(dtype)
    _check(lib.attn_bwd_set_tile(dt, int(tile)), "attn_bwd_set_tile")


def attn_bwd_set_tile_shape(dtype, br, bc) -> None:
    """Q tile rows Br and KV tile rows Bc of later bf16 calls: (128, 128)
    (default, or (0, 0)), (64, 64) or (64, 128)."""
    dt = DTYPES[dtype] if isinstance(dtype, str) else int(dtype)
    _check(lib.attn_bwd_set_tile_shape(dt, int(br), int(bc)), "attn_bwd_set_tile_shape")


def attn_bwd_tile_shape(dtype):
    """(Br, Bc) of later calls in `dtype`."""
    dt = DTYPES[dtype] if isinstance(dtype, str) else int(dtype)
    br, bc = ctypes.c_int(), ctypes.c_int()
    _check(lib.attn_bwd_tile_shape(dt, ctypes.byref(br), ctypes.byref(bc)), "attn_bwd_tile_shape")
    return br.value, bc.value


def attn_bwd_set_timing(on: bool) -> int:
    return lib.attn_bwd_set_timing(int(bool(on)))


def attn_bwd_get_kernel_times():
    a, b_, c = ctypes.c_float(), ctypes.c_float(), ctypes.c_float()
    _check(lib.attn_bwd_get_kernel_times(ctypes.byref(a), ctypes.byref(b_), ctypes.byref(c)),
           "attn_bwd_get_kernel_times")
    return a.value, b_.value, c.value


PLACEMENTS = {"global": 0, "xcd": 1}


def attn_bwd_set_placement(mode) -> None:
    """Work placement of later deterministic calls: "xcd" (per-XCD queues,
    the default) or "global" (one queue)."""
    _check(lib.attn_bwd_set_placement(PLACEMENTS[mode] if isinstance(mode, str) else int(mode)),
           "attn_bwd_set_placement")


MAIN_KERNELS = {"four_wave": 0, "pair": 1, "auto": 2}


def attn_bwd_set_main_kernel(kernel) -> None:
    """Main kernel of later deterministic bf16 calls with 128 x 128 tiles:
    "four_wave", "pair" (eight waves, two per SIMD) or "auto" (the default:
    pair under the causal mask at d = 128); all give the same bits."""
    _check(lib.attn_bwd_set_main_kernel(MAIN_KERNELS[kernel] if isinstance(kernel, str) else int(kernel)),
           "attn_bwd_set_main_kernel")


def attn_bwd_resolve_main_kernel(d, causal, dtype="bf16", schedule="shift") -> str:
    """The main kernel ("four_wave" or "pair") a call with this head dimension,
    mask, element type and schedule runs under the current settings."""
    dt = DTYPES[dtype] if isinstance(dtype, str) else int(dtype)
    sc = SCHEDULES[schedule] if isinstance(schedule, str) else int(schedule)
    code = _check(lib.attn_bwd_resolve_main_kernel(int(d), int(bool(causal)), dt, sc), "attn_bwd_resolve_main_kernel")
    return {v: k for k, v in MAIN_KERNELS.items()}[code]


def attn_bwd_main_kernel() -> str:
    """The setting of attn_bwd_set_main_kernel ("four_wave", "pair" or "auto")."""
    code = lib.attn_bwd_main_kernel()
    return {v: k for k, v in MAIN_KERNELS.items()}[code]


def attn_bwd_set_wait_stats(on: bool) -> int:
    return lib.attn_bwd_set_wait_stats(int(bool(on)))


def attn_bwd_get_wait_stats():
    a, b_, c = ctypes.c_ulonglong(), ctypes.c_ulonglong(), ctypes.c_ulonglong()
    _check(lib.attn_bwd_get_wait_stats(ctypes.byref(a), ctypes.byref(b_), ctypes.byref(c)),
           "attn_bwd_get_wait_stats")
    return a.value, b_.value, c.value


def attn_bwd_get_call_times(max_calls=4096):
    """Per-call (total ms, main-kernel ms) lists of the current timing
    recording."""
    tot = (ctypes.c_float * max_calls)()
    mai = (ctypes.c_float * max_calls)()
    n = ctypes.c_int()
    _check(lib.attn_bwd_get_call_times(tot, mai, max_calls, ctypes.byref(n)), "attn_bwd_get_call_times")
    return list(tot[:n.value]), list(mai[:n.value])


def attn_bwd_resolve_schedule(b, h, s, d, causal, dtype="bf16") -> str:
    """Name of the schedule "auto" resolves to for this shape on the current device."""
    dt = DTYPES[dtype] if isinstance(dtype, str) else int(dtype)
    rc = _check(lib.attn_bwd_resolve_schedule(b, h, s, d, int(causal), dt), "attn_bwd_resolve_schedule")
    return {v: k for k, v in SCHEDULES.items()}[rc]


def attn_bwd_handoff_latency(pong: int, iters: int = 2000, mode: int = 0, buf=None):
    """Nanoseconds per dQ hand-off between work group 0 and work group
    `pong` (mode 0: flag only; 1: a 64 KiB tile through the XCD's L2; 2: the
    tile written through to memory), with the XCDs the two groups ran on:
    returns (ns, xcd_ping, xcd_pong)."""
    import torch
    if buf is None:
        buf = torch.empty(int(lib.attn_bwd_handoff_bytes()) // 4, dtype=torch.float32, device="cuda")
    ns, a, b = ctypes.c_double(), ctypes.c_int(), ctypes.c_int()
    stream = torch.cuda.current_stream().cuda_stream
    _check(lib.attn_bwd_handoff_latency(ctypes.c_void_p(buf.data_ptr()), buf.numel() * buf.element_size(), int(pong),
                                        int(iters), int(mode), ctypes.c_void_p(stream), ctypes.byref(ns),
                                        ctypes.byref(a), ctypes.byref(b)), "attn_bwd_handoff_latency")
    return ns.value, a.value, b.value


def attn_bwd_get_wait_hist():
    """Flag-wait cycles of the last call made with wait statistics on, as a
    64 x 128 nested list: [work item of the head mod 64][task position in
    the item, capped at 127]."""
    buf = (ctypes.c_ulonglong * (64 * 128))()
    _check(lib.attn_bwd_get_wait_hist(buf), "attn_bwd_get_wait_hist")
    return [list(buf[r * 128:(r + 1) * 128]) for r in range(64)]


def attn_bwd_get_clock() -> float:
    """Shader clock (MHz) of the last call made with wait statistics on."""
    mhz = ctypes.c_double()
    _check(lib.attn_bwd_get_clock(ctypes.byref(mhz)), "attn_bwd_get_clock")
    return mhz.value


def attn_bwd_atomic_rate(acc, tasks: int):
    """fp32 atomic adds per second in the ATOMIC variant's dQ pattern, on
    `acc` (a device float32 tensor of at least 64 KiB, overwritten) and the
    current stream: returns (ms of the timed launch, adds made)."""
    import torch
    if not _on_device(acc) or acc.dtype != torch.float32 or not acc.is_contiguous():
        raise AttnError(-1, "attn_bwd_atomic_rate", "acc must be a contiguous float32 device tensor")
    ms, adds = ctypes.c_float(), ctypes.c_double()
    stream = torch.cuda.current_stream().cuda_stream
    _check(lib.attn_bwd_atomic_rate(ctypes.c_void_p(acc.data_ptr()), acc.numel() * 4, int(tasks),
                                    ctypes.c_void_p(stream), ctypes.byref(ms), ctypes.byref(adds)),
           "attn_bwd_atomic_rate")
    return ms.value, adds.value


def attn_bwd_set_debug(spin_limit=0, wait_offset=0, delay_seed=0) -> None:
    """Test hooks: flag-wait poll limit (0: default), an offset that makes
    every wait unsatisfiable, and a seed for random delays before each
    reduction phase (0: off)."""
    _check(lib.attn_bwd_set_debug(int(spin_limit), int(wait_offset), int(delay_seed)), "attn_bwd_set_debug")


def attn_sched_size(n, causal, schedule):
    ni, nt = ctypes.c_int(), ctypes.c_int()
    _check(lib.attn_sched_size(n, int(causal), _sched_id(schedule), ctypes.byref(ni),
                               ctypes.byref(nt)), "attn_sched_size")
    return ni.value, nt.value


def attn_sched_get(n, causal, schedule):
    """Returns dict of NumPy int32 arrays: item_begin, task_kv, task_q, rank (n x n), count."""
    ni, nt = attn_sched_size(n, causal, schedule)
    out = {"item_begin": np.zeros(ni + 1, np.int32), "task_kv": np.zeros(nt, np.int32),
           "task_q": np.zeros(nt, np.int32), "rank": np.zeros((n, n), np.int32),
           "count": np.zeros(n, np.int32)}
    P = lambda a: a.ctypes.data_as(ctypes.POINTER(ctypes.c_int))
    _check(lib.attn_sched_get(n, int(causal), _sched_id(schedule), P(out["item_begin"]),
                              P(out["task_kv"]), P(out["task_q"]), P(out["rank"]),
                              P(out["count"])), "attn_sched_get")
    return out


def attn_sched_min_workers(n, causal, schedule) -> int:
    return _check(lib.attn_sched_min_workers(n, int(causal), _sched_id(schedule)),
                  "attn_sched_min_workers")


def attn_dagsim(n, causal, schedule, heads, workers, placement, c, r):
    """Returns (makespan, wait_time, busy_time); raises AttnError on deadlock."""
    m, w, b_ = ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
    _check(lib.attn_dagsim(n, int(causal), _sched_id(schedule), heads, workers, placement,
                           float(c), float(r), ctypes.byref(m), ctypes.byref(w), ctypes.byref(b_)),
           "attn_dagsim")
    return m.value, w.value, b_.value


def attn_dagsim_edge(n, causal, schedule, heads, workers, placement, c, r, e):
    """Returns (makespan, wait_time, busy_time); raises AttnError on deadlock."""
    m, w, b_ = ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
    _check(lib.attn_dagsim_edge(n, int(causal), _sched_id(schedule), heads, workers, placement, float(c),
                                float(r), float(e), ctypes.byref(m), ctypes.byref(w), ctypes.byref(b_)),
           "attn_dagsim_edge")
    return m.value, w.value, b_.value


def attn_sched_get_rect(n, ratio, causal, schedule):
    """Rectangular tiles: n KV tiles, ratio Q tiles per KV tile.  Returns
    dict of NumPy int32 arrays: item_begin, task_kv, task_q, rank
    (n x ratio*n), count (ratio*n)."""
    ni, nt = ctypes.c_int(), ctypes.c_int()
    _check(lib.attn_sched_size_rect(n, ratio, int(causal), _sched_id(schedule), ctypes.byref(ni), ctypes.byref(nt)),
           "attn_sched_size_rect")
    out = {"item_begin": np.zeros(ni.value + 1, np.int32), "task_kv": np.zeros(nt.value, np.int32),
           "task_q": np.zeros(nt.value, np.int32), "rank": np.zeros((n, ratio * n), np.int32),
           "count": np.zeros(ratio * n, np.int32)}
    P = lambda a: a.ctypes.data_as(ctypes.POINTER(ctypes.c_int))
    _check(lib.attn_sched_get_rect(n, ratio, int(causal), _sched_id(schedule), P(out["item_begin"]),
                                   P(out["task_kv"]), P(out["task_q"]), P(out["rank"]), P(out["count"])),
           "attn_sched_get_rect")
    return out


def attn_dagsim_rect(n, ratio, causal, schedule, heads, workers, placement, c, r, e=0.0):
    """attn_dagsim_edge for rectangular tiles.  Returns (makespan, wait_time,
    busy_time); raises AttnError on deadlock."""
    m, w, b_ = ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
    _check(lib.attn_dagsim_rect(n, ratio, int(causal), _sched_id(schedule), heads, workers, placement, float(c),
                                float(r), float(e), ctypes.byref(m), ctypes.byref(w), ctypes.byref(b_)),
           "attn_dagsim_rect")
    return m.value, w.value, b_.value


def attn_sched_select(n, causal, heads, workers, c, r, e=0.0, placement=1):
    """Returns (schedule name, simulated makespan).  placement as in
    attn_dagsim (1: one ticket queue, 2: the kernel's XCD placement)."""
    sch, ms = ctypes.c_int(), ctypes.c_double()
    _check(lib.attn_sched_select(n, int(causal), heads, workers, int(placement), float(c), float(r), float(e),
                                 ctypes.byref(sch), ctypes.byref(ms)), "attn_sched_select")
    name = {v: k for k, v in SCHEDULES.items()}[sch.value]
    return name, ms.value


def attn_sched_fit(samples, placement=1):
    """samples: iterable of (n, causal, schedule, heads, workers, measured).
    Returns (c, r, e, rms relative error) of the model with `placement`."""
    samples = list(samples)
    k = len(samples)
    I = ctypes.c_int * k
    cols = [I(*[int(s[0]) for s in samples]), I(*[int(bool(s[1])) for s in samples]),
            I(*[_sched_id(s[2]) for s in samples]), I(*[int(s[3]) for s in samples]),
            I(*[int(s[4]) for s in samples])]
    meas = (ctypes.c_double * k)(*[float(s[5]) for s in samples])
    c, r, e, rms = ctypes.c_double(), ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
    _check(lib.attn_sched_fit(k, *cols, int(placement), meas, ctypes.byref(c), ctypes.byref(r),
                              ctypes.byref(e), ctypes.byref(rms)), "attn_sched_fit")
    return c.value, r.value, e.value, rms.value


# ---------------------------------------------------------------------------
# Torch convenience wrapper (allocation and stream only)
# ---------------------------------------------------------------------------
def _on_device(t) -> bool:
    """Whether a tensor lives in device memory (the kernels dereference every
    pointer on the GPU)."""
    return bool(t.is_cuda)


def _require(t, name, shape, dtype, device):
    """Raise ValueError unless `t` is a contiguous device tensor of `shape`
    and `dtype` on `device`: a wrong size, type or placement would make the
    kernels read or write outside the tensor."""
    if t is None:
        raise ValueError(f"{name} is missing")
    if not _on_device(t) or t.device != device:
        raise ValueError(f"{name} must be a device tensor on {device}, got {t.device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must have dtype {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _require_inputs(q, names_tensors):
    import torch
    if q.dim() != 4:
        raise ValueError(f"q must be [b, h, s, d], got shape {tuple(q.shape)}")
    if q.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("q must be bfloat16 or float32")
    if not _on_device(q):
        raise ValueError("q must be a device tensor")
    for name, t in names_tensors:
        _require(t, name, q.shape, q.dtype, q.device)


def _require_workspace(workspace, device):
    """A caller workspace: contiguous device memory on `device`; returns
    (pointer, bytes)."""
    if workspace is None:
        return 0, 0
    if not _on_device(workspace) or workspace.device != device:
        raise ValueError(f"workspace must be a device tensor on {device}")
    if not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    return workspace.data_ptr(), workspace.numel() * workspace.element_size()


def forward(q, k, v, causal: bool, scale=None, out=None, stream=None):
    """Attention forward on torch tensors [b, h, s, d] (bf16 or fp32,
    contiguous, on the current HIP device).  Returns (o, lse) with lse
    [b, h, s] fp32, allocated unless `out` gives them.  Asynchronous on
    `stream` (default: torch's current stream)."""
    import torch
    _require_inputs(q, (("q", q), ("k", k), ("v", v)))
    b, h, s, d = q.shape
    dtype = {torch.bfloat16: "bf16", torch.float32: "fp32"}[q.dtype]
    if out is None:
        out = (torch.empty_like(q), torch.empty((b, h, s), dtype=torch.float32, device=q.device))
    o, lse = out
    _require(o, "out[0] (o)", q.shape, q.dtype, q.device)
    _require(lse, "out[1] (lse)", (b, h, s), torch.float32, q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    _check(attn_fwd(q, k, v, o, lse, b, h, s, d, causal, dtype, scale, stream), "attn_fwd")
    return o, lse


def backward(q, k, v, o, do, lse, causal: bool, schedule="shift", scale=None, out=None,
             workspace=None, stream=None):
    """Run the backward on torch tensors [b, h, s, d] (bf16 or fp32, contiguous,
    on the current HIP device) with lse [b, h, s] fp32.  Returns (dq, dk, dv),
    allocated unless `out` gives them.  The call is asynchronous on `stream`
    (default: torch's current stream)."""
    import torch
    _require_inputs(q, (("q", q), ("k", k), ("v", v), ("o", o), ("do", do)))
    b, h, s, d = q.shape
    _require(lse, "lse", (b, h, s), torch.float32, q.device)
    dtype = {torch.bfloat16: "bf16", torch.float32: "fp32"}[q.dtype]
    if out is None:
        out = (torch.empty_like(q), torch.empty_like(q), torch.empty_like(q))
    dq, dk, dv = out
    for name, t in (("out[0] (dq)", dq), ("out[1] (dk)", dk), ("out[2] (dv)", dv)):
        _require(t, name, q.shape, q.dtype, q.device)
    ws_ptr, ws_bytes = _require_workspace(workspace, q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    rc = attn_bwd_deterministic_ex(q, k, v, o, do, lse, dq, dk, dv, b, h, s, d, causal, schedule,
                                   dtype, scale, ws_ptr, ws_bytes, stream)
    _check(rc, "attn_bwd_deterministic_ex")
    return dq, dk, dv
