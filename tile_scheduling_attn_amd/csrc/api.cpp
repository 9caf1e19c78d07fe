// C ABI of libattn_bwd.so: argument checks, workspace, cached device
// schedule tables and the launch of the backward kernels.  The functions
// are declared, with their contracts, in include/attn_bwd.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <tuple>
#include <vector>

#include "attn_bwd.h"
#include "internal.h"

namespace attn {

static thread_local std::string g_last_error;

int fail(int code, const char* msg) {
    g_last_error = msg ? msg : "";
    return code;
}

int fail_internal(const char* msg) noexcept {
    try {
        g_last_error = msg;
    } catch (...) {
        g_last_error.clear();
    }
    return ATTN_ERR_INTERNAL;
}

static int fail_hip(hipError_t e, const char* what) {
    g_last_error = std::string(what) + ": " + hipGetErrorString(e);
    return ATTN_ERR_HIP;
}

constexpr size_t kAlign = 256;
constexpr size_t kHandoffBytes = 256 + 2 * 65536;  // flag words, then two 64 KiB tiles
constexpr int kPadRows = 128;     // s is padded to a multiple of this
constexpr int kMinTile = 64;      // smallest tile: bounds the flag count
constexpr int kCounterWords = 64; // ticket + wait statistics
// wait histogram (when wait statistics are on): u64 wait cycles per
// (item of the head mod kHistItems, task position in the item, capped)
constexpr int kHistItems = 64, kHistSteps = 128;
// Accepted sizes: s up to kMaxTiles tiles of the largest tile edge (128), and
// b*h within an int (the kernels index heads with ints).
constexpr int kMaxSeq = kMaxTiles * 128;
constexpr long long kMaxHeads = (1LL << 31) - 1;

static size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct WsLayout {
    size_t s_pad, acc, delta, flags, counters, hist, total;
    int nflags;
};

// acc_heads: heads of fp32 accumulator (H, or kQueues copies of an XCD
// plan's slots)
static bool ws_layout(long long H, long long s, int d, long long acc_heads, WsLayout& w) {
    if (H < 0 || s < 0 || (d != 64 && d != 128)) return false;
    w.s_pad = (size_t)((s + kPadRows - 1) / kPadRows) * kPadRows;
    const size_t nmax = w.s_pad / kMinTile;
    w.nflags = (int)(H * nmax);
    w.acc = 0;
    w.delta = align_up(w.acc + (size_t)acc_heads * w.s_pad * d * sizeof(float));
    // D, then lse * log2(e), [H][s_pad] each
    w.flags = align_up(w.delta + 2 * (size_t)H * w.s_pad * sizeof(float));
    w.counters = align_up(w.flags + (size_t)w.nflags * sizeof(unsigned));
    w.hist = align_up(w.counters + kCounterWords * sizeof(unsigned));
    w.total = align_up(w.hist + (size_t)kHistItems * kHistSteps * sizeof(unsigned long long));
    return true;
}

struct DevSchedule {
    // item_begin (items+1 ints, padded to a multiple of 4) | one 16-byte
    // record per task: {kv tile, q tile, rank, item of the q tile's next
    // contributor or -1 for its last}
    int* buf = nullptr;           // device copy (null until uploaded)
    std::vector<int> table;       // host copy of the same
    int items = 0, tasks = 0, n = 0, min_workers = 1;
    std::vector<int> item_begin;  // host copy
};

struct DevState {
    bool init = false;
    int num_cus = 0;
    bool xcd_ok = false;  // work group b runs on XCD b % kQueues
    void* ws = nullptr;
    size_t ws_bytes = 0;
    // the library workspace is shared by every call on the device: a call on
    // another stream than the previous user first waits for its completion
    hipEvent_t ws_done = nullptr;
    void* ws_stream = nullptr;
    bool ws_used = false;
    unsigned* status = nullptr;
    std::map<std::tuple<int, int, int, int>, DevSchedule> schedules;
    // ATTN_SCHED_AUTO: the schedule picked per (n, causal, heads, d, dtype)
    std::map<std::tuple<int, int, long long, int, int>, int> auto_pick;
    // kernel timing: 4 events per recorded call (before preprocess, before
    // main, after main, after finalize)
    std::vector<hipEvent_t> ev_pool;
    std::vector<char> ev_finalize;   // per recorded call: finalize launched
    size_t ev_used = 0;
    void* last_counters = nullptr;
    void* last_hist = nullptr;
    bool stats_valid = false;
};

constexpr size_t kMaxTimedCalls = 4096;

std::mutex g_mutex;
static std::map<int, DevState> g_dev;
static bool g_timing = false;
static bool g_wait_stats = false;
static bool g_xcd_placement = true;
static std::atomic<int> g_main_kernel{ATTN_KERNEL_AUTO};
static int g_last_dev = -1;
// test hooks (attn_bwd_set_debug)
static unsigned g_spin_limit = 0;
static int g_wait_offset = 0;
static unsigned g_delay_seed = 0;

// First use of a device: its CU count, the device status word (a device
// variable of the library, so no allocation) and the XCD dispatch probe
// (into `probe_buf` when given, else a buffer of its own).
static int dev_init(int dev, DevState& ds, void* probe_buf = nullptr) {
    if (ds.init) return ATTN_OK;
    hipDeviceProp_t prop;
    hipError_t e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return fail_hip(e, "hipGetDeviceProperties");
    ds.num_cus = prop.multiProcessorCount;
    int rc = status_word_address(&ds.status);
    if (rc != ATTN_OK) return rc;
    e = hipMemset(ds.status, 0, sizeof(unsigned));
    if (e != hipSuccess) return fail_hip(e, "hipMemset(status)");
    if (!probe_buf || 16 * (size_t)ds.num_cus <= kNoAllocProbeBytes) {
        rc = probe_xcd_dispatch(ds.num_cus, &ds.xcd_ok, static_cast<unsigned*>(probe_buf));
        if (rc != ATTN_OK) return rc;
    }
    ds.init = true;
    return ATTN_OK;
}

// The schedule tables of (n, mask, schedule), built once per device and
// cached; `upload` also makes the device copy (an allocation).
// n KV tiles, `ratio` Q tiles per KV tile.
static int get_schedule(DevState& ds, int n, int ratio, bool causal, int schedule, DevSchedule** out,
                        bool upload = true) {
    auto key = std::make_tuple(n, ratio, (int)causal, schedule);
    auto it = ds.schedules.find(key);
    if (it != ds.schedules.end()) {
        DevSchedule& d = it->second;
        if (upload && !d.buf) {
            hipError_t e = hipMalloc(&d.buf, d.table.size() * sizeof(int));
            if (e != hipSuccess) {
                d.buf = nullptr;
                return fail_hip(e, "hipMalloc(schedule)");
            }
            e = hipMemcpy(d.buf, d.table.data(), d.table.size() * sizeof(int), hipMemcpyHostToDevice);
            if (e != hipSuccess) return fail_hip(e, "hipMemcpy(schedule)");
        }
        *out = &d;
        return ATTN_OK;
    }
    Schedule sc;
    int rc = build_schedule(n, causal, schedule, sc, ratio);
    if (rc == ATTN_ERR_UNSUPPORTED)
        return fail(rc, "unsupported schedule shape (symmetric shift under the causal mask needs an even number of "
                        "KV tiles; rectangular tiles allow at most 256 KV tiles under Shift and 2048 Q tiles)");
    if (rc != ATTN_OK) return fail(rc, "invalid schedule");
    const int nq = sc.nq;
    std::vector<int> host(sc.item_begin.begin(), sc.item_begin.end());
    host.resize((host.size() + 3) / 4 * 4, 0);
    // item that makes contribution `rank` to Q tile q: item_of[q * n + rank]
    std::vector<int> item_of((size_t)nq * n, -1);
    for (int it = 0; it < sc.num_items(); ++it)
        for (int t = sc.item_begin[it]; t < sc.item_begin[it + 1]; ++t) {
            const int r = sc.rank[(size_t)sc.task_kv[t] * nq + sc.task_q[t]];
            if (r >= 0) item_of[(size_t)sc.task_q[t] * n + r] = it;
        }
    for (size_t t = 0; t < sc.task_kv.size(); ++t) {
        const int kv = sc.task_kv[t], q = sc.task_q[t];
        const int r = sc.rank[(size_t)kv * nq + q];
        host.push_back(kv);
        host.push_back(q);
        host.push_back(r);
        host.push_back(r >= 0 && r + 1 < sc.count[q] ? item_of[(size_t)q * n + r + 1] : -1);
    }
    DevSchedule d;
    if (upload) {
        hipError_t e = hipMalloc(&d.buf, host.size() * sizeof(int));
        if (e != hipSuccess) return fail_hip(e, "hipMalloc(schedule)");
        e = hipMemcpy(d.buf, host.data(), host.size() * sizeof(int), hipMemcpyHostToDevice);
        if (e != hipSuccess) {
            (void)hipFree(d.buf);
            return fail_hip(e, "hipMemcpy(schedule)");
        }
    }
    d.table = std::move(host);
    d.items = sc.num_items();
    d.item_begin = sc.item_begin;
    d.tasks = (int)sc.task_kv.size();
    d.n = nq;
    d.min_workers = min_workers(sc);
    auto res = ds.schedules.emplace(key, d);
    *out = &res.first->second;
    return ATTN_OK;
}

// Tile shape of later bf16 calls (attn_bwd_set_tile, attn_bwd_set_tile_shape):
// Q tile rows Br in the high half, KV tile rows Bc in the low half; 128 x 128
// by default, or 64 x 64, or 64 x 128.  fp32 runs 64 x 64.
static std::atomic<int> g_shape_bf16{(128 << 16) | 128};
struct TileShape {
    int br, bc;
    int ratio() const { return bc / br; }
};
static TileShape shape_for(int dtype) {
    if (dtype == ATTN_FP32) return {64, 64};
    const int v = g_shape_bf16.load();
    return {v >> 16, v & 0xffff};
}
static int tile_for(int dtype) { return shape_for(dtype).bc; }

// Task costs of the DAG model fitted to the main kernels on MI355X
// (microseconds per compute phase c and reduction phase r, and per reduction
// hand-off e between XCDs; simulator placement 2), per head dimension and
// tile edge.  The 128 x 128 fits come from launches with the default kernel
// choice (the pair kernel under the causal mask at d = 128).
// Each tile edge has a fit of its own: scaling the 128-row costs to 64 rows
// (c by the T^2 d matrix work, r by the T d accumulator bytes) predicts the
// 64-row makespans 30-50% short, because at 64 rows the ordered dQ traffic
// and the flag hand-offs, not the matrix work, set the pace.  fp32 (64-row
// tiles only) takes the bf16 64-row costs: only their ratios matter here.
struct FittedCosts {
    double c, r, e;
};
static FittedCosts fitted_costs(int d, TileShape t) {
    if (t.bc == 64) return d == 64 ? FittedCosts{0.385, 1.859, 0.0} : FittedCosts{0.889, 3.206, 0.348};
    const FittedCosts f = d == 64 ? FittedCosts{3.144, 2.358, 0.0} : FittedCosts{3.430, 3.430, 3.022};
    // 64-row Q tiles against 128-row KV tiles: half the matrix work and half
    // the accumulator bytes of a square task (no fit of their own)
    if (t.br != t.bc) return {f.c * t.br / t.bc, f.r * t.br / t.bc, f.e};
    return f;
}

// ATTN_SCHED_AUTO.  The review page ("If this is right") has an
// implementation select one of the complementary schedules per
// configuration; here the DAG model with the fitted costs and the kernel's
// XCD placement simulates every deterministic schedule the shape admits on
// the device's resident work groups and takes the shortest makespan.
static int resolve_auto(DevState& ds, int n, bool causal, long long H, int d, int dtype, int* out) {
    const TileShape shape = shape_for(dtype);
    const auto key = std::make_tuple(n, (int)causal, H, d, (dtype * 1000 + shape.br) * 1000 + shape.bc);
    auto it = ds.auto_pick.find(key);
    if (it != ds.auto_pick.end()) {
        *out = it->second;
        return ATTN_OK;
    }
    const FittedCosts fc = fitted_costs(d, shape);
    const int workers = std::max(1, ds.num_cus);
    const int heads = (int)std::min<long long>(H, 1 << 20);
    int pick = -1;
    double best = 0;
    for (int sc : {ATTN_SCHED_NAIVE, ATTN_SCHED_DESCENDING, ATTN_SCHED_SHIFT, ATTN_SCHED_SYMMETRIC_SHIFT}) {
        Schedule sch;
        if (build_schedule(n, causal, sc, sch, shape.ratio()) != ATTN_OK) continue;
        if (min_workers(sch) > workers) continue;
        // large problems: simulate a head count that keeps the simulation
        // small but fills every worker several times (the makespan per head
        // is what is compared)
        const long long per_head = (long long)sch.task_kv.size();
        int hs = heads;
        while (hs > 8 && (long long)hs * per_head > (1LL << 22)) hs /= 2;
        double t = 0;
        if (simulate(sch, hs, workers, 2, fc.c, fc.r, fc.e, &t, nullptr, nullptr) != ATTN_OK) continue;
        if (pick < 0 || t < best * (1 - 1e-9)) {
            pick = sc;
            best = t;
        }
    }
    if (pick < 0) return fail(ATTN_ERR_COSCHEDULE, "no deterministic schedule fits the resident work groups");
    ds.auto_pick[key] = pick;
    *out = pick;
    return ATTN_OK;
}

// XCD placement of a deterministic call, planned for one resident work group
// per CU (the main kernel's LDS allows no more; a launch with more resident
// work groups only has more per queue)
static XcdPlan placement_plan(const DevState& ds, const DevSchedule& sch, int schedule, long long H) {
    if (schedule == ATTN_SCHED_ATOMIC || !g_xcd_placement || !ds.xcd_ok) return XcdPlan{};
    return xcd_plan(sch.item_begin, sch.min_workers, std::min<long long>(ds.num_cus, H * sch.items), H);
}

// One backward call.  `na` (the no-allocation entry point): every device
// buffer comes from that area (XCD probe at its start, the schedule table,
// then the workspace), the single global queue is used, no kernel timing is
// recorded, and nothing is allocated.
int backward(const void* q, const void* k, const void* v, const void* o, const void* dO,
             const float* lse, void* dq, void* dk, void* dv, int b, int h, int s, int d,
             int causal, int schedule, int dtype, float scale, void* workspace,
             size_t workspace_bytes, void* stream, const NoAllocArea* na) {
    g_last_error.clear();
    if (b < 0 || h < 0 || s < 0) return fail(ATTN_ERR_INVALID_ARG, "b, h and s must be >= 0");
    if (causal != 0 && causal != 1) return fail(ATTN_ERR_INVALID_ARG, "causal must be 0 or 1");
    if (schedule < ATTN_SCHED_NAIVE || schedule > ATTN_SCHED_AUTO)
        return fail(ATTN_ERR_INVALID_ARG, "unknown schedule");
    if (dtype != ATTN_BF16 && dtype != ATTN_FP32) return fail(ATTN_ERR_INVALID_ARG, "unknown dtype");
    if (!std::isfinite(scale) || !(scale > 0))
        return fail(ATTN_ERR_INVALID_ARG, "scale must be a positive finite number");
    if (d != 64 && d != 128) return fail(ATTN_ERR_UNSUPPORTED, "head dimension must be 64 or 128");
    const long long H = (long long)b * h;
    if (H == 0 || s == 0) return ATTN_OK;
    if (s > kMaxSeq) return fail(ATTN_ERR_UNSUPPORTED, "sequence length above 262144 is not supported");
    if (H > kMaxHeads || H * (long long)s * d >= (1LL << 40))
        return fail(ATTN_ERR_INVALID_ARG, "problem too large");
    if (!q || !k || !v || !o || !dO || !lse || !dq || !dk || !dv)
        return fail(ATTN_ERR_INVALID_ARG, "null tensor pointer");
    const uintptr_t mis = (uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o | (uintptr_t)dO |
                          (uintptr_t)dq | (uintptr_t)dk | (uintptr_t)dv;
    if (mis & 15) return fail(ATTN_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
    if (workspace && ((uintptr_t)workspace & (kAlign - 1)))
        return fail(ATTN_ERR_INVALID_ARG, "workspace must be 256-byte aligned");

    const TileShape shape = shape_for(dtype);
    const int tile = shape.bc, ratio = shape.ratio();
    // KV tiles; the Q tiles are ratio * n (at most kMaxTiles at 128-row
    // tiles; smaller tiles can exceed it, which build_schedule rejects as
    // unsupported)
    const int n = (s + tile - 1) / tile;

    std::lock_guard<std::mutex> lock(g_mutex);
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail_hip(e, "hipGetDevice");
    DevState& ds = g_dev[dev];
    int rc = dev_init(dev, ds, na ? na->base : nullptr);
    if (rc != ATTN_OK) return rc;
    if (schedule == ATTN_SCHED_AUTO) {
        rc = resolve_auto(ds, n, causal != 0, H, d, dtype, &schedule);
        if (rc != ATTN_OK) return rc;
    }
    DevSchedule* sch = nullptr;
    rc = get_schedule(ds, n, ratio, causal != 0, schedule, &sch, na == nullptr);
    if (rc != ATTN_OK) return rc;
    int* table = sch->buf;
    if (na) {
        // the schedule table after the probe area, then the workspace
        const size_t tbytes = align_up(sch->table.size() * sizeof(int));
        if (kNoAllocProbeBytes + tbytes > na->bytes)
            return fail(ATTN_ERR_WORKSPACE, "the schedule table does not fit the no-allocation area");
        table = reinterpret_cast<int*>(na->base + kNoAllocProbeBytes);
        hipError_t e = hipMemcpyAsync(table, sch->table.data(), sch->table.size() * sizeof(int),
                                      hipMemcpyHostToDevice, (hipStream_t)stream);
        if (e != hipSuccess) return fail_hip(e, "hipMemcpyAsync(schedule)");
        workspace = na->base + kNoAllocProbeBytes + tbytes;
        workspace_bytes = na->bytes - kNoAllocProbeBytes - tbytes;
    }

    // XCD placement needs an accumulator copy per XCD; a caller workspace
    // too small for it but large enough for the global queue runs with that
    WsLayout wl;
    ws_layout(H, s, d, H, wl);
    const XcdPlan plan = na ? XcdPlan{} : placement_plan(ds, *sch, schedule, H);
    WsLayout wl_xcd = wl;
    if (plan.chunks) ws_layout(H, s, d, kQueues * plan.slots, wl_xcd);
    char* ws = static_cast<char*>(workspace);
    bool use_xcd = plan.chunks > 0;
    if (ws) {
        if (workspace_bytes < wl.total)
            return fail(ATTN_ERR_WORKSPACE, na ? "problem too large for the no-allocation area"
                                               : "workspace smaller than attn_bwd_workspace_bytes()");
        use_xcd = use_xcd && workspace_bytes >= wl_xcd.total;
    }
    if (use_xcd) wl = wl_xcd;
    const bool lib_ws = ws == nullptr;
    if (lib_ws) {
        if (!ds.ws_done) {
            e = hipEventCreateWithFlags(&ds.ws_done, hipEventDisableTiming);
            if (e != hipSuccess) return fail_hip(e, "hipEventCreateWithFlags");
        }
        // order this call after the previous user of the library workspace
        if (ds.ws_used && ds.ws_stream != stream) {
            e = hipStreamWaitEvent((hipStream_t)stream, ds.ws_done, 0);
            if (e != hipSuccess) return fail_hip(e, "hipStreamWaitEvent");
        }
        if (ds.ws_bytes < wl.total) {
            if (ds.ws) {
                e = hipDeviceSynchronize();
                if (e != hipSuccess) return fail_hip(e, "hipDeviceSynchronize");
                (void)hipFree(ds.ws);
                ds.ws = nullptr;
                ds.ws_bytes = 0;
            }
            e = hipMalloc(&ds.ws, wl.total);
            if (e != hipSuccess) return fail_hip(e, "hipMalloc(workspace)");
            ds.ws_bytes = wl.total;
        }
        ws = static_cast<char*>(ds.ws);
    }

    BwdArgs a{};
    a.q = q; a.k = k; a.v = v; a.o = o; a.dO = dO; a.lse = lse;
    a.dq = dq; a.dk = dk; a.dv = dv;
    a.H = (int)H; a.s = s; a.d = d; a.n = n * ratio; a.tile = tile; a.br = shape.br;
    a.causal = causal != 0;
    a.schedule = schedule;
    a.dtype = dtype;
    a.scale = scale;
    a.stream = stream;
    a.s_pad = wl.s_pad;
    a.dq_acc = reinterpret_cast<float*>(ws + wl.acc);
    a.delta = reinterpret_cast<float*>(ws + wl.delta);
    a.flags = reinterpret_cast<unsigned*>(ws + wl.flags);
    a.counters = reinterpret_cast<unsigned*>(ws + wl.counters);
    a.acc_slots = use_xcd ? plan.slots : H;

    void** ev = nullptr;
    if (g_timing && !na && ds.ev_used < kMaxTimedCalls) {
        while (ds.ev_pool.size() < 4 * (ds.ev_used + 1)) {
            hipEvent_t x;
            e = hipEventCreate(&x);
            if (e != hipSuccess) return fail_hip(e, "hipEventCreate");
            ds.ev_pool.push_back(x);
        }
        ev = reinterpret_cast<void**>(&ds.ev_pool[4 * ds.ev_used]);
    }

    BwdLaunch L{};
    L.stream = stream;
    L.num_cus = ds.num_cus;
    L.min_workers = sch->min_workers;
    L.ev = ev;
    L.status = ds.status;
    L.stats = g_wait_stats ? reinterpret_cast<unsigned long long*>(a.counters + 2) : nullptr;
    L.whist = g_wait_stats ? reinterpret_cast<unsigned long long*>(ws + wl.hist) : nullptr;
    L.item_begin = table;
    L.tasks = L.item_begin + (sch->items + 1 + 3) / 4 * 4;
    L.items_per_head = sch->items;
    // flags, counters and the wait histogram are contiguous: one clear
    // covers them (the histogram only when it is written)
    L.nclear32 = (int)(((g_wait_stats ? wl.total : wl.hist) - wl.flags) / sizeof(unsigned));
    if (use_xcd) L.plan = plan;
    L.spin_limit = g_spin_limit;
    L.wait_offset = g_wait_offset;
    L.delay_seed = g_delay_seed;
    L.main_kernel = g_main_kernel.load();

    rc = launch_backward(a, L);
    if (rc != ATTN_OK) return rc;
    if (lib_ws) {
        e = hipEventRecord(ds.ws_done, (hipStream_t)stream);
        if (e != hipSuccess) return fail_hip(e, "hipEventRecord");
        ds.ws_stream = stream;
        ds.ws_used = true;
    }
    if (ev) {
        if (ds.ev_finalize.size() <= ds.ev_used) ds.ev_finalize.resize(ds.ev_used + 1);
        ds.ev_finalize[ds.ev_used] = schedule == ATTN_SCHED_ATOMIC;
        ds.ev_used++;
    }
    ds.last_counters = a.counters;
    ds.last_hist = ws + wl.hist;
    ds.stats_valid = g_wait_stats;
    g_last_dev = dev;
    return ATTN_OK;
}

}  // namespace attn

using namespace attn;

extern "C" int attn_bwd_deterministic(const void* q, const void* k, const void* v, const void* o,
                                      const void* dO, const float* lse, void* dq, void* dk, void* dv,
                                      int b, int h, int s, int d, int causal, int schedule) {
    return guarded([&]() -> int {
        const float scale = (d > 0) ? 1.0f / std::sqrt((float)d) : 1.0f;
        return backward(q, k, v, o, dO, lse, dq, dk, dv, b, h, s, d, causal, schedule, ATTN_BF16, scale,
                        nullptr, 0, nullptr, nullptr);
    });
}

extern "C" int attn_bwd_deterministic_ex(const void* q, const void* k, const void* v, const void* o,
                                         const void* dO, const float* lse, void* dq, void* dk, void* dv,
                                         int b, int h, int s, int d, int causal, int schedule, int dtype,
                                         float scale, void* workspace, size_t workspace_bytes, void* stream) {
    return guarded([&]() -> int {
        return backward(q, k, v, o, dO, lse, dq, dk, dv, b, h, s, d, causal, schedule, dtype, scale, workspace,
                        workspace_bytes, stream, nullptr);
    });
}

extern "C" int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int b, int h, int s,
                        int d, int causal, int dtype, float scale, void* stream) {
    return guarded([&]() -> int {
        g_last_error.clear();
        if (b < 0 || h < 0 || s < 0) return fail(ATTN_ERR_INVALID_ARG, "b, h and s must be >= 0");
        if (causal != 0 && causal != 1) return fail(ATTN_ERR_INVALID_ARG, "causal must be 0 or 1");
        if (dtype != ATTN_BF16 && dtype != ATTN_FP32) return fail(ATTN_ERR_INVALID_ARG, "unknown dtype");
        if (!std::isfinite(scale) || !(scale > 0))
            return fail(ATTN_ERR_INVALID_ARG, "scale must be a positive finite number");
        if (d != 64 && d != 128) return fail(ATTN_ERR_UNSUPPORTED, "head dimension must be 64 or 128");
        const long long H = (long long)b * h;
        if (H == 0 || s == 0) return ATTN_OK;
        if (s > kMaxSeq) return fail(ATTN_ERR_UNSUPPORTED, "sequence length above 262144 is not supported");
        if (H > kMaxHeads || H * (long long)s * d >= (1LL << 40))
            return fail(ATTN_ERR_INVALID_ARG, "problem too large");
        if (!q || !k || !v || !o || !lse) return fail(ATTN_ERR_INVALID_ARG, "null tensor pointer");
        if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15)
            return fail(ATTN_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
        if ((uintptr_t)lse & 3) return fail(ATTN_ERR_INVALID_ARG, "lse must be 4-byte aligned");
        FwdArgs a{};
        a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
        a.H = (int)H; a.s = s; a.d = d; a.causal = causal != 0; a.dtype = dtype; a.scale = scale;
        a.stream = stream;
        return launch_forward(a);
    });
}

extern "C" size_t attn_bwd_workspace_bytes(int b, int h, int s, int d, int causal, int schedule) {
    try {
        if (b < 0 || h < 0 || s < 0 || s > kMaxSeq) return 0;
        const long long H = (long long)b * h;
        if (H > kMaxHeads || H * (long long)s * d >= (1LL << 40)) return 0;
        WsLayout wl;
        if (!ws_layout(H, s, d, H, wl)) return 0;
        size_t total = wl.total;
        // what XCD placement needs on the current device (any tile shape)
        if (H > 0 && s > 0 && (causal == 0 || causal == 1) && schedule >= ATTN_SCHED_NAIVE &&
            schedule <= ATTN_SCHED_AUTO && schedule != ATTN_SCHED_ATOMIC) {
            std::lock_guard<std::mutex> lock(g_mutex);
            int dev = 0;
            if (hipGetDevice(&dev) == hipSuccess) {
                DevState& ds = g_dev[dev];
                if (dev_init(dev, ds) == ATTN_OK) {
                    for (const TileShape t : {TileShape{64, 64}, TileShape{128, 128}, TileShape{64, 128}})
                    for (int sched = ATTN_SCHED_NAIVE; sched < ATTN_SCHED_ATOMIC; ++sched) {
                        // AUTO may resolve to any deterministic schedule
                        if (schedule != ATTN_SCHED_AUTO && sched != schedule) continue;
                        const int n = (s + t.bc - 1) / t.bc;
                        Schedule sc;
                        if (build_schedule(n, causal != 0, sched, sc, t.ratio()) != ATTN_OK) continue;
                        DevSchedule shape;
                        shape.items = sc.num_items();
                        shape.item_begin = sc.item_begin;
                        shape.min_workers = min_workers(sc);
                        const XcdPlan plan = placement_plan(ds, shape, sched, H);
                        WsLayout w2;
                        if (plan.chunks && ws_layout(H, s, d, kQueues * plan.slots, w2)) total = std::max(total, w2.total);
                    }
                }
            }
            g_last_error.clear();
        }
        return total;
    } catch (...) {
        fail_internal("host memory exhausted or unexpected host-side error");
        return 0;
    }
}

extern "C" int attn_bwd_resolve_schedule(int b, int h, int s, int d, int causal, int dtype) {
    return guarded([&]() -> int {
        if (b <= 0 || h <= 0 || s <= 0 || s > kMaxSeq || (causal != 0 && causal != 1))
            return fail(ATTN_ERR_INVALID_ARG, "invalid sizes or mask");
        if (dtype != ATTN_BF16 && dtype != ATTN_FP32) return fail(ATTN_ERR_INVALID_ARG, "unknown dtype");
        if (d != 64 && d != 128) return fail(ATTN_ERR_UNSUPPORTED, "head dimension must be 64 or 128");
        const long long H = (long long)b * h;
        if (H > kMaxHeads) return fail(ATTN_ERR_INVALID_ARG, "problem too large");
        std::lock_guard<std::mutex> lock(g_mutex);
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess) return fail_hip(e, "hipGetDevice");
        DevState& ds = g_dev[dev];
        int rc = dev_init(dev, ds);
        if (rc != ATTN_OK) return rc;
        const int tile = tile_for(dtype);
        int pick = -1;
        rc = resolve_auto(ds, (s + tile - 1) / tile, causal != 0, H, d, dtype, &pick);
        return rc != ATTN_OK ? rc : pick;
    });
}

extern "C" int attn_bwd_query_status(void* stream) {
    return guarded([&]() -> int {
        g_last_error.clear();
        hipError_t e = hipStreamSynchronize((hipStream_t)stream);
        if (e != hipSuccess) return fail_hip(e, "hipStreamSynchronize");
        std::lock_guard<std::mutex> lock(g_mutex);
        int dev = 0;
        e = hipGetDevice(&dev);
        if (e != hipSuccess) return fail_hip(e, "hipGetDevice");
        auto it = g_dev.find(dev);
        if (it == g_dev.end() || !it->second.init) return ATTN_OK;
        unsigned st = 0;
        e = hipMemcpy(&st, it->second.status, sizeof(unsigned), hipMemcpyDeviceToHost);
        if (e != hipSuccess) return fail_hip(e, "hipMemcpy(status)");
        if (st) {
            e = hipMemset(it->second.status, 0, sizeof(unsigned));
            if (e != hipSuccess) return fail_hip(e, "hipMemset(status)");
            if (st & 1u) return fail(ATTN_ERR_TIMEOUT, "a dQ flag wait expired; the results of that call are invalid");
            return fail(ATTN_ERR_PLACEMENT, "XCD placement could not use the work groups as planned (an XCD "
                                            "without work groups or an unknown XCD id); the results of that call "
                                            "are invalid");
        }
        return ATTN_OK;
    });
}

extern "C" const char* attn_bwd_last_error(void) { return g_last_error.c_str(); }

extern "C" int attn_bwd_tile_size(int dtype) {
    return guarded([&]() -> int {
        if (dtype != ATTN_BF16 && dtype != ATTN_FP32) return fail(ATTN_ERR_INVALID_ARG, "unknown dtype");
        return tile_for(dtype);
    });
}

extern "C" int attn_bwd_set_timing(int on) {
    return guarded([&]() -> int {
        std::lock_guard<std::mutex> lock(g_mutex);
        g_timing = on != 0;
        if (g_timing)
            for (auto& kv : g_dev) kv.second.ev_used = 0;
        return ATTN_OK;
    });
}

extern "C" int attn_bwd_get_kernel_times(float* ms_pre, float* ms_main, float* ms_fin) {
    return guarded([&]() -> int {
        std::lock_guard<std::mutex> lock(g_mutex);
        if (ms_pre) *ms_pre = 0.f;
        if (ms_main) *ms_main = 0.f;
        if (ms_fin) *ms_fin = 0.f;
        auto it = g_dev.find(g_last_dev);
        if (it == g_dev.end() || it->second.ev_used == 0) return fail(ATTN_ERR_INVALID_ARG, "no timed call recorded");
        DevState& ds = it->second;
        const size_t calls = ds.ev_used;
        hipError_t e = hipEventSynchronize(ds.ev_pool[4 * calls - 1]);
        if (e != hipSuccess) return fail_hip(e, "hipEventSynchronize");
        double sum[3] = {0, 0, 0};
        for (size_t c = 0; c < calls; ++c) {
            hipEvent_t* ev = &ds.ev_pool[4 * c];
            for (int k = 0; k < 3; ++k) {
                if (k == 2 && !ds.ev_finalize[c]) continue;
                float t = 0.f;
                e = hipEventElapsedTime(&t, ev[k], ev[k + 1]);
                if (e != hipSuccess) return fail_hip(e, "hipEventElapsedTime");
                sum[k] += t;
            }
        }
        if (ms_pre) *ms_pre = (float)(sum[0] / calls);
        if (ms_main) *ms_main = (float)(sum[1] / calls);
        if (ms_fin) *ms_fin = (float)(sum[2] / calls);
        return ATTN_OK;
    });
}

extern "C" int attn_bwd_get_call_times(float* ms_total, float* ms_main, int max_calls, int* calls) {
    return guarded([&]() -> int {
        std::lock_guard<std::mutex> lock(g_mutex);
        if (calls) *calls = 0;
        if (max_calls < 0) return fail(ATTN_ERR_INVALID_ARG, "max_calls must be >= 0");
        auto it = g_dev.find(g_last_dev);
        if (it == g_dev.end() || it->second.ev_used == 0) return fail(ATTN_ERR_INVALID_ARG, "no timed call recorded");
        DevState& ds = it->second;
        const int n = (int)std::min<size_t>(ds.ev_used, (size_t)max_calls);
        hipError_t e = hipEventSynchronize(ds.ev_pool[4 * ds.ev_used - 1]);
        if (e != hipSuccess) return fail_hip(e, "hipEventSynchronize");
        for (int c = 0; c < n; ++c) {
            hipEvent_t* ev = &ds.ev_pool[4 * (size_t)c];
            float t = 0.f;
            if (ms_total) {
                e = hipEventElapsedTime(&t, ev[0], ev[3]);
                if (e != hipSuccess) return fail_hip(e, "hipEventElapsedTime");
                ms_total[c] = t;
            }
            if (ms_main) {
                e = hipEventElapsedTime(&t, ev[1], ev[2]);
                if (e != hipSuccess) return fail_hip(e, "hipEventElapsedTime");
                ms_main[c] = t;
            }
        }
        if (calls) *calls = n;
        return ATTN_OK;
    });
}

extern "C" int attn_bwd_set_debug(unsigned spin_limit, int wait_offset, unsigned delay_seed) {
    return guarded([&]() -> int {
        if (wait_offset < 0 || wait_offset > 0xffff) return fail(ATTN_ERR_INVALID_ARG, "wait_offset must be in [0, 65535]");
        std::lock_guard<std::mutex> lock(g_mutex);
        g_spin_limit = spin_limit;
        g_wait_offset = wait_offset;
        g_delay_seed = delay_seed;
        return ATTN_OK;
    });
}

extern "C" int attn_bwd_get_clock(double* mhz) {
    return guarded([&]() -> int {
        std::lock_guard<std::mutex> lock(g_mutex);
        if (mhz) *mhz = 0;
        auto it = g_dev.find(g_last_dev);
        if (it == g_dev.end() || !it->second.stats_valid || !it->second.last_counters)
            return fail(ATTN_ERR_INVALID_ARG, "no call with wait statistics recorded");
        hipError_t e = hipDeviceSynchronize();
        if (e != hipSuccess) return fail_hip(e, "hipDeviceSynchronize");
        unsigned long long v[5] = {0, 0, 0, 0, 0};
        e = hipMemcpy(v, static_cast<unsigned*>(it->second.last_counters) + 2, sizeof(v), hipMemcpyDeviceToHost);
        if (e != hipSuccess) return fail_hip(e, "hipMemcpy(stats)");
        int wall_khz = 0;
        e = hipDeviceGetAttribute(&wall_khz, hipDeviceAttributeWallClockRate, g_last_dev);
        if (e != hipSuccess) return fail_hip(e, "hipDeviceGetAttribute(wall clock rate)");
        if (v[4] == 0 || wall_khz <= 0) return fail(ATTN_ERR_INVALID_ARG, "no clock span recorded");
        if (mhz) *mhz = (double)v[3] / (double)v[4] * wall_khz / 1e3;
        return ATTN_OK;
    });
}

extern "C" int attn_bwd_atomic_rate(void* acc, size_t acc_bytes, int tasks, void* stream, float* ms, double* adds) {
    return guarded([&]() -> int {
        if (ms) *ms = 0;
        if (adds) *adds = 0;
        if (!acc || ((uintptr_t)acc & (kAlign - 1))) return fail(ATTN_ERR_INVALID_ARG, "acc must be a 256-byte aligned device pointer");
        if (acc_bytes < 65536) return fail(ATTN_ERR_INVALID_ARG, "acc must hold at least one 128x128 fp32 tile");
        if (tasks < 1 || tasks > 65536) return fail(ATTN_ERR_INVALID_ARG, "tasks must be in 1..65536");
        const int ntiles = (int)std::min<size_t>(acc_bytes / 65536, (size_t)1 << 30);
        int dev = 0, cus = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return fail_hip(e, "device query");
        if (cus < 1) return fail(ATTN_ERR_HIP, "no compute units reported");
        hipEvent_t ev[2] = {nullptr, nullptr};
        for (auto& x : ev)
            if ((e = hipEventCreate(&x)) != hipSuccess) break;
        int rc = e == hipSuccess ? ATTN_OK : fail_hip(e, "hipEventCreate");
        if (rc == ATTN_OK) rc = launch_atomic_rate(static_cast<float*>(acc), ntiles, cus, tasks, stream);
        if (rc == ATTN_OK && (e = hipEventRecord(ev[0], (hipStream_t)stream)) != hipSuccess) rc = fail_hip(e, "hipEventRecord");
        if (rc == ATTN_OK) rc = launch_atomic_rate(static_cast<float*>(acc), ntiles, cus, tasks, stream);
        if (rc == ATTN_OK && (e = hipEventRecord(ev[1], (hipStream_t)stream)) != hipSuccess) rc = fail_hip(e, "hipEventRecord");
        if (rc == ATTN_OK && (e = hipEventSynchronize(ev[1])) != hipSuccess) rc = fail_hip(e, "hipEventSynchronize");
        float t = 0;
        if (rc == ATTN_OK && (e = hipEventElapsedTime(&t, ev[0], ev[1])) != hipSuccess) rc = fail_hip(e, "hipEventElapsedTime");
        for (auto& x : ev)
            if (x) (void)hipEventDestroy(x);
        if (rc != ATTN_OK) return rc;
        if (ms) *ms = t;
        if (adds) *adds = (double)cus * tasks * 128.0 * 128.0;
        return ATTN_OK;
    });
}

extern "C" int attn_bwd_handoff_latency(void* buf, size_t buf_bytes, int pong, int iters, int mode, void* stream,
                                        double* ns, int* xcd_ping, int* xcd_pong) {
    return guarded([&]() -> int {
        if (ns) *ns = 0;
        if (!buf || ((uintptr_t)buf & (kAlign - 1))) return fail(ATTN_ERR_INVALID_ARG, "buf must be a 256-byte aligned device pointer");
        if (buf_bytes < kHandoffBytes) return fail(ATTN_ERR_INVALID_ARG, "buf smaller than attn_bwd_handoff_bytes");
        if (pong < 1 || pong > 63) return fail(ATTN_ERR_INVALID_ARG, "pong must be in 1..63");
        if (iters < 2 || iters > (1 << 20)) return fail(ATTN_ERR_INVALID_ARG, "iters must be in 2..2^20");
        if (mode < 0 || mode > 2) return fail(ATTN_ERR_INVALID_ARG, "mode must be 0, 1 or 2");
        int dev = 0, khz = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e == hipSuccess) e = hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev);
        if (e != hipSuccess) return fail_hip(e, "device query");
        if (khz <= 0) return fail(ATTN_ERR_HIP, "no constant-rate clock reported");
        unsigned* words = static_cast<unsigned*>(buf);
        float* tiles = reinterpret_cast<float*>(static_cast<char*>(buf) + 256);
        e = hipMemsetAsync(words, 0, 256, (hipStream_t)stream);
        if (e != hipSuccess) return fail_hip(e, "hipMemsetAsync");
        int rc = launch_handoff(words, tiles, pong, iters, mode, stream);
        if (rc != ATTN_OK) return rc;
        unsigned h[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        e = hipMemcpyAsync(h, words, sizeof(h), hipMemcpyDeviceToHost, (hipStream_t)stream);
        if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
        if (e != hipSuccess) return fail_hip(e, "hand-off result copy");
        if (h[3]) return fail(ATTN_ERR_TIMEOUT, "a hand-off wait gave up");
        if (xcd_ping) *xcd_ping = (int)h[1];
        if (xcd_pong) *xcd_pong = (int)h[2];
        const unsigned long long span = (unsigned long long)h[4] | ((unsigned long long)h[5] << 32);
        if (ns) *ns = (double)span / khz * 1e6 / iters;
        return ATTN_OK;
    });
}

extern "C" size_t attn_bwd_handoff_bytes(void) { return kHandoffBytes; }

extern "C" int attn_bwd_set_tile_shape(int dtype, int br, int bc) {
    return guarded([&]() -> int {
        if (dtype != ATTN_BF16)
            return fail(ATTN_ERR_UNSUPPORTED, "attn_bwd_set_tile_shape: only bf16 has a choice of tile");
        if (br == 0 && bc == 0) br = bc = 128;
        if (!((br == 128 && bc == 128) || (br == 64 && bc == 64) || (br == 64 && bc == 128)))
            return fail(ATTN_ERR_INVALID_ARG,
                        "attn_bwd_set_tile_shape: (Br, Bc) must be (0, 0) (default), (128, 128), (64, 64) or (64, 128)");
        std::lock_guard<std::mutex> lock(g_mutex);
        g_shape_bf16 = (br << 16) | bc;
        return ATTN_OK;
    });
}

extern "C" int attn_bwd_set_tile(int dtype, int tile) {
    return guarded([&]() -> int {
        if (dtype != ATTN_BF16) return fail(ATTN_ERR_UNSUPPORTED, "attn_bwd_set_tile: only bf16 has a choice of tile");
        if (tile != 0 && tile != 64 && tile != 128)
            return fail(ATTN_ERR_INVALID_ARG, "attn_bwd_set_tile: tile must be 0 (default), 64 or 128");
        return attn_bwd_set_tile_shape(dtype, tile, tile);
    });
}

extern "C" int attn_bwd_tile_shape(int dtype, int* br, int* bc) {
    return guarded([&]() -> int {
        if (dtype != ATTN_BF16 && dtype != ATTN_FP32) return fail(ATTN_ERR_INVALID_ARG, "unknown dtype");
        const TileShape t = shape_for(dtype);
        if (br) *br = t.br;
        if (bc) *bc = t.bc;
        return ATTN_OK;
    });
}

extern "C" int attn_bwd_set_placement(int mode) {
    return guarded([&]() -> int {
        if (mode != ATTN_PLACE_GLOBAL && mode != ATTN_PLACE_XCD)
            return fail(ATTN_ERR_INVALID_ARG, "attn_bwd_set_placement: mode must be ATTN_PLACE_GLOBAL or ATTN_PLACE_XCD");
        std::lock_guard<std::mutex> lock(g_mutex);
        g_xcd_placement = mode == ATTN_PLACE_XCD;
        return ATTN_OK;
    });
}

extern "C" int attn_bwd_set_main_kernel(int kernel) {
    return guarded([&]() -> int {
        if (kernel != ATTN_KERNEL_FOUR_WAVE && kernel != ATTN_KERNEL_PAIR && kernel != ATTN_KERNEL_AUTO)
            return fail(ATTN_ERR_INVALID_ARG, "attn_bwd_set_main_kernel: unknown kernel");
        g_main_kernel.store(kernel);
        return ATTN_OK;
    });
}

extern "C" int attn_bwd_main_kernel(void) { return g_main_kernel.load(); }

// The rule the launch applies (launch_all in bwd_kernels.hip): the pair kernel
// for deterministic bf16 calls with 128 x 128 tiles, when forced or, by
// default, under the causal mask at d = 128.
extern "C" int attn_bwd_resolve_main_kernel(int d, int causal, int dtype, int schedule) {
    return guarded([&]() -> int {
        if ((causal != 0 && causal != 1) || (dtype != ATTN_BF16 && dtype != ATTN_FP32) || schedule < ATTN_SCHED_NAIVE ||
            schedule > ATTN_SCHED_AUTO)
            return fail(ATTN_ERR_INVALID_ARG, "invalid mask, dtype or schedule");
        if (d != 64 && d != 128) return fail(ATTN_ERR_UNSUPPORTED, "head dimension must be 64 or 128");
        const TileShape t = shape_for(dtype);
        const int mk = g_main_kernel.load();
        return runs_pair_kernel(dtype == ATTN_BF16, t.br, t.bc, schedule != ATTN_SCHED_ATOMIC, mk, causal != 0, d)
                   ? ATTN_KERNEL_PAIR
                   : ATTN_KERNEL_FOUR_WAVE;
    });
}

extern "C" int attn_bwd_set_wait_stats(int on) {
    return guarded([&]() -> int {
        std::lock_guard<std::mutex> lock(g_mutex);
        g_wait_stats = on != 0;
        return ATTN_OK;
    });
}

extern "C" int attn_bwd_get_wait_hist(unsigned long long* cycles) {
    return guarded([&]() -> int {
        if (!cycles) return fail(ATTN_ERR_INVALID_ARG, "null histogram buffer");
        std::lock_guard<std::mutex> lock(g_mutex);
        auto it = g_dev.find(g_last_dev);
        if (it == g_dev.end() || !it->second.stats_valid || !it->second.last_hist)
            return fail(ATTN_ERR_INVALID_ARG, "no call with wait statistics recorded");
        hipError_t e = hipDeviceSynchronize();
        if (e != hipSuccess) return fail_hip(e, "hipDeviceSynchronize");
        e = hipMemcpy(cycles, it->second.last_hist, (size_t)kHistItems * kHistSteps * sizeof(unsigned long long),
                      hipMemcpyDeviceToHost);
        if (e != hipSuccess) return fail_hip(e, "hipMemcpy(wait histogram)");
        return ATTN_OK;
    });
}

extern "C" int attn_bwd_get_wait_stats(unsigned long long* wait_cycles, unsigned long long* item_cycles,
                                       unsigned long long* polls) {
    return guarded([&]() -> int {
        std::lock_guard<std::mutex> lock(g_mutex);
        auto it = g_dev.find(g_last_dev);
        if (it == g_dev.end() || !it->second.stats_valid || !it->second.last_counters)
            return fail(ATTN_ERR_INVALID_ARG, "no call with wait statistics recorded");
        hipError_t e = hipDeviceSynchronize();
        if (e != hipSuccess) return fail_hip(e, "hipDeviceSynchronize");
        unsigned long long v[3] = {0, 0, 0};
        e = hipMemcpy(v, static_cast<unsigned*>(it->second.last_counters) + 2, sizeof(v), hipMemcpyDeviceToHost);
        if (e != hipSuccess) return fail_hip(e, "hipMemcpy(stats)");
        if (wait_cycles) *wait_cycles = v[0];
        if (item_cycles) *item_cycles = v[1];
        if (polls) *polls = v[2];
        return ATTN_OK;
    });
}
