// Internal declarations shared by the host sources of libattn_bwd.so.
#pragma once

#include <cstddef>
#include <new>
#include <vector>

#include "attn_bwd.h"

namespace attn {

// Largest number of tiles per sequence the host side accepts: a head's task
// table holds n^2 records of 16 bytes (64 MiB at n = 2048, twice that during
// its construction), and every 32-bit offset of the kernels (per-head buffer
// resources over s rows of d elements, accumulator offsets) stays far inside
// its range.
constexpr int kMaxTiles = 2048;
// Largest problem the DAG simulator accepts: heads times tasks per head, and
// the number of workers (both bound its memory and run time).
constexpr long long kMaxSimTasks = 1LL << 27;
constexpr int kMaxWorkers = 1 << 20;

// One head's schedule pattern (see attn_sched_get in attn_bwd.h).
struct Schedule {
    int n = 0;                    // KV tiles (items' tiles)
    int nq = 0;                   // Q tiles: ratio * n (n for square tiles)
    bool causal = false;
    int schedule = 0;
    std::vector<int> item_begin;  // num_items + 1
    std::vector<int> task_kv, task_q;
    std::vector<int> rank;        // [kv * nq + q], -1 = masked (or ATOMIC)
    std::vector<int> count;       // nq: contributors per Q tile
    int round_size = 0;           // Shift: KV tiles per round (0: not Shift)
    int num_items() const { return (int)item_begin.size() - 1; }
};

// Shift cuts a head's KV tiles into rounds of at most this many tiles (the
// work groups MI355X keeps resident: one per CU), so that a round's items,
// which wait on each other cyclically, always run together.
constexpr int kShiftRound = 256;

// n KV tiles, `ratio` Q tiles per KV tile (Bc = ratio * Br; 1 = square tiles)
int build_schedule(int n, bool causal, int schedule, Schedule& out, int ratio = 1);
int min_workers(const Schedule& sc);
int simulate(const Schedule& sc, int heads, int workers, int placement, double c, double r, double e,
             double* makespan, double* wait_time, double* busy_time);

// Records `msg` as the calling thread's last error and returns `code`.
int fail(int code, const char* msg);
// fail(ATTN_ERR_INTERNAL, msg) that never throws (used while handling an
// exception, when even the message may not fit in memory).
int fail_internal(const char* msg) noexcept;

// Runs f() (returning a status) and turns any C++ exception into a status
// code, so that none crosses the C ABI: host memory exhaustion and other
// host-side failures become ATTN_ERR_INTERNAL.
template <class F>
int guarded(F&& f) noexcept {
    try {
        return f();
    } catch (const std::bad_alloc&) {
        return fail_internal("host memory exhausted");
    } catch (...) {
        return fail_internal("unexpected host-side error");
    }
}

// Parameters of one backward launch (device pointers).
struct BwdArgs {
    const void *q, *k, *v, *o, *dO;
    const float* lse;
    void *dq, *dk, *dv;
    int H, s, d, n, tile;  // n: Q tiles per head; tile: KV tile rows (Bc)
    int br;                // Q tile rows (Br; = tile for square tiles)
    bool causal;
    int schedule;
    int dtype;
    float scale;
    void* stream;
    // workspace carve-out
    float* dq_acc;
    float* delta;         // D [H][s_pad], then lse * log2(e) [H][s_pad]
    unsigned* flags;
    unsigned* counters;   // [0] ticket, [1] abort, [2..] wait statistics, [kQueueWord..] XCD queues
    long long acc_slots;  // heads of dq_acc: H, or kQueues copies of XcdPlan::slots
    size_t s_pad;
};

// Work queues of XCD placement (one per XCD of MI355X).
constexpr int kQueues = 8;

// XCD placement of a deterministic launch: a head's items split into
// `chunks` contiguous runs, chunk c = items [bounds[c], bounds[c + 1]); queue
// q serves chunk q % chunks of the heads g, g + groups, ... (g = q / chunks,
// groups = kQueues / chunks).  Each XCD keeps its own dQ accumulator of
// `slots` heads (head h in slot h / groups).
struct XcdPlan {
    int chunks = 0, groups = 0, max_chunk = 0;
    int bounds[kQueues + 1] = {};
    long long slots = 0;
};
// The plan for `grid` resident work groups, or chunks == 0 when the launch
// keeps the global queue.  item_begin: the schedule's items_per_head + 1
// task offsets (the work of each item).
XcdPlan xcd_plan(const std::vector<int>& item_begin, int min_workers, long long grid, long long heads);
// Whether work group b of a launch runs on XCD b % kQueues on this device.
// `buf`: device memory for the probe's 4 * num_cus words, or null to
// allocate it.
int probe_xcd_dispatch(int num_cus, bool* ok, unsigned* buf = nullptr);
// Device address of the library's device status word (a device variable).
int status_word_address(unsigned** ptr);
// fp32 atomic-add throughput kernel (tasks 128x128 tiles per work group into
// acc, which holds ntiles such tiles)
int launch_atomic_rate(float* acc, int ntiles, int grid, int tasks, void* stream);
// dQ hand-off latency kernel between work group 0 and work group `pong`
// (words: 8 u32 cleared by the caller; tiles: 2 x 64 KiB)
int launch_handoff(unsigned* words, float* tiles, int pong, int iters, int mode, void* stream);

// A device area that a call uses for every buffer it needs instead of
// allocating (the no-allocation entry point): XCD probe words at its start
// (kNoAllocProbeBytes), then the schedule table, then the workspace.
struct NoAllocArea {
    char* base;
    size_t bytes;
};
constexpr size_t kNoAllocProbeBytes = 64 * 1024;
int backward(const void* q, const void* k, const void* v, const void* o, const void* dO, const float* lse,
             void* dq, void* dk, void* dv, int b, int h, int s, int d, int causal, int schedule, int dtype,
             float scale, void* workspace, size_t workspace_bytes, void* stream, const NoAllocArea* na);

// Launch-time context prepared by the API layer (device pointers).
struct BwdLaunch {
    void* stream;                 // hipStream_t
    int num_cus;
    int min_workers;              // resident work groups the schedule needs
    void** ev;                    // 4 hipEvent_t to record, or null
    unsigned* status;             // device status word (bit 0: wait expired)
    unsigned long long* stats;    // wait statistics or null
    unsigned long long* whist;    // wait histogram [64][128] or null
    const int* item_begin;        // per item pattern: first task, items+1 entries
    const int* tasks;             // 4 ints per task: kv, q, rank, contributors
    int items_per_head;
    int nclear32;                 // flags + counters words to clear
    XcdPlan plan;                 // XCD placement (chunks == 0: one global queue)
    unsigned spin_limit = 0;      // test hooks (attn_bwd_set_debug); 0: default
    int wait_offset = 0;
    unsigned delay_seed = 0;
    int main_kernel = 2;          // attn_main_kernel_t (bf16 d = 128, 128 x 128 tiles)
};

// Whether a launch runs the eight-wave pair kernel: bf16, 128 x 128 tiles, an
// ordered (deterministic) schedule, and the pair kernel either forced or, by
// default, the causal mask at d = 128.  The launch and
// attn_bwd_resolve_main_kernel both decide through this one rule.
inline bool runs_pair_kernel(bool bf16, int br, int bc, bool det, int main_kernel, bool causal, int d) {
    return bf16 && br == 128 && bc == 128 && det &&
           (main_kernel == ATTN_KERNEL_PAIR || (main_kernel == ATTN_KERNEL_AUTO && causal && d == 128));
}

// first counter word of the per-XCD work queues
constexpr int kQueueWord = 48;

int launch_backward(const BwdArgs& a, const BwdLaunch& L);

// Parameters of one forward launch (device pointers; validated by the caller).
struct FwdArgs {
    const void *q, *k, *v;
    void* o;
    float* lse;
    int H, s, d;
    bool causal;
    int dtype;
    float scale;
    void* stream;
};

int launch_forward(const FwdArgs& a);

}  // namespace attn
