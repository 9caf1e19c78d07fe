/*
 * attn_bwd.h - C ABI of libattn_bwd.so, a deterministic attention backward
 * pass for AMD Instinct MI355X (gfx950) scheduled with DASH.
 *
 * Source of the method: "DASH: Deterministic Attention Scheduling for
 * High-throughput Reproducible LLM Training" (arXiv 2601.21824), as
 * described by its summary page (sections Problem, Approach, Key results)
 * and its pith.science review page (sections "What carries the argument",
 * "Core claim", Axiom ledger, Fig. 1, 3, 4, 6, 7 captions).
 *
 * The backward computes, per head, the exact softmax-attention gradient
 *   D_i = <dO_i, O_i>,  P_ij = exp(scale <q_i,k_j> - lse_i),
 *   dS_ij = P_ij (<dO_i, v_j> - D_i),
 *   dV_j = sum_i P_ij dO_i,  dK_j = scale sum_i dS_ij q_i,
 *   dQ_i = scale sum_j dS_ij k_j
 * tiled into square T x T tiles (T = 128 for bf16, 64 for fp32; bf16 also
 * offers 64 x 64 and 64-row Q tiles against 128-row KV tiles, see
 * attn_bwd_set_tile_shape).  Each work
 * group owns one KV tile at a time (Fig. 1: local dK/dV accumulation) and
 * adds its partial dQ of every Q tile into a global fp32 accumulator in an
 * order fixed by the schedule (Problem section: the serialised dQ
 * reduction), so the results are bitwise reproducible.
 *
 * Conventions shared by every entry point:
 *  - Tensors are contiguous [b][h][s][d] (lse is [b][h][s], fp32, natural
 *    log of the scaled logits, as produced by the forward pass).
 *  - All tensor pointers are DEVICE pointers of the current HIP device,
 *    16-byte aligned.  The caller owns every tensor and the stream; the
 *    library never frees caller memory.  dq, dk, dv are fully overwritten.
 *  - Under the causal mask query i sees keys j <= i (s_q = s_k).
 *  - Calls are asynchronous on the stream; device-side failures (a bounded
 *    flag wait that expired) are reported by attn_bwd_query_status().
 *  - Return value: ATTN_OK (0) or a negative attn_status_t.  No C++
 *    exception crosses the ABI (every entry point catches them and returns
 *    ATTN_ERR_INTERNAL).  attn_bwd_last_error() gives a message for the last
 *    failure on the calling thread.
 *  - Accepted sizes: s <= 262144 (at most 2048 tiles of 128 rows; with
 *    64-row tiles, at most 2048 Q tiles, i.e. s <= 131072), b*h below
 *    2^31 and b*h*s*d below 2^40; larger problems return
 *    ATTN_ERR_UNSUPPORTED (s) or ATTN_ERR_INVALID_ARG (the others).
 *  - scale must be a positive finite number (ATTN_ERR_INVALID_ARG
 *    otherwise): masked logits are -inf before scaling.
 */
#ifndef ATTN_BWD_H
#define ATTN_BWD_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Schedules.  NAIVE is the FlashAttention-3 order (Fig. 3: Q tiles ascending,
 * dQ accumulated in ascending KV order).  DESCENDING is Descending Q-Tile
 * Iteration (Fig. 4; same dQ order as NAIVE).  SHIFT is Shift Scheduling
 * (Fig. 6: the owner of KV tile i visits Q tiles i, i+1, ..., wrapping; dQ_j
 * accumulated in visiting order); with more than 256 KV tiles (more than the
 * work groups MI355X keeps resident) the KV tiles are cut into equal rounds
 * of at most 256 consecutive tiles and dQ_j is accumulated round by round,
 * inside a round in visiting order (Axiom ledger: KV tiles != SMs is handled
 * by refining heads).  SYMMETRIC_SHIFT is Symmetric Shift
 * Scheduling with two-phase workload folding for the causal mask (Fig. 7;
 * equals SHIFT under the full mask; needs an even tile count when causal).
 * ATOMIC is the non-deterministic comparison point: unordered fp32 atomic
 * dQ additions (Problem section: the non-deterministic counterpart).  AUTO
 * picks one of the four deterministic schedules per configuration (review
 * page, "If this is right": the schedules are complementary and an
 * implementation selects one per configuration): the DAG model with task
 * costs fitted on MI355X simulates each schedule the shape admits under the
 * kernel's XCD placement and the shortest makespan wins.
 * attn_bwd_resolve_schedule tells which one a call gets;
 * the choice is deterministic for a shape, so AUTO is as reproducible as
 * the schedule it resolves to. */
typedef enum {
    ATTN_SCHED_NAIVE = 0,
    ATTN_SCHED_DESCENDING = 1,
    ATTN_SCHED_SHIFT = 2,
    ATTN_SCHED_SYMMETRIC_SHIFT = 3,
    ATTN_SCHED_ATOMIC = 4,
    ATTN_SCHED_AUTO = 5
} attn_schedule_t;

typedef enum { ATTN_BF16 = 0, ATTN_FP32 = 1 } attn_dtype_t;

typedef enum {
    ATTN_OK = 0,
    ATTN_ERR_INVALID_ARG = -1,  /* null pointer, negative size, bad enum    */
    ATTN_ERR_UNSUPPORTED = -2,  /* d not 64/128, odd tile count for the fold */
    ATTN_ERR_COSCHEDULE = -3,   /* the schedule needs more resident work
                                   groups than the device can hold at once */
    ATTN_ERR_HIP = -4,          /* a HIP runtime call failed                */
    ATTN_ERR_TIMEOUT = -5,      /* a device-side flag wait expired          */
    ATTN_ERR_WORKSPACE = -6,    /* caller workspace too small               */
    ATTN_ERR_DEADLOCK = -7,     /* simulator: the schedule cannot finish    */
    ATTN_ERR_PLACEMENT = -8,    /* XCD placement found work groups it could
                                   not use as planned: an XCD without work
                                   groups or an unknown XCD id (results of
                                   that call invalid)                       */
    ATTN_ERR_INTERNAL = -9      /* host memory exhausted, or another host-side
                                   failure caught at the ABI boundary        */
} attn_status_t;

/* ------------------------------------------------------------------------
 * Backward pass.
 * ------------------------------------------------------------------------ */

/* attn_bwd_deterministic - bf16 backward with scale = 1/sqrt(d), on the null
 * stream, with a library-owned workspace (allocated on first use and grown
 * as needed; one per device).  Every call that uses the library workspace is
 * ordered after the previous such call on the device: a call on another
 * stream first waits (hipStreamWaitEvent) for the previous one to finish.
 *   q, k, v, o, dO : const bf16 [b][h][s][d]
 *   lse            : const float [b][h][s]
 *   dq, dk, dv     : bf16 [b][h][s][d], written
 *   b, h, s >= 0 (any zero: nothing to do, returns ATTN_OK); d in {64, 128}
 *   causal         : 0 full mask, 1 causal mask
 *   schedule       : attn_schedule_t */
int attn_bwd_deterministic(const void* q, const void* k, const void* v, const void* o,
                           const void* dO, const float* lse, void* dq, void* dk, void* dv,
                           int b, int h, int s, int d, int causal, int schedule);

/* attn_bwd_deterministic_ex - as above with explicit element type (tensors
 * q..dv are bf16 or fp32 per `dtype`; lse is always fp32), softmax scale,
 * stream (a hipStream_t, NULL for the null stream) and an optional caller
 * workspace.  workspace == NULL uses the library-owned one (ordered across
 * streams as above); otherwise it must be device memory of at least
 * attn_bwd_workspace_bytes(...) bytes (ATTN_ERR_WORKSPACE if smaller),
 * 256-byte aligned, owned by the caller and not used concurrently by another
 * call (the library does not order calls that share a caller workspace). */
int attn_bwd_deterministic_ex(const void* q, const void* k, const void* v, const void* o,
                              const void* dO, const float* lse, void* dq, void* dk, void* dv,
                              int b, int h, int s, int d, int causal, int schedule,
                              int dtype, float scale, void* workspace, size_t workspace_bytes,
                              void* stream);

/* attn_bwd_deterministic_noalloc - for callers that cannot allocate device
 * memory (code under stream capture, tight serving loops, harnesses that
 * forbid hipMalloc): attn_bwd_deterministic_ex without a workspace argument,
 * which allocates nothing.  Every buffer the call needs beyond its inputs
 * and outputs (schedule table, fp32 dQ accumulator, D, lse*log2(e), flags,
 * counters) comes from a fixed device array of the library,
 * attn_bwd_noalloc_capacity() bytes (64 MiB) per device, held by every
 * device the library runs on until the process ends.  The call uses the
 * single global work queue (no per-XCD accumulator copies), records no
 * kernel timing, and gives the same bits as the other entry points for the
 * same schedule.  Problems whose workspace and schedule table do not fit
 * return ATTN_ERR_WORKSPACE before anything is launched (the accumulator
 * alone is b*h*ceil(s/128)*128*d*4 bytes).  Every call on a device shares
 * that device's array: calls that overlap on one device (other streams or
 * host threads without ordering) race and give wrong results; calls in
 * sequence on one stream are safe.  Other arguments, errors and
 * asynchrony as for attn_bwd_deterministic_ex. */
int attn_bwd_deterministic_noalloc(const void* q, const void* k, const void* v, const void* o,
                                   const void* dO, const float* lse, void* dq, void* dk, void* dv,
                                   int b, int h, int s, int d, int causal, int schedule, int dtype,
                                   float scale, void* stream);

/* Size in bytes of the device array attn_bwd_deterministic_noalloc uses. */
size_t attn_bwd_noalloc_capacity(void);

/* Bytes of workspace a call with these sizes needs on the current device:
 * fp32 dQ accumulator (b*h*s_pad*d*4, or the per-XCD copies of XCD
 * placement, for either element type), per-(head, Q tile) flags,
 * D = rowsum(dO*O) and lse*log2(e) (b*h*s_pad*4 each), counters.  s_pad is
 * s rounded up to 128.  Without a
 * usable device, or under ATTN_PLACE_GLOBAL, the size for the single global
 * queue, which is also the smallest workspace a call accepts.  Returns 0
 * for invalid sizes. */
size_t attn_bwd_workspace_bytes(int b, int h, int s, int d, int causal, int schedule);

/* The deterministic schedule ATTN_SCHED_AUTO resolves to for these sizes,
 * mask and element type on the current device (an attn_schedule_t >= 0), or
 * a negative status (ATTN_ERR_INVALID_ARG, ATTN_ERR_UNSUPPORTED,
 * ATTN_ERR_COSCHEDULE, ATTN_ERR_HIP).  Initialises the device state on
 * first use; launches nothing. */
int attn_bwd_resolve_schedule(int b, int h, int s, int d, int causal, int dtype);

/* Synchronises `stream` (hipStream_t or NULL), then reports and clears the
 * device status word: ATTN_OK, or ATTN_ERR_TIMEOUT if a bounded flag wait
 * expired in any call since the last query (results of that call are
 * invalid), or ATTN_ERR_HIP if the synchronisation failed. */
int attn_bwd_query_status(void* stream);

/* Message describing the last failure on the calling thread ("" if none).
 * The string is owned by the library and valid until the next call. */
const char* attn_bwd_last_error(void);

/* KV tile rows Bc the backward uses for `dtype` (bf16: 128 unless
 * attn_bwd_set_tile or attn_bwd_set_tile_shape chose 64; fp32: 64). */
int attn_bwd_tile_size(int dtype);

/* Tile granularity of later bf16 calls (review page, "What would settle it"
 * and "Where Pith is reading between the lines": vary the tile granularity
 * and compare the measured makespan with the DAG model): tile = 128 (the
 * default; 0 selects it) or 64, square tiles Br = Bc = T, the same
 * schedules over n = ceil(s/T) tiles.  The 64-row kernel keeps 16 KV rows
 * per wave (half the operand reuse of the 128-row one) and runs the
 * compiler-scheduled sub-step.  Changing the tile changes the partial sums
 * and so the bits, never determinism.  Returns ATTN_OK,
 * ATTN_ERR_UNSUPPORTED (dtype not bf16) or ATTN_ERR_INVALID_ARG. */
int attn_bwd_set_tile(int dtype, int tile);

/* Rectangular tiles for later bf16 calls: Q tiles of Br rows against KV
 * tiles of Bc rows (variable tile shapes, Br != Bc; the pages draw square
 * tiles).  (Br, Bc) = (128, 128) (the default; (0, 0) selects
 * it), (64, 64), or (64, 128): then every KV tile meets ratio = 2 Q tiles
 * of its rows, the schedules run over n = ceil(s/Bc) KV tiles and 2n Q
 * tiles as attn_sched_get_rect defines them (Symmetric Shift folds KV p
 * with KV n-1-p into 2n + 2 tasks), the kernel takes one 64-row sub-step
 * per task and accumulates dQ per 64-row Q tile.  The ordered dQ traffic,
 * s^2 * d * 8 / Bc bytes per head, depends on Bc alone, so it is that of the
 * square 128-row tiles (and half that of the 64-row ones), with twice their
 * tasks and flag hand-offs.  attn_bwd_set_tile(dtype, T)
 * equals attn_bwd_set_tile_shape(dtype, T, T).  Returns ATTN_OK,
 * ATTN_ERR_UNSUPPORTED (dtype not bf16) or ATTN_ERR_INVALID_ARG. */
int attn_bwd_set_tile_shape(int dtype, int br, int bc);

/* The (Br, Bc) tile shape the backward uses for `dtype`; either pointer may
 * be NULL.  Returns ATTN_OK or ATTN_ERR_INVALID_ARG (unknown dtype). */
int attn_bwd_tile_shape(int dtype, int* br, int* bc);

/* Kernel timing.  attn_bwd_set_timing(1) starts a recording: every later
 * backward call (up to 4096) records HIP events on its own stream around
 * each kernel it launches; attn_bwd_set_timing(0) stops recording.
 * attn_bwd_get_kernel_times waits for the recorded events and writes the
 * mean milliseconds per call of the preprocess, main and finalize kernels
 * (finalize: mean over the calls that launched it; 0 if none).  Returns
 * ATTN_OK, ATTN_ERR_INVALID_ARG (nothing recorded) or ATTN_ERR_HIP. */
int attn_bwd_set_timing(int on);
int attn_bwd_get_kernel_times(float* ms_preprocess, float* ms_main, float* ms_finalize);

/* Work placement of the deterministic main kernel for later calls.
 * ATTN_PLACE_XCD (the default): one work queue per XCD of MI355X, served by
 * the work groups running on that XCD; a head's items are split into the
 * fewest contiguous chunks (1, 2, 4 or 8) that fit one XCD's work groups,
 * each chunk on one XCD.  Every XCD keeps its own copy of the fp32 dQ
 * accumulator: a hand-off between work groups of one XCD stays in its L2,
 * only a hand-off to another XCD goes through memory.  The copies make the
 * accumulator part of the workspace about `chunks` times larger (see
 * attn_bwd_workspace_bytes).  Used when the device deals work groups evenly
 * over 8 XCDs (checked once per device) and the launch has at least 8
 * resident work groups and, for the Shift family, a chunk that fits one
 * XCD; otherwise, and for a caller workspace too small for the copies, the
 * call keeps the single global queue.  ATTN_PLACE_GLOBAL: always the one
 * global queue and one accumulator, every hand-off through memory.  Results
 * are bitwise the same under both: the reduction order comes from the
 * schedule alone.  Returns ATTN_OK or ATTN_ERR_INVALID_ARG (unknown mode). */
typedef enum { ATTN_PLACE_GLOBAL = 0, ATTN_PLACE_XCD = 1 } attn_placement_t;
int attn_bwd_set_placement(int mode);

/* Main kernel of later deterministic bf16 calls with 128 x 128 tiles (the
 * other tile shapes, fp32 and ATOMIC always use the four-wave kernel).  ATTN_KERNEL_FOUR_WAVE: four waves per work group, one per SIMD,
 * each owning 32 KV rows of the tile.  ATTN_KERNEL_PAIR: eight waves, two
 * per SIMD; the two waves of a SIMD hold the same 32 KV rows and split each
 * 64-row step of query rows by role (one computes S, dP and the softmax of
 * the first 32 query rows and accumulates dV, the other does the same for
 * the last 32 and accumulates dK), exchanging one operand through LDS.
 * ATTN_KERNEL_AUTO (the default): the pair kernel under the causal mask at
 * d = 128, the four-wave kernel otherwise (measured on MI355X: at d = 128,
 * s = 8192 and 16384, the pair kernel is about 3% faster under the causal
 * mask and 1-4% slower under the full mask; at d = 64, s = 2048, 8-19%
 * slower).  Both kernels perform every addition in
 * the same order: the outputs are bitwise the same.  Process-wide; read at
 * each launch.  attn_bwd_main_kernel returns the current setting.  Returns
 * ATTN_OK or ATTN_ERR_INVALID_ARG. */
typedef enum { ATTN_KERNEL_FOUR_WAVE = 0, ATTN_KERNEL_PAIR = 1, ATTN_KERNEL_AUTO = 2 } attn_main_kernel_t;
int attn_bwd_set_main_kernel(int kernel);
int attn_bwd_main_kernel(void);

/* The main kernel a later call with this head dimension, mask, element type
 * and schedule runs under the current settings (attn_bwd_set_main_kernel
 * and the tile shape): ATTN_KERNEL_FOUR_WAVE or ATTN_KERNEL_PAIR; host only,
 * launches nothing.  Returns ATTN_ERR_INVALID_ARG for a bad mask, dtype or
 * schedule and ATTN_ERR_UNSUPPORTED for d not 64 or 128. */
int attn_bwd_resolve_main_kernel(int d, int causal, int dtype, int schedule);

/* Per-call times of the recording started by attn_bwd_set_timing(1): for
 * the first min(calls recorded, max_calls) calls, ms_total[i] (preprocess to
 * the end of the last kernel) and ms_main[i] (main kernel), either array may
 * be NULL; *calls receives the count written.  Waits for the recorded
 * events.  Returns ATTN_OK, ATTN_ERR_INVALID_ARG (nothing recorded,
 * max_calls < 0) or ATTN_ERR_HIP. */
int attn_bwd_get_call_times(float* ms_total, float* ms_main, int max_calls, int* calls);

/* Flag-wait instrumentation.  When enabled, the main kernel of later calls
 * accumulates, per launch, the clock cycles its work groups spent inside
 * dQ flag waits, the cycles spent in whole work items, and the number of
 * wait polls.  attn_bwd_get_wait_stats synchronises the device and returns
 * the totals of the last call. */
int attn_bwd_set_wait_stats(int on);
int attn_bwd_get_wait_stats(unsigned long long* wait_cycles, unsigned long long* item_cycles,
                            unsigned long long* polls);

/* Where the waits of the last call with wait statistics happened: cycles[64 *
 * 128] (caller's host buffer) receives, for each (work item of the head
 * modulo 64, position of the task in its item, positions past 127 counted as
 * 127), the clock cycles work groups spent waiting for that task's dQ flag,
 * summed over heads.  A schedule's reduction chains show up as the steps and
 * items where waits pile up.  Synchronises the device.  Returns ATTN_OK,
 * ATTN_ERR_INVALID_ARG (null buffer, no such call) or ATTN_ERR_HIP. */
int attn_bwd_get_wait_hist(unsigned long long* cycles);

/* The shader clock the main kernel of the last call with wait statistics
 * ran at, in MHz: each work group's span on the shader clock counter
 * (s_memtime) divided by its span on the constant-rate clock
 * (s_memrealtime, hipDeviceAttributeWallClockRate), summed over work
 * groups.  Returns ATTN_OK, ATTN_ERR_INVALID_ARG (no such call) or
 * ATTN_ERR_HIP. */
int attn_bwd_get_clock(double* mhz);

/* Reference rate for the ATOMIC schedule: fp32 global atomic adds without
 * return value on the current device, in the pattern of the ATOMIC main
 * kernel's dQ (one instruction adds 64 contiguous bytes to each of four rows
 * of a 128x128 fp32 tile; one work group of 256 threads per CU adds `tasks`
 * whole tiles, tile (group * 7 + task) mod ntiles of acc).  acc: device
 * buffer of acc_bytes (at least 65536, 256-byte aligned, overwritten;
 * ntiles = acc_bytes / 65536).  Runs one untimed and one timed launch on
 * `stream` (hipStream_t; NULL = default stream) and waits for them; *ms
 * receives the timed launch's duration, *adds its number of adds (either
 * may be NULL).  Measurement only: touches no attention state.  Returns
 * ATTN_OK, ATTN_ERR_INVALID_ARG (null or misaligned acc, acc_bytes < 65536,
 * tasks outside 1..65536) or ATTN_ERR_HIP. */
int attn_bwd_atomic_rate(void* acc, size_t acc_bytes, int tasks, void* stream, float* ms, double* adds);

/* Latency of one dQ hand-off between two work groups, for calibrating the
 * DAG model's reduction cost r and release edge e (the flag latency per
 * XCD distance, which the review page's cost model leaves open).  Work
 * group 0 and work group `pong` (1..63) take turns `iters` times (2..2^20):
 * a turn waits for a flag in device memory to reach its number (relaxed
 * agent-scope loads), then, for mode 1 or 2, reads the previous turn's
 * 64 KiB fp32 tile, adds to it and writes its own, waits for its stores and
 * moves the flag on (relaxed agent-scope store) - the main kernel's R phase.
 * mode 0: the flag alone; 1: the tile through the L2 of the XCD (plain
 * stores, L2-scope loads; meaningful when both groups share an XCD); 2: the
 * tile written through to memory and read from it, as between XCDs.  The
 * device deals work groups to its XCDs in turn, so `pong` selects the XCD
 * distance; *xcd_ping and *xcd_pong receive the XCD each group ran on.
 * buf: device buffer of at least attn_bwd_handoff_bytes() bytes, 256-byte
 * aligned, overwritten.  Runs on `stream` and waits for it; *ns receives
 * the time per turn in nanoseconds.  Every wait is bounded.  Returns
 * ATTN_OK, ATTN_ERR_INVALID_ARG, ATTN_ERR_TIMEOUT (a wait gave up) or
 * ATTN_ERR_HIP.  Measurement only: touches no attention state. */
int attn_bwd_handoff_latency(void* buf, size_t buf_bytes, int pong, int iters, int mode, void* stream,
                             double* ns, int* xcd_ping, int* xcd_pong);
size_t attn_bwd_handoff_bytes(void);

/* Test hooks for the failure and race paths (they change timing, never the
 * reduction order).  spin_limit: polls before a dQ flag wait gives up
 * (0: the default of 2^20).  wait_offset (0..65535, normally 0): added to
 * the flag value every wait looks for, so that with wait_offset > 0 no wait
 * is ever satisfied and every call reports ATTN_ERR_TIMEOUT through
 * attn_bwd_query_status once its bounded waits expire (results invalid; the
 * kernel still ends).  delay_seed (0: off): before each reduction phase a
 * work group sleeps a pseudo-random 0..8k cycles drawn from the seed, the
 * work item and the task, so that hand-offs happen at other times and in
 * other relative orders; results must stay bitwise the same.  Apply to
 * later calls.  Returns ATTN_OK or ATTN_ERR_INVALID_ARG. */
int attn_bwd_set_debug(unsigned spin_limit, int wait_offset, unsigned delay_seed);

/* ------------------------------------------------------------------------
 * Attention forward (device).  Not on the pages, which take O and lse as
 * given: Fig. 1 of the paper (review page caption) shows the tiled
 * FlashAttention whose forward this is, and the summary page's Experimental
 * setup benchmarks the backward, which consumes O and lse.  Computes, per
 * (b, h) and query row i, S_ij = scale * q_i . k_j (keys j > i masked when
 * causal), lse_i = log sum_j exp(S_ij) (natural log, fp32) and
 * O_i = sum_j exp(S_ij - lse_i) v_j, with online softmax over key tiles.
 * q, k, v, o: contiguous [b][h][s][d] device tensors of `dtype` (16-byte
 * aligned); lse: [b][h][s] fp32 device tensor (written).  Each work group
 * owns a block of output rows, so the result is bitwise reproducible and
 * independent of how work groups are scheduled.  Asynchronous on `stream`
 * (hipStream_t; NULL = default stream).  Returns ATTN_OK,
 * ATTN_ERR_INVALID_ARG (negative sizes, null or misaligned pointers, bad
 * causal or dtype, scale not positive and finite), ATTN_ERR_UNSUPPORTED (d
 * not 64 or 128, s > 262144) or ATTN_ERR_HIP (launch failure).  b*h == 0 or
 * s == 0 is a no-op.
 * ------------------------------------------------------------------------ */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int b, int h, int s, int d,
             int causal, int dtype, float scale, void* stream);

/* ------------------------------------------------------------------------
 * Schedule generator (host, no GPU needed).
 * Within one head with n = ceil(s/T) tiles, a schedule is a list of work
 * items; each item is an ordered list of (KV tile, Q tile) tasks and runs on
 * one work group; all tasks of one KV tile are contiguous in one item
 * (Axiom ledger: operations of a KV tile run contiguously on one SM).
 * rank[kv*n + q] is the position of KV tile kv in Q tile q's dQ
 * accumulation order (-1 for a task the causal mask removes), count[q] the
 * number of contributors of Q tile q.  Every head uses the same pattern.
 * ------------------------------------------------------------------------ */

/* Sizes of the schedule: number of work items per head and total tasks per
 * head.  Returns ATTN_OK, ATTN_ERR_INVALID_ARG or ATTN_ERR_UNSUPPORTED. */
int attn_sched_size(int n, int causal, int schedule, int* num_items, int* num_tasks);

/* Fills the schedule.  item_begin: num_items+1 ints (task range of each
 * item); task_kv, task_q: num_tasks ints each; rank: n*n ints; count: n ints.
 * Any output pointer may be NULL to skip it.  ATTN_SCHED_ATOMIC describes
 * the NAIVE visiting order with rank = -1 for every task (no order). */
int attn_sched_get(int n, int causal, int schedule, int* item_begin, int* task_kv, int* task_q,
                   int* rank, int* count);

/* Smallest number of simultaneously resident work groups with which the
 * schedule always makes progress when items are handed out in increasing
 * order: 1 for NAIVE, DESCENDING and ATOMIC (every wait points to an
 * earlier item), the KV tiles of a round for SHIFT (n up to 256, else
 * ceil(n / ceil(n / 256))) and the items per head for SYMMETRIC_SHIFT
 * (cyclic waits inside a round or a head).  Returns a negative status on
 * bad arguments. */
int attn_sched_min_workers(int n, int causal, int schedule);

/* Rectangular tiles: n KV tiles of Bc rows and ratio * n Q tiles of
 * Br = Bc / ratio rows (ratio 1..8; ratio 1 is the square case above).  Q
 * tile q sees KV tile kv under the causal mask when ratio * kv <= q.
 * NAIVE and DESCENDING keep their orders; SHIFT visits Q tiles
 * (ratio * kv + t) mod (ratio * n), so a head's items are on distinct Q tiles
 * at every step, and accumulates dQ in visiting order (no rounds: n <= 256);
 * SYMMETRIC_SHIFT (causal, n even) folds KV p with KV n-1-p into an item of
 * ratio * n + ratio tasks: phase 1 (KV p, Q ratio*h + (ratio*p + t) mod
 * (ratio*h)) for t < ratio*h, h = n/2; phase 2, with x = ratio*p + u for
 * u < ratio*h + ratio: (KV p, Q x) while x < ratio*h, else (KV n-1-p,
 * Q 3*ratio*h - 1 - x); dQ in step order.  rank: n * (ratio*n) ints,
 * [kv * ratio*n + q]; count: ratio*n ints.  Same returns as the square
 * calls. */
int attn_sched_size_rect(int n, int ratio, int causal, int schedule, int* num_items, int* num_tasks);
int attn_sched_get_rect(int n, int ratio, int causal, int schedule, int* item_begin, int* task_kv, int* task_q,
                        int* rank, int* count);
int attn_sched_min_workers_rect(int n, int ratio, int causal, int schedule);

/* ------------------------------------------------------------------------
 * DAG critical-path simulator (host).  Models the pages' DAG: every task is
 * a compute phase of cost c followed by a reduction phase of cost r; the
 * reduction of a task waits for the previous contributor to the same dQ
 * tile; a worker runs one phase at a time and blocks while waiting (review
 * page, "What carries the argument" and Axiom ledger).  `heads` copies of
 * the schedule run on `workers` workers; placement 0 deals items
 * round-robin in head-major order, placement 1 hands the next item to the
 * first worker that becomes free (the kernel's global ticket queue),
 * placement 2 models the kernel's XCD placement (worker w serves the queue
 * of XCD w % 8 with the chunks the kernel would use for this shape, and the
 * global queue when the kernel would fall back to it).
 * Outputs (any may be NULL): makespan, the summed time workers spent
 * blocked on waits, and the summed busy time (compute + reduction).
 * Returns ATTN_OK, ATTN_ERR_DEADLOCK or an argument error.
 * ------------------------------------------------------------------------ */
int attn_dagsim(int n, int causal, int schedule, int heads, int workers, int placement,
                double c, double r, double* makespan, double* wait_time, double* busy_time);

/* Same, with an edge cost: a reduction that follows another contributor's
 * reduction of the same dQ tile starts no earlier than e after it ended (the
 * time a release takes to reach the next contributor; under placement 2
 * only between workers of different XCDs, a hand-off within an XCD costing
 * nothing more).  The pages' model has e = 0 (review page, "Load-bearing
 * premise": zero-cost synchronisation edges); attn_dagsim is this with
 * e = 0. */
int attn_dagsim_edge(int n, int causal, int schedule, int heads, int workers, int placement,
                     double c, double r, double e, double* makespan, double* wait_time,
                     double* busy_time);

/* attn_dagsim_edge for rectangular tiles (n KV tiles, ratio Q tiles per KV
 * tile, as for attn_sched_get_rect); c and r are the costs of one
 * rectangular task. */
int attn_dagsim_rect(int n, int ratio, int causal, int schedule, int heads, int workers, int placement,
                     double c, double r, double e, double* makespan, double* wait_time, double* busy_time);

/* ------------------------------------------------------------------------
 * Schedule selection (host).  The review page ("If this is right") calls the
 * schedules complementary and has an implementation pick one per
 * configuration; this picks, among NAIVE, DESCENDING, SHIFT and
 * SYMMETRIC_SHIFT, the one with the smallest simulated makespan
 * (attn_dagsim_edge with the given placement) for `heads` heads of n tiles
 * on `workers` resident work groups with task costs c, r and edge cost e.  Schedules that
 * the shape does not admit (SYMMETRIC_SHIFT with odd n under the causal
 * mask) or that need more resident work groups than `workers` are skipped;
 * ties go to the lower schedule id.  Outputs (may be NULL): the schedule and
 * its makespan.  Returns ATTN_OK, ATTN_ERR_INVALID_ARG, or
 * ATTN_ERR_UNSUPPORTED when no schedule qualifies.
 * ------------------------------------------------------------------------ */
int attn_sched_select(int n, int causal, int heads, int workers, int placement, double c, double r,
                      double e, int* schedule, double* makespan);

/* ------------------------------------------------------------------------
 * Cost calibration of the DAG model (host).  The review page ("What would
 * settle it") asks whether measured kernels reach the model's bound
 * m*n*(c+r), and its editorial notes extend the model with synchronisation
 * costs; this fits the costs to measurements.  Sample k is a launch of
 * heads[k] heads of n[k] tiles with mask causal[k] and schedule schedule[k]
 * on workers[k] resident work groups that took measured[k] (> 0, any time
 * unit).  Returns c, r and e (per task or edge, same unit) minimising the
 * RMS relative error between the simulated makespans (attn_dagsim_edge with
 * the given placement) and the measurements, and that error.  r/c and e/c are
 * searched in [1e-4, 1e2] (e may also be 0): grids, then a pattern search.
 * Arrays are host memory of `count` elements, read only.  Returns ATTN_OK,
 * ATTN_ERR_INVALID_ARG, or ATTN_ERR_UNSUPPORTED when a sample cannot be
 * simulated (unsupported schedule, deadlock).
 * ------------------------------------------------------------------------ */
int attn_sched_fit(int count, const int* n, const int* causal, const int* schedule, const int* heads,
                   const int* workers, int placement, const double* measured, double* c, double* r,
                   double* e, double* rms);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_BWD_H */
