// The main backward kernel of the deterministic attention backward for
// gfx950 and the host templates that launch it, shared by the translation
// units that instantiate it (bwd_kernels.hip: d = 128 and the fp32 tiles;
// bwd_kernels_d64.hip: bf16 d = 64, compiled with the MFMA results in
// architectural registers).
//
// Method: DASH ("DASH: Deterministic Attention Scheduling for
// High-throughput Reproducible LLM Training").  Fig. 1 of the paper (as
// captioned on the pith.science review page) shows the tiled backward: the
// owner of a KV tile accumulates dK/dV locally while partial dQ tiles are
// reduced globally; the Problem section of the summary page says the
// deterministic mode serialises those dQ additions in a fixed order.
// The per-tile arithmetic is the softmax-attention gradient (no formulas are
// printed on the pages; this is the standard definition):
//   S = Q_j K_i^T,  P = exp(scale*S - lse_j),  dP = dO_j V_i^T,
//   dS = P o (dP - D_j),  dV_i += P^T dO_j,  dK_i += dS^T Q_j,
//   dQ_j += dS K_i  (scale applied to dK and dQ at the end).
//
// Mapping onto gfx950.  A work group of 4 wave64s owns one KV tile of T rows
// (T = 128 for bf16, 64 for fp32).  Wave w keeps K and V rows
// [w*T/4, (w+1)*T/4) of the tile in registers as MFMA B operands, its dK/dV
// accumulators in registers for the whole tile, and a K^T slice of D/4
// columns for the dQ contraction.  Q tiles stream through LDS in 64-row
// sub-steps, both row-major (A operands of S and dP) and transposed (B
// operands of dV and dK, whose contraction runs over query rows).  All five
// contractions use v_mfma_f32_16x16x32_bf16 (fp32 inputs: eight
// v_mfma_f32_16x16x4_f32 over the same 32-wide k slice).  The 16x16 output
// layout (lane l holds column l%16, rows 4*(l/16)..+3) is reused directly as
// the A operand of the next contraction by permuting the contraction index
// consistently in both operands, so P and dS never leave registers for dV
// and dK.  dS goes through LDS once for dQ.
//
// dQ reduction (the R phase of the pages' DAG).  Deterministic mode: the
// work group waits until the tile's flag equals its rank in the schedule's
// fixed order, adds its partial into the fp32 accumulator (rank 0 stores,
// the last contributor writes the output dQ in the output type), and
// publishes rank+1.  No float atomics.  Work groups of one head run on all
// eight XCDs, whose L2 caches are not coherent with each other, so every
// access to the accumulator and the flags is an agent-scope coherent access
// (the sc1 cache policy, which is how the gfx942-family memory model
// implements relaxed agent-scope atomics): such loads never return a stale
// L2 line and such stores are acknowledged only once visible device-wide.
// Release is therefore "sc1 stores; s_waitcnt vmcnt(0); barrier; sc1 flag
// store", acquire is "sc1 flag poll; barrier; sc1 loads", and no L2
// write-back or invalidate is needed (a buffer_wbl2 per release costs far
// more than the data it protects).  Atomic mode: unordered fp32 atomic adds,
// then a finalize kernel.
//
// Persistent grid: every work group takes work items from a ticket counter
// in increasing order; items are numbered head-major, so a head's items are
// all resident before any of them waits (see attn_sched_min_workers).
#pragma once

#include "attn_bwd.h"
#include "attn_device.h"
#include "internal.h"

namespace attn {

// A flag wait gives up after a bounded number of polls (by default 2^20;
// each poll sleeps ~64 cycles plus a memory round trip, so well under a
// second in all), sets the call's abort word and the device status word,
// and continues; once the abort word is set every later wait of the call is
// skipped, so a broken schedule ends the kernel quickly instead of hanging
// the device.
constexpr unsigned kSpinLimit = 1u << 20;

// Test hooks (attn_bwd_set_debug).  delay_seed != 0: before every R phase
// thread 0 sleeps a pseudo-random 0..31 x 256 cycles drawn from a hash of
// the seed, the work item and the task, so that hand-offs happen in other
// relative orders and at other times than in an undisturbed run; the
// results must not change.  wait_offset != 0: every wait looks for a flag
// value that is never published, so that the bounded wait expires.
__device__ inline unsigned mix32(unsigned x) {
    x ^= x >> 16;
    x *= 0x7feb352dU;
    x ^= x >> 15;
    x *= 0x846ca68bU;
    x ^= x >> 16;
    return x;
}

// XCD placement.  A work group takes its items from the queue of the XCD it
// runs on (HW_REG_XCC_ID), so a head's items run on one or a few XCDs and
// consecutive contributors of a dQ tile mostly share an L2.  The hardware
// deals the work groups of a launch to the eight XCDs of MI355X in turn
// (from an XCD that depends on the hardware queue), so every XCD holds at
// least grid / 8 of them, which the plan's chunk size fits.  The last work
// group to finish checks that every queue handed out all of its items.
// Each XCD keeps its own
// copy of the accumulator, written only through its own L2: a hand-off
// between work groups of one XCD stays in that L2 (plain stores, loads that
// skip only the CU's L1), and only a hand-off to another XCD is written
// through to memory and read from there.  One writer per copy means no
// line of a copy is ever dirty in two L2s, so no write-back can overwrite a
// newer value.  A flag word holds the
// contributions made so far (bits 0-23), the XCD id (bits 24-27) and queue
// (bits 28-30) of the last contributor, and whether it wrote its partial
// through to memory (bit 31).
constexpr unsigned kRankMask = 0xffffffu, kWroteThrough = 1u << 31;

struct KParams {
    const void *q, *k, *v, *dO;
    const float* lse2;   // lse * log2(e) [H][s_pad] (workspace; zero past s)
    const float* delta;  // -D = -rowsum(dO * O) [H][s_pad] (workspace; zero past s)
    void *dq, *dk, *dv;
    float* dq_acc;
    unsigned* flags;
    unsigned* ticket;   // counters[0]: next work item (one global queue)
    unsigned* queues;   // kQueues per-XCD tickets, then a count of finished work groups
    unsigned* abort;    // counters[1]: a wait of this call expired
    unsigned* status;   // device status word, reported by attn_bwd_query_status
    unsigned long long* stats;  // null unless wait statistics are on
    unsigned long long* whist;  // wait cycles per (item of the head mod 64, task position), or null
    const int* item_begin;
    const i32x4* tasks;  // {kv tile, q tile, rank, contributors} per task
    int H, s, n, items_per_head, s_pad;
    // XCD placement (XcdPlan; chunks == 0: one global queue and one
    // accumulator, every hand-off through memory)
    int chunks, groups;
    int bounds[kQueues + 1];  // chunk c of a head = items [bounds[c], bounds[c + 1])
    int chunk_shift, group_shift;  // log2 of chunks and of groups (both powers of two)
    long long acc_slots;  // heads of one XCD's accumulator copy
    long long total_items;
    float scale, scale_log2;
    unsigned spin_limit;   // polls before a flag wait gives up
    int wait_offset;       // test hook: added to the awaited flag value
    unsigned delay_seed;   // test hook: pseudo-random sleep before each R phase
};

// LDS of one work group:
//   sQ[2], sdO[2]  padded [BQ][D]   query rows of a sub-step (double buffer)
//   sK             padded [TILE][D] keys of the current KV tile (dQ operand)
//   sdS            [BR][TILE] (+pad) dS of the current task as [query][key], or
//                  (DST, bf16 and square tiles only) as [key][query]: a lane's
//                  four query rows of one key are then 8 contiguous bytes, one
//                  64-bit store
// TILE is the KV tile's rows (Bc), BR the Q tile's (Br); BR = TILE but for the
// rectangular 64-row Q tiles against 128-row KV tiles.
//   slse[2] (lse * log2 e), sdelta[2] (-D) [BQ]
//   the current item's task records, MAXT at a time (plus the next one)
//   a 1 KiB sink for copy slots with nothing to copy
template <typename T, int D, int TILE, int BR = TILE>
struct Layout {
    // query rows per sub-step (fp32 at d=128 halves it to stay within LDS)
    static constexpr int BQ = (sizeof(T) == 4 && D == 128) ? 32 : 64;
    // Q/dO buffers and sK are whole numbers of 1 KiB blocks: the last block
    // of a tile load writes (zeros) up to its end
    static constexpr int QB = (BQ * Pad<T, D>::RS + 1023) / 1024 * 1024;    // one Q (or dO) buffer
    static constexpr int KB = (TILE * Pad<T, D>::RS + 1023) / 1024 * 1024;  // sK
    static constexpr int LDSS = TILE + Elem<T>::kPad;
    static constexpr int SB = BR * LDSS * (int)sizeof(T);
    static constexpr int OFF_Q = 0, OFF_DO = 2 * QB, OFF_K = 4 * QB, OFF_S = OFF_K + KB;
    static constexpr int OFF_LSE = OFF_S + SB, OFF_DEL = OFF_LSE + 2 * BQ * 4;
    static constexpr int MAXT = 256;  // task records of an item held in LDS at a time
    static constexpr int OFF_TASK = OFF_DEL + 2 * BQ * 4;
    // 1 KiB that copy slots with nothing to copy write (nobody reads it)
    static constexpr int OFF_SINK = OFF_TASK + (MAXT + 1) * 16;
    static constexpr size_t bytes = OFF_SINK + 1024;
    static_assert(bytes <= 160 * 1024 - 64, "LDS budget of a gfx950 work group exceeded");
    static_assert(BR % BQ == 0 && TILE % BR == 0 && BQ % 32 == 0, "sub-step and tile shapes");
};

// Four waves per work group and one work group per CU (the LDS above allows
// no second), so each wave has a SIMD to itself and the SIMD's whole register
// file (512 per lane, VGPRs and AGPRs).  A wave owns TILE/4 KV rows: 32 for
// bf16, so every Q/dO operand fetched from LDS feeds two MFMAs, and the
// registers left over hold several operand fetches in flight.
constexpr int kWaves = 4, kThreads = 64 * kWaves;

// DST: dS in LDS as [key][query] (bf16 only).  Its stores take a quarter of
// the instructions of the sub-step's [query][key] ones, and the dQ contraction
// reads it through transposing reads (twice the instructions there); the two
// layouts give the same operands, so the same bits.  Measured, the balance
// favours it under Symmetric Shift at d = 128 (whose one-step reduction
// chains carry every sub-step's length) and not under the other schedules.
template <typename T, int D, int TILE, bool CAUSAL, bool DET, bool DST, int BR>
__global__ __launch_bounds__(kThreads, 1) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_main_kernel(KParams p) {
    static_assert(!DST || (sizeof(T) == 2 && BR == TILE), "the [key][query] dS layout is a bf16 square-tile layout");
    using E = Elem<T>;
    using V8 = typename E::vec8;
    using V4 = typename E::vec4;
    using L = Layout<T, D, TILE, BR>;
    constexpr int NW = kWaves;
    constexpr int BQ = L::BQ, NSUB = BR / BQ;  // sub-steps per task
    constexpr int RW = TILE / NW, NT = RW / 16;  // KV rows per wave, 16-row tiles
    constexpr int DW = D / NW, NDT = DW / 16;    // dQ columns per wave
    static_assert(RW % 16 == 0 && DW % 16 == 0, "wave shares must be whole 16-wide MFMA tiles");
    constexpr int KSD = D / 32, KSQ = BQ / 32, KSKV = TILE / 32;
    constexpr int MT = BQ / 16, DT = D / 16, MTT = BR / 16;  // MTT: 16-row tiles of a Q tile
    constexpr int LDSS = L::LDSS;

    extern __shared__ __align__(16) unsigned char smem[];
    lds_u8* const lsm = (lds_u8*)smem;  // LDS address space: no per-use conversion
    const unsigned lds_base = lds_addr(smem);
    unsigned char* sK = smem + L::OFF_K;
    T* sdS = reinterpret_cast<T*>(smem + L::OFF_S);
    __shared__ long long s_item;
    __shared__ unsigned s_prev;  // flag word left by the previous contributor

    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, c16 = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, in an SGPR
    // (kThreads per work group: lets the compiler drop the sink selection of
    // copy slots that never reach past a tile)
    __builtin_assume(w >= 0 && w < NW);
    const T* gK = static_cast<const T*>(p.k);
    const T* gV = static_cast<const T*>(p.v);
    T* gdQ = static_cast<T*>(p.dq);
    T* gdK = static_cast<T*>(p.dk);
    T* gdV = static_cast<T*>(p.dv);
    const int s = p.s, n = p.n;
    unsigned xcc;  // this work group's XCD
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
    xcc &= 0xfu;
    const int queue = (int)(xcc % kQueues);  // XCD placement: this XCD's queue
    // the items of a head that this queue serves: [chunk_lo(), chunk_hi())
    auto chunk_lo = [&]() { return p.bounds[queue & (p.chunks - 1)]; };
    auto chunk_hi = [&]() { return p.bounds[(queue & (p.chunks - 1)) + 1]; };
    if (DET && p.chunks && xcc >= (unsigned)kQueues && tid == 0) atomicOr(p.status, 2u);

    unsigned long long wait_cycles = 0, polls = 0, item_cycles = 0;
    // shader clock (s_memtime) and constant 100 MHz clock (s_memrealtime) at
    // the start: their spans give the clock the kernel actually ran at
    const unsigned long long clk0 = p.stats ? __builtin_readcyclecounter() : 0;
    const unsigned long long rt0 = p.stats ? __builtin_amdgcn_s_memrealtime() : 0;

    // dQ^T (deterministic) or dQ (atomic) of the task's whole Q tile, as
    // NSUB parts of BQ query rows, for this wave's DW columns, contracted
    // over the whole KV tile: A = K^T from sK (transposed reads), B = dS rows
    // from sdS (b128 reads of [query][key], or transposed reads of [key][query]
    // under DST).  Deterministic: C[d][q], a lane holds 4 consecutive d of one
    // query row (16-byte accumulator accesses).  Atomic: C[q][d], 16 lanes
    // hold 16 consecutive d of one row (64 contiguous bytes per atomic
    // instruction).  The loop runs over (32-key step, part) pairs, part
    // fastest, so each K^T operand feeds every part; the dS operands are
    // read two pairs ahead and the K^T operands one key step ahead of the
    // MFMAs that use them.  hook(std::integral_constant<int, pair>) runs at
    // the start of each pair, so that a caller can spread other instructions
    // over them.
    auto dq_tile = [&](f32x4 (&acc)[NSUB][NDT][MT], auto&& hook) {
#pragma unroll
        for (int part = 0; part < NSUB; ++part)
#pragma unroll
            for (int dtw = 0; dtw < NDT; ++dtw)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) acc[part][dtw][mt] = zero_vec<f32x4>();
        constexpr int NP = KSKV * NSUB;
        auto load_b = [&](auto pc, V8 (&b)[MT]) {
            constexpr int pi = decltype(pc)::value, ks = pi / NSUB, part = pi % NSUB;
            if constexpr (DST) {
                // keys 32ks + 8g .. +7 of query row part*BQ + 16mt + c16, down a
                // column of the [key][query] tile: two transposing reads
                constexpr int SRS = LDSS * 2;  // bytes per key row
                const lds_u8* ts = lsm + L::OFF_S + (8 * g + (c16 >> 2)) * SRS + 8 * (c16 & 3);
                static_for<0, MT>([&](auto mc) {
                    constexpr int o = ks * 32 * SRS + (part * BQ + decltype(mc)::value * 16) * 2;
                    b[decltype(mc)::value] = tr_frag<o, o + 4 * SRS>(ts);
                });
            } else {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    b[mt] = *reinterpret_cast<const V8*>(sdS + (part * BQ + mt * 16 + c16) * LDSS + ks * 32 + 8 * g);
            }
        };
        auto mm = [&](int part, const V8 (&a)[NDT], const V8 (&b)[MT]) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int dtw = 0; dtw < NDT; ++dtw)
                    acc[part][dtw][mt] = DET ? E::mma(acc[part][dtw][mt], a[dtw], b[mt])
                                             : E::mma(acc[part][dtw][mt], b[mt], a[dtw]);
        };
        V8 b[3][MT];  // dS operands, ring of three pairs
        load_b(std::integral_constant<int, 0>{}, b[0]);
        if constexpr (NP > 1) load_b(std::integral_constant<int, 1>{}, b[1]);
        if constexpr (sizeof(T) == 2) {
            using P = Pad<T, D>;
            const lds_u8* tk = lsm + L::OFF_K + (8 * g + (c16 >> 2)) * P::RS + (w * DW + 4 * (c16 & 3)) * 2;
            auto fetch = [&](auto ksc, V8 (&a)[NDT]) {
                constexpr int ks = decltype(ksc)::value;
                static_for<0, NDT>([&](auto jc) {
                    constexpr int o = ks * 32 * P::RS + decltype(jc)::value * 32;
                    a[decltype(jc)::value] = tr_frag<o, o + 4 * P::RS>(tk);
                });
            };
            V8 a[2][NDT];  // K^T operands, ring of two key steps
            fetch(std::integral_constant<int, 0>{}, a[0]);
            static_for<0, NP>([&](auto pc) {
                constexpr int pi = decltype(pc)::value, ks = pi / NSUB, part = pi % NSUB;
                if constexpr (part == 0 && ks + 1 < KSKV) fetch(std::integral_constant<int, ks + 1>{}, a[(ks + 1) % 2]);
                if constexpr (pi + 2 < NP) load_b(std::integral_constant<int, pi + 2>{}, b[(pi + 2) % 3]);
                hook(pc);
                mm(part, a[ks % 2], b[pi % 3]);
            });
        } else {
            V8 a[NDT];
            static_for<0, NP>([&](auto pc) {
                constexpr int pi = decltype(pc)::value, ks = pi / NSUB, part = pi % NSUB;
                if constexpr (part == 0) {
#pragma unroll
                    for (int dtw = 0; dtw < NDT; ++dtw)
                        a[dtw] = frag_col<T, D>(sK, ks * 32 + 8 * g, ks * 32 + 8 * g + 4, w * DW + dtw * 16, c16);
                }
                if constexpr (pi + 2 < NP) load_b(std::integral_constant<int, pi + 2>{}, b[(pi + 2) % 3]);
                hook(pc);
                mm(part, a, b[pi % 3]);
            });
        }
    };

    // The next work item (head * items_per_head + item of the head), or
    // total_items when there is none.  XCD placement: queue q belongs to
    // group q / chunks of `chunks` queues and serves chunk q % chunks of the
    // group's heads (heads g, g + groups, ...), in head order; every queue
    // of a group serves the same heads in the same order.
    auto next_item = [&]() -> long long {
        if (!DET || p.chunks == 0) return (long long)atomicAdd(p.ticket, 1u);
        const int grp = queue >> p.chunk_shift, lo = chunk_lo(), size = chunk_hi() - lo;
        if (size <= 0) return p.total_items;
        const unsigned k = atomicAdd(p.queues + queue, 1u);
        const long long head = grp + (long long)p.groups * (k / (unsigned)size);
        if (head >= p.H) return p.total_items;
        return head * p.items_per_head + lo + (int)(k % (unsigned)size);
    };

    for (;;) {
        if (tid == 0) s_item = next_item();
        __syncthreads();
        const long long item = s_item;
        __syncthreads();
        if (item >= p.total_items) break;
        const unsigned long long t_item0 = p.stats ? __builtin_readcyclecounter() : 0;
        const int head = (int)(item / p.items_per_head);
        const int pat = (int)(item % p.items_per_head);
        const size_t hoff = (size_t)head * s * D;
        const int t_beg = p.item_begin[pat], t_end = p.item_begin[pat + 1];
        // the item's task records, MAXT at a time plus the one after them, in
        // LDS: one broadcast LDS read per task instead of dependent scalar
        // loads, and the next task's Q tile (for the prefetch) always at hand
        i32x4* stask = reinterpret_cast<i32x4*>(smem + L::OFF_TASK);
        auto load_tasks = [&](int t0) {
            __syncthreads();  // readers of the previous records are done
            for (int i = tid; i <= L::MAXT && t0 + i < t_end; i += kThreads) stask[i] = p.tasks[t0 + i];
            __syncthreads();
        };
        auto next_q_of = [&](int t) {  // q tile of task t + 1 (< t_end)
            return __builtin_amdgcn_readfirstlane(stask[(t - t_beg) % L::MAXT + 1][1]);
        };

        // release of the last accumulator update, not yet published: every
        // wave waits for its sc1 stores to be acknowledged (device-wide
        // visible), then after a barrier one thread moves the flag on
        unsigned* pend_flag = nullptr;
        unsigned pend_val = 0;
        auto publish = [&]() {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            if (tid == 0) __hip_atomic_store(pend_flag, pend_val, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            pend_flag = nullptr;
        };
        // Q/dO double buffer: `buf` is the buffer the next sub-step reads;
        // `staged` says whether its rows were already requested
        int buf = 0;
        bool staged = false;
        // buffer resources over this head's rows (rows past s read as zero)
        const unsigned head_bytes = (unsigned)((size_t)s * D * sizeof(T));
        const u32x4 rq = rsrc_words(static_cast<const T*>(p.q) + hoff, head_bytes);
        const u32x4 rdo = rsrc_words(static_cast<const T*>(p.dO) + hoff, head_bytes);
        const u32x4 rk = rsrc_words(gK + hoff, head_bytes);
        const u32x4 rlse = rsrc_words(p.lse2 + (size_t)head * p.s_pad, (unsigned)(p.s_pad * 4));
        const u32x4 rdel = rsrc_words(p.delta + (size_t)head * p.s_pad, (unsigned)(p.s_pad * 4));
        // The copies of one sub-step's rows, as NSLOT issue slots per wave: the
        // wave's blocks of the Q tile, of the dO tile, then one slot for the
        // lse (wave 0) or D (wave 1) values of the rows.  A sub-step spreads
        // the slots of the next sub-step's prefetch over its first MFMA steps
        // instead of issuing them in one burst.
        constexpr int QITS = (L::QB / 1024 + NW - 1) / NW, NSLOT = 2 * QITS + 1;
        const unsigned sink = lds_base + L::OFF_SINK;
        auto issue_slot = [&](auto slotc, int b, int q0) {
            constexpr int slot = decltype(slotc)::value;
            // (d = 128: the destination add folded into the m0 write, measured
            // 2.7% faster under the causal mask; at d = 64 1% slower)
            if constexpr (slot < QITS) {
                const unsigned tile = lds_base + L::OFF_Q + b * L::QB;
                if constexpr (D == 128)
                    load_tile_block_c<T, D, BQ, NW, slot>(tile, tile + w * 1024, sink, rq, q0, w, lane);
                else
                    load_tile_block<T, D, BQ, NW>(tile, sink, rq, q0, w, lane, slot);
            } else if constexpr (slot < 2 * QITS) {
                const unsigned tile = lds_base + L::OFF_DO + b * L::QB;
                if constexpr (D == 128)
                    load_tile_block_c<T, D, BQ, NW, slot - QITS>(tile, tile + w * 1024, sink, rdo, q0, w, lane);
                else
                    load_tile_block<T, D, BQ, NW>(tile, sink, rdo, q0, w, lane, slot - QITS);
            } else if constexpr (BQ == 64) {
                const bool lw = w == 0, dw = w == 1;
                copy4_to_lds(lw ? rlse : rdel, lw || dw ? (unsigned)((q0 + lane) * 4) : kOutOfRange,
                             lw ? lds_base + L::OFF_LSE + b * BQ * 4 : (dw ? lds_base + L::OFF_DEL + b * BQ * 4 : sink));
            } else {
                if (w == 0) load_vec_async(lds_base + L::OFF_LSE + b * BQ * 4, rlse, q0, BQ, lane);
                if (w == 1) load_vec_async(lds_base + L::OFF_DEL + b * BQ * 4, rdel, q0, BQ, lane);
            }
        };
        auto issue_q = [&](int b, int q0) { static_for<0, NSLOT>([&](auto sc) { issue_slot(sc, b, q0); }); };
        // part `part` of NPART of the slots
        auto issue_q_part = [&](auto partc, auto npartc, int b, int q0) {
            constexpr int part = decltype(partc)::value, npart = decltype(npartc)::value;
            constexpr int per = (NSLOT + npart - 1) / npart;
            constexpr int lo = part * per, hi = (part + 1) * per < NSLOT ? (part + 1) * per : NSLOT;
            static_for<lo, hi>([&](auto sc) { issue_slot(sc, b, q0); });
        };
        f32x4 dK[NT][DT], dV[NT][DT];
        V8 Kr[NT][KSD], Vr[NT][KSD];
        // initial value of S in this lane's key column: 0, or -inf for a key
        // row past s, so that P = 0 there.  (Query rows past s need nothing:
        // their Q, dO, lse and D read as zero, so dS = 0 on them, and no
        // output row past s is stored.)
        float s_init[NT];

        // dK and dV of the run's KV tile to the outputs.  A lane's fragment
        // holds four rows of one column, so the values go through LDS (this
        // wave's rows of the K tile's region, free once every wave is done
        // with the run's last task) and leave as 16-byte row chunks: 1 KiB per
        // store instruction instead of four 32-byte row pieces.
        auto store_dkdv = [&](int kvt) {
            using P = Pad<T, D>;
            constexpr int CH = 16 / (int)sizeof(T);  // elements per 16-byte chunk
            constexpr int CPR = D / CH;              // chunks per row
            constexpr int RPI = 64 / CPR;            // rows per wave-wide instruction
            static_assert(RW % RPI == 0, "a wave's rows as whole instructions");
            using VC = T __attribute__((ext_vector_type(CH)));
            __syncthreads();  // every wave is done with sK and sdS
            unsigned char* stage = smem + L::OFF_K;
            auto put = [&](const f32x4 (&acc)[NT][DT], float mul, T* out) {
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            *reinterpret_cast<T*>(stage + (w * RW + nt * 16 + 4 * g + i) * P::RS +
                                                  (dt * 16 + c16) * (int)sizeof(T)) = E::from_f(mul * acc[nt][dt][i]);
#pragma unroll
                for (int j = 0; j < RW / RPI; ++j) {
                    const int lr = w * RW + j * RPI + lane / CPR, chunk = lane % CPR;
                    const VC v = *reinterpret_cast<const VC*>(stage + lr * P::RS + chunk * 16);
                    const int row = kvt * TILE + lr;
                    if (row < s) *reinterpret_cast<VC*>(out + hoff + (size_t)row * D + chunk * CH) = v;
                }
            };
            put(dV, 1.f, gdV);
            put(dK, p.scale, gdK);  // (this wave's rows only: no barrier between the two)
        };

        // The item's tasks, as runs of consecutive tasks on one KV tile: the
        // run keeps the tile's K/V operands and dK/dV accumulators in
        // registers and stores dK/dV at its end.
        load_tasks(t_beg);
        int t = t_beg;
        while (t < t_end) {
            const int kv = __builtin_amdgcn_readfirstlane(stask[(t - t_beg) % L::MAXT][0]);
            // this wave's K and V rows: B operands of S and dP for the run
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const int row = kv * TILE + w * RW + nt * 16 + c16;
                const size_t roff = hoff + (size_t)min(row, s - 1) * D;
#pragma unroll
                for (int ks = 0; ks < KSD; ++ks) {
                    Kr[nt][ks] = *reinterpret_cast<const V8*>(gK + roff + ks * 32 + 8 * g);
                    Vr[nt][ks] = *reinterpret_cast<const V8*>(gV + roff + ks * 32 + 8 * g);
                }
#pragma unroll
                for (int ks = 0; ks < KSD; ++ks)
                    if (row >= s) {
                        Kr[nt][ks] = zero_vec<V8>();
                        Vr[nt][ks] = zero_vec<V8>();
                    }
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    dK[nt][dt] = zero_vec<f32x4>();
                    dV[nt][dt] = zero_vec<f32x4>();
                }
                s_init[nt] = row < s ? 0.f : -__builtin_inff();
            }
            // the whole K tile in LDS (A operand of dQ^T), once every wave is
            // done with the previous tile's
            __syncthreads();
            load_tile_async<T, D, TILE, NW>(lds_base + L::OFF_K, rk, kv * TILE, w, lane);

            bool more;
            do {
                const i32x4 rec = stask[(t - t_beg) % L::MAXT];
                const int qt = __builtin_amdgcn_readfirstlane(rec[1]);

                // Causal mask: key column kloc of the KV tile is kept for query
                // row qloc of the Q tile when kloc <= qloc + qt * BR - kv * TILE,
                // which holds for every element once diag_off >= TILE - 1 (the
                // tasks the mask leaves have diag_off >= 0).
                const int diag_off = qt * BR - kv * TILE;

                const int rank = DET ? __builtin_amdgcn_readfirstlane(rec[2]) : 0;
                // item of the Q tile's next contributor (-1: this is the last)
                const int succ = DET ? __builtin_amdgcn_readfirstlane(rec[3]) : -1;
                unsigned* flag = p.flags + (size_t)head * n + qt;
                unsigned early = 0;  // tid 0: the flag as read before the last sub-step
                float* acc = p.dq_acc + (size_t)head * p.s_pad * D;  // atomic variant

#pragma unroll 1
                for (int sub = 0; sub < NSUB; ++sub) {
                    const int q0 = qt * BR + sub * BQ;
                    // ---- the Q/dO rows [q0, q0+BQ) are in buffer `buf` (prefetched
                    // during the previous sub-step, or loaded now at an item start)
                    if (!staged) issue_q(buf, q0);
                    // first row of the next sub-step (of this task or the next; at
                    // the item's end, a harmless copy of these rows again, which
                    // the item waits for before it ends)
                    const int q_next = sub + 1 < NSUB ? q0 + BQ : (t + 1 < t_end ? next_q_of(t) * BR : q0);
                    // landed for every wave, every wave done with the previous
                    // sub-step's dS, and the previous release's stores acknowledged
                    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                    __syncthreads();
                    // the next sub-step's rows go to the other buffer, issued
                    // during this sub-step's first MFMA steps
                    const int pf_buf = buf ^ 1;
                    staged = true;
                    // publish the previous release; then read this task's flag early:
                    // its latency hides behind the last sub-step (and a wait usually
                    // finds it already set).  Nothing waits on either here.
                    if (pend_flag) {
                        if (tid == 0) __hip_atomic_store(pend_flag, pend_val, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        pend_flag = nullptr;
                    }
                    if (DET && sub == NSUB - 1 && rank > 0 && tid == 0)
                        early = __hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    const unsigned char* sQ = smem + L::OFF_Q + buf * L::QB;
                    const unsigned char* sdO = smem + L::OFF_DO + buf * L::QB;
                    const float* slse = reinterpret_cast<const float*>(smem + L::OFF_LSE) + buf * BQ;
                    const float* sdelta = reinterpret_cast<const float*>(smem + L::OFF_DEL) + buf * BQ;
                    buf ^= 1;

                    // ---- the sub-step, in groups of 32 query rows.  Per group: S and
                    // dP (phase 1), P and dS (softmax), dV and dK (phase 2).  The
                    // source order below lets the scheduler overlap one group's
                    // MFMAs with the other group's softmax; the dS stores to LDS
                    // come last, so that no LDS store sits between the loads of
                    // the two groups.
                    f32x4 S[KSQ][2][NT], dP[KSQ][2][NT];
                    V8 aP[KSQ][NT], aS[KSQ][NT];
                    // S = Q K^T and dP = dO V^T (rows: queries, cols: this wave's keys)
                    auto phase1 = [&](auto gqc) {
                        constexpr int GQ = decltype(gqc)::value;
#pragma unroll
                        for (int m = 0; m < 2; ++m)
#pragma unroll
                            for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
                                for (int i = 0; i < 4; ++i) S[GQ][m][nt][i] = s_init[nt];
                                dP[GQ][m][nt] = zero_vec<f32x4>();
                            }
                        // LDS operands one 32-wide step ahead of the MFMAs that use them
                        V8 aq[2][2], ao[2][2];
                        auto fetch = [&](auto ksc) {
                            constexpr int ks = decltype(ksc)::value;
#pragma unroll
                            for (int m = 0; m < 2; ++m) {
                                aq[ks % 2][m] = frag_row<T, D>(sQ, (2 * GQ + m) * 16 + c16, ks * 32 + 8 * g);
                                ao[ks % 2][m] = frag_row<T, D>(sdO, (2 * GQ + m) * 16 + c16, ks * 32 + 8 * g);
                            }
                        };
                        fetch(std::integral_constant<int, 0>{});
                        static_for<0, KSD>([&](auto ksc) {
                            constexpr int ks = decltype(ksc)::value;
                            if constexpr (GQ == 0) issue_q_part(ksc, std::integral_constant<int, KSD>{}, pf_buf, q_next);
                            if constexpr (ks + 1 < KSD) fetch(std::integral_constant<int, ks + 1>{});
#pragma unroll
                            for (int m = 0; m < 2; ++m)
#pragma unroll
                                for (int nt = 0; nt < NT; ++nt) {
                                    S[GQ][m][nt] = E::mma(S[GQ][m][nt], aq[ks % 2][m], Kr[nt][ks]);
                                    dP[GQ][m][nt] = E::mma(dP[GQ][m][nt], ao[ks % 2][m], Vr[nt][ks]);
                                }
                        });
                    };
                    // P = exp(scale*S - lse), dS = P (dP - D), as the A operands of
                    // phase 2.  The contraction index (query row) is permuted alike
                    // in both operands there: slot (g, e) is row 32gq + 16(e/4) +
                    // 4g + e%4, which is where the 16x16 output layout of S left P
                    // and dS.
                    auto softmax = [&](auto gqc) {
                        constexpr int GQ = decltype(gqc)::value;
#pragma unroll
                        for (int m = 0; m < 2; ++m)
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                const int ql = (2 * GQ + m) * 16 + 4 * g + i;
                                const float l2 = slse[ql], dl = sdelta[ql];  // dl = -D
#pragma unroll
                                for (int nt = 0; nt < NT; ++nt) {
                                    float pv = __builtin_amdgcn_exp2f(S[GQ][m][nt][i] * p.scale_log2 - l2);
                                    if constexpr (CAUSAL)
                                        pv = (w * RW + nt * 16 + c16 <= sub * BQ + ql + diag_off) ? pv : 0.f;
                                    aP[GQ][nt][4 * m + i] = E::from_f(pv);
                                    aS[GQ][nt][4 * m + i] = E::from_f(pv * (dP[GQ][m][nt][i] + dl));
                                }
                            }
                    };
                    // dV += P^T dO, dK += dS^T Q over the group's rows
                    auto phase2 = [&](auto gqc) {
                        constexpr int GQ = decltype(gqc)::value;
                        if constexpr (sizeof(T) == 2) {
                            // dO and Q column operands PF 16-column steps ahead of
                            // the MFMAs that use them
                            using P = Pad<T, D>;
                            constexpr int ODO = L::OFF_DO - L::OFF_Q;
                            const lds_u8* tq = (const lds_u8*)sQ + (4 * g + (c16 >> 2)) * P::RS + 8 * (c16 & 3);
                            auto fetch = [&](auto dtc, V8& vq, V8& vo) {
                                constexpr int o = GQ * 32 * P::RS + decltype(dtc)::value * 32;
                                vq = tr_frag<o, o + 16 * P::RS>(tq);
                                vo = tr_frag<o + ODO, o + ODO + 16 * P::RS>(tq);
                            };
                            constexpr int PF = 2;  // steps in flight ahead of the MFMAs
                            V8 rq[PF + 1], ro[PF + 1];
                            static_for<0, (PF < DT ? PF : DT)>([&](auto jc) {
                                fetch(jc, rq[decltype(jc)::value], ro[decltype(jc)::value]);
                            });
                            static_for<0, DT>([&](auto dtc) {
                                constexpr int dt = decltype(dtc)::value;
                                if constexpr (dt + PF < DT)
                                    fetch(std::integral_constant<int, dt + PF>{}, rq[(dt + PF) % (PF + 1)],
                                          ro[(dt + PF) % (PF + 1)]);
#pragma unroll
                                for (int nt = 0; nt < NT; ++nt) {
                                    dV[nt][dt] = E::mma(dV[nt][dt], aP[GQ][nt], ro[dt % (PF + 1)]);
                                    dK[nt][dt] = E::mma(dK[nt][dt], aS[GQ][nt], rq[dt % (PF + 1)]);
                                }
                            });
                        } else {
                            const int rA = GQ * 32 + 4 * g, rB = GQ * 32 + 16 + 4 * g;
#pragma unroll
                            for (int dt = 0; dt < DT; ++dt) {
                                const V8 vq = frag_col<T, D>(sQ, rA, rB, dt * 16, c16);
                                const V8 vo = frag_col<T, D>(sdO, rA, rB, dt * 16, c16);
#pragma unroll
                                for (int nt = 0; nt < NT; ++nt) {
                                    dV[nt][dt] = E::mma(dV[nt][dt], aP[GQ][nt], vo);
                                    dK[nt][dt] = E::mma(dK[nt][dt], aS[GQ][nt], vq);
                                }
                            }
                        }
                    };
                    // dS to LDS for the dQ contraction, in the layout DST selects
                    auto store_ds = [&](auto gqc) {
                        constexpr int GQ = decltype(gqc)::value;
#pragma unroll
                        for (int m = 0; m < 2; ++m)
#pragma unroll
                            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                                for (int i = 0; i < 4; ++i) {
                                    const int q = sub * BQ + (2 * GQ + m) * 16 + 4 * g + i, key = w * RW + nt * 16 + c16;
                                    sdS[DST ? key * LDSS + q : q * LDSS + key] = aS[GQ][nt][4 * m + i];
                                }
                    };
                    if constexpr (sizeof(T) == 2 && NT == 2 && KSQ == 2) {
                        // The bf16 sub-step as an explicit instruction schedule.  The
                        // wave is alone on its SIMD, so no other wave hides its LDS
                        // latency or overlaps its VALU work with the matrix core.
                        // The sub-step is a sequence of MFMA slots (phase 1 of both
                        // groups, then phase 2 of both); each slot carries the work
                        // placed beside its MFMA: LDS operand reads two MFMA steps
                        // ahead of their use, the next sub-step's copies, a pair of
                        // softmax values of the other group (phase 2 of a group
                        // needs its whole softmax, phase 1 of the next does not),
                        // and the dS stores.  A scheduling fence closes each slot.
                        using P = Pad<T, D>;
                        constexpr int A = 8 * KSD, B = 4 * DT, NMF = 2 * A + 2 * B;
                        constexpr int ODO = L::OFF_DO - L::OFF_Q;
                        // phase-1 operands, PF1 steps ahead (a ring of PF1 + 1): [step][m]
                        constexpr int PF1 = 2, R1 = PF1 + 1;
                        V8 q1[R1][2], o1[R1][2];
                        // phase-2 operands, PF2 steps ahead of their MFMAs (a ring of
                        // PF2 + 1 steps): [step][Q/dO][lo/hi].  A wave's LDS throughput
                        // is what it has in flight over the LDS latency (~270 cycles
                        // under load), and a transposing read moves 512 bytes, so the
                        // 2 KiB that a phase-2 step consumes per 64 MFMA cycles need
                        // several steps in flight.
                        constexpr int PF2 = 4, R2 = PF2 + 1;
                        s16x4 t2[R2][2][2];
                        f32x4 lsev[2][2];  // [group][m]: lse * log2 e of rows 4g..4g+3
                        const lds_u8* tq = (const lds_u8*)sQ + (4 * g + (c16 >> 2)) * P::RS + 8 * (c16 & 3);
                        // read k (0..3) of phase-1 step j = (group, 32-wide d step)
                        auto rd1 = [&](auto jc, auto kc) {
                            constexpr int j = decltype(jc)::value, k = decltype(kc)::value;
                            constexpr int G = j / KSD, ks = j % KSD, m = k % 2;
                            if constexpr (k < 2)
                                q1[j % R1][m] = frag_row<T, D>(sQ, (2 * G + m) * 16 + c16, ks * 32 + 8 * g);
                            else
                                o1[j % R1][m] = frag_row<T, D>(sdO, (2 * G + m) * 16 + c16, ks * 32 + 8 * g);
                        };
                        // transposed read k (0..3) of phase-2 step u = (group, 16-wide d step)
                        auto rd2 = [&](auto uc, auto kc) {
                            constexpr int u = decltype(uc)::value, k = decltype(kc)::value;
                            constexpr int G = u / DT, dt = u % DT, isdo = k / 2, hi = k % 2;
                            constexpr int o = G * 32 * P::RS + dt * 32 + isdo * ODO + hi * 16 * P::RS;
                            t2[u % R2][isdo][hi] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tq + o));
                        };
                        auto op2 = [&](int slot, int isdo) {
                            return __builtin_bit_cast(V8, __builtin_shufflevector(t2[slot][isdo][0], t2[slot][isdo][1], 0,
                                                                                 1, 2, 3, 4, 5, 6, 7));
                        };
                        auto rd_lse = [&](auto Gc, auto kc) {
                            constexpr int G = decltype(Gc)::value, k = decltype(kc)::value, m = k % 2;
                            if constexpr (k < 2)
                                lsev[G][m] = *reinterpret_cast<const f32x4*>(slse + (2 * G + m) * 16 + 4 * g);
                        };
                        // softmax pair k (0..7) of group G: rows (m, 2ip..2ip+1), key tile nt
                        auto sm_pair = [&](auto Gc, auto kc) {
                            constexpr int G = decltype(Gc)::value, k = decltype(kc)::value;
                            constexpr int m = k / 4, nt = (k / 2) % 2, ip = k % 2;
#pragma unroll
                            for (int i = 2 * ip; i < 2 * ip + 2; ++i) {
                                const float pv = __builtin_amdgcn_exp2f(S[G][m][nt][i] * p.scale_log2 - lsev[G][m][i]);
                                aP[G][nt][4 * m + i] = E::from_f(pv);
                                aS[G][nt][4 * m + i] = E::from_f(pv * dP[G][m][nt][i]);  // dP holds dP - D
                            }
                        };
                        // dS stores.  DST ([key][query]): store k (0..7) = group, m, key
                        // tile; the lane's four query rows 4g..4g+3 of its key are two
                        // packed bf16 pairs of the phase-2 operand and 8 contiguous
                        // bytes: one 64-bit store.  Otherwise ([query][key]): store k
                        // (0..31) = group, m, key tile, row, each value its half of the
                        // packed pair (no second conversion; see the empty asm below).
                        constexpr int NDS = DST ? 8 : 32;
                        auto st_ds = [&](auto kc) {
                            constexpr int k = decltype(kc)::value;
                            if constexpr (DST) {
                                constexpr int G = k / 4, m = (k / 2) % 2, nt = k % 2;
                                const u32x4 words = __builtin_bit_cast(u32x4, aS[G][nt]);
                                const u32x2 pr = {words[2 * m], words[2 * m + 1]};
                                *reinterpret_cast<lds_u32x2*>(
                                    lsm + L::OFF_S + ((w * RW + nt * 16 + c16) * LDSS + sub * BQ + (2 * G + m) * 16 + 4 * g) * 2) = pr;
                            } else {
                                constexpr int G = k / 16, m = (k / 8) % 2, nt = (k / 4) % 2, i = k % 4;
                                constexpr int e = 4 * m + i;
                                const unsigned pair = __builtin_bit_cast(u32x4, aS[G][nt])[e / 2];
                                sdS[(sub * BQ + (2 * G + m) * 16 + 4 * g + i) * LDSS + w * RW + nt * 16 + c16] =
                                    __builtin_bit_cast(T, (unsigned short)(e % 2 ? pair >> 16 : pair));
                            }
                        };
                        auto mfma = [&](auto ic) {
                            constexpr int i = decltype(ic)::value;
                            if constexpr (i < 2 * A) {
                                constexpr int G = i / A, r = i % A, ks = r / 8, m = (r % 8) / 4, nt = (r % 4) / 2;
                                constexpr int j = G * KSD + ks;
                                if constexpr (r % 2 == 0)
                                    S[G][m][nt] = E::mma(S[G][m][nt], q1[j % R1][m], Kr[nt][ks]);
                                else
                                    dP[G][m][nt] = E::mma(dP[G][m][nt], o1[j % R1][m], Vr[nt][ks]);
                            } else {
                                constexpr int i2 = i - 2 * A, G = i2 / B, r = i2 % B, dt = r / 4, nt = (r % 4) / 2;
                                constexpr int u = G * DT + dt;
                                if constexpr (r % 2 == 0)
                                    dV[nt][dt] = E::mma(dV[nt][dt], aP[G][nt], op2(u % R2, 1));
                                else
                                    dK[nt][dt] = E::mma(dK[nt][dt], aS[G][nt], op2(u % R2, 0));
                            }
                        };
                        // S starts at 0, or at -inf where P must be 0: key rows
                        // past s, and (on the diagonal tile only) keys after the
                        // query, so the slots below need no mask
                        const bool diag = CAUSAL && diag_off < TILE;
#pragma unroll
                        for (int G = 0; G < 2; ++G)
#pragma unroll
                            for (int m = 0; m < 2; ++m) {
                                // dP's accumulation starts at -D of the lane's rows, so
                                // dS = P (dP - D) is one multiply per element in the
                                // softmax (the VALU work there does not shrink with d)
                                const f32x4 d0 = *reinterpret_cast<const f32x4*>(sdelta + (2 * G + m) * 16 + 4 * g);
#pragma unroll
                                for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
                                    for (int i = 0; i < 4; ++i) S[G][m][nt][i] = s_init[nt];
                                    dP[G][m][nt] = d0;
                                }
                            }
                        if (diag) {
#pragma unroll
                            for (int G = 0; G < 2; ++G)
#pragma unroll
                                for (int m = 0; m < 2; ++m)
#pragma unroll
                                    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                                        for (int i = 0; i < 4; ++i)
                                            if (w * RW + nt * 16 + c16 > sub * BQ + (2 * G + m) * 16 + 4 * g + i + diag_off)
                                                S[G][m][nt][i] = -__builtin_inff();
                        }
                        using I0 = std::integral_constant<int, 0>;
                        using I1 = std::integral_constant<int, 1>;
                        static_for<0, PF1>([&](auto jc) {
                            static_for<0, 4>([&](auto kc) { rd1(jc, kc); });
                        });
                        static_for<0, NMF>([&](auto ic) {
                            constexpr int i = decltype(ic)::value;
                            // a group's packed dS, once its softmax is complete and before
                            // phase 2 reads it, passes an empty asm that hides its origin
                            // from the optimiser: the dS stores then take their halves from
                            // these registers instead of converting the fp32 values again
                            // (emits no instruction, and no copy: nothing reads it earlier)
                            if constexpr (i == 2 * A || i == 2 * A + B) {
                                constexpr int G = i == 2 * A ? 0 : 1;
                                asm volatile("" : "+v"(aS[G][0]));  // (NT == 2 on this path)
                                asm volatile("" : "+v"(aS[G][1]));
                            }
                            mfma(ic);
                            // the next sub-step's copies, one every DSTEP slots of phase 1
                            constexpr int DSTEP = (2 * A - 8) / NSLOT;
                            if constexpr (i % DSTEP == 1 && i / DSTEP < NSLOT)
                                issue_slot(std::integral_constant<int, i / DSTEP>{}, pf_buf, q_next);
                            // phase-1 operands: step j during step j - PF1, one read per two MFMAs
                            if constexpr (i < 2 * A - 8 * PF1 && i % 2 == 0)
                                rd1(std::integral_constant<int, i / 8 + PF1>{}, std::integral_constant<int, (i % 8) / 2>{});
                            // lse and D of a group, a step before its softmax starts
                            if constexpr (i % 2 == 1 && i >= A - 16 && i < A - 8)
                                rd_lse(I0{}, std::integral_constant<int, (i - (A - 16)) / 2>{});
                            if constexpr (i % 2 == 1 && i >= 2 * A - 16 && i < 2 * A - 8)
                                rd_lse(I1{}, std::integral_constant<int, (i - (2 * A - 16)) / 2>{});
                            // phase-2 operands: steps 0 .. PF2-1 during the last PF2 / 2
                            // phase-1 steps, step u during step u - PF2
                            if constexpr (i >= 2 * A - 4 * PF2 && i < 2 * A)
                                rd2(std::integral_constant<int, (i - (2 * A - 4 * PF2)) / 4>{}, std::integral_constant<int, i % 4>{});
                            if constexpr (i >= 2 * A && i < 2 * A + 2 * B - 4 * PF2)
                                rd2(std::integral_constant<int, (i - 2 * A) / 4 + PF2>{}, std::integral_constant<int, i % 4>{});
                            // softmax of group 0 beside phase 1 of group 1, of group 1
                            // beside phase 2 of group 0
                            if constexpr (i >= A && i < 2 * A && (i - A) % (A / 8) == 0)
                                sm_pair(I0{}, std::integral_constant<int, (i - A) / (A / 8)>{});
                            if constexpr (i >= 2 * A && i < 2 * A + B && (i - 2 * A) % (B / 8) == 0)
                                sm_pair(I1{}, std::integral_constant<int, (i - 2 * A) / (B / 8)>{});
                            // dS stores spread over phase 2 of group 1
                            if constexpr (i >= 2 * A + B) {
                                constexpr int r = i - 2 * A - B;
                                if constexpr (NDS >= B) {
                                    static_for<0, NDS / B>([&](auto jc) {
                                        st_ds(std::integral_constant<int, r * (NDS / B) + decltype(jc)::value>{});
                                    });
                                } else if constexpr (r % (B / NDS) == 0) {
                                    st_ds(std::integral_constant<int, r / (B / NDS)>{});
                                }
                            }
                            __builtin_amdgcn_sched_barrier(0);
                        });
                    } else {
                        static_for<0, KSQ>([&](auto gqc) { phase1(gqc); });
                        static_for<0, KSQ>([&](auto gqc) {
                            softmax(gqc);
                            phase2(gqc);
                        });
                        static_for<0, KSQ>([&](auto gqc) { store_ds(gqc); });
                    }
                }

                // ---- R phase.  One barrier ends the last sub-step (all of dS is in
                // LDS) and, for rank > 0, the wait for this tile's turn: thread 0
                // waits for the flag before arriving.
                if (p.delay_seed && tid == 0) {
                    const unsigned nap = mix32(p.delay_seed ^ mix32((unsigned)item * 0x9e3779b9u + (unsigned)t)) & 31u;
                    for (unsigned z = 0; z < nap; ++z) __builtin_amdgcn_s_sleep(4);
                }
                if (DET && rank > 0 && tid == 0) {
                    const unsigned long long t0 = p.stats ? __builtin_readcyclecounter() : 0;
                    unsigned spins = 0;
                    unsigned seen = early;
                    const unsigned want = (unsigned)(rank + p.wait_offset) & kRankMask;
                    while ((seen & kRankMask) != want) {
                        if ((spins & 1023u) == 0 && __hip_atomic_load(p.abort, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
                            break;
                        __builtin_amdgcn_s_sleep(1);
                        if (++spins >= p.spin_limit) {
                            atomicOr(p.abort, 1u);
                            atomicOr(p.status, 1u);
                            break;
                        }
                        seen = __hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    }
                    if (p.stats) {
                        const unsigned long long dw = __builtin_readcyclecounter() - t0;
                        wait_cycles += dw;
                        polls += spins + 1;
                        atomicAdd(p.whist + (pat & 63) * 128 + min(t - t_beg, 127), dw);
                    }
                    s_prev = seen;
                }
                // d = 128: settle the early flag read in every lane here.  Left
                // pending (lanes other than thread 0 never use it), it makes the
                // compiler wait for every outstanding memory operation at the
                // next task's first LDS read, which then also waits for this R
                // phase's accumulator stores instead of letting them drain
                // behind the task setup (full-mask Shift at s = 8192 runs 2-3%
                // faster).  The d = 64 kernels have no such wait, and there the
                // settling wait, which also covers the prefetch of the next
                // rows, measured 2-9% slower.
                if constexpr (D == 128) asm volatile("" ::"v"(early));
                __syncthreads();
                if (DET) {
                    // this head's accumulator in the copy of queue qc
                    auto acc_copy = [&](unsigned qc) {
                        const size_t slot = p.chunks ? (size_t)qc * p.acc_slots + (head >> p.group_shift) : (size_t)head;
                        return make_rsrc(p.dq_acc + slot * p.s_pad * D, (unsigned)(p.s_pad * D * sizeof(float)));
                    };
                    // the previous contribution: from this XCD's L2 when it was made
                    // on this XCD, else from memory (where the contributor wrote it
                    // through; a hand-off between XCDs that was not written through
                    // means the work groups did not run where placement put them)
                    const unsigned pflag = rank > 0 ? __builtin_amdgcn_readfirstlane(s_prev) : 0u;
                    const bool same = ((pflag >> 24) & 0xfu) == xcc;
                    if (rank > 0 && !same && !(pflag & kWroteThrough) && tid == 0) atomicOr(p.status, 2u);
                    const __amdgpu_buffer_rsrc_t rprev = acc_copy((pflag >> 28) & 7u), racc = acc_copy(queue);
                    // write through unless the next contributor's item is served
                    // by this work group's queue
                    const bool wt = !p.chunks || succ < chunk_lo() || succ >= chunk_hi();
                    const int col0 = w * DW + 4 * g;
                    // The accumulator is stored as whole 16x16 tiles in the MFMA
                    // output layout (lane l's 4 values at 16*l bytes of the
                    // tile's 1 KiB), so every load and store instruction covers
                    // one contiguous KiB.
                    auto acc_off = [&](int mtt, int dtw) {
                        return (unsigned)((((qt * MTT + mtt) * (D / 16) + w * NDT + dtw) * 64 + lane) * 16);
                    };
                    // the accumulator rows of the whole tile, requested a few at a
                    // time between the 32-key steps of the dQ contraction, so that
                    // their issue and latency overlap it; every part's contraction
                    // comes before the first use of them
                    constexpr int NPREV = NDT * MTT, NSTEP = NSUB * KSKV, PER = (NPREV + NSTEP - 1) / NSTEP;
                    f32x4 prev[NDT][MTT];
                    f32x4 dq[NSUB][NDT][MT];
                    // one copy of the contraction per load policy (a policy is an
                    // immediate of the load: no branch between the MFMAs)
                    auto contract = [&](auto polc) {
                        constexpr int POL = decltype(polc)::value;
                        dq_tile(dq, [&](auto pc) {
                            // (rank 0 does not use them: no branch for it)
                            constexpr int step = decltype(pc)::value;
                            static_for<0, PER>([&](auto jc) {
                                constexpr int i = step * PER + decltype(jc)::value;
                                if constexpr (i < NPREV)
                                    prev[i / MTT][i % MTT] = __builtin_bit_cast(
                                        f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                   rprev, (int)acc_off(i % MTT, i / MTT), 0, POL));
                            });
                            // keep them here: the scheduler would otherwise sink
                            // every load below the contraction
                            __builtin_amdgcn_sched_barrier(0);
                        });
                    };
                    if (same)
                        contract(std::integral_constant<int, kCpolSc0>{});
                    else
                        contract(std::integral_constant<int, kCpolSc1>{});
                    // the sums, as the output dQ (last contributor), or stored
                    // through to memory, or into this XCD's L2: one copy each
                    auto emit = [&](auto modec) {
                        constexpr int MODE = decltype(modec)::value;  // 0 output, 1 through, 2 L2
#pragma unroll
                        for (int part = 0; part < NSUB; ++part) {
#pragma unroll
                            for (int dtw = 0; dtw < NDT; ++dtw)
#pragma unroll
                                for (int mt = 0; mt < MT; ++mt) {
                                    const int mtt = part * MT + mt;  // 16-row tile of the task's Q tile
                                    f32x4 v = dq[part][dtw][mt];
                                    if (rank > 0) v = prev[dtw][mtt] + v;
                                    if constexpr (MODE == 0) {
                                        // dQ = scale * sum in the output type
                                        const int row = qt * BR + mtt * 16 + c16;
                                        V4 o;
#pragma unroll
                                        for (int e = 0; e < 4; ++e) o[e] = E::from_f(p.scale * v[e]);
                                        if (row < s)
                                            *reinterpret_cast<V4*>(gdQ + hoff + (size_t)row * D + col0 + dtw * 16) = o;
                                    } else if constexpr (MODE == 1) {
                                        store_sc1(racc, acc_off(mtt, dtw), v);
                                    } else {
                                        store_l2(racc, acc_off(mtt, dtw), v);
                                    }
                                }
                        }
                    };
                    if (succ < 0)
                        emit(std::integral_constant<int, 0>{});
                    else if (wt)
                        emit(std::integral_constant<int, 1>{});
                    else
                        emit(std::integral_constant<int, 2>{});
                    if (succ >= 0) {
                        // published after the next barrier that follows a full
                        // s_waitcnt (next task's staging, or the end of the item)
                        pend_flag = flag;
                        pend_val = (unsigned)(rank + 1) | (xcc << 24) | ((unsigned)queue << 28) | (wt ? kWroteThrough : 0u);
                    }
                } else {
                    f32x4 dq[NSUB][NDT][MT];
                    dq_tile(dq, [](auto) {});
#pragma unroll
                    for (int part = 0; part < NSUB; ++part)
#pragma unroll
                        for (int dtw = 0; dtw < NDT; ++dtw)
#pragma unroll
                            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                                for (int i = 0; i < 4; ++i)
                                    unsafeAtomicAdd(acc + (size_t)(qt * BR + part * BQ + mt * 16 + 4 * g + i) * D + w * DW +
                                                        dtw * 16 + c16,
                                                    dq[part][dtw][mt][i]);
                }
                ++t;
                more = false;
                if (t < t_end) {
                    if ((t - t_beg) % L::MAXT == 0) load_tasks(t);
                    more = __builtin_amdgcn_readfirstlane(stask[(t - t_beg) % L::MAXT][0]) == kv;
                }
            } while (more);
            // The run's last release goes out now, once its stores are
            // acknowledged, not at the next run's first staging barrier: that
            // barrier comes only after the dK/dV stores and the next run's K/V
            // loads, and when the next contributor is itself on the last task
            // of its run (a reduction chain of run ends, as under Symmetric
            // Shift's fold) every link would add that delay to the chain.
            if (pend_flag) publish();
            store_dkdv(kv);
        }
        // the prefetch issued by the item's last sub-step lands before the
        // next item's first copies are issued
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        if (pend_flag) publish();
        if (p.stats) item_cycles += __builtin_readcyclecounter() - t_item0;
    }
    // XCD placement: the last work group to finish checks that every queue
    // handed out all of its items (an XCD without work groups would leave
    // its items undone)
    if (DET && p.chunks && tid == 0 && atomicAdd(p.queues + kQueues, 1u) == gridDim.x - 1) {
        for (int q = 0; q < kQueues; ++q) {
            const int grp = q / p.chunks, size = p.bounds[q % p.chunks + 1] - p.bounds[q % p.chunks];
            const long long heads = grp < p.H ? (p.H - grp + p.groups - 1) / p.groups : 0;
            const unsigned handed = __hip_atomic_load(p.queues + q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (size > 0 && (long long)handed < heads * size) atomicOr(p.status, 2u);
        }
    }
    if (p.stats && tid == 0) {
        atomicAdd(p.stats + 0, wait_cycles);
        atomicAdd(p.stats + 1, item_cycles);
        atomicAdd(p.stats + 2, polls);
        atomicAdd(p.stats + 3, __builtin_readcyclecounter() - clk0);
        atomicAdd(p.stats + 4, __builtin_amdgcn_s_memrealtime() - rt0);
    }
}

template <typename T, int D, int TILE, bool CAUSAL, bool DET, bool DST = false, int BR = TILE>
static int launch_main_t(const KParams& kp, const BwdLaunch& L) {
    auto kern = bwd_main_kernel<T, D, TILE, CAUSAL, DET, DST, BR>;
    const size_t smem = Layout<T, D, TILE, BR>::bytes;
    static bool attr_set = false;  // per instantiation; attribute is per device-function
    if (!attr_set) {
        if (hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem) != hipSuccess)
            return fail(ATTN_ERR_HIP, "hipFuncSetAttribute failed for the main kernel");
        attr_set = true;
    }
    int per_cu = 0;
    constexpr int nthreads = kThreads;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)kern, nthreads, smem) != hipSuccess ||
        per_cu < 1)
        return fail(ATTN_ERR_HIP, "occupancy query failed for the main kernel");
    const long long resident = (long long)per_cu * L.num_cus;
    if (L.min_workers > resident)
        return fail(ATTN_ERR_COSCHEDULE,
                    "schedule needs more simultaneously resident work groups than the device holds");
    const long long grid = std::min<long long>(resident, kp.total_items);
    if (grid <= 0) return ATTN_OK;
    KParams k = kp;
    // the XCD plan was made for one work group per CU: it holds for any
    // larger grid (checked anyway; the accumulator always has room for the
    // global queue's one copy)
    const XcdPlan& pl = L.plan;
    if (DET && pl.chunks && grid / kQueues >= 1 && (L.min_workers <= 1 || pl.max_chunk <= grid / kQueues)) {
        k.chunks = pl.chunks;
        for (int c = 0; c <= kQueues; ++c) k.bounds[c] = pl.bounds[c];
        k.groups = pl.groups;
        k.acc_slots = pl.slots;
        k.chunk_shift = __builtin_ctz((unsigned)pl.chunks);
        k.group_shift = __builtin_ctz((unsigned)pl.groups);
    }
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(nthreads), smem, (hipStream_t)L.stream, k);
    if (hipGetLastError() != hipSuccess) return fail(ATTN_ERR_HIP, "main kernel launch failed");
    return ATTN_OK;
}

template <typename T, int D, int TILE, int BR = TILE>
static int launch_main_d(const KParams& kp, const BwdLaunch& L, bool causal, bool det, bool dst) {
    if constexpr (sizeof(T) == 2 && D == 128 && TILE == 128 && BR == TILE) {
        if (causal && det && dst) return launch_main_t<T, D, TILE, true, true, true>(kp, L);
    }
    if (causal)
        return det ? launch_main_t<T, D, TILE, true, true, false, BR>(kp, L)
                   : launch_main_t<T, D, TILE, true, false, false, BR>(kp, L);
    return det ? launch_main_t<T, D, TILE, false, true, false, BR>(kp, L)
               : launch_main_t<T, D, TILE, false, false, false, BR>(kp, L);
}

}  // namespace attn
