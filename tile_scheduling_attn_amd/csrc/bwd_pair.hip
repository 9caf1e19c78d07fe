// The deterministic main kernel for bf16, d = 64 or 128, 128 x 128 tiles,
// with two waves per SIMD ("pair" kernel).
//
// Same method, same task records, flags, accumulator layout and XCD
// placement as bwd_main_kernel (bwd_main.h); what differs is how a work group
// spreads a task over its waves.  bwd_main_kernel gives each of its four
// waves 32 KV rows and a SIMD of its own, and with one wave per SIMD nothing
// overlaps that wave's softmax, LDS reads and copies with its MFMAs: a
// 64-row sub-step issues about 630 instructions per wave against 2048 cycles
// of matrix work, at one instruction per four cycles.  Here eight waves run
// as four pairs; both waves of pair sl hold K and V of the same 32 KV rows
// (rows [32 sl, 32 sl + 32) of the tile) as MFMA B operands, and the pair
// splits each 64-row sub-step by role:
//
//   role 0: S, dP and the softmax of query rows 0..31 of the sub-step
//           (group 0), and dV of the pair's rows over all 64 query rows;
//   role 1: the same for query rows 32..63 (group 1), and dK.
//
// A role needs one operand of the other group: role 0 takes P of group 1
// and role 1 takes dS of group 0, through LDS, after one barrier in the
// middle of the sub-step.  dS goes to LDS anyway (the dQ contraction reads
// it); P of group 1 takes an extra 8 KiB exchange area.  Each wave keeps 64
// accumulator registers (dV or dK) instead of 128, which is what lets two
// waves share a SIMD's 512 registers per lane; per pair the LDS operand
// traffic is that of one bwd_main_kernel wave (each role reads the Q/dO rows
// of its own group for S and dP, and dO or Q of both groups for dV or dK).
//
// The sums run in the same order as in bwd_main_kernel: S and dP over the
// 32-wide d steps in order, dV and dK over group 0 then group 1 of each
// sub-step, dQ over the 32-key steps in order, and the accumulator in the
// schedule's rank order.  Every MFMA sees the same operands, so the outputs
// are bitwise those of bwd_main_kernel.
//
// Both waves of a pair run the same code; the role only selects addresses
// and which A operand of phase 2 comes from registers.  Two waves per SIMD
// leave each 256 registers: the K/V operands (64) and the dV or dK
// accumulators (64) stay resident, and the rest of a phase must fit beside
// them, which is why per-lane addresses are re-derived at each phase and the
// kernel parameters of the reduction phase are read where they are used.
// Measured on MI355X at s = 8192 and 16384, d = 128, against bwd_main_kernel:
// without the reduction phase the sub-steps are 11-13% slower (the single
// wave's explicit instruction schedule hides its softmax under its own MFMAs,
// while here the two waves of a SIMD meet the exchange barrier together), the
// reduction phase is faster (eight waves keep more accumulator loads and
// stores in flight), and whole launches are 0-2% faster under the causal mask
// (Descending most) and about 4% slower under the full mask, hence the
// default choice of the library (the pair kernel under the causal mask at
// d = 128).  At d = 64 it is 8-19% slower than the four-wave kernel of that
// head dimension.
//
// Method: DASH (Deterministic Attention Scheduling), Fig. 1 of the paper as
// captioned on the pith.science review page (tiled backward: dK/dV local to
// the owner of a KV tile, dQ reduced globally) and the Problem section of the
// summary page (the deterministic mode serialises the dQ additions in a
// fixed order).
#include "bwd_main.h"

namespace attn {

namespace {

constexpr int kPairWaves = 8, kPairThreads = 64 * kPairWaves;

// LDS of one work group:
//   sQ[2], sdO[2]  padded [64][128]  query rows of a sub-step (double buffer)
//   sK             padded [128][128] keys of the current KV tile (dQ operand)
//   sdS            [128 keys][128 queries + 16]: dS of the task as
//                  [key][query] (a lane's four query rows of one key are 8
//                  contiguous bytes); at a run's end, the dK staging rows
//   sP             [128 keys][32 queries + 4]: P of the sub-step's group 1
//   slse[2], sdelta[2] (-D) [64]
//   the current item's task records, MAXT at a time (plus the next one)
//   a 1 KiB sink for copy slots with nothing to copy
template <int D>
struct PairLayout {
    using P = Pad<bf16, D>;
    static constexpr int BQ = 64;
    static constexpr int QB = (BQ * P::RS + 1023) / 1024 * 1024;
    static constexpr int KB = (128 * P::RS + 1023) / 1024 * 1024;
    static constexpr int LDSS = 128 + 16;
    static constexpr int SB = 128 * LDSS * 2;
    // P rows of 72 bytes: the 16 keys of a 16-lane group's 8-byte accesses
    // then start 18 dwords apart and fall in distinct banks (measured: 10%
    // fewer LDS bank-conflict cycles per launch than 80-byte rows, 25% fewer
    // than 96-byte rows)
    static constexpr int PSS = 32 + 4;
    static constexpr int PB = 128 * PSS * 2;
    static constexpr int OFF_Q = 0, OFF_DO = 2 * QB, OFF_K = 4 * QB, OFF_S = OFF_K + KB, OFF_P = OFF_S + SB;
    static constexpr int OFF_LSE = OFF_P + PB, OFF_DEL = OFF_LSE + 2 * BQ * 4;
    static constexpr int MAXT = 64;
    static constexpr int OFF_TASK = OFF_DEL + 2 * BQ * 4;
    static constexpr int OFF_SINK = OFF_TASK + (MAXT + 1) * 16;
    static constexpr size_t bytes = OFF_SINK + 1024;
    static_assert(bytes <= 160 * 1024 - 64, "LDS budget of a gfx950 work group exceeded");
    static_assert(SB >= 128 * P::RS && KB >= 128 * P::RS, "dV and dK staging rows at a run's end");
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kPairThreads, 1) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_pair_kernel(KParams p) {
    using T = bf16;
    using E = Elem<T>;
    using V8 = bf16x8;
    using V4 = bf16x4;
    using L = PairLayout<D>;
    using P = Pad<T, D>;
    constexpr int TILE = 128, BR = 128, BQ = 64, NSUB = 2, NW = kPairWaves;
    constexpr int KSD = D / 32, DT = D / 16, MTT = BR / 16, KSKV = TILE / 32;  // 32-wide steps over d and over keys
    constexpr int DW = D / 4, NDT = DW / 16, MT = 4;  // dQ per wave: D/4 d columns x 64 query rows
    constexpr int LDSS = L::LDSS, SRS = LDSS * 2, PRS = L::PSS * 2;
    constexpr int ODO = L::OFF_DO - L::OFF_Q;
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;

    extern __shared__ __align__(16) unsigned char smem[];
    lds_u8* const lsm = (lds_u8*)smem;
    const unsigned lds_base = lds_addr(smem);
    __shared__ long long s_item;
    __shared__ unsigned s_prev;

    const int tid = threadIdx.x;
    // lane, g (lane / 16) and c16 (lane % 16) are re-derived from an opaque copy of
    // the lane id at the start of every phase: the compiler would otherwise hoist
    // every per-lane address out of the loops and hold it for the whole kernel
    int lane = tid & 63, g = lane >> 4, c16 = lane & 15;
    auto relane = [&]() {
        int l = tid & 63;
        asm volatile("" : "+v"(l));
        lane = l;
        g = l >> 4;
        c16 = l & 15;
    };
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    __builtin_assume(w >= 0 && w < NW);
    const int sl = w & 3;     // the pair: KV rows [32 sl, 32 sl + 32) of the tile
    const int role = w >> 2;  // query group of each sub-step; 0: dV, 1: dK
    const int dblk = w & 3, part = w >> 2;  // dQ: d columns [DW dblk, +DW), query rows [64 part, +64)
    const T* gK = static_cast<const T*>(p.k);
    const T* gV = static_cast<const T*>(p.v);
    T* gdQ = static_cast<T*>(p.dq);
    const int s = p.s, n = p.n;
    unsigned xcc;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
    xcc &= 0xfu;
    const int queue = (int)(xcc % kQueues);
    auto chunk_lo = [&]() { return p.bounds[queue & (p.chunks - 1)]; };
    auto chunk_hi = [&]() { return p.bounds[(queue & (p.chunks - 1)) + 1]; };
    if (p.chunks && xcc >= (unsigned)kQueues && tid == 0) atomicOr(p.status, 2u);
    // the parameters through an opaque pointer: a field read through it is
    // loaded (scalar cache) where it is used instead of occupying a scalar
    // register for the whole kernel
    // (KParams is the kernel's only argument, at the start of its kernarg
    // segment)
    auto kpar = [&]() -> const KParams& {
        const __attribute__((address_space(4))) KParams* r =
            (const __attribute__((address_space(4))) KParams*)__builtin_amdgcn_kernarg_segment_ptr();
        asm volatile("" : "+s"(r));
        return *(const KParams*)r;
    };

    unsigned long long wait_cycles = 0, polls = 0, item_cycles = 0;
    const unsigned long long clk0 = p.stats ? __builtin_readcyclecounter() : 0;
    const unsigned long long rt0 = p.stats ? __builtin_amdgcn_s_memrealtime() : 0;

    // the next work item (as in bwd_main_kernel)
    auto next_item = [&]() -> long long {
        if (p.chunks == 0) return (long long)atomicAdd(p.ticket, 1u);
        const int grp = queue >> p.chunk_shift, lo = chunk_lo(), size = chunk_hi() - lo;
        if (size <= 0) return p.total_items;
        const unsigned k = atomicAdd(p.queues + queue, 1u);
        const long long head = grp + (long long)p.groups * (k / (unsigned)size);
        if (head >= p.H) return p.total_items;
        return head * p.items_per_head + lo + (int)(k % (unsigned)size);
    };

    // The copies of a sub-step's Q (or dO) rows as 1 KiB blocks of the padded
    // LDS tile dealt over the waves: block w + NW * IT of this wave, lane l
    // writing its bytes [16 l, 16 l + 16).  cvoff[IT] is the lane's source
    // offset relative to the rows' start (out of range where the lane falls
    // in a row's padding or past the tile: the copy then writes zeros), fixed
    // for the kernel.
    constexpr int QTOTAL = BQ * P::RS, QBLOCKS = (QTOTAL + 1023) / 1024;
    constexpr int QITS = (L::QB / 1024 + NW - 1) / NW, NSLOT = 2 * QITS + 1;
    unsigned cvoff[QITS];
#pragma unroll
    for (int it = 0; it < QITS; ++it) {
        const int byte = (w + NW * it) * 1024 + lane * 16;
        const int row = byte / P::RS, inrow = byte % P::RS;
        cvoff[it] = (byte < QTOTAL && inrow < P::RB) ? (unsigned)(row * P::RB + inrow) : kOutOfRange;
    }

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
        i32x4* stask = reinterpret_cast<i32x4*>(smem + L::OFF_TASK);
        auto load_tasks = [&](int t0) {
            __syncthreads();
            for (int i = tid; i <= L::MAXT && t0 + i < t_end; i += kPairThreads) stask[i] = p.tasks[t0 + i];
            __syncthreads();
        };
        auto next_q_of = [&](int t) { return __builtin_amdgcn_readfirstlane(stask[(t - t_beg) % L::MAXT + 1][1]); };

        unsigned* pend_flag = nullptr;
        unsigned pend_val = 0;
        auto publish = [&]() {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            if (tid == 0) __hip_atomic_store(pend_flag, pend_val, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            pend_flag = nullptr;
        };
        int buf = 0;
        bool staged = false;
        const unsigned head_bytes = (unsigned)((size_t)s * D * sizeof(T));
        const u32x4 rq = rsrc_words(static_cast<const T*>(p.q) + hoff, head_bytes);
        const u32x4 rdo = rsrc_words(static_cast<const T*>(p.dO) + hoff, head_bytes);
        const u32x4 rk = rsrc_words(gK + hoff, head_bytes);
        const u32x4 rlse = rsrc_words(p.lse2 + (size_t)head * p.s_pad, (unsigned)(p.s_pad * 4));
        const u32x4 rdel = rsrc_words(p.delta + (size_t)head * p.s_pad, (unsigned)(p.s_pad * 4));
        // the copies of one sub-step's rows as NSLOT issue slots per wave: the
        // wave's 1 KiB blocks of the Q rows, of the dO rows, then the lse (wave
        // 0) or D (wave 1) values of the rows
        const unsigned sink = lds_base + L::OFF_SINK;
        auto issue_slot = [&](auto slotc, int b, int q0) {
            constexpr int slot = decltype(slotc)::value;
            if constexpr (slot < 2 * QITS) {
                // block IT of this wave in the Q (or dO) rows [q0, q0 + 64): the
                // lane's precomputed offset plus the rows' start
                constexpr int IT = slot % QITS;
                const unsigned tile = lds_base + (slot < QITS ? L::OFF_Q : L::OFF_DO) + b * L::QB;
                const unsigned voff = cvoff[IT] + (unsigned)(q0 * P::RB);
                if constexpr (NW - 1 + NW * IT < QBLOCKS)
                    copy16_to_lds_at<(unsigned)(NW * IT * 1024)>(slot < QITS ? rq : rdo, voff, tile + w * 1024);
                else
                    copy16_to_lds(slot < QITS ? rq : rdo, voff, w + NW * IT < QBLOCKS ? tile + (w + NW * IT) * 1024 : sink);
            } else {
                const bool lw = w == 0, dw = w == 1;
                copy4_to_lds(lw ? rlse : rdel, lw || dw ? (unsigned)((q0 + lane) * 4) : kOutOfRange,
                             lw ? lds_base + L::OFF_LSE + b * BQ * 4 : (dw ? lds_base + L::OFF_DEL + b * BQ * 4 : sink));
            }
        };
        auto issue_q = [&](int b, int q0) { static_for<0, NSLOT>([&](auto sc) { issue_slot(sc, b, q0); }); };

        // dV (role 0) or dK (role 1) of the pair's 32 KV rows, fp32
        f32x4 acc2[2][DT];
        V8 Kr[2][KSD], Vr[2][KSD];
        float s_init[2];

        // dV and dK of the run's KV tile to the outputs, through LDS (role 0
        // stages dV in the K tile's region, role 1 dK in the dS region; both
        // are free once every wave is done with the run's last task), leaving
        // as 16-byte row chunks
        auto store_dkdv = [&](int kvt) {
            constexpr int CH = 8, CPR = D / CH, RPI = 64 / CPR;
            using VC = T __attribute__((ext_vector_type(CH)));
            __syncthreads();
            relane();
            unsigned char* stage = smem + (role ? L::OFF_S : L::OFF_K);
            const float mul = role ? p.scale : 1.f;
            T* out = static_cast<T*>(role ? p.dk : p.dv);
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        *reinterpret_cast<T*>(stage + (sl * 32 + nt * 16 + 4 * g + i) * P::RS + (dt * 16 + c16) * 2) =
                            E::from_f(mul * acc2[nt][dt][i]);
#pragma unroll
            for (int j = 0; j < 32 / RPI; ++j) {
                const int lr = sl * 32 + j * RPI + lane / CPR, chunk = lane % CPR;
                const VC v = *reinterpret_cast<const VC*>(stage + lr * P::RS + chunk * 16);
                const int row = kvt * TILE + lr;
                if (row < s) *reinterpret_cast<VC*>(out + hoff + (size_t)row * D + chunk * CH) = v;
            }
        };

        load_tasks(t_beg);
        int t = t_beg;
        while (t < t_end) {
            const int kv = __builtin_amdgcn_readfirstlane(stask[(t - t_beg) % L::MAXT][0]);
            relane();
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                const int row = kv * TILE + sl * 32 + nt * 16 + c16;
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
                for (int dt = 0; dt < DT; ++dt) acc2[nt][dt] = zero_vec<f32x4>();
                s_init[nt] = row < s ? 0.f : -__builtin_inff();
            }
            __syncthreads();
            load_tile_async<T, D, TILE, NW>(lds_base + L::OFF_K, rk, kv * TILE, w, lane);

            bool more;
            do {
                const i32x4 rec = stask[(t - t_beg) % L::MAXT];
                const int qt = __builtin_amdgcn_readfirstlane(rec[1]);
                const int diag_off = qt * BR - kv * TILE;
                const int rank = __builtin_amdgcn_readfirstlane(rec[2]);
                const int succ = __builtin_amdgcn_readfirstlane(rec[3]);
                unsigned* flag = p.flags + (size_t)head * n + qt;
                unsigned early = 0;

#pragma unroll 1
                for (int sub = 0; sub < NSUB; ++sub) {
                    const int q0 = qt * BR + sub * BQ;
                    if (!staged) issue_q(buf, q0);
                    const int q_next = sub + 1 < NSUB ? q0 + BQ : (t + 1 < t_end ? next_q_of(t) * BR : q0);
                    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                    __syncthreads();
                    const int pf_buf = buf ^ 1;
                    staged = true;
                    if (pend_flag) {
                        if (tid == 0) __hip_atomic_store(pend_flag, pend_val, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        pend_flag = nullptr;
                    }
                    if (sub == NSUB - 1 && rank > 0 && tid == 0)
                        early = __hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    const unsigned char* sQ = smem + L::OFF_Q + buf * L::QB;
                    const unsigned char* sdO = smem + L::OFF_DO + buf * L::QB;
                    const float* slse = reinterpret_cast<const float*>(smem + L::OFF_LSE) + buf * BQ;
                    const float* sdelta = reinterpret_cast<const float*>(smem + L::OFF_DEL) + buf * BQ;
                    buf ^= 1;

                    // ---- first half, the same code for both roles: S, dP and the
                    // softmax of the role's 32 query rows (qr0 = 32 * role within the
                    // sub-step); dS (and for role 1, P) to LDS
                    const int qr0 = role * 32;
                    f32x4 S[2][2], dP[2][2];  // [m][nt]: rows qr0 + 16m.., keys 16nt..
#pragma unroll
                    for (int m = 0; m < 2; ++m) {
                        // dP starts at -D of the lane's rows (as in the four-wave
                        // kernel, so the two give the same bits)
                        const f32x4 d0 = *reinterpret_cast<const f32x4*>(sdelta + qr0 + m * 16 + 4 * g);
#pragma unroll
                        for (int nt = 0; nt < 2; ++nt) {
#pragma unroll
                            for (int i = 0; i < 4; ++i) S[m][nt][i] = s_init[nt];
                            dP[m][nt] = d0;
                        }
                    }
                    if (CAUSAL && diag_off < TILE) {
#pragma unroll
                        for (int m = 0; m < 2; ++m)
#pragma unroll
                            for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                                for (int i = 0; i < 4; ++i)
                                    if (sl * 32 + nt * 16 + c16 > sub * BQ + qr0 + m * 16 + 4 * g + i + diag_off)
                                        S[m][nt][i] = -__builtin_inff();
                    }
                    // the step's Q and dO operands are read at the step (the other
                    // wave of the SIMD covers their latency)
                    const unsigned char* sQr = sQ + qr0 * P::RS;
                    const unsigned char* sdOr = sdO + qr0 * P::RS;
                    static_for<0, KSD>([&](auto ksc) {
                        constexpr int ks = decltype(ksc)::value;
                        // the next sub-step's copies, spread over phase 1
                        constexpr int per = (NSLOT + KSD - 1) / KSD;
                        static_for<ks * per, ((ks + 1) * per < NSLOT ? (ks + 1) * per : NSLOT)>(
                            [&](auto sc) { issue_slot(sc, pf_buf, q_next); });
                        V8 aq[2], ao[2];
#pragma unroll
                        for (int m = 0; m < 2; ++m) {
                            aq[m] = frag_row<T, D>(sQr, m * 16 + c16, ks * 32 + 8 * g);
                            ao[m] = frag_row<T, D>(sdOr, m * 16 + c16, ks * 32 + 8 * g);
                        }
#pragma unroll
                        for (int m = 0; m < 2; ++m)
#pragma unroll
                            for (int nt = 0; nt < 2; ++nt) {
                                S[m][nt] = E::mma(S[m][nt], aq[m], Kr[nt][ks]);
                                dP[m][nt] = E::mma(dP[m][nt], ao[m], Vr[nt][ks]);
                            }
                        __builtin_amdgcn_sched_barrier(0);
                    });
                    // P and dS as phase-2 A operands: slot (g, e) of the contraction
                    // is query row 16(e/4) + 4g + e%4 of the group, where the 16x16
                    // output layout of S left it
                    V8 aP[2], aS[2];
#pragma unroll
                    for (int m = 0; m < 2; ++m) {
                        // lse * log2 e of the lane's four rows of this half
                        const f32x4 lsev = *reinterpret_cast<const f32x4*>(slse + qr0 + m * 16 + 4 * g);
#pragma unroll
                        for (int i = 0; i < 4; ++i)
#pragma unroll
                            for (int nt = 0; nt < 2; ++nt) {
                                const float pv = __builtin_amdgcn_exp2f(S[m][nt][i] * p.scale_log2 - lsev[i]);
                                aP[nt][4 * m + i] = E::from_f(pv);
                                aS[nt][4 * m + i] = E::from_f(pv * dP[m][nt][i]);  // dP holds dP - D
                            }
                        __builtin_amdgcn_sched_barrier(0);
                    }
                    // dS as [key][query] (the lane's four query rows of its key are 8
                    // contiguous bytes); role 1 also P of its rows to the exchange
                    const int key0 = sl * 32 + c16;
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt) {
                        const u32x4 ws = __builtin_bit_cast(u32x4, aS[nt]);
#pragma unroll
                        for (int m = 0; m < 2; ++m)
                            *reinterpret_cast<lds_u32x2*>(
                                lsm + L::OFF_S + ((key0 + nt * 16) * LDSS + sub * BQ + qr0 + m * 16 + 4 * g) * 2) =
                                u32x2{ws[2 * m], ws[2 * m + 1]};
                    }
                    if (role) {
#pragma unroll
                        for (int nt = 0; nt < 2; ++nt) {
                            const u32x4 wp = __builtin_bit_cast(u32x4, aP[nt]);
#pragma unroll
                            for (int m = 0; m < 2; ++m)
                                *reinterpret_cast<lds_u32x2*>(lsm + L::OFF_P + (key0 + nt * 16) * PRS + (m * 16 + 4 * g) * 2) =
                                    u32x2{wp[2 * m], wp[2 * m + 1]};
                        }
                    }
                    // B operands of phase 2: dO (role 0) or Q (role 1) rows, transposed
                    const lds_u8* tq = (const lds_u8*)sQ + (role ? 0 : ODO) + (4 * g + (c16 >> 2)) * P::RS + 8 * (c16 & 3);
                    auto phase2 = [&](auto gc, const V8 (&a)[2]) {
                        constexpr int G = decltype(gc)::value;
                        static_for<0, DT>([&](auto dtc) {
                            constexpr int dt = decltype(dtc)::value, o = G * 32 * P::RS + dt * 32;
                            const V8 b = tr_frag<o, o + 16 * P::RS>(tq);
#pragma unroll
                            for (int nt = 0; nt < 2; ++nt) acc2[nt][dt] = E::mma(acc2[nt][dt], a[nt], b);
                            if constexpr (dt % 2 == 1) __builtin_amdgcn_sched_barrier(0);
                        });
                    };
                    // role 0: dV += P^T dO over group 0 from its own registers while
                    // role 1 finishes its softmax (the older waves of a SIMD win
                    // issue ties, so role 0 gets there first)
                    if (role == 0) phase2(I0{}, aP);
                    // dS of both groups and P of group 1 are in LDS
                    __syncthreads();
                    // ---- second half: role 0 dV += P^T dO over group 1 (P from the
                    // exchange); role 1 dK += dS^T Q over group 0, then group 1 (dS
                    // from LDS)
                    {
                        const lds_u8* pr0 = lsm + L::OFF_S + ((sl * 32 + c16) * LDSS + sub * BQ + 4 * g) * 2;
                        const lds_u8* pr1 = role ? pr0 + 64 : lsm + L::OFF_P + (sl * 32 + c16) * PRS + 8 * g;
                        const int rs1 = role ? SRS : PRS;
                        V8 a0[2], a1[2];
#pragma unroll
                        for (int nt = 0; nt < 2; ++nt) {
                            const u32x2 lo1 = *reinterpret_cast<const lds_u32x2*>(pr1 + nt * 16 * rs1);
                            const u32x2 hi1 = *reinterpret_cast<const lds_u32x2*>(pr1 + nt * 16 * rs1 + 32);
                            a1[nt] = __builtin_bit_cast(V8, u32x4{lo1[0], lo1[1], hi1[0], hi1[1]});
                        }
                        if (role) {
#pragma unroll
                            for (int nt = 0; nt < 2; ++nt) {
                                const u32x2 lo0 = *reinterpret_cast<const lds_u32x2*>(pr0 + nt * 16 * SRS);
                                const u32x2 hi0 = *reinterpret_cast<const lds_u32x2*>(pr0 + nt * 16 * SRS + 32);
                                a0[nt] = __builtin_bit_cast(V8, u32x4{lo0[0], lo0[1], hi0[0], hi0[1]});
                            }
                            phase2(I0{}, a0);
                        }
                        phase2(I1{}, a1);
                    }
                }

                // ---- R phase: wait for the tile's turn, dQ^T of this wave's
                // D/4 d columns and 64 query rows, the ordered sum, the release
                const KParams& pr = kpar();
                if (pr.delay_seed && tid == 0) {
                    const unsigned nap = mix32(pr.delay_seed ^ mix32((unsigned)item * 0x9e3779b9u + (unsigned)t)) & 31u;
                    for (unsigned z = 0; z < nap; ++z) __builtin_amdgcn_s_sleep(4);
                }
                if (rank > 0 && tid == 0) {
                    const unsigned long long t0 = pr.stats ? __builtin_readcyclecounter() : 0;
                    unsigned spins = 0;
                    unsigned seen = early;
                    const unsigned want = (unsigned)(rank + pr.wait_offset) & kRankMask;
                    while ((seen & kRankMask) != want) {
                        if ((spins & 1023u) == 0 && __hip_atomic_load(pr.abort, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
                            break;
                        __builtin_amdgcn_s_sleep(1);
                        if (++spins >= pr.spin_limit) {
                            atomicOr(pr.abort, 1u);
                            atomicOr(pr.status, 1u);
                            break;
                        }
                        seen = __hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    }
                    if (pr.stats) {
                        const unsigned long long dw = __builtin_readcyclecounter() - t0;
                        wait_cycles += dw;
                        polls += spins + 1;
                        atomicAdd(pr.whist + (pat & 63) * 128 + min(t - t_beg, 127), dw);
                    }
                    s_prev = seen;
                }
                __syncthreads();
                relane();
                {
                    auto acc_copy = [&](unsigned qc) {
                        const size_t slot = pr.chunks ? (size_t)qc * pr.acc_slots + (head >> pr.group_shift) : (size_t)head;
                        return make_rsrc(pr.dq_acc + slot * pr.s_pad * D, (unsigned)(pr.s_pad * D * sizeof(float)));
                    };
                    const unsigned pflag = rank > 0 ? __builtin_amdgcn_readfirstlane(s_prev) : 0u;
                    const bool same = ((pflag >> 24) & 0xfu) == xcc;
                    if (rank > 0 && !same && !(pflag & kWroteThrough) && tid == 0) atomicOr(pr.status, 2u);
                    const __amdgpu_buffer_rsrc_t rprev = acc_copy((pflag >> 28) & 7u), racc = acc_copy(queue);
                    const bool wt = !pr.chunks || succ < pr.bounds[queue & (pr.chunks - 1)] || succ >= pr.bounds[(queue & (pr.chunks - 1)) + 1];
                    const int col0 = dblk * DW + 4 * g;
                    // the accumulator as 16x16 tiles in MFMA output order, as in
                    // bwd_main_kernel (lane l's 4 values at 16*l bytes of a tile); a
                    // tile's offset is the access's scalar offset, the lane's 16
                    // bytes its vector offset
                    auto acc_soff = [&](int mtt, int dtw) {
                        return (int)((((qt * MTT + mtt) * (D / 16) + dblk * NDT + dtw) * 64) * 16);
                    };
                    const int acc_voff = lane * 16;
                    typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
                    // the previous contribution's 8 tiles of the wave's block, all
                    // requested before the contraction
                    f32x4 prev[NDT][MT];
                    auto load_prev = [&](auto polc) {
                        constexpr int POL = decltype(polc)::value;
                        static_for<0, NDT * MT>([&](auto ic) {
                            constexpr int i = decltype(ic)::value, hf = i / (NDT * 2), r = i % (NDT * 2);
                            constexpr int dtw = r / 2, mt = hf * 2 + r % 2;
                            prev[dtw][mt] = __builtin_bit_cast(
                                f32x4, __builtin_amdgcn_raw_buffer_load_b128(rprev, acc_voff, acc_soff(part * MT + mt, dtw), POL));
                        });
                    };
                    if (rank > 0) {
                        if (same)
                            load_prev(std::integral_constant<int, kCpolSc0>{});
                        else
                            load_prev(std::integral_constant<int, kCpolSc1>{});
                    }
                    // dQ^T = K^T dS^T of the wave's block over the tile's 128 keys in
                    // 32-key steps (A = K^T from transposed reads of sK, B = dS^T from
                    // transposed reads of [key][query]), then the sums: the output dQ
                    // (last contributor, MODE 0), written through to memory (MODE 1)
                    // or into this XCD's L2 (MODE 2)
                    const lds_u8* tk = lsm + L::OFF_K + (8 * g + (c16 >> 2)) * P::RS + (dblk * DW + 4 * (c16 & 3)) * 2;
                    const lds_u8* ts = lsm + L::OFF_S + (8 * g + (c16 >> 2)) * SRS + 8 * (c16 & 3) + part * BQ * 2;
                    auto sum_out = [&](auto modec) {
                        constexpr int MODE = decltype(modec)::value;
                        f32x4 dq[NDT][MT];
#pragma unroll
                        for (int dtw = 0; dtw < NDT; ++dtw)
#pragma unroll
                            for (int j = 0; j < MT; ++j) dq[dtw][j] = zero_vec<f32x4>();
                        static_for<0, KSKV>([&](auto ksc) {
                            constexpr int ks = decltype(ksc)::value;
                            V8 a[NDT], b[MT];
                            static_for<0, NDT>([&](auto jc) {
                                constexpr int o = ks * 32 * P::RS + decltype(jc)::value * 32;
                                a[decltype(jc)::value] = tr_frag<o, o + 4 * P::RS>(tk);
                            });
                            static_for<0, MT>([&](auto jc) {
                                constexpr int o = ks * 32 * SRS + decltype(jc)::value * 16 * 2;
                                b[decltype(jc)::value] = tr_frag<o, o + 4 * SRS>(ts);
                            });
#pragma unroll
                            for (int j = 0; j < MT; ++j)
#pragma unroll
                                for (int dtw = 0; dtw < NDT; ++dtw) dq[dtw][j] = E::mma(dq[dtw][j], a[dtw], b[j]);
                            __builtin_amdgcn_sched_barrier(0);
                        });
#pragma unroll
                        for (int dtw = 0; dtw < NDT; ++dtw)
#pragma unroll
                            for (int mt = 0; mt < MT; ++mt) {
                                const int mtt = part * MT + mt;
                                f32x4 v = dq[dtw][mt];
                                if (rank > 0) v = prev[dtw][mt] + v;
                                if constexpr (MODE == 0) {
                                    const int row = qt * BR + mtt * 16 + c16;
                                    V4 o;
#pragma unroll
                                    for (int e = 0; e < 4; ++e) o[e] = E::from_f(pr.scale * v[e]);
                                    if (row < s) *reinterpret_cast<V4*>(gdQ + hoff + (size_t)row * D + col0 + dtw * 16) = o;
                                } else if constexpr (MODE == 1) {
                                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), racc, acc_voff, acc_soff(mtt, dtw), kCpolSc1);
                                } else {
                                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), racc, acc_voff, acc_soff(mtt, dtw), 0);
                                }
                            }
                    };
                    if (succ < 0)
                        sum_out(std::integral_constant<int, 0>{});
                    else if (wt)
                        sum_out(std::integral_constant<int, 1>{});
                    else
                        sum_out(std::integral_constant<int, 2>{});
                    if (succ >= 0) {
                        pend_flag = flag;
                        pend_val = (unsigned)(rank + 1) | (xcc << 24) | ((unsigned)queue << 28) | (wt ? kWroteThrough : 0u);
                    }
                }
                ++t;
                more = false;
                if (t < t_end) {
                    if ((t - t_beg) % L::MAXT == 0) load_tasks(t);
                    more = __builtin_amdgcn_readfirstlane(stask[(t - t_beg) % L::MAXT][0]) == kv;
                }
            } while (more);
            // the run's last release goes out before the dK/dV epilogue (as in
            // bwd_main_kernel)
            if (pend_flag) publish();
            store_dkdv(kv);
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        if (pend_flag) publish();
        if (p.stats) item_cycles += __builtin_readcyclecounter() - t_item0;
    }
    if (p.chunks && tid == 0 && atomicAdd(p.queues + kQueues, 1u) == gridDim.x - 1) {
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

template <int D, bool CAUSAL>
int launch_pair_t(const KParams& kp, const BwdLaunch& L) {
    auto kern = bwd_pair_kernel<D, CAUSAL>;
    const size_t smem = PairLayout<D>::bytes;
    static bool attr_set = false;
    if (!attr_set) {
        if (hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem) != hipSuccess)
            return fail(ATTN_ERR_HIP, "hipFuncSetAttribute failed for the pair kernel");
        attr_set = true;
    }
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)kern, kPairThreads, smem) != hipSuccess ||
        per_cu < 1)
        return fail(ATTN_ERR_HIP, "occupancy query failed for the pair kernel");
    const long long resident = (long long)per_cu * L.num_cus;
    if (L.min_workers > resident)
        return fail(ATTN_ERR_COSCHEDULE, "schedule needs more simultaneously resident work groups than the device holds");
    const long long grid = std::min<long long>(resident, kp.total_items);
    if (grid <= 0) return ATTN_OK;
    KParams k = kp;
    const XcdPlan& pl = L.plan;
    if (pl.chunks && grid / kQueues >= 1 && (L.min_workers <= 1 || pl.max_chunk <= grid / kQueues)) {
        k.chunks = pl.chunks;
        for (int c = 0; c <= kQueues; ++c) k.bounds[c] = pl.bounds[c];
        k.groups = pl.groups;
        k.acc_slots = pl.slots;
        k.chunk_shift = __builtin_ctz((unsigned)pl.chunks);
        k.group_shift = __builtin_ctz((unsigned)pl.groups);
    }
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kPairThreads), smem, (hipStream_t)L.stream, k);
    if (hipGetLastError() != hipSuccess) return fail(ATTN_ERR_HIP, "pair kernel launch failed");
    return ATTN_OK;
}

}  // namespace

// The deterministic bf16 128 x 128 backward through the pair kernel (d = 64 or 128).
int launch_main_bf16_pair(const KParams& kp, const BwdLaunch& L, bool causal, int d) {
    if (d == 64) return causal ? launch_pair_t<64, true>(kp, L) : launch_pair_t<64, false>(kp, L);
    return causal ? launch_pair_t<128, true>(kp, L) : launch_pair_t<128, false>(kp, L);
}

}  // namespace attn
