// Preprocess and finalize kernels, the device status word, the XCD probe and
// the launch of one backward call for gfx950.  The main kernel itself is in
// bwd_main.h.
#include "bwd_main.h"

namespace attn {

// bf16 d = 64 main kernels (bwd_kernels_d64.hip)
int launch_main_bf16_d64(const KParams& kp, const BwdLaunch& L, bool causal, bool det, int tile);

// -D[head][row] = -<dO_row, O_row> in fp32 (negated: the bf16 main kernels
// start dP's accumulation from it, so dP - D needs no subtraction)
// and lse2[head][row] = lse * log2(e) (both zero for padded rows, the
// softmax's exp2 argument then needs no multiply per use); clears the flags and counters of the call and, for the
// atomic variant, the dQ accumulator.  Each lane reads 32 bytes of a row of
// O and of dO (kPreLanes<T, D> lanes per row: 4 for bf16 at d = 64, 8 at
// d = 128).  Measured at s = 2048, d = 64, b*h = 64: 16 lanes of 8-byte reads
// 12.4 us, 8 lanes of 16 bytes 10.2 us, 4 of 32 bytes 9.2 us; at s = 8192,
// d = 128, b*h = 32: 31.5 us with 16-byte reads, 29.5 us with 32-byte ones.
template <typename T, int D>
constexpr int kPreLanes = D * (int)sizeof(T) / 32;
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_preprocess_kernel(const T* __restrict__ o, const T* __restrict__ dO,
                                                              const float* __restrict__ lse, float* __restrict__ delta,
                                                              float* __restrict__ lse2, int H, int s, int s_pad,
                                                              unsigned* __restrict__ clear32, int nclear32,
                                                              float* __restrict__ zero_acc, size_t nzero4) {
    constexpr int LPR = kPreLanes<T, D>, PER = D / LPR;
    static_assert(LPR >= 1 && LPR <= 64 && (LPR & (LPR - 1)) == 0 && 256 % LPR == 0, "lanes per row");
    const size_t rows = (size_t)H * s_pad;
    const size_t gtid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t row = gtid / LPR;
    const int part = (int)(gtid % LPR);
    if (row < rows) {
        const int hh = (int)(row / s_pad), r = (int)(row % s_pad);
        float acc = 0.f;
        if (r < s) {
            const size_t off = ((size_t)hh * s + r) * D + part * PER;
#pragma unroll
            for (int e = 0; e < PER; ++e) acc += Elem<T>::to_f(o[off + e]) * Elem<T>::to_f(dO[off + e]);
        }
#pragma unroll
        for (int m = LPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, LPR);
        if (part == 0) {
            delta[row] = -acc;
            lse2[row] = r < s ? lse[(size_t)hh * s + r] * kLog2e : 0.f;
        }
    }
    const size_t nthreads = (size_t)gridDim.x * blockDim.x;
    for (size_t i = gtid; i < (size_t)nclear32; i += nthreads) clear32[i] = 0u;
    if (zero_acc) {
        f32x4* z = reinterpret_cast<f32x4*>(zero_acc);
        for (size_t i = gtid; i < nzero4; i += nthreads) z[i] = zero_vec<f32x4>();
    }
}

// Atomic variant only: dQ = scale * accumulator, converted to the output type.
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_finalize_kernel(const float* __restrict__ acc, T* __restrict__ dq,
                                                            int H, int s, int s_pad, float scale) {
    const size_t total4 = (size_t)H * s * D / 4;
    const size_t nthreads = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total4; i += nthreads) {
        const size_t e0 = i * 4;
        const size_t hh = e0 / ((size_t)s * D), rem = e0 % ((size_t)s * D);
        const f32x4 a = *reinterpret_cast<const f32x4*>(acc + hh * (size_t)s_pad * D + rem);
        typename Elem<T>::vec4 out;
#pragma unroll
        for (int e = 0; e < 4; ++e) out[e] = Elem<T>::from_f(scale * a[e]);
        *reinterpret_cast<typename Elem<T>::vec4*>(dq + e0) = out;
    }
}

// ---------------------------------------------------------------------------
// Launch
// ---------------------------------------------------------------------------
// The device status word that attn_bwd_query_status reports (bit 0: a flag
// wait expired, bit 1: XCD placement could not run as planned); one copy per
// device, found with hipGetSymbolAddress while that device is current.
__device__ unsigned g_status_word;

int status_word_address(unsigned** ptr) {
    const hipError_t e = hipGetSymbolAddress((void**)ptr, HIP_SYMBOL(g_status_word));
    if (e != hipSuccess) return fail(ATTN_ERR_HIP, "hipGetSymbolAddress(status word)");
    return ATTN_OK;
}

// Records the XCD of every work group (one wave each).
__global__ __launch_bounds__(64) void xcd_probe_kernel(unsigned* out) {
    unsigned x;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(x));
    if (threadIdx.x == 0) out[blockIdx.x] = x & 0xfu;
}

// Placement needs XCD ids 0..kQueues-1, each dealt an equal share of a grid.
int probe_xcd_dispatch(int num_cus, bool* ok, unsigned* buf) {
    *ok = false;
    if (num_cus < kQueues || num_cus % kQueues) return ATTN_OK;
    const int grid = 4 * num_cus;
    unsigned* d = buf;
    if (!d && hipMalloc(&d, grid * sizeof(unsigned)) != hipSuccess) return fail(ATTN_ERR_HIP, "hipMalloc(xcd probe)");
    std::vector<unsigned> h(grid, ~0u);
    hipLaunchKernelGGL(xcd_probe_kernel, dim3(grid), dim3(64), 0, 0, d);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess) e = hipMemcpy(h.data(), d, grid * sizeof(unsigned), hipMemcpyDeviceToHost);
    const hipError_t ef = buf ? hipSuccess : hipFree(d);
    if (ef != hipSuccess || e != hipSuccess) return fail(ATTN_ERR_HIP, "XCD probe kernel failed");
    std::vector<int> per(kQueues, 0);
    bool all = true;
    for (int b = 0; b < grid; ++b) {
        all = all && h[b] < (unsigned)kQueues;
        if (h[b] < (unsigned)kQueues) per[h[b]]++;
    }
    for (int q = 0; q < kQueues; ++q) all = all && per[q] == grid / kQueues;
    *ok = all;
    return ATTN_OK;
}

// bf16 d = 64 main kernels (bwd_kernels_d64.hip) for Q tiles of br rows
int launch_main_bf16_d64_rect(const KParams& kp, const BwdLaunch& L, bool causal, bool det);
// deterministic bf16 128 x 128 tiles, eight waves (bwd_pair.hip)
int launch_main_bf16_pair(const KParams& kp, const BwdLaunch& L, bool causal, int d);

template <typename T, int TILE, int BR = TILE>
static int launch_all(const BwdArgs& a, const BwdLaunch& L, KParams& kp) {
    const T* o = static_cast<const T*>(a.o);
    const T* dO = static_cast<const T*>(a.dO);
    const bool det = a.schedule != ATTN_SCHED_ATOMIC;
    hipStream_t st = (hipStream_t)L.stream;

    // preprocess
    if (L.ev && hipEventRecord((hipEvent_t)L.ev[0], st) != hipSuccess) return fail(ATTN_ERR_HIP, "hipEventRecord failed");
    {
        const size_t rows = (size_t)a.H * a.s_pad;
        const size_t threads = rows * (a.d == 64 ? kPreLanes<T, 64> : kPreLanes<T, 128>);
        const unsigned blocks = (unsigned)((threads + 255) / 256);
        const size_t nzero4 = det ? 0 : (size_t)a.H * a.s_pad * a.d / 4;
        float* lse2 = a.delta + (size_t)a.H * a.s_pad;
        if (a.d == 64)
            hipLaunchKernelGGL((bwd_preprocess_kernel<T, 64>), dim3(blocks), dim3(256), 0, st, o, dO, a.lse, a.delta, lse2, a.H,
                               a.s, (int)a.s_pad, a.flags, L.nclear32, det ? nullptr : a.dq_acc, nzero4);
        else
            hipLaunchKernelGGL((bwd_preprocess_kernel<T, 128>), dim3(blocks), dim3(256), 0, st, o, dO, a.lse, a.delta, lse2, a.H,
                               a.s, (int)a.s_pad, a.flags, L.nclear32, det ? nullptr : a.dq_acc, nzero4);
        if (hipGetLastError() != hipSuccess) return fail(ATTN_ERR_HIP, "preprocess kernel launch failed");
    }
    if (L.ev && hipEventRecord((hipEvent_t)L.ev[1], st) != hipSuccess) return fail(ATTN_ERR_HIP, "hipEventRecord failed");
    // Symmetric Shift (causal; under the full mask it runs Shift) with dS as
    // [key][query] at d = 128 (measured: 8% faster at s = 8192; at d = 64,
    // s = 2048 the row layout is 3% faster)
    const bool dst = a.schedule == ATTN_SCHED_SYMMETRIC_SHIFT && BR == TILE;
    int rc;
    // the eight-wave pair kernel (bf16 128 x 128 tiles, deterministic): forced,
    // or by default under the causal mask at d = 128
    const bool pair = runs_pair_kernel(sizeof(T) == 2, BR, TILE, det, L.main_kernel, a.causal, a.d);
    if (pair) {
        rc = launch_main_bf16_pair(kp, L, a.causal, a.d);
    } else if (a.d == 64) {
        if constexpr (sizeof(T) == 2 && BR != TILE)
            rc = launch_main_bf16_d64_rect(kp, L, a.causal, det);
        else if constexpr (sizeof(T) == 2)
            rc = launch_main_bf16_d64(kp, L, a.causal, det, TILE);
        else
            rc = launch_main_d<T, 64, TILE>(kp, L, a.causal, det, dst);
    } else {
        rc = launch_main_d<T, 128, TILE, BR>(kp, L, a.causal, det, dst);
    }
    if (rc != ATTN_OK) return rc;
    if (L.ev && hipEventRecord((hipEvent_t)L.ev[2], st) != hipSuccess) return fail(ATTN_ERR_HIP, "hipEventRecord failed");
    if (!det) {
        const size_t total4 = (size_t)a.H * a.s * a.d / 4;
        const unsigned blocks = (unsigned)std::min<size_t>((total4 + 255) / 256, 65536);
        if (a.d == 64)
            hipLaunchKernelGGL((bwd_finalize_kernel<T, 64>), dim3(blocks), dim3(256), 0, st, a.dq_acc,
                               static_cast<T*>(a.dq), a.H, a.s, (int)a.s_pad, a.scale);
        else
            hipLaunchKernelGGL((bwd_finalize_kernel<T, 128>), dim3(blocks), dim3(256), 0, st, a.dq_acc,
                               static_cast<T*>(a.dq), a.H, a.s, (int)a.s_pad, a.scale);
        if (hipGetLastError() != hipSuccess) return fail(ATTN_ERR_HIP, "finalize kernel launch failed");
    }
    if (L.ev && hipEventRecord((hipEvent_t)L.ev[3], st) != hipSuccess) return fail(ATTN_ERR_HIP, "hipEventRecord failed");
    return ATTN_OK;
}

int launch_backward(const BwdArgs& a, const BwdLaunch& L) {
    KParams kp{};
    kp.q = a.q; kp.k = a.k; kp.v = a.v; kp.dO = a.dO;
    kp.lse2 = a.delta + (size_t)a.H * a.s_pad;
    kp.delta = a.delta;
    kp.dq = a.dq; kp.dk = a.dk; kp.dv = a.dv;
    kp.dq_acc = a.dq_acc;
    kp.flags = a.flags;
    kp.ticket = a.counters;
    kp.queues = a.counters + kQueueWord;
    kp.abort = a.counters + 1;
    kp.status = L.status;
    kp.stats = L.stats;
    kp.whist = L.whist;
    kp.item_begin = L.item_begin;
    kp.tasks = reinterpret_cast<const i32x4*>(L.tasks);
    kp.H = a.H;
    kp.s = a.s;
    kp.n = a.n;
    kp.items_per_head = L.items_per_head;
    kp.s_pad = (int)a.s_pad;
    kp.total_items = (long long)a.H * L.items_per_head;
    kp.scale = a.scale;
    kp.scale_log2 = a.scale * kLog2e;
    kp.spin_limit = L.spin_limit ? L.spin_limit : kSpinLimit;
    kp.wait_offset = L.wait_offset;
    kp.delay_seed = L.delay_seed;
    if (a.dtype == ATTN_BF16) {
        if (a.tile == 64 && a.br == 64) return launch_all<bf16, 64>(a, L, kp);
        if (a.tile == 128 && a.br == 64) return launch_all<bf16, 128, 64>(a, L, kp);
        if (a.tile == 128 && a.br == 128) return launch_all<bf16, 128>(a, L, kp);
        return fail(ATTN_ERR_UNSUPPORTED, "bf16 tile shape must be 128x128, 64x64 or 64x128 (Br x Bc)");
    }
    if (a.tile != 64 || a.br != 64) return fail(ATTN_ERR_UNSUPPORTED, "fp32 tiles are 64x64");
    return launch_all<float, 64>(a, L, kp);
}

}  // namespace attn
