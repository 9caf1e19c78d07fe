// HIP kernel of the attention forward pass for gfx950 (CDNA4): O and the
// log-sum-exp lse that the deterministic backward consumes.
//
// The pages do not print the forward; Fig. 1 of the DASH paper (as captioned
// on the pith.science review page) shows tiled FlashAttention, whose forward
// is the one computed here, and the summary page's Experimental setup runs a
// FlashAttention backward benchmark, which needs O and lse as inputs.  Per
// query row i: S_ij = scale * q_i . k_j (keys after i masked under the causal
// mask), lse_i = log sum_j exp(S_ij), O_i = sum_j exp(S_ij - lse_i) v_j.
//
// Mapping onto gfx950.  A work group of 4 wave64s owns one tile of 128 query
// rows; wave w owns rows [32w, 32w+32) as two 16-row tiles and keeps their Q
// values in registers for the whole pass.  K and V stream through LDS in
// tiles of 64 rows (double-buffered global-to-LDS copies).  Every wave forms
// S^T = K Q^T (A = K rows from LDS, B = its Q rows): in the 16x16 MFMA output
// layout a lane then holds 4 keys of one query column, so a query's running
// maximum and sum are reduced over the lane's values and the 4 lanes that
// share the column.  O^T = V^T P^T follows with P^T as the B operand in the
// same register layout (the contraction index, the key, is permuted alike in
// both operands) and V^T read from the row-major V tile by transposing LDS
// reads; in the O^T accumulator a lane holds 4 consecutive d of one query
// row, the same query column as its statistics.  Online softmax in base 2
// with the running maximum m: alpha = 2^(m_old - m_new) rescales O^T and the
// partial sums.  Each work group owns its output rows, so the result does
// not depend on the order in which work groups run.
#include "attn_bwd.h"
#include "attn_device.h"
#include "internal.h"

namespace attn {

namespace {

constexpr int kFwdWaves = 4, kFwdThreads = 64 * kFwdWaves;
constexpr int kFwdBQ = 128;  // query rows per work group
constexpr int kFwdBK = 64;   // key rows per LDS tile

template <typename T, int D>
struct FwdLayout {
    static constexpr int KB = (kFwdBK * Pad<T, D>::RS + 1023) / 1024 * 1024;  // one K (or V) buffer
    static constexpr int OFF_K = 0, OFF_V = 2 * KB;
    static constexpr size_t bytes = 4 * KB;
    static_assert(bytes <= 160 * 1024, "LDS budget of a gfx950 work group exceeded");
};

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(kFwdThreads, 1) void fwd_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                            const T* __restrict__ v, T* __restrict__ o,
                                                            float* __restrict__ lse, int s, int nq, float scale_log2) {
    using E = Elem<T>;
    using V8 = typename E::vec8;
    using V4 = typename E::vec4;
    using L = FwdLayout<T, D>;
    constexpr int KSD = D / 32, DT = D / 16, NK = kFwdBK / 16, KK = kFwdBK / 32;
    extern __shared__ __align__(16) unsigned char smem[];
    const unsigned lds_base = lds_addr(smem);

    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, c16 = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    // heavier query tiles first under the causal mask
    const int head = blockIdx.x / nq;
    const int qt = CAUSAL ? nq - 1 - (int)(blockIdx.x % nq) : (int)(blockIdx.x % nq);
    const size_t hoff = (size_t)head * s * D;
    const int q0 = qt * kFwdBQ + 32 * w;  // first query row of this wave

    // this wave's query rows as B operands of S^T (column = query, 8 d per lane group)
    V8 qb[2][KSD];
#pragma unroll
    for (int mq = 0; mq < 2; ++mq) {
        const int row = q0 + 16 * mq + c16;
        const size_t roff = hoff + (size_t)min(row, s - 1) * D;
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks) {
            qb[mq][ks] = *reinterpret_cast<const V8*>(q + roff + ks * 32 + 8 * g);
            if (row >= s) qb[mq][ks] = zero_vec<V8>();
        }
    }

    const unsigned head_bytes = (unsigned)((size_t)s * D * sizeof(T));
    const u32x4 rk = rsrc_words(k + hoff, head_bytes), rv = rsrc_words(v + hoff, head_bytes);
    // key tiles this work group visits: all, or up to its last query row
    const int last_row = min(s, (qt + 1) * kFwdBQ) - 1;
    const int ntiles = CAUSAL ? last_row / kFwdBK + 1 : (s + kFwdBK - 1) / kFwdBK;
    auto issue = [&](int b, int t) {
        load_tile_async<T, D, kFwdBK, kFwdWaves>(lds_base + L::OFF_K + b * L::KB, rk, t * kFwdBK, w, lane);
        load_tile_async<T, D, kFwdBK, kFwdWaves>(lds_base + L::OFF_V + b * L::KB, rv, t * kFwdBK, w, lane);
    };

    f32x4 ot[DT][2];  // O^T: [d tile][query tile]
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int mq = 0; mq < 2; ++mq) ot[dt][mq] = zero_vec<f32x4>();
    float mrun[2] = {-__builtin_inff(), -__builtin_inff()};  // running max of scale*log2e*S
    float lrun[2] = {0.f, 0.f};                              // this lane's part of the running sum

    issue(0, 0);
    for (int t = 0; t < ntiles; ++t) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();  // tile t landed for every wave; every wave done with tile t-1
        if (t + 1 < ntiles) issue((t + 1) & 1, t + 1);
        const unsigned char* sK = smem + L::OFF_K + (t & 1) * L::KB;
        const unsigned char* sV = smem + L::OFF_V + (t & 1) * L::KB;
        const int k0 = t * kFwdBK;

        // S^T = K Q^T over d; key rows past s and (causal) keys after the
        // query start at -inf
        f32x4 st[NK][2];
        const bool edge = k0 + kFwdBK > s || (CAUSAL && k0 + kFwdBK - 1 > q0);
#pragma unroll
        for (int nk = 0; nk < NK; ++nk)
#pragma unroll
            for (int mq = 0; mq < 2; ++mq) {
                st[nk][mq] = zero_vec<f32x4>();
                if (edge) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int kg = k0 + 16 * nk + 4 * g + i, qg = q0 + 16 * mq + c16;
                        if (kg >= s || (CAUSAL && kg > qg)) st[nk][mq][i] = -__builtin_inff();
                    }
                }
            }
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks)
#pragma unroll
            for (int nk = 0; nk < NK; ++nk) {
                const V8 a = frag_row<T, D>(sK, 16 * nk + c16, ks * 32 + 8 * g);
#pragma unroll
                for (int mq = 0; mq < 2; ++mq) st[nk][mq] = E::mma(st[nk][mq], a, qb[mq][ks]);
            }

        // online softmax per query column: max over this lane's keys, then
        // over the 4 lanes of the column (lanes c16 + 16g)
        V8 pb[KK][2];
#pragma unroll
        for (int mq = 0; mq < 2; ++mq) {
            float mx = -__builtin_inff();
#pragma unroll
            for (int nk = 0; nk < NK; ++nk)
#pragma unroll
                for (int i = 0; i < 4; ++i) mx = fmaxf(mx, st[nk][mq][i]);
            mx *= scale_log2;
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float mnew = fmaxf(mrun[mq], mx);
            const float muse = mnew == -__builtin_inff() ? 0.f : mnew;  // fully masked so far
            const float alpha = __builtin_amdgcn_exp2f(mrun[mq] - muse);
            mrun[mq] = mnew;
            float sum = 0.f;
#pragma unroll
            for (int nk = 0; nk < NK; ++nk)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float pv = __builtin_amdgcn_exp2f(st[nk][mq][i] * scale_log2 - muse);
                    sum += pv;
                    // key slot of P^T as the B operand of O^T: k step nk/2,
                    // element 4*(nk%2) + i
                    pb[nk / 2][mq][4 * (nk % 2) + i] = E::from_f(pv);
                }
            lrun[mq] = lrun[mq] * alpha + sum;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) ot[dt][mq] = ot[dt][mq] * alpha;
        }

        // O^T += V^T P^T over this tile's keys
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const V8 a = frag_col<T, D>(sV, 32 * kk + 4 * g, 32 * kk + 16 + 4 * g, 16 * dt, c16);
#pragma unroll
                for (int mq = 0; mq < 2; ++mq) ot[dt][mq] = E::mma(ot[dt][mq], a, pb[kk][mq]);
            }
    }

    // O = O^T / l (a lane: 4 consecutive d of query row q0 + 16mq + c16) and
    // lse = ln 2 * (m + log2 l)
#pragma unroll
    for (int mq = 0; mq < 2; ++mq) {
        float l = lrun[mq];
        l += __shfl_xor(l, 16);
        l += __shfl_xor(l, 32);
        const int row = q0 + 16 * mq + c16;
        const float inv = 1.f / l;
        if (row < s) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                V4 out;
#pragma unroll
                for (int e = 0; e < 4; ++e) out[e] = E::from_f(ot[dt][mq][e] * inv);
                *reinterpret_cast<V4*>(o + hoff + (size_t)row * D + 16 * dt + 4 * g) = out;
            }
            if (g == 0) lse[(size_t)head * s + row] = (mrun[mq] + __builtin_amdgcn_logf(l)) * 0.6931471805599453f;
        }
    }
}

template <typename T, int D>
int launch_fwd_t(const FwdArgs& a) {
    const int nq = (a.s + kFwdBQ - 1) / kFwdBQ;
    const long long grid = (long long)a.H * nq;
    if (grid <= 0) return ATTN_OK;
    if (grid > 0x7fffffffLL) return fail(ATTN_ERR_INVALID_ARG, "problem too large");
    const size_t smem = FwdLayout<T, D>::bytes;
    auto kern = a.causal ? fwd_kernel<T, D, true> : fwd_kernel<T, D, false>;
    if (hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem) != hipSuccess)
        return fail(ATTN_ERR_HIP, "hipFuncSetAttribute failed for the forward kernel");
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kFwdThreads), smem, (hipStream_t)a.stream,
                       static_cast<const T*>(a.q), static_cast<const T*>(a.k), static_cast<const T*>(a.v),
                       static_cast<T*>(a.o), a.lse, a.s, nq, a.scale * kLog2e);
    if (hipGetLastError() != hipSuccess) return fail(ATTN_ERR_HIP, "forward kernel launch failed");
    return ATTN_OK;
}

}  // namespace

int launch_forward(const FwdArgs& a) {
    if (a.dtype == ATTN_BF16) return a.d == 64 ? launch_fwd_t<bf16, 64>(a) : launch_fwd_t<bf16, 128>(a);
    return a.d == 64 ? launch_fwd_t<float, 64>(a) : launch_fwd_t<float, 128>(a);
}

}  // namespace attn
