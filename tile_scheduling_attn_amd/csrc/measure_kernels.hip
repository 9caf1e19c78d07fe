// Measurement kernels beside the backward: the fp32 atomic-add rate the
// ATOMIC schedule is held against, and the latency of one dQ hand-off
// between two work groups at a chosen XCD distance.  Neither touches
// attention state.
#include <hip/hip_runtime.h>

#include "attn_bwd.h"
#include "attn_device.h"
#include "internal.h"

namespace attn {

// Throughput of fp32 atomic adds without return value in the pattern of the
// atomic variant's dQ: per task a work group adds one 128x128 fp32 tile into
// tile (group * 7 + task) mod ntiles of acc, each instruction covering 64
// contiguous bytes of four rows.  A measurement kernel: the ATOMIC schedule's
// main kernel is compared with the rate it reaches.
__global__ __launch_bounds__(256) void atomic_rate_kernel(float* acc, int ntiles, int tasks) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    for (int t = 0; t < tasks; ++t) {
        const int tile = (int)(((long long)blockIdx.x * 7 + t) % ntiles);
        float* base = acc + (size_t)tile * 128 * 128;
#pragma unroll 4
        for (int i = 0; i < 64; ++i) {
            const int row = (i >> 1) * 4 + (lane >> 4);
            const int col = w * 32 + (i & 1) * 16 + (lane & 15);
            unsafeAtomicAdd(base + row * 128 + col, 1.0f);
        }
    }
}

int launch_atomic_rate(float* acc, int ntiles, int grid, int tasks, void* stream) {
    hipLaunchKernelGGL(atomic_rate_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream, acc, ntiles, tasks);
    if (hipGetLastError() != hipSuccess) return fail(ATTN_ERR_HIP, "atomic rate kernel launch failed");
    return ATTN_OK;
}

// Latency of one dQ hand-off between two work groups, in the main kernel's
// protocol: a turn waits for the flag to reach its number (relaxed
// agent-scope loads, one thread, s_sleep between polls), reads the previous
// turn's 64 KiB fp32 tile, adds to it, writes its own tile, waits for its
// stores and moves the flag on with a relaxed agent-scope store.  Work
// group 0 takes the even turns and work group `pong` the odd ones; the
// dispatcher deals work groups to XCDs in turn, so `pong` picks the XCD
// distance (each group records its XCD).  MODE 0: the flag alone; 1: the
// tile through the L2 of the XCD (plain stores, sc0 loads: meaningful when
// both groups share an XCD); 2: the tile written through to memory and read
// from it (sc1), as hand-offs between XCDs are.  Every wait gives up after
// kHandoffPolls polls and records it in words[3].
// words: [0] flag, [1] XCD of group 0, [2] XCD of group pong, [3] error,
// [4..5] group 0's span on the constant-rate clock (u64).
constexpr unsigned kHandoffPolls = 1u << 20;
template <int MODE>
__global__ __launch_bounds__(256) void handoff_kernel(unsigned* words, float* tiles, int pong, int iters) {
    const int b = blockIdx.x;
    if (b != 0 && b != pong) return;
    const bool ping = b == 0;
    __shared__ unsigned s_err;
    unsigned x;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(x));
    if (threadIdx.x == 0) {
        words[ping ? 1 : 2] = x & 0xfu;
        s_err = 0;
    }
    const __amdgpu_buffer_rsrc_t rt = make_rsrc(tiles, 2u * 65536u);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
    __syncthreads();
    for (int k = ping ? 0 : 1; k < iters; k += 2) {
        if (threadIdx.x == 0) {
            unsigned polls = 0;
            while (__hip_atomic_load(words, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != (unsigned)k) {
                __builtin_amdgcn_s_sleep(1);
                if (++polls >= kHandoffPolls) {
                    s_err = 1;
                    atomicOr(words + 3, 1u);
                    break;
                }
            }
        }
        __syncthreads();
        if (s_err) break;
        if constexpr (MODE > 0) {
            // 16 KiB per wave: 16 instructions of 1 KiB, as the R phase's
            f32x4 v[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const unsigned off = (unsigned)(((k + 1) & 1) * 65536 + (w * 16 + i) * 1024 + lane * 16);
                v[i] = k == 0 ? zero_vec<f32x4>() : (MODE == 1 ? load_sc0(rt, off) : load_sc1(rt, off));
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const unsigned off = (unsigned)((k & 1) * 65536 + (w * 16 + i) * 1024 + lane * 16);
                const f32x4 u = v[i] + 1.f;
                if constexpr (MODE == 1)
                    store_l2(rt, off, u);
                else
                    store_sc1(rt, off, u);
            }
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }
        __syncthreads();
        if (threadIdx.x == 0) __hip_atomic_store(words, (unsigned)(k + 1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (ping && threadIdx.x == 0) {
        // the span ends when the last turn (possibly the other group's) is done
        for (unsigned polls = 0; !s_err && __hip_atomic_load(words, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) !=
                                              (unsigned)iters;) {
            __builtin_amdgcn_s_sleep(1);
            if (++polls >= kHandoffPolls) atomicOr(words + 3, 1u), s_err = 1;
        }
        const unsigned long long span = __builtin_amdgcn_s_memrealtime() - t0;
        words[4] = (unsigned)span;
        words[5] = (unsigned)(span >> 32);
    }
}

int launch_handoff(unsigned* words, float* tiles, int pong, int iters, int mode, void* stream) {
    hipStream_t st = (hipStream_t)stream;
    if (mode == 0)
        hipLaunchKernelGGL(handoff_kernel<0>, dim3(pong + 1), dim3(256), 0, st, words, tiles, pong, iters);
    else if (mode == 1)
        hipLaunchKernelGGL(handoff_kernel<1>, dim3(pong + 1), dim3(256), 0, st, words, tiles, pong, iters);
    else
        hipLaunchKernelGGL(handoff_kernel<2>, dim3(pong + 1), dim3(256), 0, st, words, tiles, pong, iters);
    if (hipGetLastError() != hipSuccess) return fail(ATTN_ERR_HIP, "hand-off kernel launch failed");
    return ATTN_OK;
}

}  // namespace attn
