// Device helpers shared by the attention kernels for gfx950: element types
// and MFMA wrappers, coherent buffer accesses, padded LDS tiles filled by
// global-to-LDS copies, and MFMA operand fetches from LDS.
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>

namespace attn {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) u32x2 lds_u32x2;

template <typename T> struct Elem;

template <> struct Elem<bf16> {
    using vec8 = bf16x8;  // MFMA operand: 8 k values of one row or column
    using vec4 = bf16x4;
    static constexpr int kPad = 16;  // LDS row padding in elements (32 bytes)
    __device__ static inline f32x4 mma(f32x4 c, vec8 a, vec8 b) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    __device__ static inline bf16 from_f(float x) { return (bf16)x; }
    __device__ static inline float to_f(bf16 x) { return (float)x; }
};

template <> struct Elem<float> {
    using vec8 = f32x8;
    using vec4 = f32x4;
    static constexpr int kPad = 8;  // 32 bytes
    // the same 32-wide k slice as the bf16 instruction, as 8 steps of k=4:
    // step e takes element e of every lane, so lane group l/16 supplies k
    // slot l/16 of step e for both operands alike.
    __device__ static inline f32x4 mma(f32x4 c, vec8 a, vec8 b) {
#pragma unroll
        for (int e = 0; e < 8; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[e], c, 0, 0, 0);
        return c;
    }
    __device__ static inline float from_f(float x) { return x; }
    __device__ static inline float to_f(float x) { return x; }
};

// 16-byte accesses through a raw buffer resource (dword 3 = 0x00020000 is
// the raw-buffer format word of the gfx9 family; out-of-range offsets read 0
// and drop writes) with a cache policy: sc1 is agent scope (a load misses
// every cache that is not coherent device-wide, a store is written through
// to memory), sc0 alone is the scope of the L2 of the issuing XCD (a load
// misses the CU's L1 and may hit that L2).
constexpr int kCpolSc1 = 16;
constexpr int kCpolSc0 = 1;
__device__ inline f32x4 load_sc0(__amdgpu_buffer_rsrc_t r, unsigned off) {
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kCpolSc0));
}
// plain store: written to the XCD's L2 (written back to memory later)
__device__ inline void store_l2(__amdgpu_buffer_rsrc_t r, unsigned off, f32x4 v) {
    typedef unsigned u32x4_ __attribute__((ext_vector_type(4)));
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_, v), r, (int)off, 0, 0);
}
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(void* base, unsigned bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(base, 0, (int)bytes, 0x00020000);
}
__device__ inline f32x4 load_sc1(__amdgpu_buffer_rsrc_t r, unsigned off) {
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kCpolSc1));
}
__device__ inline void store_sc1(__amdgpu_buffer_rsrc_t r, unsigned off, f32x4 v) {
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, (int)off, 0, kCpolSc1);
}

template <typename V>
__device__ inline V zero_vec() {
    V z;
#pragma unroll
    for (int e = 0; e < (int)(sizeof(V) / sizeof(z[0])); ++e) z[e] = 0;
    return z;
}

// Row-major LDS tile of rows of D elements with 32 bytes of padding per row
// (row stride RS = row bytes + 32: the 16 rows read by one 16-lane operand
// fetch start 8 banks apart; measured on gfx950, a 16-row x 16-byte
// ds_read_b128 gather runs 1.5x faster than with a 16-byte pad and close to
// a contiguous read).  It is filled straight from global
// memory by global_load_lds_dwordx4: each wave-wide load fills 1 KiB of LDS,
// lane l writing bytes [16l, 16l+16); a lane whose slot falls in a row's
// padding is switched off.
template <typename T, int D>
struct Pad {
    static constexpr int RB = D * (int)sizeof(T);  // data bytes per row
    static constexpr int RS = RB + 32;            // row stride in bytes
    __device__ static inline int off(int row, int col) { return row * RS + col * (int)sizeof(T); }
};

typedef __attribute__((address_space(3))) unsigned char lds_u8;
constexpr unsigned kOutOfRange = 0x80000000u;  // a buffer offset past any tensor

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// The words of a raw buffer resource over [base, base + bytes) (the same
// descriptor as make_rsrc), for the copy instructions below.
__device__ inline u32x4 rsrc_words(const void* base, unsigned bytes) {
    const unsigned long long a = (unsigned long long)base;
    return u32x4{(unsigned)a, (unsigned)(a >> 32) & 0xffffu, bytes, 0x00020000u};
}

// Global-to-LDS copies (buffer_load_dword[x4] ... lds): the element at byte
// offset voff of the resource lands at LDS address m0 + 4 * lane (dword) or
// m0 + 16 * lane (dwordx4).  They are written as inline assembly so that the
// compiler does not know an LDS copy is in flight: otherwise it makes every
// transposing LDS read (which it cannot tell apart from the copy's
// destination) wait for all outstanding vector-memory operations, which
// would stall each sub-step until the prefetch of the next one had landed.
// Readers of a copied tile are ordered after it by an explicit
// s_waitcnt vmcnt(0) and a barrier.  A write of m0 needs one wait state
// before the copy reads it.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ inline void copy16_to_lds(u32x4 rsrc, unsigned voff, unsigned lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(rsrc), "s"(__builtin_amdgcn_readfirstlane(lds))
                 : "memory", "m0");
}
// As copy16_to_lds, to LDS byte address base + OFF: the add is the m0 write
// itself (one scalar instruction instead of an add and a move).
template <unsigned OFF>
__device__ inline void copy16_to_lds_at(u32x4 rsrc, unsigned voff, unsigned base) {
    asm volatile("s_add_u32 m0, %2, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(rsrc), "s"(__builtin_amdgcn_readfirstlane(base)), "i"(OFF)
                 : "memory", "m0", "scc");
}
__device__ inline void copy4_to_lds(u32x4 rsrc, unsigned voff, unsigned lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(rsrc), "s"(__builtin_amdgcn_readfirstlane(lds))
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// LDS byte address of a pointer into the work group's LDS.
__device__ inline unsigned lds_addr(const void* p) {
    return (unsigned)(size_t)(const lds_u8*)p;
}

// Issue the loads of rows [row0, row0 + ROWS) of one head's [s][D] tensor
// into a padded LDS tile, 1 KiB blocks dealt round-robin over the NW waves.
// `rsrc` covers exactly that head's s rows, so rows past the end read as
// zero; slots that fall in a row's padding or past the tile are pointed out
// of range (and write zeros), so the destination region must extend to a
// whole number of 1 KiB blocks.  Completion: s_waitcnt vmcnt(0), then a
// barrier.
template <typename T, int D, int ROWS, int NW>
__device__ inline void load_tile_async(unsigned tile, u32x4 rsrc, int row0, int w, int lane) {
    using P = Pad<T, D>;
    constexpr int TOTAL = ROWS * P::RS;
    constexpr int BLOCKS = (TOTAL + 1023) / 1024;
#pragma unroll
    for (int it = 0; it < (BLOCKS + NW - 1) / NW; ++it) {
        const int blk = w + NW * it;
        if (blk < BLOCKS) {
            const int byte = blk * 1024 + lane * 16;
            const int row = byte / P::RS, inrow = byte % P::RS;
            const unsigned voff = (byte < TOTAL && inrow < P::RB) ? (unsigned)((row0 + row) * P::RB + inrow)
                                                                 : kOutOfRange;
            copy16_to_lds(rsrc, voff, tile + blk * 1024);
        }
    }
}

// Block `it` of this wave in load_tile_async, without a branch: a block
// index past the tile is sent to `sink` (1 KiB of LDS that nobody reads)
// with every lane out of range.
template <typename T, int D, int ROWS, int NW>
__device__ inline void load_tile_block(unsigned tile, unsigned sink, u32x4 rsrc, int row0, int w, int lane, int it) {
    using P = Pad<T, D>;
    constexpr int TOTAL = ROWS * P::RS;
    constexpr int BLOCKS = (TOTAL + 1023) / 1024;
    const int blk = w + NW * it;
    const int byte = blk * 1024 + lane * 16;
    const int row = byte / P::RS, inrow = byte % P::RS;
    const unsigned voff = (byte < TOTAL && inrow < P::RB) ? (unsigned)((row0 + row) * P::RB + inrow) : kOutOfRange;
    copy16_to_lds(rsrc, voff, blk < BLOCKS ? tile + blk * 1024 : sink);
}

// load_tile_block for a block index IT known at compile time, from
// tile_w = tile + w * 1024 (this wave's first block): where no wave's block
// IT reaches past the tile, no sink selection and one scalar instruction for
// the destination.
template <typename T, int D, int ROWS, int NW, int IT>
__device__ inline void load_tile_block_c(unsigned tile, unsigned tile_w, unsigned sink, u32x4 rsrc, int row0, int w,
                                         int lane) {
    using P = Pad<T, D>;
    constexpr int TOTAL = ROWS * P::RS;
    constexpr int BLOCKS = (TOTAL + 1023) / 1024;
    if constexpr (NW - 1 + NW * IT < BLOCKS) {
        const int byte = (w + NW * IT) * 1024 + lane * 16;
        const int row = byte / P::RS, inrow = byte % P::RS;
        const unsigned voff = (byte < TOTAL && inrow < P::RB) ? (unsigned)((row0 + row) * P::RB + inrow) : kOutOfRange;
        copy16_to_lds_at<(unsigned)(NW * IT * 1024)>(rsrc, voff, tile_w);
    } else {
        load_tile_block<T, D, ROWS, NW>(tile, sink, rsrc, row0, w, lane, IT);
    }
}

// n consecutive fp32 values of a per-row vector (rows [row0, row0 + n),
// n <= 64) into LDS, by one wave; rows past the resource read as zero.
__device__ inline void load_vec_async(unsigned dst, u32x4 rsrc, int row0, int n, int lane) {
    if (lane < n) copy4_to_lds(rsrc, (unsigned)((row0 + lane) * 4), dst);
}

// MFMA operand whose contraction index runs ALONG a row of a padded tile:
// lane (16g + i) gets row `row`, elements col .. col+7 (col = 8-aligned).
template <typename T, int D>
__device__ inline typename Elem<T>::vec8 frag_row(const unsigned char* tile, int row, int col) {
    using S = Pad<T, D>;
    using V8 = typename Elem<T>::vec8;
    if constexpr (sizeof(T) == 2) {
        return *reinterpret_cast<const V8*>(tile + S::off(row, col));
    } else {
        const f32x4 a = *reinterpret_cast<const f32x4*>(tile + S::off(row, col));
        const f32x4 b = *reinterpret_cast<const f32x4*>(tile + S::off(row, col + 4));
        return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
    }
}

// MFMA operand whose contraction index runs DOWN the columns of a padded
// tile: lane (16g + i) receives column col + i at rows rowA..rowA+3
// (elements 0..3) and rowB..rowB+3 (elements 4..7), rowA/rowB chosen per
// lane group.  For bf16, ds_read_b64_tr_b16 transposes within each 16-lane
// group: result lane i, element e is element i%4 of the 4-vector read by
// lane i/4 + 4e of the group, so lane j of the group reads row rowX + j/4,
// columns col + 4*(j%4) .. +3.  fp32 uses plain scalar reads.
template <typename T, int D>
__device__ inline typename Elem<T>::vec8 frag_col(const unsigned char* tile, int rowA, int rowB, int col, int c16) {
    using S = Pad<T, D>;
    typename Elem<T>::vec8 r;
    if constexpr (sizeof(T) == 2) {
        const int rr = c16 >> 2, cc = col + 4 * (c16 & 3);
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tile + S::off(rowA + rr, cc)));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tile + S::off(rowB + rr, cc)));
        const s16x4 both[2] = {lo, hi};
        r = *reinterpret_cast<const typename Elem<T>::vec8*>(both);
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            r[e] = *reinterpret_cast<const float*>(tile + S::off(rowA + e, col + c16));
            r[4 + e] = *reinterpret_cast<const float*>(tile + S::off(rowB + e, col + c16));
        }
    }
    return r;
}

// Compile-time loop: f(std::integral_constant<int, I>) for I in [B, E).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

// The bf16 column operand of frag_col, as two ds_read_b64_tr_b16 at
// compile-time byte offsets OLO and OHI from a per-lane pointer (row
// rowX + lane/4, column col + 4*(lane%4) of the 16-lane group).
template <int OLO, int OHI>
__device__ inline bf16x8 tr_frag(const lds_u8* p) {
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + OLO));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + OHI));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

}  // namespace attn
