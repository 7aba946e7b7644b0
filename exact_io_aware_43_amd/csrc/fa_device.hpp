// Device-side building blocks for the gfx950 attention kernels: vector types,
// the 32x32x16 MFMA wrappers and their register layouts, and small load/store
// helpers.
//
// MFMA v_mfma_f32_32x32x16_{bf16,f16} register layout (wave64), used by every
// kernel here. Lane l, with c = l % 32 and kg = l / 32:
//   A (32 x 16, M x K): lane l holds A[m = c][k = 8*kg + e], e = 0..7
//   B (16 x 32, K x N): lane l holds B[k = 8*kg + e][n = c], e = 0..7
//   C (32 x 32, fp32):  acc[4*i + j] = C[m = 8*i + 4*kg + j][n = c], i, j = 0..3
// Only the pairing matters for the K index: the kernels give element e of lane
// l the same k in A and in B, so any consistent k permutation is a valid
// contraction.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "fa_internal.hpp"

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Last word of a raw buffer descriptor (no stride, no swizzle; 32-bit data
// format) as the CDNA3/CDNA4 buffer instructions expect it.
constexpr int kBufferWord3 = 0x00020000;

template <typename T>
struct Mfma;

template <>
struct Mfma<__bf16> {
    using V8 = bf16x8;
    static __device__ __forceinline__ f32x16 mma(V8 a, V8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};

template <>
struct Mfma<_Float16> {
    using V8 = f16x8;
    static __device__ __forceinline__ f32x16 mma(V8 a, V8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
};

template <typename T>
using V8 = typename Mfma<T>::V8;

// Round-to-nearest-even conversion of 8 fp32 values into one MFMA operand.
template <typename T>
__device__ __forceinline__ V8<T> pack8(float x0, float x1, float x2, float x3, float x4, float x5,
                                       float x6, float x7) {
    V8<T> r;
    r[0] = (T)x0; r[1] = (T)x1; r[2] = (T)x2; r[3] = (T)x3;
    r[4] = (T)x4; r[5] = (T)x5; r[6] = (T)x6; r[7] = (T)x7;
    return r;
}

// Four fp32 values -> four 16-bit values in 8 bytes (RNE).
template <typename T>
__device__ __forceinline__ uint2 pack4(float x0, float x1, float x2, float x3) {
    typedef T T4 __attribute__((ext_vector_type(4)));
    T4 r;
    r[0] = (T)x0; r[1] = (T)x1; r[2] = (T)x2; r[3] = (T)x3;
    return __builtin_bit_cast(uint2, r);
}

template <typename T>
__device__ __forceinline__ V8<T> as_v8(uint4 u) {
    return __builtin_bit_cast(V8<T>, u);
}

__device__ __forceinline__ uint4 ld_g16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ uint4 ld_s16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// tanh x = 1 - 2 / (e^(2x) + 1), with e^(2x) = 2^(2x log2 e): one exponential
// and one reciprocal. Saturates to +-1 (e^(2x) = inf or 0); near 0 the
// subtraction leaves an absolute error of a few fp32 ulps of 1.
__device__ __forceinline__ float tanh_fast(float x) {
    const float e = exp2_fast(x * (2.f * kLog2e));
    return 1.f - 2.f * __builtin_amdgcn_rcpf(e + 1.f);
}

// acc + x0 + x1 for a packed pair of 16-bit values (x0, x1), with one v_dot2
// against (1, 1): the products are exact and the sum is taken in fp32.
template <typename T>
__device__ __forceinline__ float add_pair(uint32_t pair, float acc);
template <>
__device__ __forceinline__ float add_pair<__bf16>(uint32_t pair, float acc) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pair), one, acc, false);
}
template <>
__device__ __forceinline__ float add_pair<_Float16>(uint32_t pair, float acc) {
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
    const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, pair), one, acc, false);
}

// Philox-4x32 with 10 rounds (Salmon, Moraes, Dror, Shaw, "Parallel Random
// Numbers: As Easy as 1, 2, 3", SC'11): a bijection of the 128-bit counter
// (c0, c1, c2, c3) under the 64-bit key (k0, k1). Each round takes the 64-bit
// products of c0 and c2 with the multipliers 0xD2511F53 and 0xCD9E8D57, mixes
// their high halves with the other words and the key, and bumps the key by
// the Weyl constants 0x9E3779B9 and 0xBB67AE85. The key is wave-uniform, so
// its schedule runs on the scalar unit.
__device__ __forceinline__ uint4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                                               uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
        const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
        const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        c0 = hi1 ^ c1 ^ k0;
        c1 = lo1;
        c2 = hi0 ^ c3 ^ k1;
        c3 = lo0;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    return make_uint4(c0, c1, c2, c3);
}

// Keep mask of two 16-bit values from two random bytes of `word` (bytes
// 2 * hi and 2 * hi + 1): each 16-bit half is 0xFFFF when its byte is below
// K (`k2` = K | K << 16, K <= 256) and 0 otherwise. The bytes are spread to
// the halves, K subtracted in 16-bit lanes and the sign bit replicated.
__device__ __forceinline__ uint32_t keep_mask2(uint32_t word, int hi, uint32_t k2) {
    typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
    typedef short i16x2 __attribute__((ext_vector_type(2)));
    const uint32_t x = __builtin_amdgcn_perm(0u, word, hi ? 0x0c030c02u : 0x0c010c00u);
    const u16x2 d = __builtin_bit_cast(u16x2, x) - __builtin_bit_cast(u16x2, k2);
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(i16x2, d) >> (short)15);
}

// Maximum / sum of x over lanes l and l ^ 32 with v_permlane32_swap (a
// register exchange between the two halves of the wave, no LDS round trip).
// Both lanes get the same value, with the same rounding.
__device__ __forceinline__ float max_xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Transposing LDS read (ds_read_b64_tr_b16). Within each group of 16 lanes,
// lane 4a + c receives element c of the 8-byte chunks addressed by lanes
// a, a + 4, a + 8 and a + 12 of the group, in that order. If lane r of a group
// addresses row (row0 + r / 4), columns (col0 + 4 * (r % 4)) .. +3 of a
// row-major 16-bit tile, lane r receives column (col0 + r) of rows
// row0 .. row0 + 3: four consecutive rows of one column.
__device__ __forceinline__ uint2 ld_s8_tr(const uint16_t* p) {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4*)((__attribute__((address_space(3))) uint16_t*)p));
    return __builtin_bit_cast(uint2, v);
}

// Load of a wave-uniform, kernel-invariant value through the scalar cache
// (s_load): unlike a vector load it is not counted by vmcnt, so waiting for it
// does not also wait for the direct loads in flight.
__device__ __forceinline__ float ld_uniform(const float* p) {
#if defined(__HIP_DEVICE_COMPILE__)
    return *(const __attribute__((address_space(4))) float*)p;
#else
    return *p;
#endif
}

// Swizzled 16-bit tile in LDS: rows of exactly D elements, and the 16-byte chunk
// c of row r stored at chunk position c ^ f(r), f(r) = ((r & 3) * D / 32) ^ ((r >> 2) & 3).
// With it, three access patterns are free of bank conflicts: 16-byte reads of
// one chunk from 32 consecutive rows (row-major MFMA operands), the transposing
// 8-byte reads of 4 rows x 64 bytes per half-wave (transposed operands), and
// 16-byte writes of whole rows by consecutive lanes. `col` is a multiple of 4.
template <int D>
__host__ __device__ constexpr int swz(int row, int col) {
    const int f = ((row & 3) * (D / 32)) ^ ((row >> 2) & 3);
    return row * D + (((col >> 3) ^ f) << 3) + (col & 7);
}

// Row-major operand read from a swizzled tile: element offset of (row, col) for
// row = 32 * blk + (lane % 32), col = 16 * kk + 8 * (lane / 32). The block
// part is the constant 32 * blk * D because the swizzle depends on row % 16
// only; this returns the lane part, to be kept in a register for each kk.
template <int D>
__host__ __device__ constexpr int swz_row_off(int lane, int kk) {
    return swz<D>(lane & 31, 16 * kk + 8 * (lane >> 5));
}

// Transposed operand read from a swizzled tile: the MFMA A operand whose
// contraction index runs along the rows (for example V^T from V[key][d]),
// built from two transposing reads (ld_s8_tr). Lane l gets column
// 32 * db + (l % 32) of rows {4 kg .. 4 kg + 3} (half = 0) and
// {8 + 4 kg .. 8 + 4 kg + 3} (half = 1) of a 16-row chunk, kg = l / 32: the k
// order the score accumulator hands to its transposed operand. This returns
// the lane part of each read's offset; chunk c adds the constant 16 * c * D.
template <int D>
__host__ __device__ constexpr int swz_tr_off(int lane, int db, int half) {
    const int r = lane & 15, grp = lane >> 4;
    return swz<D>(8 * half + 4 * (grp >> 1) + (r >> 2), 32 * db + 16 * (grp & 1) + 4 * (r & 3));
}

// XOR forms of the two lane offsets. A row starts at a multiple of D elements
// and the swizzled chunk bits sit below D, so the kk (or db, half) part of an
// offset enters as an XOR with a constant of the lane's base offset (kk = 0,
// db = half = 0), plus 8 D per half. One v_xor per read then replaces a
// register per operand group.
template <int D>
__host__ __device__ constexpr int swz_row_x(int rbase, int kk) {
    return rbase ^ (16 * kk);
}
template <int D>
__host__ __device__ constexpr int swz_tr_x(int tbase, int db, int half) {
    return (tbase ^ (32 * db + 16 * half)) + 8 * half * D;
}
template <int D>
constexpr bool swz_xor_forms_hold() {
    for (int lane = 0; lane < 64; ++lane) {
        for (int kk = 0; kk < D / 16; ++kk)
            if (swz_row_x<D>(swz_row_off<D>(lane, 0), kk) != swz_row_off<D>(lane, kk)) return false;
        for (int db = 0; db < D / 32; ++db)
            for (int half = 0; half < 2; ++half)
                if (swz_tr_x<D>(swz_tr_off<D>(lane, 0, 0), db, half) != swz_tr_off<D>(lane, db, half)) return false;
    }
    return true;
}
static_assert(swz_xor_forms_hold<32>() && swz_xor_forms_hold<64>() && swz_xor_forms_hold<128>() &&
                  swz_xor_forms_hold<256>(),
              "XOR forms of the swizzled offsets");

// Direct global -> LDS staging (buffer_load_dwordx4 ... lds) of a [ROWS x D]
// 16-bit tile into a swizzled LDS tile. Each instruction of a wave fills 1 KB
// of LDS, lane L writing bytes 16 L .. 16 L + 15; the lane fetches from global
// memory the 16-byte chunk that belongs at that position, at a byte offset
// from the tile's first row that is fixed for the kernel (precomputed once).
// Per tile only a buffer descriptor is built (scalar code): its base is the
// tile's first row and its size ends with the last element of row `nrows` - 1
// in memory, so the hardware range check turns the chunks of rows at or past
// `nrows` into zeros. Every
// kernel masks such rows (P = 0), and zero rows contribute exactly zero. `NW`
// waves share the tile; a tile of fewer 1 KB instructions than waves (small
// head dims) is issued by the first INSTR waves alone. The loads complete
// asynchronously (vmcnt); callers wait and barrier before reading the tile.
template <int D, int ROWS, int NW>
struct DmaTile {
    static constexpr int INSTR = ROWS * D * 2 / 1024;
    static constexpr bool PARTIAL = INSTR < NW;  // waves at or past INSTR issue nothing
    static constexpr int PER_WAVE = PARTIAL ? 1 : INSTR / NW;
    static_assert(INSTR >= 1 && (PARTIAL || INSTR % NW == 0), "tile must split evenly over the waves");
    // the immediate offset field reaches 4 KB: one LDS base per 4 instructions
    static_assert(PER_WAVE <= 4 || PER_WAVE % 4 == 0, "instructions per wave: 1..4 or a multiple of 4");
    // byte offset of this lane's chunk of instruction i from the tile's first
    // row (row stride `ld`), less the instruction's immediate offset 1024 i
    uint32_t boff[PER_WAVE];
    uint32_t ld2;             // row stride in bytes
    uint32_t rowb;            // bytes of one row in memory (2 dl)

    // `dl`: elements per row in memory (D, or fewer for a tile whose upper
    // columns are padding): chunks at or past it take an offset beyond any
    // buffer range, so the range check stores zeros there and nothing is read.
    // The range ends after the last valid row's dl elements: with a row stride
    // below 2 D bytes (head dim 16 in the 32-wide tiles, one head) an end at D
    // elements would take in the first chunks of the row after it, past the
    // end of the tensor for the last row.
    __device__ __forceinline__ void init(int wave, int lane, size_t ld, int dl = D) {
        ld2 = (uint32_t)(ld * 2);
        rowb = 2u * (uint32_t)dl;
#pragma unroll
        for (int i = 0; i < PER_WAVE; ++i) {
            const int p = (wave * PER_WAVE + i) * 64 + lane;  // chunk index in LDS order
            const int row = p / (D / 8), pos = p % (D / 8);
            const int f = ((row & 3) * (D / 32)) ^ ((row >> 2) & 3);
            const int gc = pos ^ f;  // chunk of the row in memory
            boff[i] = 8 * gc < dl ? (uint32_t)row * ld2 + 16u * (uint32_t)gc - 1024u * (uint32_t)(i % 4) : 0x80000000u;
        }
    }

    // Rows [row_start, row_start + ROWS) of `base` (16-bit elements, any
    // 16-bit type viewed as uint16_t); rows at or past `nrows` read as zero.
    __device__ __forceinline__ void issue(uint16_t* tile, const uint16_t* base, int row_start, int nrows,
                                          int wave) const {
#if defined(__HIP_DEVICE_COMPILE__)  // the buffer descriptor type exists for the GPU target only
        if (PARTIAL && wave >= INSTR) return;
        const int valid = min(nrows - row_start, ROWS);
        const uint32_t bytes = valid > 0 ? (uint32_t)(valid - 1) * ld2 + rowb : 0u;
        const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t*>(base) + (size_t)row_start * (ld2 / 2), (short)0, (int)bytes, kBufferWord3);
        // One LDS base (M0) per wave, tile and group of 4 instructions: the
        // immediate offset 1024 (i % 4) of instruction i moves both the global
        // and the LDS address, so M0 is set once per group instead of once per
        // instruction from a vector register.
        typedef __attribute__((address_space(3))) void lds_void;
#pragma unroll
        for (int g0 = 0; g0 < PER_WAVE; g0 += 4) {
            lds_void* dst =
                (lds_void*)((__attribute__((address_space(3))) uint16_t*)(tile + (wave * PER_WAVE + g0) * 512));
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, dst, 16, boff[g0], 0, 0, 0);
            if constexpr (PER_WAVE > 1) __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, dst, 16, boff[g0 + 1], 0, 1024, 0);
            if constexpr (PER_WAVE > 2) __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, dst, 16, boff[g0 + 2], 0, 2048, 0);
            if constexpr (PER_WAVE > 3) __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, dst, 16, boff[g0 + 3], 0, 3072, 0);
        }
#else
        (void)tile, (void)base, (void)row_start, (void)nrows, (void)wave;
#endif
    }
};

// Direct global -> LDS load of `count` (<= 64) consecutive fp32 values (one wave,
// 4 bytes per lane) from `src` into dst[0 .. 64): the buffer range ends after
// `count` values, so lanes at or past it read nothing from memory and store
// zero. Buffer form, like the tiles: the FLAT-encoded global_load_lds would
// also count against lgkmcnt, after which the compiler can no longer count LDS
// reads exactly and waits for all of them before every MFMA, defeating the
// operand prefetch rings.
__device__ __forceinline__ void dma_vec(float* dst, const float* src, int lane, int count) {
#if defined(__HIP_DEVICE_COMPILE__)  // the buffer descriptor type exists for the GPU target only
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(src), (short)0, count * 4, kBufferWord3);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rsrc, (__attribute__((address_space(3))) void*)((__attribute__((address_space(3))) float*)dst), 4,
        (uint32_t)lane * 4u, 0, 0, 0);
#else
    (void)dst, (void)src, (void)lane, (void)count;
#endif
}

// The double-buffered tile loop shared by the kernels: body(stage, i) runs for
// i in [0, n) while issue(other stage, i + 1) prefetches the next tile. The two
// stages are distinct __shared__ arrays so that the compiler can tell the
// prefetch's LDS writes apart from the body's LDS reads and does not wait for
// the prefetch before reading.
template <class Issue, class Body>
__device__ __forceinline__ void two_stage_loop(uint16_t* A, uint16_t* B, int n, Issue&& issue, Body&& body) {
    issue(A, 0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int i = 0; i < n; i += 2) {
        if (i + 1 < n) issue(B, i + 1);
        body(static_cast<const uint16_t*>(A), i);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (i + 1 >= n) break;
        if (i + 2 < n) issue(A, i + 2);
        body(static_cast<const uint16_t*>(B), i + 1);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }
}

// Query head of grid column x. Workgroups are dealt to the eight XCDs (each
// with its own L2) in turn, so with H a multiple of 8 column x runs on XCD
// x % 8. Numbering the columns kv-head-major (x = g + Hkv * i for query head
// G g + i) puts the G query heads that read one kv head's K and V on the same
// XCD whenever Hkv divides 8 or is a multiple of it; with G = 1 it is the
// identity.
__device__ __forceinline__ int query_head(const Args& a, int x) { return (x % a.Hkv) * a.G + x / a.Hkv; }

// Sequence base row and length of batch entry / packed sequence b; lengths are
// clamped to [0, N] so a malformed cu_seqlens cannot enlarge the grid's work.
__device__ __forceinline__ void seq_bounds(const Args& a, int b, int& row0, int& len) {
    if (a.cu) {
        row0 = a.cu[b];
        len = a.cu[b + 1] - row0;
        len = len < 0 ? 0 : (len > a.N ? a.N : len);
    } else {
        row0 = b * a.N;
        len = a.N;
    }
}

}  // namespace fa
