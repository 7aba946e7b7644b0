// FP8 (e4m3) forward attention with power-of-two block scales and an optional
// Walsh-Hadamard rotation of Q and K, on the gfx950 32x32x64 f8f6f4 MFMA.
//
// Method: "FlashAttention: Faster Attention Without Dropping a Single
// Interaction", Method Deep Dive, Key design 4 (the FlashAttention-3 row: FP8
// with block quantization and incoherent processing) on top of Key designs 1
// and 2 (tiling, the mergeable softmax state). The details are this library's
// reading of techniques the page only names:
//
//   Q, K: one power-of-two scale 2^e per (sequence, head, 128 tokens), the
//         smallest with amax <= 448 * 2^e, so x * 2^-e is exact; optionally each
//         row first multiplied by caller-given signs and the unnormalized
//         Walsh-Hadamard matrix (fp32 butterflies, stages h = 1, 2, 4, ...),
//         after which Q'K'^T = d QK^T and the softmax scale is divided by d.
//   V:    one power-of-two scale per (sequence, kv head, channel), folded into
//         O at the end (O[:, c] = 2^e_c sum_j P_j V8[j, c]); stored transposed
//         ([B, Hkv, d, NP], NP = N rounded up to a whole 128-key tile, keys
//         permuted within 64-key chunks) so that each MFMA lane's 32 keys of a
//         chunk are contiguous bytes.
//   P:    rounded to e4m3 for the second product (P <= 448 by the sum bound of
//         the maximum-free path); O is divided by the sum of exactly those
//         rounded values, lse uses the fp32 sum. The rounded sums come from the
//         matrix cores as well: one 16x16x128 product per 64-key chunk of a
//         constant 0 / 1 operand with the P operand as it stands.
//
// e4m3 here is the OCP "fn" encoding that v_cvt_pk_fp8_f32 produces (round to
// nearest even; values past 464 would become NaN, which the scaling rules out).
//
// Forward work decomposition as the 16-bit kernel: 8 waves, 256 query rows per
// workgroup, 32 per wave; K and V^T tiles of 128 keys double buffered in LDS
// with direct loads (byte rows handled as 16-bit pairs by the same swizzled
// tile code). Per tile and wave: S^T = K Q^T in 8 MFMAs of 32x32x64 (head dim
// 128), the softmax, O^T += V^T P^T in 8 more.
#include <type_traits>

#include "fa_device.hpp"

namespace fa {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int QB = 128;  // tokens per Q / K scale block

// 32x32x64 e4m3 x e4m3 -> fp32 (operand formats 0 and 0, unit E8M0 scales).
__device__ __forceinline__ f32x16 mma_f8(v8i a, v8i b, f32x16 c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// 16x16x128 e4m3 x e4m3 -> fp32.
__device__ __forceinline__ f32x4 mma_f8_16(v8i a, v8i b, f32x4 c) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// Smallest e >= -127 with amax <= 448 * 2^e, from the bits of amax = m 2^E,
// m in [1, 2): E - 8 when m <= 1.75, E - 7 otherwise; 0 for amax = 0. The
// floor keeps 2^e and 2^-e finite in fp32; it also covers subnormal amax, whose
// exponent field reads as E = -127.
__device__ __forceinline__ int block_exp(float amax) {
    const uint32_t u = __float_as_uint(amax);
    if (amax == 0.f) return 0;
    const int E = (int)((u >> 23) & 0xFF) - 127;
    return max((u & 0x7FFFFF) <= 0x600000u ? E - 8 : E - 7, -127);
}

// e4m3 codes of (x0, x1) into bytes 0, 1 (HI = false) or 2, 3 (HI = true) of old.
template <bool HI>
__device__ __forceinline__ uint32_t cvt2(float x0, float x1, uint32_t old) {
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, (int)old, HI);
}

// Eight 16-bit values of one 16-byte load as fp32 (exact).
template <typename T>
__device__ __forceinline__ void unpack8(const uint4 u, float* f) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if constexpr (std::is_same_v<T, __bf16>) {
            f[2 * i] = __uint_as_float(w[i] << 16);
            f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
        } else {
            f[2 * i] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] & 0xFFFF));
            f[2 * i + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] >> 16));
        }
    }
}

// 16 fp32 values (already scaled into e4m3 range) as 16 codes in one uint4.
__device__ __forceinline__ uint4 pack16(const float* x) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = cvt2<true>(x[4 * i + 2], x[4 * i + 3], cvt2<false>(x[4 * i], x[4 * i + 1], 0u));
    return make_uint4(w[0], w[1], w[2], w[3]);
}

// ---------------------------------------------------------------- Q, K
// One workgroup of 2 waves per (head, 128-token block, sequence); each lane owns
// one row: the sign flips and all log2(D) butterfly stages in registers (no
// cross-lane traffic), then the block maximum over both waves, the scale and
// the codes. Rows of one head lie H d elements apart, so the block's rows pass
// through LDS both ways: D / 8 consecutive lanes move one row's 16-byte chunks
// (row-contiguous loads and stores), and each lane reads back its own row.
template <typename T, int D, bool ROT>
__global__ __launch_bounds__(128) void quant_qk_kernel(const T* __restrict__ x, uint8_t* __restrict__ codes,
                                                       float* __restrict__ scales, int N, int H,
                                                       unsigned long long s0, unsigned long long s1) {
    constexpr int CPR = D / 8;          // 16-byte input chunks per row
    constexpr int RPP = QB / CPR;       // rows per pass of the workgroup
    constexpr int LDR = 2 * D + 16;     // staged row pitch in bytes (padded against bank conflicts)
    __shared__ float wmax[2];
    __shared__ __attribute__((aligned(16))) uint8_t stage[QB * LDR];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    // grid x = head: workgroups dispatched together read the neighbouring head
    // slices of the same token rows (contiguous memory) rather than rows H d
    // elements apart
    const int h = blockIdx.x, blk = blockIdx.y, b = blockIdx.z;
    const int nb = (N + QB - 1) / QB;
    {
        // pass p: row p * RPP + threadIdx.x / CPR, chunk threadIdx.x % CPR; rows
        // past N stage zeros. Loads in groups of 16 so that d = 256 stays in
        // registers.
        const int cc = threadIdx.x % CPR, r0 = threadIdx.x / CPR;
        constexpr int NP = QB / RPP, GRP = NP < 16 ? NP : 16;
#pragma unroll
        for (int p0 = 0; p0 < NP; p0 += GRP) {
            uint4 u[GRP];
#pragma unroll
            for (int p = 0; p < GRP; ++p) {
                const int rr = (p0 + p) * RPP + r0, tt = blk * QB + rr;
                u[p] = make_uint4(0, 0, 0, 0);
                if (tt < N) u[p] = *reinterpret_cast<const uint4*>(x + (((size_t)b * N + tt) * H + h) * D + 8 * cc);
            }
#pragma unroll
            for (int p = 0; p < GRP; ++p)
                *reinterpret_cast<uint4*>(stage + ((p0 + p) * RPP + r0) * LDR + 16 * cc) = u[p];
        }
    }
    __syncthreads();
    float r[D];
#pragma unroll
    for (int c = 0; c < CPR; ++c)
        unpack8<T>(*reinterpret_cast<const uint4*>(stage + threadIdx.x * LDR + 16 * c), r + 8 * c);
    if (ROT) {
        // signs (bit i % 64 of word i / 64 set: -1), then stages h = 1, 2, 4, ...:
        // the pair (i, i + h) of every 2h-block becomes (a + b, a - b)
#pragma unroll
        for (int i = 0; i < D; ++i) {
            const unsigned long long wd = i < 64 ? s0 : s1;
            r[i] = __uint_as_float(__float_as_uint(r[i]) ^ ((uint32_t)((wd >> (i & 63)) & 1ull) << 31));
        }
#pragma unroll
        for (int hh = 1; hh < D; hh *= 2) {
#pragma unroll
            for (int i = 0; i < D; ++i) {
                if (i & hh) continue;
                const float p = r[i], q = r[i + hh];
                r[i] = p + q;
                r[i + hh] = p - q;
            }
        }
    }
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < D; ++i) amax = fmaxf(amax, fabsf(r[i]));
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m));
    if (lane == 0) wmax[wave] = amax;
    __syncthreads();
    amax = fmaxf(wmax[0], wmax[1]);
    const int e = block_exp(amax);
    const float inv = __builtin_ldexpf(1.f, -e);
    if (threadIdx.x == 0) scales[((size_t)b * H + h) * nb + blk] = __builtin_ldexpf(1.f, e);
#pragma unroll
    for (int i = 0; i < D; ++i) r[i] *= inv;
    // the codes of this lane's row over its own staged row (only this lane
    // reads or writes it until the barrier), then row-contiguous stores
#pragma unroll
    for (int c = 0; c < D / 16; ++c)
        *reinterpret_cast<uint4*>(stage + threadIdx.x * LDR + 16 * c) = pack16(r + 16 * c);
    __syncthreads();
    {
        constexpr int CPO = D / 16, RPO = QB / CPO;  // 16-byte code chunks per row, rows per pass
        const int cc = threadIdx.x % CPO, r0 = threadIdx.x / CPO;
#pragma unroll
        for (int p = 0; p < QB / RPO; ++p) {
            const int rr = p * RPO + r0, tt = blk * QB + rr;
            if (tt < N)
                *reinterpret_cast<uint4*>(codes + (((size_t)b * N + tt) * H + h) * D + 16 * cc) =
                    *reinterpret_cast<const uint4*>(stage + rr * LDR + 16 * cc);
        }
    }
}

// ---------------------------------------------------------------- V
// Pass 1: per-channel |v| maximum over the sequence, as float bits (order-
// preserving for non-negative values) with atomic max into `scales`, which the
// clear kernel zeroed first. Pass 2 turns it into 2^e and writes the codes.
__global__ void clear_kernel(float* p, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0.f;
}

// One workgroup per (kv head, 256 rows, sequence): a thread reads 8 channels of
// every (256 / (D / 8))-th row with 16-byte loads; lanes of equal channels
// reduce by shuffles, the four waves through LDS, then one atomic per channel.
template <typename T, int D>
__global__ __launch_bounds__(256) void v_amax_kernel(const T* __restrict__ v, float* __restrict__ scales, int N,
                                                     int Hkv) {
    constexpr int CG = D / 8;        // 16-byte chunks per row
    constexpr int RPI = 256 / CG;    // rows per iteration of the workgroup
    __shared__ float part[4][D];
    const int g = blockIdx.x, b = blockIdx.z;  // grid x = kv head (as the Q/K quantizer)
    const int cg = threadIdx.x % CG, r0 = threadIdx.x / CG;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int t0 = blockIdx.y * 256, t1 = min(N, t0 + 256);
    // all 256 / RPI loads of a thread issued before the first is used; a row
    // past t1 re-reads row t1 - 1, which leaves every maximum unchanged
    uint4 u[256 / RPI];
#pragma unroll
    for (int it = 0; it < 256 / RPI; ++it) {
        const int t = min(t0 + r0 + it * RPI, t1 - 1);
        u[it] = *reinterpret_cast<const uint4*>(v + (((size_t)b * N + t) * Hkv + g) * D + 8 * cg);
    }
    float m[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int it = 0; it < 256 / RPI; ++it) {
        float f[8];
        unpack8<T>(u[it], f);
#pragma unroll
        for (int i = 0; i < 8; ++i) m[i] = fmaxf(m[i], fabsf(f[i]));
    }
#pragma unroll
    for (int msk = CG; msk < 64; msk *= 2)
#pragma unroll
        for (int i = 0; i < 8; ++i) m[i] = fmaxf(m[i], __shfl_xor(m[i], msk));
    if (lane < CG)
#pragma unroll
        for (int i = 0; i < 8; ++i) part[wave][8 * lane + i] = m[i];
    __syncthreads();
    if (threadIdx.x < D) {
        const int c = threadIdx.x;
        const float mm = fmaxf(fmaxf(part[0][c], part[1][c]), fmaxf(part[2][c], part[3][c]));
        atomicMax(reinterpret_cast<unsigned int*>(scales) + ((size_t)b * Hkv + g) * D + c, __float_as_uint(mm));
    }
}

// One workgroup per (kv head, 128-key tile, sequence). Key n = 32 b + 8 i + 4 kg + j
// of a 64-key chunk goes to byte 32 kg + 16 b + 4 i + j of each channel's
// 64-byte chunk row; keys at or past N are zero. The tile goes through LDS as
// fp32 (rows padded to keep 16-byte alignment; column reads are conflict-free);
// each thread then writes 16 codes of one channel with one 16-byte store.
template <typename T, int D>
__global__ __launch_bounds__(256) void v_quant_kernel(const T* __restrict__ v, uint8_t* __restrict__ codes_t,
                                                      const float* __restrict__ amax, int N, int Hkv, int NP) {
    constexpr int CG = D / 8, LD = D + 4;
    __shared__ __attribute__((aligned(16))) float tile[128 * LD];
    const int g = blockIdx.x, tt = blockIdx.y, b = blockIdx.z;  // grid x = kv head
    const int k0 = tt * 128;
    // every load of the thread in flight before the first LDS store; keys past
    // the end read key N - 1 and store zeros
    constexpr int NL = 128 * CG / 256;
    uint4 u[NL];
#pragma unroll
    for (int it = 0; it < NL; ++it) {
        const int ci = threadIdx.x + 256 * it, kk = ci / CG, cg = ci % CG;
        const int t = min(k0 + kk, N - 1);
        u[it] = *reinterpret_cast<const uint4*>(v + (((size_t)b * N + t) * Hkv + g) * D + 8 * cg);
    }
#pragma unroll
    for (int it = 0; it < NL; ++it) {
        const int ci = threadIdx.x + 256 * it, kk = ci / CG, cg = ci % CG;
        float f[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (k0 + kk < N) unpack8<T>(u[it], f);
        *reinterpret_cast<float4*>(tile + kk * LD + 8 * cg) = make_float4(f[0], f[1], f[2], f[3]);
        *reinterpret_cast<float4*>(tile + kk * LD + 8 * cg + 4) = make_float4(f[4], f[5], f[6], f[7]);
    }
    __syncthreads();
    // group gi: channel gi / 8, 16-byte group gi % 8 of the channel's 128 bytes
    // (64-key chunk ch2 = group / 4, bytes 16 q .. 16 q + 15 of it, q = group % 4:
    // kg = q / 2, b = q % 2)
#pragma unroll
    for (int it = 0; it < D * 8 / 256; ++it) {
        const int gi = threadIdx.x + 256 * it, c = gi / 8, grp = gi % 8;
        const int ch2 = grp >> 2, kg = (grp >> 1) & 1, b2 = grp & 1;
        const float inv = __builtin_ldexpf(1.f, -block_exp(amax[((size_t)b * Hkv + g) * D + c]));
        float x[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int key = 64 * ch2 + 32 * b2 + 8 * (u >> 2) + 4 * kg + (u & 3);
            x[u] = tile[key * LD + c] * inv;
        }
        *reinterpret_cast<uint4*>(codes_t + (((size_t)b * Hkv + g) * D + c) * NP + k0 + 16 * grp) = pack16(x);
    }
}

__global__ void v_scale_kernel(float* scales, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) scales[i] = __builtin_ldexpf(1.f, block_exp(scales[i]));
}

// ---------------------------------------------------------------- forward
constexpr int F8_BC = 128;  // keys per K / V^T tile (one K scale block)

struct Fp8Args {
    const uint8_t* q;   // [B, N, H, D]
    const uint8_t* k;   // [B, N, Hkv, D]
    const uint8_t* vt;  // [B, Hkv, D, NP]
    const float* qs;    // [B, H, nb]
    const float* ks;    // [B, Hkv, nb]
    const float* vs;    // [B, Hkv, D]
    void* out;          // [B, N, H, D]
    float* lse;         // [B, H, N]
    int B, H, Hkv, N, G, NP, nb;
    float scale_log2;   // softmax scale * log2(e) (already divided by D under the rotation)
};

// NW waves of 32 query rows each; with NW = 4 two workgroups share a CU
template <typename TO, int D, bool CAUSAL, int NW>
__global__ __launch_bounds__(64 * NW, NW == 4 ? 2 : 1) void fwd_fp8_kernel(Fp8Args a) {
    constexpr int F8_BR = 32 * NW, F8_NT = 64 * NW;
    // byte tiles viewed as 16-bit rows of D / 2 (K: keys x D bytes) and
    // F8_BC / 2 (V^T: channels x F8_BC bytes) elements, swizzled like the
    // 16-bit tiles; two named stages
    constexpr int KT = F8_BC * D / 2, VT = D * F8_BC / 2;  // uint16 elements
    constexpr int DK = D / 2, DV = F8_BC / 2;               // 16-bit row lengths
    __shared__ __attribute__((aligned(16))) uint16_t stA[KT + VT];
    __shared__ __attribute__((aligned(16))) uint16_t stB[KT + VT];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int col = lane & 31, kg = lane >> 5;
    const int h = (blockIdx.x % a.Hkv) * a.G + blockIdx.x / a.Hkv;  // kv-head-major columns
    const int b = blockIdx.y;
    const int qt = CAUSAL ? (int)(gridDim.z - 1 - blockIdx.z) : (int)blockIdx.z;
    const int len = a.N;
    const int q0 = qt * F8_BR;
    if (q0 >= len) return;
    const int g = h / a.G;
    const int qw = q0 + wave * 32, qi = qw + col;
    const bool wave_live = qw < len;

    // Q^T operand: lane (query qi, kg) holds bytes 64 kk + 32 kg .. + 31 of the row
    constexpr int NKK = D / 64;
    v8i qf[NKK];
    {
        const uint8_t* qr = a.q + (((size_t)b * a.N + qi) * a.H + h) * D;
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
            uint4 lo = make_uint4(0, 0, 0, 0), hi = lo;
            if (qi < len) {
                lo = *reinterpret_cast<const uint4*>(qr + 64 * kk + 32 * kg);
                hi = *reinterpret_cast<const uint4*>(qr + 64 * kk + 32 * kg + 16);
            }
            qf[kk] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        }
    }
    // the wave's 32 queries lie in one Q scale block (128 = 4 x 32, aligned)
    const float sq = wave_live ? a.qs[((size_t)b * a.H + h) * a.nb + qw / QB] : 0.f;

    // operand offsets (16-bit units) of a lane's two 16-byte chunks: K row
    // 32 kb + col, byte column 64 kk + 32 kg; V^T row 32 db + col, byte column
    // 64 m + 32 kg (chunk m of the tile)
    int koff[NKK][2], voff[2][2];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
        koff[kk][0] = swz<DK>(col, 32 * kk + 16 * kg);
        koff[kk][1] = swz<DK>(col, 32 * kk + 16 * kg + 8);
    }
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        voff[m][0] = swz<DV>(col, 32 * m + 16 * kg);
        voff[m][1] = swz<DV>(col, 32 * m + 16 * kg + 8);
    }

    const int kend = CAUSAL ? min(len, q0 + F8_BR) : len;
    const int nkt = (kend + F8_BC - 1) / F8_BC;
    const uint16_t* Kg = reinterpret_cast<const uint16_t*>(a.k + ((size_t)b * a.N * a.Hkv + g) * D);
    const uint16_t* Vg = reinterpret_cast<const uint16_t*>(a.vt + ((size_t)b * a.Hkv + g) * D * (size_t)a.NP);
    DmaTile<DK, F8_BC, F8_NT / 64> kdma;
    kdma.init(wave, lane, (size_t)a.Hkv * DK);
    DmaTile<DV, D, F8_NT / 64> vdma;
    vdma.init(wave, lane, (size_t)a.NP / 2);
    // K block scale of each stage's tile, read when the tile is issued (a read
    // inside the compute step would wait on the next tile's loads as well)
    const float* ksb = a.ks + ((size_t)b * a.Hkv + g) * a.nb;
    float ksA = 0.f, ksB = 0.f;
    auto issue = [&](uint16_t* st, int kt) {
        if (st == stA)
            ksA = ksb[kt];
        else
            ksB = ksb[kt];
        kdma.issue(st, Kg, kt * F8_BC, len, wave);
        // V^T rows are channels: the tile is columns kt * F8_BC .. of every row
        vdma.issue(st + KT, Vg + kt * (F8_BC / 2), 0, D, wave);
    };

    f32x16 oacc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16{};
    float m_ref = -INFINITY, l_run = 0.f;
    const float c2q = a.scale_log2 * sq;
    // Row sums of the rounded P: A = 1 where (row < 8) == (lane group even),
    // so output rows 0-7 sum the lanes c, c + 32 (query c) and rows 8-15 the
    // lanes c + 16, c + 48 (query c + 16) of column c. Lane L then holds the sum
    // of query L for L < 16 or L >= 48 and that of lane L ^ 48 for 16 <= L < 48.
    const int onew = (((lane & 15) < 8) == (((lane >> 4) & 1) == 0)) ? 0x38383838 : 0;  // e4m3 1.0 = 0x38
    const v8i ones = {onew, onew, onew, onew, onew, onew, onew, onew};
    const int xlane = ((lane >> 4) == 1 || (lane >> 4) == 2) ? lane ^ 48 : lane;
    f32x4 lacc = {};

    auto compute = [&](const uint16_t* S, int kt) {
        const int k0 = kt * F8_BC;
        if (!(wave_live && (!CAUSAL || k0 <= qw + 31))) return;
        const uint16_t* Ks = S;
        const uint16_t* Vs = S + KT;
        const float c2 = c2q * (S == stA ? ksA : ksB);  // scale x log2(e) x Q block scale x K block scale

        f32x16 s[F8_BC / 32];
        auto score_product = [&]() {
#pragma unroll
            for (int kb = 0; kb < F8_BC / 32; ++kb) {
                s[kb] = f32x16{};
#pragma unroll
                for (int kk = 0; kk < NKK; ++kk) {
                    const uint4 lo = ld_s16(Ks + 32 * kb * DK + koff[kk][0]);
                    const uint4 hi = ld_s16(Ks + 32 * kb * DK + koff[kk][1]);
                    const v8i kf = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                                    (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
                    s[kb] = mma_f8(kf, qf[kk], s[kb]);
                }
            }
        };
        score_product();

        const bool edge = (k0 + F8_BC > len) || (CAUSAL && k0 + F8_BC - 1 > qw);
        float ls = 0.f;
        bool need_max = true;
        if (kt != 0 && !edge) {
            // maximum-free: P against the reference; every P of a lane at most
            // its sum, which must stay within e4m3 (448)
            need_max = false;
#pragma unroll
            for (int kb = 0; kb < F8_BC / 32; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float p = exp2_fast(fmaf(s[kb][r], c2, -m_ref));
                    s[kb][r] = p;
                    ls += p;
                }
            if (__any(!(ls <= 448.f))) {
                // a fresh product from LDS: without the clobber the compiler keeps
                // partial products of the first one live across the exponentials
                asm volatile("" ::: "memory");
                score_product();
                need_max = true;
                ls = 0.f;
            }
        }
        if (need_max) {
            const int lim_len = len - k0 - 4 * kg, lim_q = qi - k0 - 4 * kg;
            float mt = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < F8_BC / 32; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float t = s[kb][r] * c2;
                    const int kofs = 32 * kb + 8 * (r >> 2) + (r & 3);
                    if (edge && (kofs >= lim_len || (CAUSAL && kofs > lim_q))) t = -INFINITY;
                    s[kb][r] = t;
                    mt = fmaxf(mt, t);
                }
            mt = max_xor32(mt);
            const bool raise = mt > m_ref + 8.f;
            if (__any(raise)) {
                const float m_new = raise ? mt : m_ref;
                const float alpha = raise ? exp2_fast(m_ref - mt) : 1.f;
                l_run *= alpha;
                lacc *= __shfl(alpha, xlane);
#pragma unroll
                for (int db = 0; db < D / 32; ++db) oacc[db] *= alpha;
                m_ref = m_new;
            }
            const float m_use = (m_ref == -INFINITY) ? 0.f : m_ref;
#pragma unroll
            for (int kb = 0; kb < F8_BC / 32; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float p = exp2_fast(s[kb][r] - m_use);
                    s[kb][r] = p;
                    ls += p;
                }
        }
        l_run += ls;

        // P^T as e4m3, chunk m of 64 keys: byte e = 16 b + r is element r of s[2m + b]
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            uint32_t w[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int bb = q >> 2, r0 = 4 * (q & 3);
                const f32x16& sv = s[2 * m + bb];
                // word q is written over element q of s[2m], an input already
                // converted by then: the eight words land in eight consecutive
                // registers, as the MFMA operand needs, without moves or zeroing
                w[q] = cvt2<true>(sv[r0 + 2], sv[r0 + 3], cvt2<false>(sv[r0], sv[r0 + 1], __float_as_uint(s[2 * m][q])));
            }
            const v8i pf = {(int)w[0], (int)w[1], (int)w[2], (int)w[3], (int)w[4], (int)w[5], (int)w[6], (int)w[7]};
            lacc = mma_f8_16(ones, pf, lacc);
#pragma unroll
            for (int db = 0; db < D / 32; ++db) {
                const uint4 lo = ld_s16(Vs + 32 * db * DV + voff[m][0]);
                const uint4 hi = ld_s16(Vs + 32 * db * DV + voff[m][1]);
                const v8i vf = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                                (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
                oacc[db] = mma_f8(vf, pf, oacc[db]);
            }
        }
    };

    two_stage_loop(stA, stB, nkt, issue, compute);

    const float l_tot = sum_xor32(l_run);
    const float lr_tot = __shfl(lacc[0], xlane);
    if (qi < len) {
        const float inv = 1.f / lr_tot;
        const float* vsc = a.vs + ((size_t)b * a.Hkv + g) * D;
        TO* O = reinterpret_cast<TO*>(a.out) + (((size_t)b * a.N + qi) * a.H + h) * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int d0 = 32 * db + 8 * i + 4 * kg;
                const float4 sc = *reinterpret_cast<const float4*>(vsc + d0);
                *reinterpret_cast<uint2*>(O + d0) =
                    pack4<TO>(oacc[db][4 * i] * inv * sc.x, oacc[db][4 * i + 1] * inv * sc.y,
                              oacc[db][4 * i + 2] * inv * sc.z, oacc[db][4 * i + 3] * inv * sc.w);
            }
        }
        if (kg == 0) a.lse[((size_t)b * a.H + h) * a.N + qi] = (m_ref + __log2f(l_tot)) * kLn2;
    }
}

template <typename T, int D>
hipError_t quant_qk_d(const void* x, uint8_t* codes, float* scales, int B, int N, int H,
                      const unsigned long long* signs, hipStream_t s) {
    dim3 grid(H, (N + QB - 1) / QB, B);
    if (signs)
        hipLaunchKernelGGL((quant_qk_kernel<T, D, true>), grid, dim3(QB), 0, s, reinterpret_cast<const T*>(x), codes,
                           scales, N, H, signs[0], D > 64 ? signs[1] : 0ull);
    else
        hipLaunchKernelGGL((quant_qk_kernel<T, D, false>), grid, dim3(QB), 0, s, reinterpret_cast<const T*>(x),
                           codes, scales, N, H, 0ull, 0ull);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t quant_v_d(const void* v, uint8_t* codes_t, float* scales, int B, int N, int Hkv, hipStream_t s) {
    const int n = B * Hkv * D;
    const int NP = fp8_keys_padded(N);
    hipLaunchKernelGGL(clear_kernel, dim3((n + 255) / 256), dim3(256), 0, s, scales, n);
    hipLaunchKernelGGL((v_amax_kernel<T, D>), dim3(Hkv, (N + 255) / 256, B), dim3(256), 0, s,
                       reinterpret_cast<const T*>(v), scales, N, Hkv);
    hipLaunchKernelGGL((v_quant_kernel<T, D>), dim3(Hkv, NP / 128, B), dim3(256), 0, s,
                       reinterpret_cast<const T*>(v), codes_t, scales, N, Hkv, NP);
    hipLaunchKernelGGL(v_scale_kernel, dim3((n + 255) / 256), dim3(256), 0, s, scales, n);
    return hipGetLastError();
}

template <typename TO, int D, bool CAUSAL, int NW>
hipError_t fwd_nw(const Fp8Args& a, hipStream_t s) {
    dim3 grid(a.H, a.B, (a.N + 32 * NW - 1) / (32 * NW));
    hipLaunchKernelGGL((fwd_fp8_kernel<TO, D, CAUSAL, NW>), grid, dim3(64 * NW), 0, s, a);
    return hipGetLastError();
}

// Four waves (two workgroups per CU) at head dim 64 and for causal masks, eight
// for non-causal head dim 128; outputs are the same either way. Measured on
// the GPT-2-medium shape (d 64): 4 waves 15% faster; causal d 128 at 8192 keys
// with GQA: 6% faster, at 16384 keys even; non-causal d 128: 4% slower.
template <typename TO, int D>
hipError_t fwd_d(const Fp8Args& a, bool causal, hipStream_t s) {
    if (causal) return fwd_nw<TO, D, true, 4>(a, s);
    if constexpr (D == 64)
        return fwd_nw<TO, D, false, 4>(a, s);
    else
        return fwd_nw<TO, D, false, 8>(a, s);
}

}  // namespace

hipError_t launch_quant_qk(const void* x, uint8_t* codes, float* scales, int B, int N, int H, int d,
                           const unsigned long long* signs, int dtype, hipStream_t s) {
    if (dtype == 2)
        return d == 64 ? quant_qk_d<__bf16, 64>(x, codes, scales, B, N, H, signs, s)
                       : quant_qk_d<__bf16, 128>(x, codes, scales, B, N, H, signs, s);
    return d == 64 ? quant_qk_d<_Float16, 64>(x, codes, scales, B, N, H, signs, s)
                   : quant_qk_d<_Float16, 128>(x, codes, scales, B, N, H, signs, s);
}

hipError_t launch_quant_v(const void* v, uint8_t* codes_t, float* scales, int B, int N, int Hkv, int d, int dtype,
                          hipStream_t s) {
    if (dtype == 2)
        return d == 64 ? quant_v_d<__bf16, 64>(v, codes_t, scales, B, N, Hkv, s)
                       : quant_v_d<__bf16, 128>(v, codes_t, scales, B, N, Hkv, s);
    return d == 64 ? quant_v_d<_Float16, 64>(v, codes_t, scales, B, N, Hkv, s)
                   : quant_v_d<_Float16, 128>(v, codes_t, scales, B, N, Hkv, s);
}

hipError_t launch_fwd_fp8(const uint8_t* q, const uint8_t* k, const uint8_t* vt, const float* qs, const float* ks,
                          const float* vs, void* out, float* lse, int B, int H, int Hkv, int N, int d,
                          float scale_log2, bool causal, int out_dtype, hipStream_t s) {
    Fp8Args a{};
    a.q = q;
    a.k = k;
    a.vt = vt;
    a.qs = qs;
    a.ks = ks;
    a.vs = vs;
    a.out = out;
    a.lse = lse;
    a.B = B;
    a.H = H;
    a.Hkv = Hkv;
    a.N = N;
    a.G = H / Hkv;
    a.NP = fp8_keys_padded(N);
    a.nb = (N + QB - 1) / QB;
    a.scale_log2 = scale_log2;
    if (out_dtype == 2) return d == 64 ? fwd_d<__bf16, 64>(a, causal, s) : fwd_d<__bf16, 128>(a, causal, s);
    return d == 64 ? fwd_d<_Float16, 64>(a, causal, s) : fwd_d<_Float16, 128>(a, causal, s);
}

}  // namespace fa
