// Backward attention for 16-bit inputs on gfx950 MFMA.
//
// Method: "FlashAttention: Faster Attention Without Dropping a Single
// Interaction", Method Deep Dive, Key design 3. Nothing quadratic is read back:
// every score tile is rebuilt from Q, K and the saved L = m + ln(l)
// (P_ij = exp(S_ij - L_i)), and the softmax backward uses
// D_i = dO_i . O_i, so dS = P o (dP - D). Three launches run in stream order:
//
//   1. bwd_dsum:  D_i = sum_c dO_ic O_ic in fp32 (memory bound, one pass over
//                 O and dO; O is the stored forward output).
//   2. bwd_dkdv:  one workgroup per (128-key tile, kv head, sequence). K and V
//                 of the tile stay in registers; the workgroup walks every
//                 query head of the kv group and every 64-query tile that can
//                 see the keys, accumulating dV = P^T dO and dK = dS^T Q in
//                 registers. No atomics: each dK / dV row has one owner, and
//                 the GQA group sum happens in the accumulators.
//   3. bwd_dq:    one workgroup of 8 waves per (256-query tile, query head,
//                 sequence); Q and dO stay in registers and 64-key K, V tiles
//                 stream through LDS, shared by all 8 waves; dQ = dS K is
//                 accumulated in registers. Two waves run on each SIMD (one
//                 workgroup of 4 waves, one per SIMD, where registers need
//                 it: see dq_waves).
// Splitting dQ from dK/dV recomputes S and dP twice but needs no atomic
// reduction, so the result is bitwise reproducible (the deterministic option
// the page's Limitations section discusses).
//
// Register orientation follows the MFMA layout notes in fa_device.hpp. The
// dK/dV kernel computes S = Q K^T (queries x keys) so that each lane owns one
// key column, and accumulates dV^T = dO^T P and dK^T = Q^T dS with P and dS as
// B operands taken straight from the accumulators. The dQ kernel computes
// S^T = K Q^T so that each lane owns one query, and accumulates
// dQ^T = K^T dS^T. Tiles are staged with direct global-to-LDS loads into
// row-major LDS tiles whose 16-byte chunks are XOR-swizzled per row; the
// transposed operands (dO^T, Q^T, K^T) come from the transposing LDS read.
//
// Variants: a sliding window (runtime bounds) limits the visited tiles and
// masks per key on the tiles that cross a bound; softcapping (compiled
// instances) recomputes t = cap tanh(u / cap) and multiplies dS by the
// derivative 1 - tanh^2 before it meets K or Q.
//
// Workspace: D followed by L * log2(e), fp32 [B, H, N64] each (N64 = N rounded
// up to 64), both written by the pre-pass; positions past a sequence's end get
// L * log2(e) = +inf and D = 0, so any row the later kernels read there
// contributes exactly zero.
#include <type_traits>

#include "fa_device.hpp"

namespace fa {
namespace {

constexpr int NT = 256;

// ---------------------------------------------------------------- D = dO . O
template <typename T, int D>
__global__ __launch_bounds__(NT) void bwd_dsum_kernel(Args a) {
    constexpr int LPR = D / 8;        // lanes per (row, head)
    constexpr int RPB = NT / LPR;     // rows per block
    // grid x = row block (up to N64 / RPB, beyond the 65535 limit of y and z),
    // y = head, z = sequence
    const int h = blockIdx.y, b = blockIdx.z;
    int row0, len;
    seq_bounds(a, b, row0, len);
    const int i = blockIdx.x * RPB + threadIdx.x / LPR;
    const int part = threadIdx.x % LPR;
    if (i >= a.N64) return;
    const int DL = D == 32 ? a.dl : D;  // head dim in memory
    float acc = 0.f;
    if (i < len && part * 8 < DL) {
        const size_t off = ((size_t)(row0 + i) * a.H + h) * DL + part * 8;
        const uint4 uo = ld_g16(reinterpret_cast<const T*>(a.o) + off);
        const uint4 ud = ld_g16(reinterpret_cast<const T*>(a.dout) + off);
        const V8<T> vo = as_v8<T>(uo), vd = as_v8<T>(ud);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc = fmaf((float)vo[e], (float)vd[e], acc);
    }
#pragma unroll
    for (int w = LPR / 2; w >= 1; w >>= 1) acc += __shfl_xor(acc, w);
    if (part == 0) {
        const size_t idx = ((size_t)b * a.H + h) * a.N64 + i;
        a.dsum[idx] = (i < len) ? acc : 0.f;
        a.lse2[idx] = (i < len) ? a.lse_in[((size_t)b * a.H + h) * a.N + i] * kLog2e : INFINITY;
    }
}

// ---------------------------------------------------------------- dQ
constexpr int DQ_BK = 64;  // keys per K/V tile

// NW waves per workgroup, 32 queries each: 8 (two per SIMD) where the kernel
// fits in 256 registers per lane. The d = 128 non-causal instances, the
// d = 128 causal instance with both ALiBi and dropout, and head dim 256 do not
// (the compiler spills them there) and run 4 waves, one per SIMD.
template <int D, bool CAUSAL, bool ALIBI, bool DROP, bool CAP>
constexpr int dq_waves() {
    return (D == 256 || (D == 128 && (!CAUSAL || (ALIBI && DROP)))) ? 4 : 8;
}

// NWO = 4 asks for 4-wave workgroups where the default is 8 (short grids: see
// the launcher).
template <typename T, int D, bool CAUSAL, bool ALIBI, bool DROP, bool CAP, int NWO = 0>
__global__ __launch_bounds__((64 * (NWO ? NWO : dq_waves<D, CAUSAL, ALIBI, DROP, CAP>())), 1) void bwd_dq_kernel(Args a) {
    constexpr int DQ_NT = 64 * (NWO ? NWO : dq_waves<D, CAUSAL, ALIBI, DROP, CAP>());
    constexpr int DQ_BQ = DQ_NT / 2;
    constexpr int TILE = DQ_BK * D;  // stage: K tile then V tile, swizzled
    __shared__ __attribute__((aligned(16))) uint16_t stA[2 * TILE];
    __shared__ __attribute__((aligned(16))) uint16_t stB[2 * TILE];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int col = lane & 31, kg = lane >> 5;
    const int h = query_head(a, blockIdx.x), b = blockIdx.y;  // kv-head-major columns
    const int qt = CAUSAL ? (int)(gridDim.z - 1 - blockIdx.z) : (int)blockIdx.z;
    int row0, len;
    seq_bounds(a, b, row0, len);
    const int q0 = qt * DQ_BQ;
    if (q0 >= len) return;

    const int g = h / a.G;
    const int DL = D == 32 ? a.dl : D;  // head dim in memory (16 runs here, zero-padded)
    const size_t ldq = (size_t)a.H * DL, ldk = (size_t)a.Hkv * DL;
    const int qw = q0 + wave * 32;
    const int qi = qw + col;
    const bool wave_live = qw < len;

    V8<T> qf[D / 16], df[D / 16];
    {
        const T* Qp = reinterpret_cast<const T*>(a.q) + (size_t)(row0 + qi) * ldq + (size_t)h * DL;
        const T* Dp = reinterpret_cast<const T*>(a.dout) + (size_t)(row0 + qi) * ldq + (size_t)h * DL;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            uint4 uq = make_uint4(0, 0, 0, 0), ud = uq;
            if (qi < len && 16 * kk + 8 * kg < DL) {
                uq = ld_g16(Qp + 16 * kk + 8 * kg);
                ud = ld_g16(Dp + 16 * kk + 8 * kg);
            }
            qf[kk] = as_v8<T>(uq);
            df[kk] = as_v8<T>(ud);
        }
    }
    const size_t vidx = ((size_t)b * a.H + h) * a.N64 + qi;
    const float lse2 = (qi < len) ? a.lse2[vidx] : INFINITY;
    const float dsum = (qi < len) ? a.dsum[vidx] : 0.f;
    const float c2 = a.scale_log2;
    const float slope2 = ALIBI ? ld_uniform(a.slopes + h) * kLog2e : 0.f;
    const uint32_t drop_row = (uint32_t)(b * a.H + h);  // dropout generator counter word 2
    const uint32_t keep2 = a.keep_k | (a.keep_k << 16);

    int roff[D / 16], toff[D / 32][2];
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) roff[kk] = swz_row_off<D>(lane, kk);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
        toff[db][0] = swz_tr_off<D>(lane, db, 0);
        toff[db][1] = swz_tr_off<D>(lane, db, 1);
    }

    f32x16 dqacc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) dqacc[db] = f32x16{};

    // window bounds (causal: nothing right of the diagonal) and the key tiles
    // some query of the workgroup can see
    const int wl = a.wl, wr = CAUSAL ? 0 : a.wr;
    const int kt_lo = max(q0 - wl, 0) / DQ_BK;
    const int kend = min(len, q0 + DQ_BQ + wr);
    const int nkt = (kend + DQ_BK - 1) / DQ_BK - kt_lo;
    const T* Kg = reinterpret_cast<const T*>(a.k) + (size_t)row0 * ldk + (size_t)g * DL;
    const T* Vg = reinterpret_cast<const T*>(a.v) + (size_t)row0 * ldk + (size_t)g * DL;

    DmaTile<D, DQ_BK, DQ_NT / 64> dma;
    dma.init(wave, lane, ldk, DL);
    auto issue = [&](uint16_t* S, int it) {
        dma.issue(S, reinterpret_cast<const uint16_t*>(Kg), (kt_lo + it) * DQ_BK, len, wave);
        dma.issue(S + TILE, reinterpret_cast<const uint16_t*>(Vg), (kt_lo + it) * DQ_BK, len, wave);
    };

    auto compute = [&](const uint16_t* S, int it) {
        const int k0 = (kt_lo + it) * DQ_BK;
        // wave-uniform: skip tiles no query of this wave can see
        if (!(wave_live && k0 <= qw + 31 + wr && k0 + DQ_BK - 1 >= qw - wl)) return;
        const uint16_t* Ks = S;
        const uint16_t* Vs = S + TILE;
        // Per 32-key block kb: S^T = K Q^T and dP^T = V dO^T, the softmax
        // backward, then dQ^T += K^T dS^T over the block's two 16-key chunks.
        // One block's scores at a time keep the wave within the register
        // budget of two waves per SIMD; the other wave on the SIMD fills the
        // MFMA pipe during this one's softmax. Operand loads run two MFMA
        // groups ahead through register rings; scheduling barriers keep the
        // order.
        constexpr int NK = D / 16, ND = D / 32;
        // masked: a compile-time flag, true for tiles with keys past the end or
        // outside some query's window (across the diagonal when causal)
        auto body = [&](auto masked_t) {
            constexpr bool masked = decltype(masked_t)::value;
            uint4 fk[3], fv[3], fkt[3];
#pragma unroll
            for (int kb = 0; kb < DQ_BK / 32; ++kb) {
                f32x16 s = f32x16{}, dp = f32x16{};
                auto load1 = [&](int kk) {
                    fk[kk % 3] = ld_s16(Ks + 32 * kb * D + roff[kk]);
                    fv[kk % 3] = ld_s16(Vs + 32 * kb * D + roff[kk]);
                };
                load1(0);
                load1(1);
#pragma unroll
                for (int kk = 0; kk < NK; ++kk) {
                    if (kk + 2 < NK) load1(kk + 2);
                    __builtin_amdgcn_sched_barrier(0);
                    s = Mfma<T>::mma(as_v8<T>(fk[kk % 3]), qf[kk], s);
                    dp = Mfma<T>::mma(as_v8<T>(fv[kk % 3]), df[kk], dp);
                    __builtin_amdgcn_sched_barrier(0);
                }
                // With dropout the gradient reaching P is dP o keep * 256 / K:
                // this lane's 16 bytes come from one generator call per 32-key
                // block (byte r for element r, as in the forward).
                uint32_t wd[4] = {0u, 0u, 0u, 0u};
                if constexpr (DROP) {
                    const uint4 w = philox4x32_10(2u * (uint32_t)(k0 / 32 + kb) + (uint32_t)kg, (uint32_t)qi,
                                                  drop_row, a.drop_offset, a.seed_lo, a.seed_hi);
                    wd[0] = w.x, wd[1] = w.y, wd[2] = w.z, wd[3] = w.w;
                }
                uint32_t keepm = 0u;  // 16-bit keep masks of the element pair (r & ~1, r | 1)
                // dS^T = P^T (dP^T - D), P^T = exp2(S^T * scale * log2(e) - L * log2(e)) [+ ALiBi]
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int kj = k0 + 32 * kb + 8 * (r >> 2) + 4 * kg + (r & 3);
                    float bias = -lse2;
                    if (ALIBI) {
                        const float dist = (float)(qi - kj);
                        bias -= slope2 * (CAUSAL ? dist : fabsf(dist));
                    }
                    float th = 0.f;  // softcapping: tanh(u / cap), for the derivative
                    if (CAP) th = tanh_fast(s[r] * a.cap_in);
                    float p = exp2_fast(CAP ? fmaf(a.cap_out, th, bias) : fmaf(s[r], c2, bias));
                    if (masked && (kj >= len || kj > qi + wr || kj < qi - wl)) p = 0.f;
                    float g = dp[r];
                    if constexpr (DROP) {
                        if ((r & 1) == 0) keepm = keep_mask2(wd[r >> 2], (r >> 1) & 1, keep2);
                        const uint32_t m = (r & 1) ? (uint32_t)((int)keepm >> 16)
                                                   : (uint32_t)((int)(keepm << 16) >> 16);
                        g = __uint_as_float(__float_as_uint(g) & m) * a.drop_scale;
                    }
                    dp[r] = CAP ? p * (g - dsum) * (1.f - th * th) : p * (g - dsum);
                }
                V8<T> dsb[2];
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2) {
                    const int r0 = 8 * h2;
                    dsb[h2] = pack8<T>(dp[r0], dp[r0 + 1], dp[r0 + 2], dp[r0 + 3], dp[r0 + 4], dp[r0 + 5], dp[r0 + 6],
                                       dp[r0 + 7]);
                }
                // dQ^T += K^T dS^T for chunks c = 2 kb, 2 kb + 1
                auto load2 = [&](int gi) {
                    const int c = 2 * kb + gi / ND, db = gi % ND;
                    const uint2 lo = ld_s8_tr(Ks + 16 * c * D + toff[db][0]);
                    const uint2 hi = ld_s8_tr(Ks + 16 * c * D + toff[db][1]);
                    fkt[gi % 3] = make_uint4(lo.x, lo.y, hi.x, hi.y);
                };
                load2(0);
                load2(1);
#pragma unroll
                for (int gi = 0; gi < 2 * ND; ++gi) {
                    if (gi + 2 < 2 * ND) load2(gi + 2);
                    __builtin_amdgcn_sched_barrier(0);
                    dqacc[gi % ND] = Mfma<T>::mma(as_v8<T>(fkt[gi % 3]), dsb[gi / ND], dqacc[gi % ND]);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        };
        if ((k0 + DQ_BK > len) || (k0 + DQ_BK - 1 > qw + wr) || (k0 < qw + 31 - wl))
            body(std::true_type{});
        else
            body(std::false_type{});
    };

    two_stage_loop(stA, stB, nkt, issue, compute);

    if (qi < len) {
        T* dQ = reinterpret_cast<T*>(a.dq) + (size_t)(row0 + qi) * ldq + (size_t)h * DL;
        const float sc = a.scale;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int d0 = 32 * db + 8 * i + 4 * kg;
                if (d0 >= DL) continue;
                const int r = 4 * i;
                *reinterpret_cast<uint2*>(dQ + d0) = pack4<T>(dqacc[db][r] * sc, dqacc[db][r + 1] * sc,
                                                              dqacc[db][r + 2] * sc, dqacc[db][r + 3] * sc);
            }
        }
    }
}

template <typename T, int D, bool CAUSAL, bool ALIBI, bool DROP, bool CAP>
hipError_t launch(const Args& a, unsigned stages, hipStream_t s) {
    if (stages & 1u) {
        constexpr int RPB = NT / (D / 8);
        dim3 grid((a.N64 + RPB - 1) / RPB, a.H, a.B);
        hipLaunchKernelGGL((bwd_dsum_kernel<T, D>), grid, dim3(NT), 0, s, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (stages & 2u) {
        hipError_t e = launch_bwd_dkdv(a, std::is_same<T, __bf16>::value ? 2 : 1, D, CAUSAL, ALIBI,
                                       DROP ? kDropout : (CAP ? kSoftcap : kPlain), s);
        if (e != hipSuccess) return e;
    }
    if (stages & 4u) {
        constexpr int nw = dq_waves<D, CAUSAL, ALIBI, DROP, CAP>();
        if constexpr ((D == 64 || D == 128) && CAUSAL && nw == 8 && !ALIBI && !DROP && !CAP) {
            // short causal grids (at most two 8-wave workgroups per compute unit):
            // 4-wave workgroups, several of which share a compute unit, and twice
            // as many of them for the longest-first order to balance the causal
            // triangle (B = 4, H = 16, N = 1024: 0.0325 against 0.0273 ms; the
            // non-causal grids were 4-13% slower with 4 waves and keep 8)
            const long long wg8 = (long long)a.H * a.B * ((a.N + 255) / 256);
            if (wg8 <= 256) {
                dim3 grid(a.H, a.B, (a.N + 127) / 128);
                hipLaunchKernelGGL((bwd_dq_kernel<T, D, CAUSAL, ALIBI, DROP, CAP, 4>), grid, dim3(256), 0, s, a);
                return hipGetLastError();
            }
        }
        dim3 grid(a.H, a.B, (a.N + 32 * nw - 1) / (32 * nw));
        hipLaunchKernelGGL((bwd_dq_kernel<T, D, CAUSAL, ALIBI, DROP, CAP>), grid, dim3(64 * nw), 0, s, a);
        return hipGetLastError();
    }
    return hipSuccess;
}

template <typename T, int D, bool DROP, bool CAP>
hipError_t launch_m(const Args& a, bool causal, bool alibi, unsigned st, hipStream_t s) {
    if (causal)
        return alibi ? launch<T, D, true, true, DROP, CAP>(a, st, s) : launch<T, D, true, false, DROP, CAP>(a, st, s);
    return alibi ? launch<T, D, false, true, DROP, CAP>(a, st, s) : launch<T, D, false, false, DROP, CAP>(a, st, s);
}

template <typename T, int D>
hipError_t launch_d(const Args& a, bool causal, bool alibi, int var, unsigned st, hipStream_t s) {
    if (var == kDropout) return launch_m<T, D, true, false>(a, causal, alibi, st, s);
    if (var == kSoftcap) return launch_m<T, D, false, true>(a, causal, alibi, st, s);
    return launch_m<T, D, false, false>(a, causal, alibi, st, s);
}

template <typename T>
hipError_t launch_t(const Args& a, int d, bool causal, bool alibi, int var, unsigned st, hipStream_t s) {
    switch (d) {
        case 32: return launch_d<T, 32>(a, causal, alibi, var, st, s);
        case 64: return launch_d<T, 64>(a, causal, alibi, var, st, s);
        case 128: return launch_d<T, 128>(a, causal, alibi, var, st, s);
        default: return launch_d<T, 256>(a, causal, alibi, var, st, s);
    }
}

}  // namespace

hipError_t launch_bwd(const Args& a, int dtype, int d, bool causal, bool alibi, int var, unsigned st,
                      hipStream_t s) {
    return dtype == 2 ? launch_t<__bf16>(a, d, causal, alibi, var, st, s)
                      : launch_t<_Float16>(a, d, causal, alibi, var, st, s);
}

}  // namespace fa
