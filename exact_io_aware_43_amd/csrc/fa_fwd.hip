// Forward attention for 16-bit inputs on gfx950 MFMA.
//
// Method: "FlashAttention: Faster Attention Without Dropping a Single
// Interaction", Method Deep Dive, Key design 1 (tiling: Q in row blocks, K and
// V in column blocks, S and P only on chip) and Key design 2 (the mergeable
// running max / running sum / output state); the loop order is the query-outer
// one of Key design 4 (one workgroup per query tile, parallel over the
// sequence), and only O and L = m + ln(l) are written.
//
// Work decomposition. One workgroup of 4 waves owns BR = 128 query rows of one
// (sequence, query head); each wave owns 32 of them. K and V of the head's kv
// head stream through LDS in tiles of BC = 64 keys, double buffered: the next
// tile's global loads are in flight while the current tile is multiplied. Two
// workgroups share a compute unit, so each SIMD interleaves the matrix work of
// one wave with the softmax of the other.
//
// Register orientation. Each wave computes the transposed score tile
// S^T = K Q^T (keys x queries) so that in the MFMA accumulator every lane holds
// scores of ONE query (its column) for 16 keys; the row max and row sum are
// in-lane reductions plus one exchange with lane l ^ 32. The output is
// accumulated transposed as well, O^T += V^T P^T, which takes P^T straight
// from the score accumulator as the B operand and keeps the per-query rescale
// factor in-lane. V stays row-major in LDS; its transposed operand comes from
// the transposing LDS read.
//
// Softmax bookkeeping. Scores are kept in log2 units (scale * log2(e) folded
// into one FMA before exp2). The reference maximum m is only raised when a
// tile's maximum exceeds it by more than TAU = 8 (a factor 256): P = 2^(t - m)
// then stays below 256, which fp32 accumulators and the 16-bit P operand hold
// with their usual relative precision, and the rescale of O and l is skipped
// for almost every tile. The result is unchanged in exact arithmetic because
// the final division uses sums taken against the same reference.
//
// Numerics: scores, sums and the O accumulator are fp32; P is rounded to the
// input type for the second product; lse is converted back to natural log.
#include "fa_device.hpp"

namespace fa {
namespace {

constexpr int BR = 128;    // query rows per workgroup
constexpr int BC = 64;     // keys per K/V tile
constexpr int NT = 256;    // threads per workgroup (4 waves)
constexpr float TAU = 8.f; // lazy-rescale threshold, log2 units

template <int D>
struct FwdLds {
    // K: row-major, pitch = D + 8 elements (b128 reads of 16 keys hit distinct banks).
    // V: row-major, pitch = D + 32 elements (the transposing b64 reads of 4 rows x 64 B
    //    per half-wave hit distinct banks).
    static constexpr int KP = D + 8;
    static constexpr int VP = D + 32;
    static constexpr int KT = BC * KP;
    static constexpr int VT = BC * VP;
    static constexpr int STAGE = KT + VT;
    static constexpr int CHUNKS = BC * D / 8;             // 16-byte chunks per tile (each of K, V)
    static constexpr int LOADS = CHUNKS / NT;             // per thread, per tensor
    static_assert(CHUNKS % NT == 0, "tile must split evenly over the workgroup");
};

template <typename T, int D, bool CAUSAL, bool ALIBI>
__global__ __launch_bounds__(NT, 2) void fwd_mfma_kernel(Args a) {
    using L = FwdLds<D>;
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * L::STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int col = lane & 31;
    const int kg = lane >> 5;

    // Grid: x = query head, y = batch / sequence, z = query tile. Causal
    // launches the longest tiles (highest index) first.
    const int h = blockIdx.x;
    const int b = blockIdx.y;
    const int qt = CAUSAL ? (int)(gridDim.z - 1 - blockIdx.z) : (int)blockIdx.z;

    int row0, len;
    seq_bounds(a, b, row0, len);
    const int q0 = qt * BR;
    if (q0 >= len) return;

    const int g = h / a.G;
    const size_t ldq = (size_t)a.H * D;
    const size_t ldk = (size_t)a.Hkv * D;
    const T* Q = reinterpret_cast<const T*>(a.q) + (size_t)row0 * ldq + (size_t)h * D;
    const T* Kg = reinterpret_cast<const T*>(a.k) + (size_t)row0 * ldk + (size_t)g * D;
    const T* Vg = reinterpret_cast<const T*>(a.v) + (size_t)row0 * ldk + (size_t)g * D;

    const int qw = q0 + wave * 32;  // first query of this wave
    const int qi = qw + col;        // this lane's query
    const bool wave_live = qw < len;

    // Q^T fragments (B operand): lane holds query qi, dims 16*kk + 8*kg + 0..7.
    V8<T> qf[D / 16];
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
        uint4 u = make_uint4(0, 0, 0, 0);
        if (qi < len) u = ld_g16(Q + (size_t)qi * ldq + 16 * kk + 8 * kg);
        qf[kk] = as_v8<T>(u);
    }

    const int kend = CAUSAL ? min(len, q0 + BR) : len;
    const int nkt = (kend + BC - 1) / BC;

    // ---- cooperative K/V staging: global -> registers -> LDS, 16 bytes per chunk.
    // Chunk c of a tile is (key c / (D/8), dims 8 * (c % (D/8))); consecutive
    // threads read consecutive 16 bytes of one key row.
    uint4 kreg[L::LOADS], vreg[L::LOADS];
    auto gload = [&](int kt) {
        const int k0 = kt * BC;
#pragma unroll
        for (int r = 0; r < L::LOADS; ++r) {
            const int c = tid + r * NT;
            const int key = k0 + c / (D / 8), dc = 8 * (c % (D / 8));
            const bool ok = key < len;
            kreg[r] = ok ? ld_g16(Kg + (size_t)key * ldk + dc) : make_uint4(0, 0, 0, 0);
            vreg[r] = ok ? ld_g16(Vg + (size_t)key * ldk + dc) : make_uint4(0, 0, 0, 0);
        }
    };
    auto swrite = [&](int stage) {
        uint16_t* Ks = smem + stage * L::STAGE;
        uint16_t* Vs = Ks + L::KT;
#pragma unroll
        for (int r = 0; r < L::LOADS; ++r) {
            const int c = tid + r * NT;
            const int key = c / (D / 8), dc = 8 * (c % (D / 8));
            st_s16(Ks + key * L::KP + dc, kreg[r]);
            st_s16(Vs + key * L::VP + dc, vreg[r]);
        }
    };

    f32x16 oacc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16{};
    float m_ref = -INFINITY;  // reference max, log2 units (same in lanes l and l ^ 32)
    float l_run = 0.f;        // this lane's share of the running sum

    const float c2 = a.scale_log2;
    const float slope2 = ALIBI ? a.slopes[h] * kLog2e : 0.f;

    gload(0);
    swrite(0);
    __syncthreads();

    for (int kt = 0; kt < nkt; ++kt) {
        const int stage = kt & 1;
        if (kt + 1 < nkt) gload(kt + 1);
        const int k0 = kt * BC;
        // wave-uniform: skip tiles that are entirely above this wave's diagonal
        const bool active = wave_live && (!CAUSAL || k0 <= qw + 31);
        if (active) {
            const uint16_t* Ks = smem + stage * L::STAGE;
            const uint16_t* Vs = Ks + L::KT;

            // S^T = K Q^T for BC keys x 32 queries (raw, unscaled scores)
            f32x16 s[BC / 32];
#pragma unroll
            for (int kb = 0; kb < BC / 32; ++kb) {
                s[kb] = f32x16{};
#pragma unroll
                for (int kk = 0; kk < D / 16; ++kk) {
                    const V8<T> kf = as_v8<T>(ld_s16(Ks + (32 * kb + col) * L::KP + 16 * kk + 8 * kg));
                    s[kb] = Mfma<T>::mma(kf, qf[kk], s[kb]);
                }
            }

            // Scores in log2 units. Plain tiles keep the raw score and fold the
            // scale into the exponent's FMA; ALiBi and edge tiles materialise
            // t = s * c2 + bias (or -inf when masked) and use scale 1 below.
            const bool edge = (k0 + BC > len) || (CAUSAL && k0 + BC - 1 > qw);
            const bool materialise = ALIBI || edge;
            float mt;
            if (materialise) {
                mt = -INFINITY;
#pragma unroll
                for (int kb = 0; kb < BC / 32; ++kb) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = k0 + 32 * kb + 8 * (r >> 2) + 4 * kg + (r & 3);
                        float t = s[kb][r] * c2;
                        if (ALIBI) {
                            const float dist = (float)(qi - key);
                            t -= slope2 * (CAUSAL ? dist : fabsf(dist));
                        }
                        if (edge && (key >= len || (CAUSAL && key > qi))) t = -INFINITY;
                        s[kb][r] = t;
                        mt = fmaxf(mt, t);
                    }
                }
            } else {
                float mx = s[0][0];
#pragma unroll
                for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
                mt = mx * c2;
            }
            mt = fmaxf(mt, __shfl_xor(mt, 32));

            // lazy rescale: raise the reference only when the tile max exceeds it by > TAU
            const bool raise = mt > m_ref + TAU;
            if (__any(raise)) {
                const float m_new = raise ? mt : m_ref;
                const float alpha = exp2_fast(m_ref - m_new);  // 0 on the first tile
                l_run *= alpha;
#pragma unroll
                for (int db = 0; db < D / 32; ++db) oacc[db] *= alpha;
                m_ref = m_new;
            }
            const float m_use = (m_ref == -INFINITY) ? 0.f : m_ref;  // rows with no key yet

            const float sc = materialise ? 1.f : c2;
            float ls = 0.f;
#pragma unroll
            for (int kb = 0; kb < BC / 32; ++kb) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float p = exp2_fast(fmaf(s[kb][r], sc, -m_use));
                    s[kb][r] = p;
                    ls += p;
                }
            }
            l_run += ls;

            // O^T += V^T P^T, 16 keys per MFMA
#pragma unroll
            for (int c = 0; c < BC / 16; ++c) {
                const int kb = c >> 1, r0 = 8 * (c & 1);
                const V8<T> pf = pack8<T>(s[kb][r0 + 0], s[kb][r0 + 1], s[kb][r0 + 2], s[kb][r0 + 3],
                                          s[kb][r0 + 4], s[kb][r0 + 5], s[kb][r0 + 6], s[kb][r0 + 7]);
#pragma unroll
                for (int db = 0; db < D / 32; ++db) {
                    const V8<T> vf = as_v8<T>(ld_s16_rows_tr(Vs, L::VP, 16 * c, 32 * db, lane));
                    oacc[db] = Mfma<T>::mma(vf, pf, oacc[db]);
                }
            }
        }
        if (kt + 1 < nkt) swrite(stage ^ 1);
        __syncthreads();
    }

    // ---- epilogue: O = O_acc / l, lse = (m + log2 l) * ln 2
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    if (qi < len) {
        const float inv = 1.f / l_tot;
        T* O = reinterpret_cast<T*>(a.out) + (size_t)row0 * ldq + (size_t)h * D + (size_t)qi * ldq;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int d0 = 32 * db + 8 * i + 4 * kg;
                *reinterpret_cast<uint2*>(O + d0) =
                    pack4<T>(oacc[db][4 * i] * inv, oacc[db][4 * i + 1] * inv, oacc[db][4 * i + 2] * inv,
                             oacc[db][4 * i + 3] * inv);
            }
        }
        if (kg == 0) a.lse[((size_t)b * a.H + h) * a.N + qi] = (m_ref + __log2f(l_tot)) * kLn2;
    }
}

template <typename T, int D, bool CAUSAL, bool ALIBI>
hipError_t launch(const Args& a, hipStream_t s) {
    const int nqt = (a.N + BR - 1) / BR;
    dim3 grid(a.H, a.B, nqt);
    hipLaunchKernelGGL((fwd_mfma_kernel<T, D, CAUSAL, ALIBI>), grid, dim3(NT), 0, s, a);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_d(const Args& a, bool causal, bool alibi, hipStream_t s) {
    if (causal) return alibi ? launch<T, D, true, true>(a, s) : launch<T, D, true, false>(a, s);
    return alibi ? launch<T, D, false, true>(a, s) : launch<T, D, false, false>(a, s);
}

}  // namespace

hipError_t launch_fwd_mfma(const Args& a, int dtype, int d, bool causal, bool alibi, hipStream_t s) {
    if (dtype == 2) return d == 64 ? launch_d<__bf16, 64>(a, causal, alibi, s) : launch_d<__bf16, 128>(a, causal, alibi, s);
    return d == 64 ? launch_d<_Float16, 64>(a, causal, alibi, s) : launch_d<_Float16, 128>(a, causal, alibi, s);
}

}  // namespace fa
