// Forward attention for 16-bit inputs on gfx950 MFMA.
//
// Method: "FlashAttention: Faster Attention Without Dropping a Single
// Interaction", Method Deep Dive, Key design 1 (tiling: Q in row blocks, K and
// V in column blocks, S and P only on chip) and Key design 2 (the mergeable
// running max / running sum / output state); the loop order is the query-outer
// one of Key design 4 (one workgroup per query tile, parallel over the
// sequence), and only O and L = m + ln(l) are written.
//
// Work decomposition (head dims 32, 64 and 128; head dim 256 below). One
// workgroup of 8 waves owns BR = 256 query rows of one
// (sequence, query head); each wave owns 32 of them. K and V of the head's kv
// head stream through LDS in tiles of BC = 128 keys, double buffered: the next
// tile's loads are in flight while the current tile is multiplied. The 8 waves
// share every tile (the direct loads that stage it cost issue time per wave,
// so sharing halves that cost against two 4-wave groups), and two waves run
// on each SIMD, which interleaves the matrix work of one with the softmax of
// the other.
//
// Register orientation. Each wave computes the transposed score tile
// S^T = K Q^T (keys x queries) so that in the MFMA accumulator every lane holds
// scores of ONE query (its column) for 16 keys; the row max and row sum are
// in-lane reductions plus one register exchange with lane l ^ 32. The output is
// accumulated transposed as well, O^T += V^T P^T, which takes P^T straight
// from the score accumulator as the B operand and keeps the per-query rescale
// factor in-lane. K and V are staged with direct global-to-LDS loads into
// row-major tiles whose 16-byte chunks are XOR-swizzled per row (free of bank
// conflicts for the row-wise K reads and the transposing V reads); the
// transposed V operand comes from the transposing LDS read.
//
// Softmax bookkeeping. Scores are kept in log2 units (scale * log2(e) folded
// into one FMA before exp2). A tile that takes its row maximum raises the
// reference m only when that maximum exceeds it by more than TAU = 8 (a factor
// 256), so the rescale of O and l is skipped for almost every tile. Plain
// tiles after the first take no maximum at all: P = 2^(t - m) is formed against
// the current reference and the tile's row sum, computed anyway, shows whether
// any P exceeded the bound the accumulators allow (then the tile is redone with
// its maximum). P keeps the relative precision of its type at any magnitude, so
// where the reference sits does not change the result, which is exact in real
// arithmetic because the final division uses sums taken against the same
// reference.
//
// Variants: a sliding window (runtime bounds; it sets the visited key range,
// the per-wave skips and the edge tiles that take the mask) and softcapping
// (compiled instances: the scaled score u becomes cap tanh(u / cap) before the
// bias, which needs the materialised path and one tanh per score).
//
// Numerics: scores, sums and the O accumulator are fp32; P is rounded to the
// input type for the second product. O is divided by the sum of exactly those
// rounded P values (so its weights sum to one and a row dominated by one key
// reproduces that key's V), while lse uses the fp32 sum of the unrounded P and
// is converted back to natural log.
#include "fa_device.hpp"

namespace fa {
namespace {

// Tile shape per head dim: 8 waves (two per SIMD) and 128-key tiles; for head
// dim 256, whose O accumulator alone takes 128 registers per lane, 4 waves (one
// per SIMD, twice the registers each) and 64-key tiles (the two K/V stages
// stay at 128 KB of LDS). Head dim 64 runs 4-wave workgroups too: their 64 KB
// of LDS and about 190 registers per lane let two share a compute unit, which
// measured 3-15% faster than one 8-wave workgroup on every shape tried (short
// and long, causal and not). Each wave owns 32 query rows.
template <int D>
struct FwdShape {
    static constexpr int NT = (D == 256 || D == 64) ? 256 : 512;  // threads per workgroup
    static constexpr int BC = D == 256 ? 64 : 128;   // keys per K/V tile
    static constexpr int BR = 32 * (NT / 64);        // query rows per workgroup
};
constexpr float TAU = 8.f; // lazy-rescale threshold, log2 units
// Largest fp32 sum of one lane's 64 P values of a tile that the path without
// a row maximum accepts. Every P is then at most this bound, which must fit the
// 16-bit type P is rounded to for the second product: 2^32 for bf16 (the O
// accumulator and the sums stay far inside fp32 range for any length) and
// 2^15 for fp16 (largest finite value 65504).
template <typename T>
constexpr float sum_bound() {
    return sizeof(T) == 2 && __is_same(T, _Float16) ? 32768.f : 4294967296.f;
}

template <typename T, int D, bool CAUSAL, bool ALIBI, bool DROP, bool CAP>
__global__ __launch_bounds__(FwdShape<D>::NT, 1) void fwd_mfma_kernel(Args a) {
    constexpr int NT = FwdShape<D>::NT, BC = FwdShape<D>::BC, BR = FwdShape<D>::BR;
    // Two named K/V stages (swizzled [BC x D] tiles, K then V): the prefetch
    // into one overlaps the reads of the other, which the compiler can only
    // prove independent when they are distinct arrays.
    constexpr int TILE = BC * D;
    __shared__ __attribute__((aligned(16))) uint16_t stA[2 * TILE];
    __shared__ __attribute__((aligned(16))) uint16_t stB[2 * TILE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int col = lane & 31;
    const int kg = lane >> 5;

    // Grid: x = query head (kv-head-major, see query_head), y = batch /
    // sequence, z = query tile. Causal launches the longest tiles (highest
    // index) first.
    const int h = query_head(a, blockIdx.x);
    const int b = blockIdx.y;
    const int qt = CAUSAL ? (int)(gridDim.z - 1 - blockIdx.z) : (int)blockIdx.z;

    int row0, len;
    seq_bounds(a, b, row0, len);
    const int q0 = qt * BR;
    if (q0 >= len) return;

    const int g = h / a.G;
    const int DL = D == 32 ? a.dl : D;  // head dim in memory (16 runs here, zero-padded)
    const size_t ldq = (size_t)a.H * DL;
    const size_t ldk = (size_t)a.Hkv * DL;
    const T* Q = reinterpret_cast<const T*>(a.q) + (size_t)row0 * ldq + (size_t)h * DL;
    const T* Kg = reinterpret_cast<const T*>(a.k) + (size_t)row0 * ldk + (size_t)g * DL;
    const T* Vg = reinterpret_cast<const T*>(a.v) + (size_t)row0 * ldk + (size_t)g * DL;

    const int qw = q0 + wave * 32;  // first query of this wave
    const int qi = qw + col;        // this lane's query
    const bool wave_live = qw < len;

    // Q^T fragments (B operand): lane holds query qi, dims 16*kk + 8*kg + 0..7.
    V8<T> qf[D / 16];
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
        uint4 u = make_uint4(0, 0, 0, 0);
        if (qi < len && 16 * kk + 8 * kg < DL) u = ld_g16(Q + (size_t)qi * ldq + 16 * kk + 8 * kg);
        qf[kk] = as_v8<T>(u);
    }

    // lane parts of the LDS operand offsets (loop invariant)
    int roff[D / 16], toff[D / 32][2];
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) roff[kk] = swz_row_off<D>(lane, kk);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
        toff[db][0] = swz_tr_off<D>(lane, db, 0);
        toff[db][1] = swz_tr_off<D>(lane, db, 1);
    }

    // window bounds (causal: nothing to the right of the diagonal) and the key
    // tiles some query of the workgroup can see
    const int wl = a.wl, wr = CAUSAL ? 0 : a.wr;
    const int kt_lo = max(q0 - wl, 0) / BC;
    const int kend = min(len, q0 + BR + wr);
    const int nkt = (kend + BC - 1) / BC - kt_lo;

    DmaTile<D, BC, NT / 64> dma;
    dma.init(wave, lane, ldk, DL);
    // With ALiBi, key tiles are visited from the last (the diagonal one under
    // the causal mask) down to the first: the bias falls with distance, so the
    // tile of a row's nearest keys holds its largest scores, and the maximum
    // taken on that first tile bounds every later one (ascending, each tile
    // would exceed the last and force the maximum path every time). Without a
    // bias the plain ascending order is kept.
    auto tile_of = [&](int it) { return kt_lo + (ALIBI ? nkt - 1 - it : it); };
    auto issue = [&](uint16_t* st, int it) {
        const int kt = tile_of(it);
        dma.issue(st, reinterpret_cast<const uint16_t*>(Kg), kt * BC, len, wave);
        dma.issue(st + TILE, reinterpret_cast<const uint16_t*>(Vg), kt * BC, len, wave);
    };

    f32x16 oacc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16{};
    float m_ref = -INFINITY;  // reference max, log2 units (same in lanes l and l ^ 32)
    float l_run = 0.f;        // this lane's share of the running sum of P (fp32, for lse)
    float l_rnd = 0.f;        // the same sum over P rounded to T (the weights the product uses)

    const float c2 = a.scale_log2;
    const float slope2 = ALIBI ? ld_uniform(a.slopes + h) * kLog2e : 0.f;
    const uint32_t drop_row = (uint32_t)(b * a.H + h);  // generator counter word 2
    const uint32_t keep2 = a.keep_k | (a.keep_k << 16);

    bool fresh = true;  // wave-uniform: no tile of this wave processed yet
    auto compute = [&](const uint16_t* Ks, int it) {
        const int kt = tile_of(it);
        const uint16_t* Vs = Ks + TILE;
        const int k0 = kt * BC;
        // wave-uniform: skip tiles no query of this wave can see (above the
        // diagonal, outside the window)
        if (!(wave_live && k0 <= qw + 31 + wr && k0 + BC - 1 >= qw - wl)) return;

        // S^T = K Q^T for BC keys x 32 queries (raw, unscaled scores). The K
        // operand loads run two (kb, kk) groups ahead of the MFMAs; scheduling
        // barriers keep that order.
        f32x16 s[BC / 32];
        // (also written out inline for the first product below: with both as
        // calls the register allocator spills the non-causal ALiBi instance)
        auto score_product = [&]() {
            constexpr int NG1 = BC / 32 * D / 16;
#pragma unroll
            for (int kb = 0; kb < BC / 32; ++kb) s[kb] = f32x16{};
            uint4 fk[3];
            auto load1 = [&](int gi) { fk[gi % 3] = ld_s16(Ks + 32 * (gi / (D / 16)) * D + roff[gi % (D / 16)]); };
            load1(0);
            load1(1);
#pragma unroll
            for (int gi = 0; gi < NG1; ++gi) {
                if (gi + 2 < NG1) load1(gi + 2);
                __builtin_amdgcn_sched_barrier(0);
                const int kb = gi / (D / 16), kk = gi % (D / 16);
                s[kb] = Mfma<T>::mma(as_v8<T>(fk[gi % 3]), qf[kk], s[kb]);
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        {
            constexpr int NG1 = BC / 32 * D / 16;
#pragma unroll
            for (int kb = 0; kb < BC / 32; ++kb) s[kb] = f32x16{};
            uint4 fk[3];
            auto load1 = [&](int gi) { fk[gi % 3] = ld_s16(Ks + 32 * (gi / (D / 16)) * D + roff[gi % (D / 16)]); };
            load1(0);
            load1(1);
#pragma unroll
            for (int gi = 0; gi < NG1; ++gi) {
                if (gi + 2 < NG1) load1(gi + 2);
                __builtin_amdgcn_sched_barrier(0);
                const int kb = gi / (D / 16), kk = gi % (D / 16);
                s[kb] = Mfma<T>::mma(as_v8<T>(fk[gi % 3]), qf[kk], s[kb]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }

        // Scores in log2 units: t = s * scale * log2(e) + bias. The ALiBi bias
        // -slope |i - j| is slope2 * (key - qi) on keys at or before the query and
        // slope2 * (qi - key) after it. Element (kb, r) of this lane has
        // key - qi = lin + off(kb, r) with lin = k0 + 4 kg - qi per tile and the
        // compile-time off = 32 kb + 8 (r / 4) + r % 4.
        // edge: some key of the tile is past the end or outside some row's window
        const bool edge = (k0 + BC > len) || (k0 + BC - 1 > qw + wr) || (k0 < qw + 31 - wl);
        const bool below = k0 + BC - 1 <= qw;  // every key <= every query of the wave
        const bool above = k0 >= qw + 31;      // every key >= every query of the wave
        const float lin = (float)(k0 + 4 * kg - qi);
        auto off = [](int kb, int r) { return (float)(32 * kb + 8 * (r >> 2) + (r & 3)); };
        float ls = 0.f;

        // Plain tiles after a wave's first tile take no row maximum: P is formed
        // against the current reference directly, and the fp32 row sum, which lse
        // needs anyway, bounds every element of the lane's share. Only if some
        // lane's sum exceeds sum_bound<T>() (or overflowed) does the wave recompute
        // the scores and take the maximum path for this tile. A wave's first tile
        // always takes the maximum path. Without a window every row of a live
        // wave sees at least one key of every tile it visits (causal: key
        // k0 <= its query), so that sets a finite reference in each row; a row
        // whose window starts later keeps an infinite reference, overflows the
        // next maximum-free sum and is redone on the maximum path.
        // ALiBi tiles qualify when the bias is linear in the key over the whole
        // tile (no key on both sides of any of the wave's queries).
        bool need_max = true;
        const bool first = fresh;
        if (!first && !edge && (!ALIBI || below || above)) {
            need_max = false;
            const float sl = ALIBI ? (below ? slope2 : -slope2) : 0.f;
            const float base = ALIBI ? fmaf(sl, lin, -m_ref) : -m_ref;
#pragma unroll
            for (int kb = 0; kb < BC / 32; ++kb) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float t = CAP ? fmaf(a.cap_out, tanh_fast(s[kb][r] * a.cap_in), base) : fmaf(s[kb][r], c2, base);
                    if (ALIBI) t = fmaf(sl, off(kb, r), t);
                    const float p = exp2_fast(t);
                    s[kb][r] = p;
                    ls += p;
                }
            }
            if (__any(!(ls <= sum_bound<T>()))) {
                score_product();
                need_max = true;
                ls = 0.f;
            }
        }
        // Maximum path: t materialised (masked keys -inf), tile maximum, lazy
        // raise of the reference. (One body with a run-time mask test: separate
        // masked and unmasked copies make the register allocator spill.)
        if (need_max) {
            // Unmasked tiles without a bias keep raw scores (the scale goes into
            // the exponent's FMA); a negative scale reverses the order of raw
            // scores, so it materialises like the others.
            const bool materialise = ALIBI || CAP || edge || !(c2 >= 0.f);
            float mt;
            if (materialise) {
                mt = -INFINITY;
                // key = k0 + 4 kg + kofs: the constant kofs against per-tile limits
                const int lim_len = len - k0 - 4 * kg, lim_r = qi + wr - k0 - 4 * kg, lim_l = qi - wl - k0 - 4 * kg;
#pragma unroll
                for (int kb = 0; kb < BC / 32; ++kb) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        float t = CAP ? a.cap_out * tanh_fast(s[kb][r] * a.cap_in) : s[kb][r] * c2;
                        if (ALIBI) {
                            const float d = lin + off(kb, r);  // key - qi, exact in fp32
                            t = fmaf(slope2, CAUSAL ? d : -fabsf(d), t);
                        }
                        const int kofs = 32 * kb + 8 * (r >> 2) + (r & 3);
                        if (edge && (kofs >= lim_len || kofs > lim_r || kofs < lim_l)) t = -INFINITY;
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
            mt = max_xor32(mt);

            // lazy rescale: raise the reference only when the tile max exceeds it by > TAU
            const bool raise = mt > m_ref + TAU;
            if (__any(raise)) {
                const float m_new = raise ? mt : m_ref;
                // 0 where the reference was -inf; 1 on rows that keep theirs (also
                // a row that has seen no key yet: a window can leave one empty)
                const float alpha = raise ? exp2_fast(m_ref - mt) : 1.f;
                l_run *= alpha;
                l_rnd *= alpha;
#pragma unroll
                for (int db = 0; db < D / 32; ++db) oacc[db] *= alpha;
                m_ref = m_new;
            }
            const float m_use = (m_ref == -INFINITY) ? 0.f : m_ref;  // rows with no key yet
            const float sc = materialise ? 1.f : c2;
#pragma unroll
            for (int kb = 0; kb < BC / 32; ++kb) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float p = exp2_fast(fmaf(s[kb][r], sc, -m_use));
                    s[kb][r] = p;
                    ls += p;
                }
            }
        }
        l_run += ls;
        fresh = false;

        // O^T += V^T P^T, 16 keys per MFMA; transposed V loads two groups ahead
        constexpr int NG2 = BC / 16 * D / 32;
        V8<T> pf[BC / 16];
#pragma unroll
        for (int c = 0; c < BC / 16; ++c) {
            const int kb = c >> 1, r0 = 8 * (c & 1);
            pf[c] = pack8<T>(s[kb][r0 + 0], s[kb][r0 + 1], s[kb][r0 + 2], s[kb][r0 + 3], s[kb][r0 + 4],
                             s[kb][r0 + 5], s[kb][r0 + 6], s[kb][r0 + 7]);
        }
        {
            float r0 = 0.f, r1 = 0.f;
#pragma unroll
            for (int c = 0; c < BC / 16; ++c) {
                const uint4 u = __builtin_bit_cast(uint4, pf[c]);
                r0 = add_pair<T>(u.x, r0);
                r1 = add_pair<T>(u.y, r1);
                r0 = add_pair<T>(u.z, r0);
                r1 = add_pair<T>(u.w, r1);
            }
            l_rnd += r0 + r1;
        }
        if constexpr (DROP) {
            // Dropout on the probabilities that multiply V (the sums above keep
            // every one): one generator call per 32-key block gives this lane's
            // 16 bytes, byte r deciding accumulator element r (key
            // k0 + 32 kb + 8 (r / 4) + 4 kg + r % 4 of query qi); the 256 / K
            // factor is applied to O at the end.
#pragma unroll
            for (int kb = 0; kb < BC / 32; ++kb) {
                const uint4 w = philox4x32_10(2u * (uint32_t)(k0 / 32 + kb) + (uint32_t)kg, (uint32_t)qi, drop_row,
                                              a.drop_offset, a.seed_lo, a.seed_hi);
                const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    uint4 u = __builtin_bit_cast(uint4, pf[2 * kb + half]);
                    u.x &= keep_mask2(wd[2 * half], 0, keep2);
                    u.y &= keep_mask2(wd[2 * half], 1, keep2);
                    u.z &= keep_mask2(wd[2 * half + 1], 0, keep2);
                    u.w &= keep_mask2(wd[2 * half + 1], 1, keep2);
                    pf[2 * kb + half] = as_v8<T>(u);
                }
            }
        }
        uint4 fv[3];
        auto load2 = [&](int gi) {
            const int c = gi / (D / 32), db = gi % (D / 32);
            const uint2 lo = ld_s8_tr(Vs + 16 * c * D + toff[db][0]);
            const uint2 hi = ld_s8_tr(Vs + 16 * c * D + toff[db][1]);
            fv[gi % 3] = make_uint4(lo.x, lo.y, hi.x, hi.y);
        };
        load2(0);
        load2(1);
#pragma unroll
        for (int gi = 0; gi < NG2; ++gi) {
            if (gi + 2 < NG2) load2(gi + 2);
            __builtin_amdgcn_sched_barrier(0);
            const int c = gi / (D / 32), db = gi % (D / 32);
            oacc[db] = Mfma<T>::mma(as_v8<T>(fv[gi % 3]), pf[c], oacc[db]);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    two_stage_loop(stA, stB, nkt, issue, compute);

    // ---- epilogue: O = O_acc / (sum of rounded P), lse = (m + log2 l) * ln 2
    const float l_tot = sum_xor32(l_run);
    const float lr_tot = sum_xor32(l_rnd);
    if (qi < len) {
        const float inv = (DROP ? a.drop_scale : 1.f) / lr_tot;
        T* O = reinterpret_cast<T*>(a.out) + (size_t)row0 * ldq + (size_t)h * DL + (size_t)qi * ldq;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int d0 = 32 * db + 8 * i + 4 * kg;
                if (d0 >= DL) continue;
                *reinterpret_cast<uint2*>(O + d0) =
                    pack4<T>(oacc[db][4 * i] * inv, oacc[db][4 * i + 1] * inv, oacc[db][4 * i + 2] * inv,
                             oacc[db][4 * i + 3] * inv);
            }
        }
        if (kg == 0) a.lse[((size_t)b * a.H + h) * a.N + qi] = (m_ref + __log2f(l_tot)) * kLn2;
    }
}

template <typename T, int D, bool CAUSAL, bool ALIBI, bool DROP, bool CAP>
hipError_t launch(const Args& a, hipStream_t s) {
    const int nqt = (a.N + FwdShape<D>::BR - 1) / FwdShape<D>::BR;
    dim3 grid(a.H, a.B, nqt);
    hipLaunchKernelGGL((fwd_mfma_kernel<T, D, CAUSAL, ALIBI, DROP, CAP>), grid, dim3(FwdShape<D>::NT), 0, s, a);
    return hipGetLastError();
}

template <typename T, int D, bool DROP, bool CAP>
hipError_t launch_m(const Args& a, bool causal, bool alibi, hipStream_t s) {
    if (causal) return alibi ? launch<T, D, true, true, DROP, CAP>(a, s) : launch<T, D, true, false, DROP, CAP>(a, s);
    return alibi ? launch<T, D, false, true, DROP, CAP>(a, s) : launch<T, D, false, false, DROP, CAP>(a, s);
}

template <typename T, int D>
hipError_t launch_d(const Args& a, bool causal, bool alibi, int var, hipStream_t s) {
    if (var == kDropout) return launch_m<T, D, true, false>(a, causal, alibi, s);
    if (var == kSoftcap) return launch_m<T, D, false, true>(a, causal, alibi, s);
    return launch_m<T, D, false, false>(a, causal, alibi, s);
}

template <typename T>
hipError_t launch_t(const Args& a, int d, bool causal, bool alibi, int var, hipStream_t s) {
    switch (d) {
        case 32: return launch_d<T, 32>(a, causal, alibi, var, s);
        case 64: return launch_d<T, 64>(a, causal, alibi, var, s);
        case 128: return launch_d<T, 128>(a, causal, alibi, var, s);
        default: return launch_d<T, 256>(a, causal, alibi, var, s);
    }
}

}  // namespace

hipError_t launch_fwd_mfma(const Args& a, int dtype, int d, bool causal, bool alibi, int var, hipStream_t s) {
    return dtype == 2 ? launch_t<__bf16>(a, d, causal, alibi, var, s) : launch_t<_Float16>(a, d, causal, alibi, var, s);
}

}  // namespace fa
