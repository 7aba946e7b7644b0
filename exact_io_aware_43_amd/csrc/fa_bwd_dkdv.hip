// dK/dV kernel of the backward pass (the three-launch structure and the method
// are described in fa_bwd.hip; "FlashAttention: Faster Attention Without
// Dropping a Single Interaction", Method Deep Dive, Key design 3).
//
// One workgroup of 8 waves (two per SIMD) per (256-key tile, kv head,
// sequence); each wave owns 32 keys. K of the wave's keys is held in registers
// as an MFMA operand; V of the workgroup's keys sits in LDS for the whole
// kernel (it is read once per query block), which keeps a wave within the 256
// registers per lane that two waves per SIMD allow next to the dK, dV
// accumulators. The workgroup walks every query head of the kv group and every
// 64-query tile that can see the keys; all 8 waves share each staged Q / dO
// tile, so a direct load feeds twice the MFMA work it would with 4 waves. Per
// 32-query block qb of a step:
//
//   S  = Q K^T, dP = dO V^T            (scores: one key column per lane)
//   P  = exp2(S * scale * log2 e - L * log2 e), dS = P o (dP - D)
//   dV^T += dO^T P,  dK^T += Q^T dS    (transposed operands via ds_read_b64_tr_b16)
//
// A sliding window narrows the query tiles a key tile walks and masks the
// steps that cross a bound; softcapping recomputes tanh(u / cap) per score and
// multiplies dS by 1 - tanh^2 before dK accumulates it.
//
// The other wave on the SIMD fills the MFMA pipe during this one's softmax.
// LDS operand loads run one MFMA group ahead through two-slot register rings,
// and scheduling barriers pin the order.
#include <type_traits>

#include "fa_device.hpp"

namespace fa {
namespace {

// Shape per head dim: 8 waves (two per SIMD) and 64-query steps; at head dim
// 256, whose dK and dV accumulators take 256 registers per lane, 4 waves (one
// per SIMD) and 32-query steps, which keeps V and the two Q / dO stages within
// LDS. NWO = 4 asks for 4-wave workgroups at a head dim that defaults to 8:
// the launcher takes them for short grids, where three such workgroups share a
// compute unit and one's set-up and epilogue overlap the others' work.
template <int D, int NWO = 0>
struct DkdvShape {
    static constexpr int NW = NWO ? NWO : (D == 256 ? 4 : 8);  // waves per workgroup
    static constexpr int NT = 64 * NW;
    static constexpr int KV_BK = 32 * NW;          // keys per workgroup (32 per wave)
    static constexpr int KV_BQ = D == 256 ? 32 : 64;  // queries per step (blocks of 32)
};

#define FA_SB() __builtin_amdgcn_sched_barrier(0)

template <typename T, int D, bool CAUSAL, bool ALIBI, bool DROP, bool CAP, int NWO = 0>
__global__ __launch_bounds__((DkdvShape<D, NWO>::NT), 1) void bwd_dkdv_kernel(Args a) {
    constexpr int NW = DkdvShape<D, NWO>::NW, KV_BK = DkdvShape<D, NWO>::KV_BK, KV_BQ = DkdvShape<D, NWO>::KV_BQ;
    // stage: Q tile, dO tile (swizzled [KV_BQ x D] each), with L*log2(e) and D
    // (fp32, KV_BQ each) in a small array of their own: the two tile stages
    // then span 64 KB, and every operand read reaches them from one set of
    // per-lane offset registers through the 16-bit immediate offset.
    constexpr int TILE = KV_BQ * D;
    constexpr int STAGE = 2 * TILE;
    __shared__ __attribute__((aligned(16))) uint16_t stA[STAGE];
    __shared__ __attribute__((aligned(16))) uint16_t stB[STAGE];
    // (64 values each: one direct load per wave fills 64 slots)
    __shared__ __attribute__((aligned(16))) float vecA[2 * 64];
    __shared__ __attribute__((aligned(16))) float vecB[2 * 64];
    __shared__ __attribute__((aligned(16))) uint16_t vt[KV_BK * D];  // V rows k0 .. k0 + KV_BK, swizzled
    // dropout: each wave's 32 x 32 block of random bytes, stored key-major
    // with the queries of one lane half (kg) contiguous (see the step below)
    __shared__ __attribute__((aligned(16))) uint8_t dmask[DROP ? NW * 32 * 32 : 16];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int kg = lane >> 5;
    const int g = blockIdx.x, b = blockIdx.y;
    const int kt = blockIdx.z;  // low key tiles see the most queries: dispatched first
    int row0, len;
    seq_bounds(a, b, row0, len);
    const int k0 = kt * KV_BK;
    if (k0 >= len) return;

    const int DL = D == 32 ? a.dl : D;  // head dim in memory (16 runs here, zero-padded)
    const size_t ldq = (size_t)a.H * DL, ldk = (size_t)a.Hkv * DL;
    const int kw = k0 + wave * 32;     // first key of this wave
    const int key = kw + (lane & 31);  // this lane's key (column of S)

    // K^T fragments as B operands: lane holds key `key`, dims 16*kk + 8*kg + 0..7.
    V8<T> kf[D / 16];
    {
        const T* Kp = reinterpret_cast<const T*>(a.k) + (size_t)(row0 + key) * ldk + (size_t)g * DL;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            uint4 uk = make_uint4(0, 0, 0, 0);
            if (key < len && 16 * kk + 8 * kg < DL) uk = ld_g16(Kp + 16 * kk + 8 * kg);
            kf[kk] = as_v8<T>(uk);
        }
    }
    // V of the workgroup's keys into LDS (rows past the end read as zero), in
    // two halves of KV_BK / 2 rows; the swizzle repeats every 16 rows, so the
    // halves form one swizzled [KV_BK x D] tile. The first wait of the loop
    // below covers these loads.
    {
        DmaTile<D, KV_BK / 2, NW> vdma;
        vdma.init(wave, lane, ldk, DL);
        const uint16_t* Vg = reinterpret_cast<const uint16_t*>(a.v) + (size_t)row0 * ldk + (size_t)g * DL;
        vdma.issue(vt, Vg, k0, len, wave);
        vdma.issue(vt + (KV_BK / 2) * D, Vg, k0 + KV_BK / 2, len, wave);
    }

    const int vrow = wave * 32 * D;  // element offset of this wave's 32 rows of V
    const int rbase = swz_row_off<D>(lane, 0), tbase = swz_tr_off<D>(lane, 0, 0);

    f32x16 dkacc[D / 32], dvacc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
        dkacc[db] = f32x16{};
        dvacc[db] = f32x16{};
    }

    // Query tiles that can see this key tile (queries i with
    // k0 - wr <= i <= k0 + KV_BK - 1 + wl; causal: wr = 0), for every query
    // head of the kv group.
    const int wl = a.wl, wr = CAUSAL ? 0 : a.wr;
    const int qt0 = max(k0 - wr, 0) / KV_BQ;
    const int nqt = (min(len, k0 + KV_BK + wl) + KV_BQ - 1) / KV_BQ;
    const int per_head = nqt - qt0;
    const int steps = a.G * per_head;
    const float c2 = a.scale_log2;
    const T* Qb = reinterpret_cast<const T*>(a.q) + (size_t)row0 * ldq;
    const T* Db = reinterpret_cast<const T*>(a.dout) + (size_t)row0 * ldq;

    auto step_coords = [&](int st, int& h, int& q0) {
        const int hh = st / per_head;
        h = g * a.G + hh;
        q0 = (qt0 + st - hh * per_head) * KV_BQ;
    };

    DmaTile<D, KV_BQ, NW> dma;
    dma.init(wave, lane, ldq, DL);
    auto issue = [&](uint16_t* S, int st) {
        int h, q0;
        step_coords(st, h, q0);
        dma.issue(S, reinterpret_cast<const uint16_t*>(Qb + (size_t)h * DL), q0, len, wave);
        dma.issue(S + TILE, reinterpret_cast<const uint16_t*>(Db + (size_t)h * DL), q0, len, wave);
        // the pre-pass filled positions [len, N64) with +inf / 0, so the KV_BQ
        // values from q0 are in bounds and padding rows get P = 0
        const size_t vbase = ((size_t)b * a.H + h) * a.N64 + q0;
        float* vec = S == stA ? vecA : vecB;
        if (wave == 0) dma_vec(vec, a.lse2 + vbase, lane, KV_BQ);
        if (wave == 1) dma_vec(vec + 64, a.dsum + vbase, lane, KV_BQ);
    };

    const uint32_t keep2 = a.keep_k | (a.keep_k << 16);
    uint8_t* dm = dmask + (DROP ? wave * 32 * 32 : 0);

    auto step = [&](const uint16_t* S, int h, int q0, auto masked) {
        constexpr bool MASKED = decltype(masked)::value;
        const uint16_t* Qs = S;
        const uint16_t* Ds = S + TILE;
        const float* lse2 = S == stA ? vecA : vecB;
        const float* dsv = lse2 + 64;
        const float slope2 = ALIBI ? ld_uniform(a.slopes + h) * kLog2e : 0.f;
        constexpr int NK = D / 16, ND = D / 32;
        // Lane parts of the LDS operand offsets in XOR form: a base per lane,
        // passed through an empty asm in every block so that the compiler cannot
        // hoist the per-group offsets out of the loop as 16 registers per lane,
        // which two waves per SIMD cannot afford. Formed here, each is one
        // v_xor, and the stage and tile bases fold into the immediate offsets.
        const uint16_t* Vw = vt + vrow;  // this wave's 32 rows of V

#pragma unroll
        for (int qb = 0; qb < KV_BQ / 32; ++qb) {
            int rb = rbase, tb = tbase;
            asm volatile("" : "+v"(rb), "+v"(tb));
            // ---- S = Q K^T and dP = dO V^T: operand groups kk = 0 .. NK - 1
            f32x16 sc = f32x16{}, dpc = f32x16{};
            uint4 fq[2], fd[2], fv[2];  // one group ahead: three operands per group
            auto load1 = [&](int kk) {
                const int o = swz_row_x<D>(rb, kk);
                fq[kk % 2] = ld_s16(Qs + 32 * qb * D + o);
                fd[kk % 2] = ld_s16(Ds + 32 * qb * D + o);
                fv[kk % 2] = ld_s16(Vw + o);
            };
            load1(0);
#pragma unroll
            for (int kk = 0; kk < NK; ++kk) {
                if (kk + 1 < NK) load1(kk + 1);
                FA_SB();
                sc = Mfma<T>::mma(as_v8<T>(fq[kk % 2]), kf[kk], sc);
                dpc = Mfma<T>::mma(as_v8<T>(fd[kk % 2]), as_v8<T>(fv[kk % 2]), dpc);
                FA_SB();
            }

            // ---- dropout bytes of this block. The generator gives 16 bytes per
            // (query, half of the wave's 32 keys), the layout the forward uses;
            // this lane owns one key, so the wave writes its block to LDS and
            // reads it back transposed. Lane (query ql, half) writes the byte of
            // key 8 i + 4 half + j to row key, column 16 ((ql / 4) % 2) + 4 (ql / 8)
            // + ql % 4; lane (key, kg) then reads its 16 queries
            // 8 i + 4 kg + j as one 16-byte row segment, byte r for element r.
            uint32_t wd[4] = {0u, 0u, 0u, 0u};
            if constexpr (DROP) {
                const int ql = lane & 31, half = lane >> 5;
                const uint4 w = philox4x32_10(2u * (uint32_t)(kw / 32) + (uint32_t)half, (uint32_t)(q0 + 32 * qb + ql),
                                              (uint32_t)(b * a.H + h), a.drop_offset, a.seed_lo, a.seed_hi);
                const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
                const int colq = 16 * ((ql >> 2) & 1) + 4 * (ql >> 3) + (ql & 3);
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    dm[(8 * (e >> 2) + 4 * half + (e & 3)) * 32 + colq] = (uint8_t)(ww[e >> 2] >> (8 * (e & 3)));
                const uint4 rd = *reinterpret_cast<const uint4*>(dm + (lane & 31) * 32 + 16 * kg);
                wd[0] = rd.x, wd[1] = rd.y, wd[2] = rd.z, wd[3] = rd.w;
            }

            // ---- softmax backward, row group i = accumulator rows 4i .. 4i + 3.
            // Query qi of element (i, j) has qi - key = qk + 8 i + j; the pair is
            // masked when that offset is below -wr (key right of the window) or
            // above wl (key left of it): two per-step limits against constants.
            const int qk = q0 + 32 * qb + 4 * kg - key;
            const int lim_hi = wl - qk, lim_lo = -wr - qk;
            float pv[16], dsr[16];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float4 l4 = *reinterpret_cast<const float4*>(lse2 + 32 * qb + 8 * i + 4 * kg);
                const float4 d4 = *reinterpret_cast<const float4*>(dsv + 32 * qb + 8 * i + 4 * kg);
                const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
                const float dv[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int r = 4 * i + j;
                    float bias = -lv[j];
                    if (ALIBI) {
                        const float dist = (float)(qk + 8 * i + j);  // qi - key
                        bias -= slope2 * (CAUSAL ? dist : fabsf(dist));
                    }
                    float th = 0.f;  // softcapping: tanh(u / cap), for the derivative
                    if (CAP) th = tanh_fast(sc[r] * a.cap_in);
                    float p = exp2_fast(CAP ? fmaf(a.cap_out, th, bias) : fmaf(sc[r], c2, bias));
                    if (MASKED && (8 * i + j > lim_hi || 8 * i + j < lim_lo)) p = 0.f;
                    pv[r] = p;
                    float g = dpc[r];
                    if constexpr (DROP) {  // the gradient reaching P: dP o keep * 256 / K
                        const uint32_t m2 = keep_mask2(wd[r >> 2], (r >> 1) & 1, keep2);
                        const uint32_t m = (r & 1) ? (uint32_t)((int)m2 >> 16) : (uint32_t)((int)(m2 << 16) >> 16);
                        g = __uint_as_float(__float_as_uint(g) & m) * a.drop_scale;
                    }
                    dsr[r] = CAP ? p * (g - dv[j]) * (1.f - th * th) : p * (g - dv[j]);
                }
            }
            V8<T> pb[2], db8[2];  // P and dS per 16-query chunk, as B operands
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                const int r0 = 8 * h2;
                pb[h2] = pack8<T>(pv[r0], pv[r0 + 1], pv[r0 + 2], pv[r0 + 3], pv[r0 + 4], pv[r0 + 5], pv[r0 + 6],
                                  pv[r0 + 7]);
                db8[h2] = pack8<T>(dsr[r0], dsr[r0 + 1], dsr[r0 + 2], dsr[r0 + 3], dsr[r0 + 4], dsr[r0 + 5],
                                   dsr[r0 + 6], dsr[r0 + 7]);
                if constexpr (DROP) {  // dV takes the dropped probabilities (scaled at the end)
                    uint4 u = __builtin_bit_cast(uint4, pb[h2]);
                    u.x &= keep_mask2(wd[2 * h2], 0, keep2);
                    u.y &= keep_mask2(wd[2 * h2], 1, keep2);
                    u.z &= keep_mask2(wd[2 * h2 + 1], 0, keep2);
                    u.w &= keep_mask2(wd[2 * h2 + 1], 1, keep2);
                    pb[h2] = as_v8<T>(u);
                }
            }

            // ---- dV^T += dO^T P, dK^T += Q^T dS: groups (chunk c of the block, db)
            uint4 fo[2], fqt[2];
            auto load2 = [&](int gi) {
                const int c = 2 * qb + gi / ND, db = gi % ND;
                const int o0 = swz_tr_x<D>(tb, db, 0), o1 = swz_tr_x<D>(tb, db, 1);
                const uint2 olo = ld_s8_tr(Ds + 16 * c * D + o0);
                const uint2 ohi = ld_s8_tr(Ds + 16 * c * D + o1);
                const uint2 qlo = ld_s8_tr(Qs + 16 * c * D + o0);
                const uint2 qhi = ld_s8_tr(Qs + 16 * c * D + o1);
                fo[gi % 2] = make_uint4(olo.x, olo.y, ohi.x, ohi.y);
                fqt[gi % 2] = make_uint4(qlo.x, qlo.y, qhi.x, qhi.y);
            };
            load2(0);
#pragma unroll
            for (int gi = 0; gi < 2 * ND; ++gi) {
                if (gi + 1 < 2 * ND) load2(gi + 1);
                FA_SB();
                const int db = gi % ND;
                dvacc[db] = Mfma<T>::mma(as_v8<T>(fo[gi % 2]), pb[gi / ND], dvacc[db]);
                dkacc[db] = Mfma<T>::mma(as_v8<T>(fqt[gi % 2]), db8[gi / ND], dkacc[db]);
                FA_SB();
            }
        }
    };

    auto compute = [&](const uint16_t* S, int st) {
        int h, q0;
        step_coords(st, h, q0);
        // wave-uniform skips: keys past the sequence end, or a query tile no
        // key of this wave is visible from (causal: entirely before the keys)
        if (!((kw < len) && kw <= q0 + KV_BQ - 1 + wr && kw + 31 >= q0 - wl)) return;
        if (kw + 31 > q0 + wr || kw < q0 + KV_BQ - 1 - wl)
            step(S, h, q0, std::true_type{});  // some pair is masked (diagonal, window)
        else
            step(S, h, q0, std::false_type{});
    };

    two_stage_loop(stA, stB, steps, issue, compute);

    // epilogue: lane owns key `key`; accumulator rows are dims 32*db + 8*i + 4*kg + 0..3
    if (key < len) {
        T* dK = reinterpret_cast<T*>(a.dk) + (size_t)(row0 + key) * ldk + (size_t)g * DL;
        T* dV = reinterpret_cast<T*>(a.dv) + (size_t)(row0 + key) * ldk + (size_t)g * DL;
        const float sc = a.scale;
        const float vs = DROP ? a.drop_scale : 1.f;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int d0 = 32 * db + 8 * i + 4 * kg;
                const int r = 4 * i;
                if (d0 >= DL) continue;
                *reinterpret_cast<uint2*>(dK + d0) = pack4<T>(dkacc[db][r] * sc, dkacc[db][r + 1] * sc,
                                                              dkacc[db][r + 2] * sc, dkacc[db][r + 3] * sc);
                *reinterpret_cast<uint2*>(dV + d0) = pack4<T>(dvacc[db][r] * vs, dvacc[db][r + 1] * vs,
                                                              dvacc[db][r + 2] * vs, dvacc[db][r + 3] * vs);
            }
        }
    }
}

#undef FA_SB

template <typename T, int D, bool CAUSAL, bool ALIBI, bool DROP, bool CAP, int NWO>
hipError_t launch_shape(const Args& a, hipStream_t s) {
    constexpr int KV_BK = DkdvShape<D, NWO>::KV_BK;
    dim3 grid(a.Hkv, a.B, (a.N + KV_BK - 1) / KV_BK);
    hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, CAUSAL, ALIBI, DROP, CAP, NWO>), grid, dim3(DkdvShape<D, NWO>::NT), 0,
                       s, a);
    return hipGetLastError();
}

// Head dim 64, plain variant: 4-wave workgroups when the 8-wave grid would give
// at most two workgroups per compute unit (measured on B = 8, H = 16, N = 1024:
// 0.089 against 0.104 ms; on longer grids the 8-wave shape was as fast or up to
// 3% faster).
constexpr int kComputeUnits = 256;
template <typename T, int D, bool CAUSAL, bool ALIBI, bool DROP, bool CAP>
hipError_t launch(const Args& a, hipStream_t s) {
    if constexpr ((D == 64 || D == 128) && !ALIBI && !DROP && !CAP) {
        const long long wg8 = (long long)a.Hkv * a.B * ((a.N + DkdvShape<D>::KV_BK - 1) / DkdvShape<D>::KV_BK);
        if (wg8 <= (D == 64 ? 2 : 1) * kComputeUnits) return launch_shape<T, D, CAUSAL, ALIBI, DROP, CAP, 4>(a, s);
    }
    return launch_shape<T, D, CAUSAL, ALIBI, DROP, CAP, 0>(a, s);
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

hipError_t launch_bwd_dkdv(const Args& a, int dtype, int d, bool causal, bool alibi, int var, hipStream_t s) {
    return dtype == 2 ? launch_t<__bf16>(a, d, causal, alibi, var, s) : launch_t<_Float16>(a, d, causal, alibi, var, s);
}

}  // namespace fa
