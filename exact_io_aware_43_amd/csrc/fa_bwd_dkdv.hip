// dK/dV kernel of the backward pass (the three-launch structure and the method
// are described in fa_bwd.hip; "FlashAttention: Faster Attention Without
// Dropping a Single Interaction", Method Deep Dive, Key design 3).
//
// One workgroup of 4 waves per (128-key tile, kv head, sequence); each wave
// owns 32 keys and keeps their K and V rows in registers as MFMA operands and
// their dK, dV accumulators in AGPRs. The workgroup walks every query head of
// the kv group and every 64-query tile that can see the keys. Per 64-query
// step, with query blocks qb = 0, 1 of 32 rows:
//
//   S  = Q K^T, dP = dO V^T            (scores: one key column per lane)
//   P  = exp2(S * scale * log2 e - L * log2 e), dS = P o (dP - D)
//   dV^T += dO^T P,  dK^T += Q^T dS    (transposed operands via ds_read_b64_tr_b16)
//
// At one wave per SIMD nothing else hides the softmax, so the step is laid out
// by hand as four phases whose VALU and MFMA work are independent and
// interleaved:
//   A: S/dP of block 0
//   B: S/dP of block 1        + softmax of block 0
//   C: dV/dK of block 0       + softmax of block 1
//   D: dV/dK of block 1
// LDS operand loads run two MFMA groups ahead through small register rings,
// and scheduling barriers pin the order.
#include <type_traits>

#include "fa_device.hpp"

namespace fa {
namespace {

constexpr int NT = 256;
constexpr int KV_BK = 128;  // keys per workgroup (32 per wave)
constexpr int KV_BQ = 64;   // queries per step (two blocks of 32)

#define FA_SB() __builtin_amdgcn_sched_barrier(0)

template <typename T, int D, bool CAUSAL, bool ALIBI>
__global__ __launch_bounds__(NT, 1) void bwd_dkdv_kernel(Args a) {
    // stage: Q tile, dO tile (swizzled [KV_BQ x D] each), then L*log2(e) and D (fp32, KV_BQ each)
    constexpr int TILE = KV_BQ * D;
    constexpr int STAGE = 2 * TILE + 2 * KV_BQ * 2;
    __shared__ __attribute__((aligned(16))) uint16_t stA[STAGE];
    __shared__ __attribute__((aligned(16))) uint16_t stB[STAGE];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int kg = lane >> 5;
    const int g = blockIdx.x, b = blockIdx.y;
    const int kt = blockIdx.z;  // low key tiles see the most queries: dispatched first
    int row0, len;
    seq_bounds(a, b, row0, len);
    const int k0 = kt * KV_BK;
    if (k0 >= len) return;

    const size_t ldq = (size_t)a.H * D, ldk = (size_t)a.Hkv * D;
    const int kw = k0 + wave * 32;     // first key of this wave
    const int key = kw + (lane & 31);  // this lane's key (column of S)

    // K^T and V^T fragments as B operands: lane holds key `key`, dims 16*kk + 8*kg + 0..7.
    V8<T> kf[D / 16], vf[D / 16];
    {
        const T* Kp = reinterpret_cast<const T*>(a.k) + (size_t)(row0 + key) * ldk + (size_t)g * D;
        const T* Vp = reinterpret_cast<const T*>(a.v) + (size_t)(row0 + key) * ldk + (size_t)g * D;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            uint4 uk = make_uint4(0, 0, 0, 0), uv = uk;
            if (key < len) {
                uk = ld_g16(Kp + 16 * kk + 8 * kg);
                uv = ld_g16(Vp + 16 * kk + 8 * kg);
            }
            kf[kk] = as_v8<T>(uk);
            vf[kk] = as_v8<T>(uv);
        }
    }

    int roff[D / 16], toff[D / 32][2];
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) roff[kk] = swz_row_off<D>(lane, kk);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
        toff[db][0] = swz_tr_off<D>(lane, db, 0);
        toff[db][1] = swz_tr_off<D>(lane, db, 1);
    }

    f32x16 dkacc[D / 32], dvacc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
        dkacc[db] = f32x16{};
        dvacc[db] = f32x16{};
    }

    // Query tiles that can see this key tile: all of them, or (causal) those
    // ending at or after k0; for every query head of the kv group.
    const int qt0 = CAUSAL ? k0 / KV_BQ : 0;
    const int nqt = (len + KV_BQ - 1) / KV_BQ;
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

    DmaTile<D, KV_BQ, NT / 64> dma;
    dma.init(wave, lane, ldq);
    auto issue = [&](uint16_t* S, int st) {
        int h, q0;
        step_coords(st, h, q0);
        dma.issue(S, reinterpret_cast<const uint16_t*>(Qb + (size_t)h * D), q0, len, wave);
        dma.issue(S + TILE, reinterpret_cast<const uint16_t*>(Db + (size_t)h * D), q0, len, wave);
        // the pre-pass filled positions [len, N64) with +inf / 0, so the 64
        // values from q0 are in bounds and padding rows get P = 0
        const size_t vbase = ((size_t)b * a.H + h) * a.N64 + q0;
        if (wave == 0) dma_vec64(reinterpret_cast<float*>(S + 2 * TILE), a.lse2 + vbase, lane);
        if (wave == 1) dma_vec64(reinterpret_cast<float*>(S + 2 * TILE) + KV_BQ, a.dsum + vbase, lane);
    };

    auto step = [&](const uint16_t* S, int h, int q0, auto masked) {
        constexpr bool MASKED = decltype(masked)::value;
        const uint16_t* Qs = S;
        const uint16_t* Ds = S + TILE;
        const float* lse2 = reinterpret_cast<const float*>(S + 2 * TILE);
        const float* dsv = lse2 + KV_BQ;
        const float slope2 = ALIBI ? ld_uniform(a.slopes + h) * kLog2e : 0.f;

        f32x16 sc[2], dpc[2];  // S and dP of blocks 0, 1
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            sc[qb] = f32x16{};
            dpc[qb] = f32x16{};
        }
        float4 l4[4], d4[4];  // L*log2(e) and D of the block being softmaxed, per row group i
        float pv[16], dsr[16];
        V8<T> pb[4], db8[4];  // packed P and dS per 16-query chunk c

        // L*log2(e) and D of rows 8i + 4kg + 0..3 of block qb (one row group)
        auto load_vec = [&](int qb, int i) {
            l4[i] = *reinterpret_cast<const float4*>(lse2 + 32 * qb + 8 * i + 4 * kg);
            d4[i] = *reinterpret_cast<const float4*>(dsv + 32 * qb + 8 * i + 4 * kg);
        };
        // softmax backward of accumulator row r of block qb: P and dS
        auto elem = [&](int qb, int r) {
            const int i = r >> 2, j = r & 3;
            const float lv = j == 0 ? l4[i].x : j == 1 ? l4[i].y : j == 2 ? l4[i].z : l4[i].w;
            const float dv = j == 0 ? d4[i].x : j == 1 ? d4[i].y : j == 2 ? d4[i].z : d4[i].w;
            const int qi = q0 + 32 * qb + 8 * i + 4 * kg + j;
            float bias = -lv;
            if (ALIBI) {
                const float dist = (float)(qi - key);
                bias -= slope2 * (CAUSAL ? dist : fabsf(dist));
            }
            float p = exp2_fast(fmaf(sc[qb][r], c2, bias));
            if (MASKED && key > qi) p = 0.f;
            float ds = p * (dpc[qb][r] - dv);
            asm volatile("" : "+v"(p), "+v"(ds));  // materialise here: keeps the VALU work in its MFMA slot
            pv[r] = p;
            dsr[r] = ds;
        };
        // P and dS of rows 8 h2 .. 8 h2 + 7 of block qb as bf16/f16 B operands
        auto pack_half = [&](int qb, int h2) {
            const int r0 = 8 * h2;
            pb[2 * qb + h2] = pack8<T>(pv[r0], pv[r0 + 1], pv[r0 + 2], pv[r0 + 3], pv[r0 + 4], pv[r0 + 5], pv[r0 + 6],
                                       pv[r0 + 7]);
            db8[2 * qb + h2] = pack8<T>(dsr[r0], dsr[r0 + 1], dsr[r0 + 2], dsr[r0 + 3], dsr[r0 + 4], dsr[r0 + 5],
                                        dsr[r0 + 6], dsr[r0 + 7]);
        };
        // elements [r0, r0 + n) of block qb, each followed by what it frees or completes:
        // the row group's vectors for block `nxt` (if >= 0) and the packed half
        auto elems = [&](int qb, int r0, int n, int nxt) {
#pragma unroll
            for (int r = r0; r < r0 + n; ++r) {
                elem(qb, r);
                if ((r & 3) == 3 && nxt >= 0) load_vec(nxt, r >> 2);
                if ((r & 7) == 7) pack_half(qb, r >> 3);
            }
        };

        // ---- S/dP operand ring: group g1 in [0, 2 * D/16): block g1 / (D/16), kk = g1 % (D/16)
        constexpr int NK = D / 16;
        uint4 fq[3], fd[3];
        auto load1 = [&](int g1) {
            const int qb = g1 / NK, kk = g1 % NK;
            fq[g1 % 3] = ld_s16(Qs + 32 * qb * D + roff[kk]);
            fd[g1 % 3] = ld_s16(Ds + 32 * qb * D + roff[kk]);
        };
        auto mma1s = [&](int g1) {
            const int qb = g1 / NK, kk = g1 % NK;
            sc[qb] = Mfma<T>::mma(as_v8<T>(fq[g1 % 3]), kf[kk], sc[qb]);
        };
        auto mma1d = [&](int g1) {
            const int qb = g1 / NK, kk = g1 % NK;
            dpc[qb] = Mfma<T>::mma(as_v8<T>(fd[g1 % 3]), vf[kk], dpc[qb]);
        };
        auto mma1 = [&](int g1) {
            mma1s(g1);
            mma1d(g1);
        };
        // ---- dV/dK operand ring: group g2 in [0, 4 * D/32): chunk c = g2 / (D/32), db = g2 % (D/32)
        constexpr int ND = D / 32;
        uint4 fo[3], fqt[3];
        auto load2 = [&](int g2) {
            const int c = g2 / ND, db = g2 % ND;
            const uint2 olo = ld_s8_tr(Ds + 16 * c * D + toff[db][0]);
            const uint2 ohi = ld_s8_tr(Ds + 16 * c * D + toff[db][1]);
            const uint2 qlo = ld_s8_tr(Qs + 16 * c * D + toff[db][0]);
            const uint2 qhi = ld_s8_tr(Qs + 16 * c * D + toff[db][1]);
            fo[g2 % 3] = make_uint4(olo.x, olo.y, ohi.x, ohi.y);
            fqt[g2 % 3] = make_uint4(qlo.x, qlo.y, qhi.x, qhi.y);
        };
        auto mma2v = [&](int g2) {
            const int c = g2 / ND, db = g2 % ND;
            dvacc[db] = Mfma<T>::mma(as_v8<T>(fo[g2 % 3]), pb[c], dvacc[db]);
        };
        auto mma2k = [&](int g2) {
            const int c = g2 / ND, db = g2 % ND;
            dkacc[db] = Mfma<T>::mma(as_v8<T>(fqt[g2 % 3]), db8[c], dkacc[db]);
        };
        auto mma2 = [&](int g2) {
            mma2v(g2);
            mma2k(g2);
        };

        // One softmax element after every MFMA of phases B and C (two for
        // D = 64): with one wave per SIMD issue is in order, and a VALU run
        // only overlaps the MFMA issued just before it.
        constexpr int EB = 16 / (2 * NK);  // elements per MFMA in phase B
        constexpr int EC = 16 / (4 * ND);  // and in phase C

        // phase A: S/dP of block 0
#pragma unroll
        for (int i = 0; i < 4; ++i) load_vec(0, i);
        load1(0);
        load1(1);
#pragma unroll
        for (int g1 = 0; g1 < NK; ++g1) {
            load1(g1 + 2);
            FA_SB();
            mma1(g1);
            FA_SB();
        }
        // phase B: S/dP of block 1, softmax of block 0 (its row-group vectors
        // are replaced by block 1's as they are used up)
#pragma unroll
        for (int g1 = NK; g1 < 2 * NK; ++g1) {
            const int e = 2 * (g1 - NK) * EB;
            if (g1 + 2 < 2 * NK) load1(g1 + 2);
            FA_SB();
            mma1s(g1);
            FA_SB();
            elems(0, e, EB, 1);
            FA_SB();
            mma1d(g1);
            FA_SB();
            elems(0, e + EB, EB, 1);
            FA_SB();
        }
        // phase C: dV/dK of block 0 (chunks 0, 1), softmax of block 1
        load2(0);
        load2(1);
#pragma unroll
        for (int g2 = 0; g2 < 2 * ND; ++g2) {
            const int e = 2 * g2 * EC;
            load2(g2 + 2);
            FA_SB();
            mma2v(g2);
            FA_SB();
            elems(1, e, EC, -1);
            FA_SB();
            mma2k(g2);
            FA_SB();
            elems(1, e + EC, EC, -1);
            FA_SB();
        }
        // phase D: dV/dK of block 1 (chunks 2, 3)
#pragma unroll
        for (int g2 = 2 * ND; g2 < 4 * ND; ++g2) {
            if (g2 + 2 < 4 * ND) load2(g2 + 2);
            FA_SB();
            mma2(g2);
            FA_SB();
        }
    };

    auto compute = [&](const uint16_t* S, int st) {
        int h, q0;
        step_coords(st, h, q0);
        // wave-uniform skips: keys past the sequence end, or (causal) a query
        // tile entirely before this wave's first key
        if (!((kw < len) && (!CAUSAL || q0 + KV_BQ - 1 >= kw))) return;
        if (CAUSAL && q0 < kw + 31)
            step(S, h, q0, std::true_type{});  // tile straddles the diagonal
        else
            step(S, h, q0, std::false_type{});
    };

    two_stage_loop(stA, stB, steps, issue, compute);

    // epilogue: lane owns key `key`; accumulator rows are dims 32*db + 8*i + 4*kg + 0..3
    if (key < len) {
        T* dK = reinterpret_cast<T*>(a.dk) + (size_t)(row0 + key) * ldk + (size_t)g * D;
        T* dV = reinterpret_cast<T*>(a.dv) + (size_t)(row0 + key) * ldk + (size_t)g * D;
        const float sc = a.scale;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int d0 = 32 * db + 8 * i + 4 * kg;
                const int r = 4 * i;
                *reinterpret_cast<uint2*>(dK + d0) = pack4<T>(dkacc[db][r] * sc, dkacc[db][r + 1] * sc,
                                                              dkacc[db][r + 2] * sc, dkacc[db][r + 3] * sc);
                *reinterpret_cast<uint2*>(dV + d0) =
                    pack4<T>(dvacc[db][r], dvacc[db][r + 1], dvacc[db][r + 2], dvacc[db][r + 3]);
            }
        }
    }
}

#undef FA_SB

template <typename T, int D, bool CAUSAL, bool ALIBI>
hipError_t launch(const Args& a, hipStream_t s) {
    dim3 grid(a.Hkv, a.B, (a.N + KV_BK - 1) / KV_BK);
    hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, CAUSAL, ALIBI>), grid, dim3(NT), 0, s, a);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_d(const Args& a, bool causal, bool alibi, hipStream_t s) {
    if (causal) return alibi ? launch<T, D, true, true>(a, s) : launch<T, D, true, false>(a, s);
    return alibi ? launch<T, D, false, true>(a, s) : launch<T, D, false, false>(a, s);
}

}  // namespace

hipError_t launch_bwd_dkdv(const Args& a, int dtype, int d, bool causal, bool alibi, hipStream_t s) {
    if (dtype == 2) return d == 64 ? launch_d<__bf16, 64>(a, causal, alibi, s) : launch_d<__bf16, 128>(a, causal, alibi, s);
    return d == 64 ? launch_d<_Float16, 64>(a, causal, alibi, s) : launch_d<_Float16, 128>(a, causal, alibi, s);
}

}  // namespace fa
