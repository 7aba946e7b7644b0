// Decode over a key/value cache: a few new queries per sequence against a long
// cache, with the keys split across workgroups and the partial states merged.
//
// Method: "FlashAttention: Faster Attention Without Dropping a Single
// Interaction", Key design 2 (the (m, l, O) state of disjoint key sets merges
// exactly: m = max m_s, l = sum l_s e^(m_s - m), O = sum O_s l_s e^(m_s - m) / l)
// applied across key splits, for the decode workload its Limitations section
// sets apart from training and prefill ("long context and inference").
//
// Rows. The G = H / Hkv query heads of a kv head read the same K and V, so the
// G * Nq query rows of one (sequence, kv head) form the 32 columns of the MFMA
// B operand (row hh * Nq + t is query head g G + hh, query t); more rows use
// more row groups. K and V are then read from HBM once per kv head, which is
// what bounds this workload: every key is touched by a handful of queries, so
// the work per byte is small.
//
// Split kernel: one workgroup of 4 waves per (kv head and row group, sequence,
// key split). Tiles of 128 keys stream through LDS (direct global-to-LDS
// loads, double buffered); wave w takes keys 32 w .. 32 w + 31 of each tile, so
// the four waves hold four states of disjoint key sets, merged through LDS at
// the end. A split writes its normalised O (fp32) and lse to the workspace, or,
// when the problem has one split, the final O and lse directly.
// Merge kernel: one workgroup per (sequence, query head, query), one lane per
// head dimension, combines the splits.
//
// Causal: query t of a sequence with L cached keys (the new tokens included)
// sits at position L - Nq + t and keeps keys j <= L - Nq + t. ALiBi adds
// -slope_h |position - j|. Every row takes its maximum on every tile and
// raises its reference whenever the maximum grows, so the largest weight is
// exactly 1 before rounding (this kernel is bound by HBM, not by the VALU).
#include "fa_device.hpp"

namespace fa {
namespace {

constexpr int DNW = 4;           // waves per split workgroup
constexpr int DNT = 64 * DNW;
constexpr int DBC = 32 * DNW;    // keys per staged tile (32 per wave)

// Sequence b's cache length, clamped to [0, Nk].
__device__ __forceinline__ int cache_len(const DecodeArgs& a, int b) {
    const int L = a.seqlens[b];
    return L < 0 ? 0 : (L > a.Nk ? a.Nk : L);
}

// Keys [kbeg, kend) of sequence b (L cached keys) for the query rows of row
// group rg of kv head g: the tile loop, the merge of the four waves' states,
// then O and lse of the range, final (direct) or as partial `slot` of the
// sequence's rows. Every wave of the workgroup calls it with the same
// arguments (it holds barriers), and it leaves the staging buffers free.
template <typename T, int D, bool CAUSAL, bool ALIBI>
__device__ __forceinline__ void decode_range(const DecodeArgs& a, uint16_t* stA, uint16_t* stB, int g, int rg, int b,
                                             int L, int kbeg, int kend, int slot, bool direct) {
    constexpr int TILE = DBC * D;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int col = lane & 31, kg = lane >> 5;
    const int G = a.H / a.Hkv;
    const int R = G * a.Nq;  // query rows of this kv head

    const int rr = rg * 32 + col;  // this lane's row
    const bool row_live = rr < R;
    const int hh = row_live ? rr / a.Nq : 0, t = row_live ? rr % a.Nq : 0;
    const int h = g * G + hh;
    const int pos = L - a.Nq + t;  // position of this lane's query in its sequence
    const int ntile = kend > kbeg ? (kend - kbeg + DBC - 1) / DBC : 0;

    const size_t ldq = (size_t)a.H * D, ldk = (size_t)a.Hkv * D;
    const T* Qp = reinterpret_cast<const T*>(a.q) + ((size_t)b * a.Nq + t) * ldq + (size_t)h * D;
    const T* Kg = reinterpret_cast<const T*>(a.k) + (size_t)b * a.Nk * ldk + (size_t)g * D;
    const T* Vg = reinterpret_cast<const T*>(a.v) + (size_t)b * a.Nk * ldk + (size_t)g * D;

    V8<T> qf[D / 16];
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
        uint4 u = make_uint4(0, 0, 0, 0);
        if (row_live) u = ld_g16(Qp + 16 * kk + 8 * kg);
        qf[kk] = as_v8<T>(u);
    }
    const float c2 = a.scale_log2;
    const float slope2 = (ALIBI && row_live) ? a.slopes[h] * kLog2e : 0.f;

    int roff[D / 16], toff[D / 32][2];
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) roff[kk] = swz_row_off<D>(lane, kk);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
        toff[db][0] = swz_tr_off<D>(lane, db, 0);
        toff[db][1] = swz_tr_off<D>(lane, db, 1);
    }

    f32x16 oacc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16{};
    float m_run = -INFINITY, l_run = 0.f;

    // Each tile is staged as two halves of DBC / 2 rows (a wave's share of a
    // whole tile would exceed the four loads one LDS base reaches); the swizzle
    // repeats every 16 rows, so the halves form one swizzled [DBC x D] tile.
    // Rows at or past the split's end read as zero (kend bounds the range
    // check), and their keys are masked below.
    DmaTile<D, DBC / 2, DNW> dma;
    dma.init(wave, lane, ldk);
    auto issue = [&](uint16_t* st, int it) {
        const int r0 = kbeg + it * DBC;
        const uint16_t* kb = reinterpret_cast<const uint16_t*>(Kg);
        const uint16_t* vb = reinterpret_cast<const uint16_t*>(Vg);
        dma.issue(st, kb, r0, kend, wave);
        dma.issue(st + (DBC / 2) * D, kb, r0 + DBC / 2, kend, wave);
        dma.issue(st + TILE, vb, r0, kend, wave);
        dma.issue(st + TILE + (DBC / 2) * D, vb, r0 + DBC / 2, kend, wave);
    };
    auto compute = [&](const uint16_t* Ks, int it) {
        const uint16_t* Vs = Ks + TILE;
        const int k0 = kbeg + it * DBC + 32 * wave;  // first key of this wave's slice
        if (k0 >= kend) return;                      // wave-uniform
        f32x16 s = f32x16{};
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
            s = Mfma<T>::mma(as_v8<T>(ld_s16(Ks + 32 * wave * D + roff[kk])), qf[kk], s);
        float mt = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int key = k0 + 8 * (r >> 2) + 4 * kg + (r & 3);
            float x = s[r] * c2;
            if (ALIBI) x -= slope2 * fabsf((float)(pos - key));
            if (key >= kend || (CAUSAL && key > pos)) x = -INFINITY;
            s[r] = x;
            mt = fmaxf(mt, x);
        }
        mt = max_xor32(mt);
        const float m_new = fmaxf(m_run, mt);
        if (__any(m_new > m_run)) {
            const float alpha = m_new > m_run ? exp2_fast(m_run - m_new) : 1.f;  // 0 from -inf
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < D / 32; ++db) oacc[db] *= alpha;
            m_run = m_new;
        }
        const float m_use = m_run == -INFINITY ? 0.f : m_run;
        float ls = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float p = exp2_fast(s[r] - m_use);
            s[r] = p;
            ls += p;
        }
        l_run += ls;
        V8<T> pf[2];
#pragma unroll
        for (int c = 0; c < 2; ++c)
            pf[c] = pack8<T>(s[8 * c], s[8 * c + 1], s[8 * c + 2], s[8 * c + 3], s[8 * c + 4], s[8 * c + 5],
                             s[8 * c + 6], s[8 * c + 7]);
#pragma unroll
        for (int c = 0; c < 2; ++c) {
#pragma unroll
            for (int db = 0; db < D / 32; ++db) {
                const uint16_t* vb = Vs + 16 * (2 * wave + c) * D;
                const uint2 lo = ld_s8_tr(vb + toff[db][0]);
                const uint2 hi = ld_s8_tr(vb + toff[db][1]);
                oacc[db] = Mfma<T>::mma(as_v8<T>(make_uint4(lo.x, lo.y, hi.x, hi.y)), pf[c], oacc[db]);
            }
        }
    };
    if (ntile > 0) two_stage_loop(stA, stB, ntile, issue, compute);
    __syncthreads();  // all waves are done with the staging buffers: reuse them for the merge

    // ---- merge the four waves' states of this row group through LDS
    float* ms = reinterpret_cast<float*>(stA);           // [DNW][32] maxima (log2 units)
    float* ls_ = ms + DNW * 32;                           // [DNW][32] sums
    float* ob = reinterpret_cast<float*>(stB);            // [DNW][32 rows][D] unnormalised O
    const float l_tot = sum_xor32(l_run);
    if (kg == 0) {
        ms[wave * 32 + col] = m_run;
        ls_[wave * 32 + col] = l_tot;
    }
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                ob[(wave * 32 + col) * D + 32 * db + 8 * i + 4 * kg + j] = oacc[db][4 * i + j];
    __syncthreads();

    // Thread tid handles (row, 32-dimension quarter) pairs: row = tid % 32,
    // dims 32 (tid / 32) ... (D / 32 quarters, so 32 * D / 32 = D threads are
    // busy; for D = 64 half of the workgroup idles here).
    const int row = tid & 31, part = tid >> 5;
    if (part < D / 32) {
        const int rrow = rg * 32 + row;
        float m = -INFINITY;
#pragma unroll
        for (int w = 0; w < DNW; ++w) m = fmaxf(m, ms[w * 32 + row]);
        float wt[DNW], lsum = 0.f;
#pragma unroll
        for (int w = 0; w < DNW; ++w) {
            const float mw = ms[w * 32 + row];
            wt[w] = mw == -INFINITY ? 0.f : exp2_fast(mw - m);
            lsum += wt[w] * ls_[w * 32 + row];
        }
        const bool seen = m != -INFINITY && lsum > 0.f;
        const float inv = seen ? 1.f / lsum : 0.f;
        const float lse = seen ? (m + __log2f(lsum)) * kLn2 : -INFINITY;
        if (rrow < R) {
            const int hq = g * G + rrow / a.Nq, tq = rrow % a.Nq;
            float o[32];
#pragma unroll
            for (int e = 0; e < 32; ++e) {
                float acc = 0.f;
#pragma unroll
                for (int w = 0; w < DNW; ++w) acc = fmaf(wt[w], ob[(w * 32 + row) * D + 32 * part + e], acc);
                o[e] = acc * inv;
            }
            const size_t orow = ((size_t)b * a.Nq + tq) * a.H + hq;  // row of O in [B, Nq, H, d]
            if (direct) {
                T* O = reinterpret_cast<T*>(a.o) + orow * D + 32 * part;
#pragma unroll
                for (int e = 0; e < 32; e += 4)
                    *reinterpret_cast<uint2*>(O + e) = pack4<T>(o[e], o[e + 1], o[e + 2], o[e + 3]);
                if (part == 0) a.lse[((size_t)b * a.H + hq) * a.Nq + tq] = lse;
            } else {
                // partial `slot`: [B, H, Nq, splits] lse and [B, H, Nq, splits, D] O
                const size_t prow = (((size_t)b * a.H + hq) * a.Nq + tq) * a.splits + slot;
                float* Op = a.part_o + prow * D + 32 * part;
#pragma unroll
                for (int e = 0; e < 32; e += 4) *reinterpret_cast<float4*>(Op + e) = make_float4(o[e], o[e + 1], o[e + 2], o[e + 3]);
                if (part == 0) a.part_lse[prow] = lse;
            }
        }
    }
    __syncthreads();  // the merge buffers are the staging buffers of a next range
}

// Key ranges of the concatenated caches in flat mode: the T keys of all
// sequences (kv head by kv head the same) cut into `parts` ranges of C keys
// (C a multiple of 32); returns C, 0 when every cache is empty.
__device__ __forceinline__ long long flat_chunk(long long T, int parts) {
    return ((T + parts - 1) / parts + 31) & ~31ll;
}

template <typename T, int D, bool CAUSAL, bool ALIBI>
__global__ __launch_bounds__(DNT, 1) void decode_split_kernel(DecodeArgs a) {
    constexpr int TILE = DBC * D;
    __shared__ __attribute__((aligned(16))) uint16_t stA[2 * TILE];
    __shared__ __attribute__((aligned(16))) uint16_t stB[2 * TILE];
    const int g = blockIdx.x % a.Hkv, rg = blockIdx.x / a.Hkv;  // kv head, row group
    if (a.flat) {
        // Balanced ranges: workgroup p takes keys [p C, (p + 1) C) of the
        // caches laid end to end, one piece per sequence its range meets, so
        // every workgroup streams the same number of keys whatever the mix of
        // cache lengths. A piece's state is partial p of its sequence.
        const int p = blockIdx.y;
        long long total = 0;
        for (int b = 0; b < a.B; ++b) total += cache_len(a, b);
        const long long C = flat_chunk(total, a.splits);
        const long long lo = (long long)p * C, hi = min(total, lo + C);
        long long off = 0;
        for (int b = 0; b < a.B && off < hi; ++b) {
            const int L = cache_len(a, b);
            const long long s0 = max(lo, off), s1 = min(hi, off + L);
            if (s1 > s0)
                decode_range<T, D, CAUSAL, ALIBI>(a, stA, stB, g, rg, b, L, (int)(s0 - off), (int)(s1 - off), p,
                                                  false);
            off += L;
        }
    } else {
        // keys of split sp: sequence b's L keys cut into `splits` ranges of
        // ceil(L / splits) keys rounded up to 32 (trailing ranges may be empty)
        const int b = blockIdx.y, sp = blockIdx.z;
        const int L = cache_len(a, b);
        const int chunk = ((L + a.splits - 1) / a.splits + 31) & ~31;
        const int kbeg = min(L, sp * chunk);
        const int kend = min(L, kbeg + chunk);
        decode_range<T, D, CAUSAL, ALIBI>(a, stA, stB, g, rg, b, L, kbeg, kend, sp, a.splits == 1);
    }
}

// One workgroup of D threads per (sequence, query head, query): combine the
// splits' (lse_s, O_s) into O = sum_s e^(lse_s - lse) O_s, lse = log sum_s e^lse_s.
template <typename T, int D>
__global__ __launch_bounds__(D) void decode_merge_kernel(DecodeArgs a) {
    const int row = blockIdx.x;  // (b * H + h) * Nq + t
    const int e = threadIdx.x;
    const int S = a.splits;
    const float* pl = a.part_lse + (size_t)row * S;
    // partials written for this row: all S ranges of its sequence, or in flat
    // mode the ranges [s_lo, s_hi] that met it (none for an empty cache)
    int s_lo = 0, s_hi = S - 1;
    if (a.flat) {
        const int bq = row / (a.H * a.Nq);
        long long total = 0, off = 0;
        for (int b = 0; b < a.B; ++b) {
            const int L = cache_len(a, b);
            if (b < bq) off += L;
            total += L;
        }
        const int L = cache_len(a, bq);
        const long long C = flat_chunk(total, S);
        s_lo = L > 0 ? (int)(off / C) : 0;
        s_hi = L > 0 ? (int)((off + L - 1) / C) : -1;
    }
    float m = -INFINITY;
    for (int s = s_lo; s <= s_hi; ++s) m = fmaxf(m, pl[s]);
    float total = 0.f, acc = 0.f;
    if (m != -INFINITY) {
        for (int s = s_lo; s <= s_hi; ++s) {
            const float ws = pl[s] == -INFINITY ? 0.f : __expf(pl[s] - m);
            total += ws;
            acc = fmaf(ws, a.part_o[((size_t)row * S + s) * D + e], acc);
        }
    }
    const int t = row % a.Nq, bh = row / a.Nq, h = bh % a.H, b = bh / a.H;
    T* O = reinterpret_cast<T*>(a.o) + (((size_t)b * a.Nq + t) * a.H + h) * D;
    O[e] = (T)(total > 0.f ? acc / total : 0.f);
    if (e == 0) a.lse[row] = total > 0.f ? m + __logf(total) : -INFINITY;
}

template <typename T, int D, bool CAUSAL, bool ALIBI>
hipError_t launch(const DecodeArgs& a, hipStream_t s) {
    const int G = a.H / a.Hkv;
    const int rgroups = (G * a.Nq + 31) / 32;
    const dim3 grid = a.flat ? dim3(a.Hkv * rgroups, a.splits, 1) : dim3(a.Hkv * rgroups, a.B, a.splits);
    hipLaunchKernelGGL((decode_split_kernel<T, D, CAUSAL, ALIBI>), grid, dim3(DNT), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || (a.splits == 1 && !a.flat)) return e;
    hipLaunchKernelGGL((decode_merge_kernel<T, D>), dim3(a.B * a.H * a.Nq), dim3(D), 0, s, a);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_d(const DecodeArgs& a, bool causal, bool alibi, hipStream_t s) {
    if (causal) return alibi ? launch<T, D, true, true>(a, s) : launch<T, D, true, false>(a, s);
    return alibi ? launch<T, D, false, true>(a, s) : launch<T, D, false, false>(a, s);
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, int dtype, int d, bool causal, bool alibi, hipStream_t s) {
    if (dtype == 2) return d == 64 ? launch_d<__bf16, 64>(a, causal, alibi, s) : launch_d<__bf16, 128>(a, causal, alibi, s);
    return d == 64 ? launch_d<_Float16, 64>(a, causal, alibi, s) : launch_d<_Float16, 128>(a, causal, alibi, s);
}

}  // namespace fa
