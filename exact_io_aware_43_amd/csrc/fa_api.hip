// C-ABI entry points of libfa (declared in include/fa.h): argument checks,
// selection of the compiled kernel instance, and the launches. Every check runs
// before the first launch, so a rejected call enqueues and writes nothing.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "../../include/fa.h"
#include "fa_internal.hpp"

namespace {

constexpr int kVersion = 1 * 10000 + 0 * 100 + 0;

// N rounded up to a multiple of 64: row pitch of the backward workspace vectors,
// which the kernels load 64 positions at a time.
int round64(int N) { return (N + 63) & ~63; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool valid_dtype(int dt) { return dt == FA_FP32 || dt == FA_FP16 || dt == FA_BF16; }

// Largest grid y / z extent of a launch.
constexpr long long kMaxTiles = 65535;

// Checks shared by forward and backward. Returns FA_OK or the status to report.
int check_common(int B, int H, int Hkv, int N, int d, float scale, int causal, int dtype) {
    if (B <= 0 || H <= 0 || Hkv <= 0 || N <= 0 || d <= 0) return FA_ERR_INVALID_ARG;
    if (H % Hkv != 0) return FA_ERR_INVALID_ARG;
    if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
    if (!std::isfinite(scale)) return FA_ERR_INVALID_ARG;
    if (!valid_dtype(dtype)) return FA_ERR_INVALID_ARG;
    if (d != 16 && d != 32 && d != 64 && d != 128 && d != 256) return FA_ERR_UNSUPPORTED;
    // element offsets of one row-block are computed in 64 bits, but per-head row
    // counts, lse indices and grid sizes are 32-bit
    const long long rows = (long long)B * N;
    if (rows * H >= (1ll << 31) || rows * Hkv >= (1ll << 31)) return FA_ERR_INVALID_ARG;
    // query and key tiles run along grid z (at most 65535 blocks): 128 rows per
    // block in the smallest 16-bit tile, 64 in the fp32 forward
    if (N > kMaxTiles * (dtype == FA_FP32 ? 64 : 128) || B > kMaxTiles) return FA_ERR_INVALID_ARG;
    return FA_OK;
}

fa::Args make_args(const void* q, const void* k, const void* v, int B, int H, int Hkv, int N, float scale,
                   const float* slopes, const int* cu) {
    fa::Args a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.slopes = slopes;
    a.cu = cu;
    a.B = B;
    a.H = H;
    a.Hkv = Hkv;
    a.N = N;
    a.G = H / Hkv;
    a.N64 = round64(N);
    a.scale = scale;
    a.scale_log2 = scale * 1.4426950408889634f;
    a.wl = a.wr = fa::kNoWindow;
    return a;
}

// Head dim of the 16-bit kernel instance that runs a head dim: 16 runs in the
// 32 instances with Args::dl = 16 (zero-padded tiles and fragments).
int kernel_d(int d) { return d == 16 ? 32 : d; }

// Sliding window and softcapping as the kernels take them (see fa::Args).
struct Masking {
    int wl = fa::kNoWindow, wr = fa::kNoWindow;
    float softcap = 0.f;  // 0: off
};

// Window bounds: -1 for an unbounded side, else >= 0; softcap: 0 (off) or a
// finite positive cap. False for anything else.
bool make_masking(int window_left, int window_right, float softcap, Masking& mk) {
    if (window_left < -1 || window_right < -1) return false;
    if (!(softcap >= 0.f) || !std::isfinite(softcap)) return false;
    mk.wl = (window_left < 0 || window_left >= fa::kNoWindow) ? fa::kNoWindow : window_left;
    mk.wr = (window_right < 0 || window_right >= fa::kNoWindow) ? fa::kNoWindow : window_right;
    mk.softcap = softcap;
    return true;
}

void set_masking(fa::Args& a, const Masking& mk, float scale) {
    a.wl = mk.wl;
    a.wr = mk.wr;
    if (mk.softcap > 0.f) {
        a.cap_in = scale / mk.softcap;
        a.cap_out = mk.softcap * 1.4426950408889634f;
    }
}

// Dropout arguments as the kernels take them. `on` is false when nothing is
// dropped (K = 256), which runs the instances without dropout.
struct Dropout {
    bool on = false;
    uint32_t seed_lo = 0, seed_hi = 0, offset = 0, keep_k = 256;
    float scale = 1.f;
};

// K = round(256 (1 - p_drop)), kept when the random byte is below K; false for
// p_drop outside [0, 1) or rounding to K = 0.
bool make_dropout(float p_drop, unsigned long long seed, unsigned int offset, Dropout& dr) {
    if (!(p_drop >= 0.f && p_drop < 1.f)) return false;
    const int K = (int)std::nearbyint(256.0 * (1.0 - (double)p_drop));
    if (K < 1 || K > 256) return false;
    dr.on = K < 256;
    dr.seed_lo = (uint32_t)(seed & 0xFFFFFFFFull);
    dr.seed_hi = (uint32_t)(seed >> 32);
    dr.offset = offset;
    dr.keep_k = (uint32_t)K;
    dr.scale = (float)(256.0 / (double)K);
    return true;
}

void set_dropout(fa::Args& a, const Dropout& dr) {
    a.seed_lo = dr.seed_lo;
    a.seed_hi = dr.seed_hi;
    a.drop_offset = dr.offset;
    a.keep_k = dr.keep_k;
    a.drop_scale = dr.scale;
}

// D and lse * log2(e), fp32 each, [B, H, N64] (see round64).
size_t workspace_rows(int B, int H, int N) { return (size_t)B * (size_t)H * (size_t)round64(N); }
size_t workspace_bytes_for(int B, int H, int N) {
    return (2 * workspace_rows(B, H, N) * sizeof(float) + 255) & ~(size_t)255;
}

int fwd_impl(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Hkv, int N, int d,
             float scale, int causal, const float* alibi_slopes, const int* cu_seqlens, fa_dtype dtype,
             const Dropout& dr, void* stream, const Masking& mk = Masking{}) {
    if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
    int st = check_common(B, H, Hkv, N, d, scale, causal, (int)dtype);
    if (st != FA_OK) return st;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
        return FA_ERR_INVALID_ARG;
    if ((alibi_slopes && !aligned16(alibi_slopes)) || (cu_seqlens && !aligned16(cu_seqlens)))
        return FA_ERR_INVALID_ARG;

    fa::Args a = make_args(q, k, v, B, H, Hkv, N, scale, alibi_slopes, cu_seqlens);
    a.out = o;
    a.lse = lse;
    a.dl = d;
    set_dropout(a, dr);
    set_masking(a, mk, scale);
    const bool cap = mk.softcap > 0.f;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    hipError_t e;
    if (dtype == FA_FP32)
        e = fa::launch_fwd_f32(a, d, causal != 0, alibi_slopes != nullptr, cap, s);
    else
        e = fa::launch_fwd_mfma(a, (int)dtype, kernel_d(d), causal != 0, alibi_slopes != nullptr,
                                dr.on ? fa::kDropout : (cap ? fa::kSoftcap : fa::kPlain), s);
    return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // namespace

extern "C" {

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Hkv, int N, int d,
           float scale, int causal, const float* alibi_slopes, const int* cu_seqlens, fa_dtype dtype,
           void* stream) {
    return fwd_impl(q, k, v, o, lse, B, H, Hkv, N, d, scale, causal, alibi_slopes, cu_seqlens, dtype, Dropout{},
                    stream);
}

int fa_fwd_dropout(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Hkv, int N,
                   int d, float scale, int causal, const float* alibi_slopes, const int* cu_seqlens, fa_dtype dtype,
                   float p_drop, unsigned long long seed, unsigned int offset, void* stream) {
    Dropout dr;
    if (!make_dropout(p_drop, seed, offset, dr)) return FA_ERR_INVALID_ARG;
    if (dr.on && dtype == FA_FP32) return FA_ERR_UNSUPPORTED;
    return fwd_impl(q, k, v, o, lse, B, H, Hkv, N, d, scale, causal, alibi_slopes, cu_seqlens, dtype, dr, stream);
}

int fa_fwd_ext(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Hkv, int N, int d,
               float scale, int causal, const float* alibi_slopes, const int* cu_seqlens, fa_dtype dtype,
               int window_left, int window_right, float softcap, float p_drop, unsigned long long seed,
               unsigned int offset, void* stream) {
    Dropout dr;
    Masking mk;
    if (!make_dropout(p_drop, seed, offset, dr) || !make_masking(window_left, window_right, softcap, mk))
        return FA_ERR_INVALID_ARG;
    if (dr.on && (dtype == FA_FP32 || mk.softcap > 0.f)) return FA_ERR_UNSUPPORTED;
    return fwd_impl(q, k, v, o, lse, B, H, Hkv, N, d, scale, causal, alibi_slopes, cu_seqlens, dtype, dr, stream, mk);
}

size_t fa_bwd_workspace_size(int B, int H, int Hkv, int N, int d, int causal, int varlen, fa_dtype dtype) {
    (void)varlen;
    if (check_common(B, H, Hkv, N, d, 1.0f, causal, (int)dtype) != FA_OK) return 0;
    return workspace_bytes_for(B, H, N);
}

}  // extern "C"

namespace {

// Argument checks of the backward entry points other than the workspace.
int check_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
              void* dq, void* dk, void* dv, int B, int H, int Hkv, int N, int d, float scale, int causal,
              const float* alibi_slopes, const int* cu_seqlens, fa_dtype dtype) {
    if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return FA_ERR_INVALID_ARG;
    int st = check_common(B, H, Hkv, N, d, scale, causal, (int)dtype);
    if (st != FA_OK) return st;
    if (dtype == FA_FP32) return FA_ERR_UNSUPPORTED;
    const void* ptrs[] = {q, k, v, o, dout, lse, dq, dk, dv};
    for (const void* p : ptrs)
        if (!aligned16(p)) return FA_ERR_INVALID_ARG;
    if ((alibi_slopes && !aligned16(alibi_slopes)) || (cu_seqlens && !aligned16(cu_seqlens)))
        return FA_ERR_INVALID_ARG;
    return FA_OK;
}

// Backward workspace kept in the library for callers that cannot allocate
// (fa_bwd_noalloc): one copy per GPU, held until the process ends. Host code
// never uses the array's name as an address; each device's address comes from
// hipGetSymbolAddress, taken once with that device current.
constexpr size_t kScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

int scratch_for_current_device(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FA_ERR_LAUNCH;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return FA_ERR_LAUNCH;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return FA_OK;
}

int bwd_launch(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
               void* dq, void* dk, void* dv, int B, int H, int Hkv, int N, int d, float scale, int causal,
               const float* alibi_slopes, const int* cu_seqlens, fa_dtype dtype, void* workspace, unsigned stages,
               void* stream, const Dropout& dr = Dropout{}, const Masking& mk = Masking{}) {
    fa::Args a = make_args(q, k, v, B, H, Hkv, N, scale, alibi_slopes, cu_seqlens);
    a.o = o;
    a.dout = dout;
    a.lse_in = lse;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.dsum = reinterpret_cast<float*>(workspace);
    a.lse2 = a.dsum + workspace_rows(B, H, N);
    a.dl = d;
    set_dropout(a, dr);
    set_masking(a, mk, scale);
    const int var = dr.on ? fa::kDropout : (mk.softcap > 0.f ? fa::kSoftcap : fa::kPlain);
    hipError_t e = fa::launch_bwd(a, (int)dtype, kernel_d(d), causal != 0, alibi_slopes != nullptr, var, stages,
                                  reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

// Key ranges per (sequence, kv head) of a decode problem. num_splits = 0
// aims at one workgroup per compute unit (measured on the decode workload:
// 4 ranges per sequence and kv head streamed the caches at 5.1 TB/s, 16 at
// 4.4 and 32 at 3.6, each range adding fixed set-up, merge and partial-write
// cost) with at least 512 keys per range of an Nk-key cache; any count is
// capped at one range per 128 keys. The device cuts each sequence's own
// length into that many ranges.
constexpr int kComputeUnits = 256;

int decode_splits(int B, int H, int Hkv, int Nq, int Nk, int num_splits) {
    const int tiles = (Nk + 127) / 128;
    int S = num_splits;
    if (S <= 0) {
        const long long rgroups = ((long long)(H / Hkv) * Nq + 31) / 32;
        const long long base = (long long)Hkv * rgroups * B;
        S = (int)((kComputeUnits + base - 1) / base);
        S = std::min(S, std::max(1, Nk / 512));
    }
    return std::max(1, std::min({S, tiles, (int)kMaxTiles}));
}

// The split kernel's grid: `parts` ranges and whether they are flat ranges of
// the caches laid end to end. The automatic choice with more than one range
// per sequence goes flat (B * S equal ranges per kv head: with caches of
// different lengths, ranges of each sequence's own length leave the
// workgroups of the longest cache running alone at the end); an explicit
// count keeps `num_splits` ranges of every sequence.
void decode_plan(int B, int H, int Hkv, int Nq, int Nk, int num_splits, int& parts, int& flat) {
    const int S = decode_splits(B, H, Hkv, Nq, Nk, num_splits);
    flat = (num_splits == 0 && S > 1) ? 1 : 0;
    parts = flat ? B * S : S;
}

size_t decode_workspace_bytes(int B, int H, int Nq, int d, int splits) {
    if (splits <= 1) return 0;
    const size_t rows = (size_t)B * H * Nq * splits;
    return (rows * (size_t)(d + 1) * sizeof(float) + 255) & ~(size_t)255;
}

int check_decode(int B, int H, int Hkv, int Nq, int Nk, int d, float scale, int causal, int dtype) {
    if (B <= 0 || H <= 0 || Hkv <= 0 || Nq <= 0 || Nk <= 0 || d <= 0) return FA_ERR_INVALID_ARG;
    if (H % Hkv != 0 || (causal != 0 && causal != 1) || !std::isfinite(scale)) return FA_ERR_INVALID_ARG;
    if (!valid_dtype(dtype)) return FA_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    if (dtype == FA_FP32) return FA_ERR_UNSUPPORTED;
    if ((long long)B * Nk * Hkv >= (1ll << 31) || (long long)B * Nq * H >= (1ll << 31)) return FA_ERR_INVALID_ARG;
    if (B > kMaxTiles) return FA_ERR_INVALID_ARG;
    return FA_OK;
}

}  // namespace

extern "C" {

size_t fa_kvcache_workspace_size(int B, int H, int Hkv, int Nq, int Nk, int d, int num_splits) {
    if (check_decode(B, H, Hkv, Nq, Nk, d, 1.0f, 0, FA_BF16) != FA_OK || num_splits < 0) return 0;
    int parts, flat;
    decode_plan(B, H, Hkv, Nq, Nk, num_splits, parts, flat);
    return decode_workspace_bytes(B, H, Nq, d, parts);
}

int fa_fwd_kvcache(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                   const int* cache_seqlens, int B, int H, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                   const float* alibi_slopes, fa_dtype dtype, int num_splits, void* workspace,
                   size_t workspace_bytes, void* stream) {
    if (!q || !k_cache || !v_cache || !o || !lse || !cache_seqlens || num_splits < 0) return FA_ERR_INVALID_ARG;
    int st = check_decode(B, H, Hkv, Nq, Nk, d, scale, causal, (int)dtype);
    if (st != FA_OK) return st;
    const void* ptrs[] = {q, k_cache, v_cache, o, lse};
    for (const void* p : ptrs)
        if (!aligned16(p)) return FA_ERR_INVALID_ARG;
    if (!aligned16(cache_seqlens) || (alibi_slopes && !aligned16(alibi_slopes))) return FA_ERR_INVALID_ARG;
    fa::DecodeArgs a{};
    decode_plan(B, H, Hkv, Nq, Nk, num_splits, a.splits, a.flat);
    const size_t need = decode_workspace_bytes(B, H, Nq, d, a.splits);
    if (need > 0 && (!workspace || !aligned16(workspace) || workspace_bytes < need)) return FA_ERR_WORKSPACE;
    a.q = q;
    a.k = k_cache;
    a.v = v_cache;
    a.o = o;
    a.lse = lse;
    a.seqlens = cache_seqlens;
    a.slopes = alibi_slopes;
    a.part_o = reinterpret_cast<float*>(workspace);
    a.part_lse = need > 0 ? a.part_o + (size_t)B * H * Nq * a.splits * d : nullptr;
    a.B = B;
    a.H = H;
    a.Hkv = Hkv;
    a.Nq = Nq;
    a.Nk = Nk;
    a.scale_log2 = scale * 1.4426950408889634f;
    hipError_t e = fa::launch_decode(a, (int)dtype, d, causal != 0, alibi_slopes != nullptr,
                                     reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

int fa_bwd_stages(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                  void* dq, void* dk, void* dv, int B, int H, int Hkv, int N, int d, float scale, int causal,
                  const float* alibi_slopes, const int* cu_seqlens, fa_dtype dtype, void* workspace,
                  size_t workspace_bytes, unsigned stages, void* stream) {
    if (stages == 0 || (stages & ~(unsigned)FA_BWD_ALL) != 0) return FA_ERR_INVALID_ARG;
    int st = check_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, H, Hkv, N, d, scale, causal, alibi_slopes, cu_seqlens,
                       dtype);
    if (st != FA_OK) return st;
    if (!workspace || !aligned16(workspace) || workspace_bytes < workspace_bytes_for(B, H, N))
        return FA_ERR_WORKSPACE;

    return bwd_launch(q, k, v, o, dout, lse, dq, dk, dv, B, H, Hkv, N, d, scale, causal, alibi_slopes, cu_seqlens,
                      dtype, workspace, stages, stream);
}

int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                   void* dq, void* dk, void* dv, int B, int H, int Hkv, int N, int d, float scale, int causal,
                   const float* alibi_slopes, const int* cu_seqlens, fa_dtype dtype, void* stream) {
    int st = check_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, H, Hkv, N, d, scale, causal, alibi_slopes, cu_seqlens,
                       dtype);
    if (st != FA_OK) return st;
    if (workspace_bytes_for(B, H, N) > kScratchBytes) return FA_ERR_SCRATCH;
    void* ws = nullptr;
    st = scratch_for_current_device(&ws);
    if (st != FA_OK) return st;
    return bwd_launch(q, k, v, o, dout, lse, dq, dk, dv, B, H, Hkv, N, d, scale, causal, alibi_slopes, cu_seqlens,
                      dtype, ws, FA_BWD_ALL, stream);
}

size_t fa_bwd_noalloc_max_bytes(void) { return kScratchBytes; }

int fa_bwd_dropout(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                   void* dq, void* dk, void* dv, int B, int H, int Hkv, int N, int d, float scale, int causal,
                   const float* alibi_slopes, const int* cu_seqlens, fa_dtype dtype, float p_drop,
                   unsigned long long seed, unsigned int offset, void* workspace, size_t workspace_bytes,
                   void* stream) {
    Dropout dr;
    if (!make_dropout(p_drop, seed, offset, dr)) return FA_ERR_INVALID_ARG;
    int st = check_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, H, Hkv, N, d, scale, causal, alibi_slopes, cu_seqlens,
                       dtype);
    if (st != FA_OK) return st;
    if (!workspace || !aligned16(workspace) || workspace_bytes < workspace_bytes_for(B, H, N))
        return FA_ERR_WORKSPACE;
    return bwd_launch(q, k, v, o, dout, lse, dq, dk, dv, B, H, Hkv, N, d, scale, causal, alibi_slopes, cu_seqlens,
                      dtype, workspace, FA_BWD_ALL, stream, dr);
}

int fa_bwd_ext(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
               void* dq, void* dk, void* dv, int B, int H, int Hkv, int N, int d, float scale, int causal,
               const float* alibi_slopes, const int* cu_seqlens, fa_dtype dtype, int window_left, int window_right,
               float softcap, float p_drop, unsigned long long seed, unsigned int offset, void* workspace,
               size_t workspace_bytes, void* stream) {
    Dropout dr;
    Masking mk;
    if (!make_dropout(p_drop, seed, offset, dr) || !make_masking(window_left, window_right, softcap, mk))
        return FA_ERR_INVALID_ARG;
    int st = check_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, H, Hkv, N, d, scale, causal, alibi_slopes, cu_seqlens,
                       dtype);
    if (st != FA_OK) return st;
    if (dr.on && mk.softcap > 0.f) return FA_ERR_UNSUPPORTED;
    if (!workspace || !aligned16(workspace) || workspace_bytes < workspace_bytes_for(B, H, N))
        return FA_ERR_WORKSPACE;
    return bwd_launch(q, k, v, o, dout, lse, dq, dk, dv, B, H, Hkv, N, d, scale, causal, alibi_slopes, cu_seqlens,
                      dtype, workspace, FA_BWD_ALL, stream, dr, mk);
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse, void* dq,
           void* dk, void* dv, int B, int H, int Hkv, int N, int d, float scale, int causal,
           const float* alibi_slopes, const int* cu_seqlens, fa_dtype dtype, void* workspace,
           size_t workspace_bytes, void* stream) {
    return fa_bwd_stages(q, k, v, o, dout, lse, dq, dk, dv, B, H, Hkv, N, d, scale, causal, alibi_slopes,
                         cu_seqlens, dtype, workspace, workspace_bytes, FA_BWD_ALL, stream);
}

int fa_fp8_v_keys(int N) { return N > 0 && N <= (1 << 30) ? fa::fp8_keys_padded(N) : 0; }

int fa_quantize_fp8_qk(const void* x, unsigned char* codes, float* scales, int B, int N, int H, int d,
                       const unsigned long long* hadamard_signs, fa_dtype dtype, void* stream) {
    if (!x || !codes || !scales || B <= 0 || N <= 0 || H <= 0 || d <= 0) return FA_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(codes) || !aligned16(scales)) return FA_ERR_INVALID_ARG;
    if (dtype != FA_FP16 && dtype != FA_BF16) return valid_dtype(dtype) ? FA_ERR_UNSUPPORTED : FA_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    if ((long long)B * N * H >= (1ll << 31) || N > kMaxTiles * 128 || B > kMaxTiles) return FA_ERR_INVALID_ARG;
    hipError_t e = fa::launch_quant_qk(x, codes, scales, B, N, H, d, hadamard_signs, (int)dtype,
                                       reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

int fa_quantize_fp8_v(const void* v, unsigned char* codes_t, float* scales, int B, int N, int Hkv, int d,
                      fa_dtype dtype, void* stream) {
    if (!v || !codes_t || !scales || B <= 0 || N <= 0 || Hkv <= 0 || d <= 0) return FA_ERR_INVALID_ARG;
    if (!aligned16(v) || !aligned16(codes_t) || !aligned16(scales)) return FA_ERR_INVALID_ARG;
    if (dtype != FA_FP16 && dtype != FA_BF16) return valid_dtype(dtype) ? FA_ERR_UNSUPPORTED : FA_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    if ((long long)B * N * Hkv >= (1ll << 31) || N > kMaxTiles * 128 || B > kMaxTiles) return FA_ERR_INVALID_ARG;
    hipError_t e = fa::launch_quant_v(v, codes_t, scales, B, N, Hkv, d, (int)dtype,
                                      reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

int fa_fwd_fp8(const unsigned char* q, const unsigned char* k, const unsigned char* v_t, const float* q_scales,
               const float* k_scales, const float* v_scales, void* o, float* lse, int B, int H, int Hkv, int N,
               int d, float scale, int causal, int rotated, fa_dtype out_dtype, void* stream) {
    const void* ptrs[] = {q, k, v_t, q_scales, k_scales, v_scales, o, lse};
    for (const void* p : ptrs)
        if (!p || !aligned16(p)) return FA_ERR_INVALID_ARG;
    if (B <= 0 || H <= 0 || Hkv <= 0 || N <= 0 || d <= 0 || H % Hkv != 0) return FA_ERR_INVALID_ARG;
    if ((causal != 0 && causal != 1) || (rotated != 0 && rotated != 1) || !std::isfinite(scale))
        return FA_ERR_INVALID_ARG;
    if (out_dtype != FA_FP16 && out_dtype != FA_BF16)
        return valid_dtype(out_dtype) ? FA_ERR_UNSUPPORTED : FA_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    if ((long long)B * N * H >= (1ll << 31) || N > kMaxTiles * 128 || B > kMaxTiles) return FA_ERR_INVALID_ARG;
    const float s_eff = rotated ? scale / (float)d : scale;  // exact: d is a power of two
    hipError_t e = fa::launch_fwd_fp8(q, k, v_t, q_scales, k_scales, v_scales, o, lse, B, H, Hkv, N, d,
                                      s_eff * 1.4426950408889634f, causal != 0, (int)out_dtype,
                                      reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

const char* fa_strerror(int status) {
    switch (status) {
        case FA_OK: return "success";
        case FA_ERR_INVALID_ARG: return "invalid argument";
        case FA_ERR_UNSUPPORTED:
            return "unsupported configuration (head dim must be 16, 32, 64, 128 or 256, and 64 or 128 for decode "
                   "and fp8; fp32 is forward only and without dropout; dropout and softcapping do not combine; "
                   "fp8 takes and returns fp16 or bf16)";
        case FA_ERR_WORKSPACE: return "workspace missing, misaligned or smaller than fa_bwd_workspace_size()";
        case FA_ERR_LAUNCH: return "kernel launch failed";
        case FA_ERR_SCRATCH: return "problem needs more backward scratch than fa_bwd_noalloc holds (fa_bwd_noalloc_max_bytes())";
        default: return "unknown status";
    }
}

int fa_version(void) { return kVersion; }

}  // extern "C"
