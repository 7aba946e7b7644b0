// Launch arguments shared by the C-ABI layer (fa_api.hip) and the kernel files.
// Host-visible only; no kernel code here.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace fa {

// One attention problem as the kernels see it. Pointers are device memory in
// the layouts documented in include/fa.h; `cu` is NULL for dense inputs.
struct Args {
    const void* q;
    const void* k;
    const void* v;
    const void* o;     // forward output / backward input
    const void* dout;  // backward only
    void* out;         // fa_fwd: O.  (backward writes dq/dk/dv below)
    float* lse;        // [B, H, N]
    const float* lse_in;
    void* dq;
    void* dk;
    void* dv;
    float* dsum;       // backward workspace: D_i = dO_i . O_i, [B, H, N64]
    float* lse2;       // backward workspace: lse * log2(e), [B, H, N64]
    const float* slopes;
    const int* cu;
    int B, H, Hkv, N, G;
    int N64;           // N rounded up to a multiple of 64: row pitch of the workspace vectors
    float scale;       // softmax scale
    float scale_log2;  // scale * log2(e)
    // dropout (instances with dropout only): Philox key, counter word 3, keep
    // threshold K (a probability is kept when its random byte is below K) and
    // the factor 256 / K applied to kept probabilities
    uint32_t seed_lo, seed_hi, drop_offset, keep_k;
    float drop_scale;
    // sliding window: key j is visible from query i when i - wl <= j <= i + wr
    // (positions within a sequence; kNoWindow for an unbounded side; causal
    // instances use wr = 0 whatever is stored here)
    int wl, wr;
    // softcapping (instances with it only): the scaled score u becomes
    // cap tanh(u / cap); the kernels take tanh(s * cap_in) with s the raw dot
    // product (cap_in = scale / cap) and scale it by cap_out = cap * log2(e)
    float cap_in, cap_out;
    // head dim as stored in memory: equal to the kernel's tile head dim, except
    // for head dim 16, which runs in the head-dim-32 instances with the upper
    // 16 columns of every staged tile and register fragment zero (row pitches,
    // loads and stores use this value)
    int dl;
};

// An unbounded window side: larger than any position difference, small enough
// that position +- kNoWindow stays inside int32.
constexpr int kNoWindow = 1 << 30;

// A decode problem: Nq new queries per sequence against a cache of up to Nk
// keys (seqlens[b] valid); each sequence's keys are cut into `splits` ranges.
struct DecodeArgs {
    const void* q;        // [B, Nq, H, d]
    const void* k;        // [B, Nk, Hkv, d]
    const void* v;
    void* o;              // [B, Nq, H, d]
    float* lse;           // [B, H, Nq]
    const int* seqlens;   // [B], device
    const float* slopes;  // [H] or NULL
    float* part_o;        // splits > 1 or flat: [B, H, Nq, splits, d] fp32
    float* part_lse;      //                     [B, H, Nq, splits]
    int B, H, Hkv, Nq, Nk, splits;
    int flat;             // 1: `splits` equal ranges of the caches laid end to end
                          // (per kv head), 0: `splits` ranges of each sequence
    float scale_log2;
};

// Score variants beyond mask and bias: one per compiled instance set.
enum Variant : int { kPlain = 0, kDropout = 1, kSoftcap = 2 };

// Each returns hipSuccess or the launch error. `dtype` follows fa_dtype;
// `var` selects the instances with dropout (16-bit only) or softcapping.
hipError_t launch_fwd_mfma(const Args& a, int dtype, int d, bool causal, bool alibi, int var, hipStream_t s);
hipError_t launch_fwd_f32(const Args& a, int d, bool causal, bool alibi, bool cap, hipStream_t s);
// The dK/dV launch alone (built in its own translation unit with its own flags).
hipError_t launch_bwd_dkdv(const Args& a, int dtype, int d, bool causal, bool alibi, int var, hipStream_t s);
// `stages`: bit 0 = D pre-pass, bit 1 = dK/dV, bit 2 = dQ (enqueued in that order).
hipError_t launch_bwd(const Args& a, int dtype, int d, bool causal, bool alibi, int var, unsigned stages,
                      hipStream_t s);
hipError_t launch_decode(const DecodeArgs& a, int dtype, int d, bool causal, bool alibi, hipStream_t s);

// FP8 path: keys of the transposed V codes, padded to whole 128-key tiles.
inline int fp8_keys_padded(int N) { return (N + 127) & ~127; }
hipError_t launch_quant_qk(const void* x, uint8_t* codes, float* scales, int B, int N, int H, int d,
                           const unsigned long long* signs, int dtype, hipStream_t s);
hipError_t launch_quant_v(const void* v, uint8_t* codes_t, float* scales, int B, int N, int Hkv, int d, int dtype,
                          hipStream_t s);
hipError_t launch_fwd_fp8(const uint8_t* q, const uint8_t* k, const uint8_t* vt, const float* qs, const float* ks,
                          const float* vs, void* out, float* lse, int B, int H, int Hkv, int N, int d,
                          float scale_log2, bool causal, int out_dtype, hipStream_t s);

}  // namespace fa
