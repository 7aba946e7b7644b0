/*
 * libfa: exact tiled scaled-dot-product attention (forward and backward) for
 * AMD Instinct MI355X (gfx950).
 *
 * Operation (page "FlashAttention: Faster Attention Without Dropping a Single
 * Interaction", Method Deep Dive, Key design 1): for every batch entry or
 * packed sequence b and query head h, with kv head g = h / (H / Hkv),
 *
 *     S_ij = scale * <q_i, k_j> + beta_ij,   P = softmax_rows(S),   O = P V,
 *
 * where beta_ij = -alibi_slopes[h] * |i - j| when slopes are given (0 otherwise)
 * and, when causal, keys j > i are removed. The forward also stores the row
 * statistic lse_i = m_i + ln(sum_j exp(S_ij - m_i)) (natural log; the saved-state
 * table of Key design 2), which is all the backward needs to rebuild P (Key
 * design 3). The N x N matrices S and P never reach device memory.
 *
 * Layouts (row-major, contiguous, element strides implied by the sizes):
 *   dense   q, o, dout, dq : [B, N, H, d]       k, v, dk, dv : [B, N, Hkv, d]
 *   packed  q, o, dout, dq : [total, H, d]      k, v, dk, dv : [total, Hkv, d]
 *           (packed when cu_seqlens != NULL; total = cu_seqlens[B])
 *   lse                    : float [B, H, N] in both modes; for packed inputs
 *                            entries at positions >= a sequence's length are
 *                            left untouched.
 *   cu_seqlens             : int32 [B + 1], device memory, cu_seqlens[0] = 0,
 *                            non-decreasing; every length must be <= N (N is
 *                            the maximum sequence length in packed mode).
 *                            The lengths live in device memory and are not
 *                            checked on the host: a length above N is
 *                            truncated to N (its rows past N are neither read
 *                            nor written) and a negative one is treated as
 *                            empty, and the call still returns FA_OK.
 *   alibi_slopes           : float [H], device memory, or NULL for no bias.
 *
 * Element types (fa_dtype): FA_BF16 and FA_FP16 store q, k, v, o, dout, dq, dk,
 * dv in that 16-bit type and accumulate in fp32; FA_FP32 stores fp32 and
 * computes in fp32 (forward only).
 *
 * Ownership and execution: every pointer is caller-owned device memory. The
 * library never allocates, frees or synchronises; all work is enqueued on
 * `stream` (a hipStream_t, NULL for the default stream) and the call returns
 * at once. Inputs are read-only; outputs must not alias inputs or each other.
 * Base pointers must be 16-byte aligned. Apart from fa_bwd_noalloc's scratch
 * (see there) the library keeps no mutable global state, so concurrent calls
 * from several host threads are safe.
 *
 * Errors: every entry returns FA_OK (0) or a negative fa_status. All argument
 * checks run before any launch; a call that fails them enqueues nothing and
 * writes nothing. FA_ERR_LAUNCH reports a failure of the launch itself.
 */
#ifndef LIBFA_FA_H
#define LIBFA_FA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fa_dtype {
    FA_FP32 = 0,
    FA_FP16 = 1,
    FA_BF16 = 2
} fa_dtype;

typedef enum fa_status {
    FA_OK = 0,
    FA_ERR_INVALID_ARG = -1, /* null pointer, bad size, H % Hkv != 0, non-finite scale, misalignment;
                                sizes: B * N * H < 2^31, B <= 65535, N <= 8388480 (65535 tiles of 128
                                rows; 4194240 for FA_FP32) */
    FA_ERR_UNSUPPORTED = -2, /* head dim or type combination not built (see fa_strerror) */
    FA_ERR_WORKSPACE = -3,   /* workspace missing or smaller than fa_bwd_workspace_size() */
    FA_ERR_LAUNCH = -4,      /* the kernel launch itself failed */
    FA_ERR_SCRATCH = -5      /* fa_bwd_noalloc: problem larger than its built-in scratch */
} fa_status;

/*
 * Forward pass: O and lse from Q, K, V (Key design 1 and 2 of the page above;
 * the tiled loop of "FlashAttention: The Algorithm That Beat the Memory Wall",
 * "A Tile, a Register File, and a Trick Called Online Softmax"; packed
 * sequences as in its "Varlen Is the Quiet Superpower").
 *
 *   B, H, Hkv, N, d : batch (number of sequences), query heads, kv heads
 *                     (H % Hkv == 0), sequence length (maximum length when
 *                     packed), head dimension (16, 32, 64, 128 or 256; the
                     usage contract's list, "paper lists 16/32/64/128", up to
                     256).
 *   scale           : multiplies Q K^T before the softmax (1/sqrt(d) is usual).
 *   causal          : 0 or 1; 1 keeps key j <= query i.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int Hkv, int N, int d, float scale, int causal,
           const float* alibi_slopes, const int* cu_seqlens, fa_dtype dtype,
           void* stream);

/*
 * Forward pass with dropout on the attention probabilities: the fused dropout
 * of the page's Key design 1 stage table, whose mask the backward regenerates
 * from the saved generator state (Key design 3). The softmax and lse use
 * every score; the probabilities that multiply V are dropped and the kept
 * ones scaled, O = (P o M * 256 / K) V.
 *
 *   p_drop : drop probability in [0, 1). K = round(256 (1 - p_drop)) must be
 *            at least 1; a probability is kept when its random byte is below
 *            K (the effective keep rate is K / 256, and the factor 256 / K
 *            keeps every expectation unchanged). K = 256 (p_drop < 1/512)
 *            drops nothing and equals fa_fwd.
 *   seed   : 64-bit key of the generator; offset: its 32-bit counter word 3
 *            (advance it between calls that share a seed).
 *
 * Mask M for sequence b, query head h, query position i and key position j
 * (positions within the sequence): the byte (j % 4) (little-endian) of output
 * word (j % 32) / 8 of Philox-4x32 with 10 rounds (Salmon, Moraes, Dror, Shaw,
 * "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11) under key
 * (seed mod 2^32, seed / 2^32) at counter
 * (2 (j / 32) + (j / 4) % 2, i, b H + h, offset). Other arguments, layouts
 * and errors as fa_fwd; FA_FP32 with dropout is FA_ERR_UNSUPPORTED, and an
 * out-of-range p_drop is FA_ERR_INVALID_ARG.
 */
int fa_fwd_dropout(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int H, int Hkv, int N, int d, float scale, int causal,
                   const float* alibi_slopes, const int* cu_seqlens, fa_dtype dtype,
                   float p_drop, unsigned long long seed, unsigned int offset,
                   void* stream);

/*
 * Forward pass with the mask variants of the page's usage contract (its mask
 * row names sliding window, ALiBi and softcapping; the formulas are this
 * library's reading) together with dropout as in fa_fwd_dropout.
 *
 *   window_left, window_right : key j is visible from query i when
 *            i - window_left <= j <= i + window_right (positions within the
 *            sequence); -1 leaves that side unbounded. causal = 1 still keeps
 *            j <= i. Values below -1 are FA_ERR_INVALID_ARG.
 *   softcap : 0 for none; else the scaled score u = scale * <q_i, k_j> becomes
 *            softcap * tanh(u / softcap) before the ALiBi bias and the masks.
 *            Must be finite and >= 0.
 *   p_drop, seed, offset : as fa_fwd_dropout (p_drop = 0: no dropout).
 *
 * The window also bounds the work: only key tiles some query can see are read.
 * Every query sees at least its own key, so lse is always finite. Dropout
 * together with softcapping, or dropout with FA_FP32, is FA_ERR_UNSUPPORTED.
 * Other arguments, layouts and errors as fa_fwd; with both windows -1 and
 * softcap = 0 the result equals fa_fwd_dropout's.
 */
int fa_fwd_ext(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int H, int Hkv, int N, int d, float scale, int causal,
               const float* alibi_slopes, const int* cu_seqlens, fa_dtype dtype,
               int window_left, int window_right, float softcap,
               float p_drop, unsigned long long seed, unsigned int offset,
               void* stream);

/*
 * Decode over a key/value cache: attention of Nq new queries per sequence
 * against a cache of keys and values (the inference workload the page's
 * Limitations section sets apart from training, "long context and inference
 * remain unsolved"). The keys are split into ranges processed in parallel,
 * and the partial states merge exactly (Key design 2: the (m, l, O) state of
 * disjoint key sets combines with m = max m_s, l = sum l_s e^(m_s - m)).
 *
 *   q             : [B, Nq, H, d]; o : [B, Nq, H, d] (written); lse : float
 *                   [B, H, Nq] (written; -inf for a query that sees no key).
 *   k_cache, v_cache : [B, Nk, Hkv, d]; sequence b uses its first
 *                   cache_seqlens[b] rows.
 *   cache_seqlens : int32 [B], device memory: L_b, the valid keys of sequence
 *                   b, the new tokens included; lengths above Nk are treated
 *                   as Nk and negative ones as 0 (not checked on the host).
 *   causal        : 1 aligns the mask to the end of the cache: query t sits at
 *                   position L_b - Nq + t and keeps keys j <= L_b - Nq + t.
 *   alibi_slopes  : float [H] or NULL; the bias is -slope_h |position - j|.
 *   num_splits    : key ranges per sequence and kv head (each sequence's
 *                   L_b keys are cut into that many ranges of ceil(L_b / S)
 *                   keys rounded up to 32); 0 lets the library pick from the
 *                   sizes: about one workgroup per compute unit, at least
 *                   512 keys per range of an Nk-key cache, and, when that
 *                   gives S > 1 ranges per sequence, B * S equal ranges per
 *                   kv head over the B caches laid end to end (a range may
 *                   cover the end of one sequence and the start of the
 *                   next), so caches of different lengths take equal work
 *                   per workgroup. At most one range per 128 keys of Nk is
 *                   used per sequence.
 *   workspace     : fp32 partial results when more than one range is used,
 *                   fa_kvcache_workspace_size(...) bytes (0: NULL allowed).
 *
 * FA_BF16 and FA_FP16 only (FA_FP32 is FA_ERR_UNSUPPORTED); d in {64, 128}.
 * Other conventions (alignment, asynchrony, errors) as fa_fwd.
 */
size_t fa_kvcache_workspace_size(int B, int H, int Hkv, int Nq, int Nk, int d,
                                 int num_splits);

int fa_fwd_kvcache(const void* q, const void* k_cache, const void* v_cache, void* o,
                   float* lse, const int* cache_seqlens, int B, int H, int Hkv,
                   int Nq, int Nk, int d, float scale, int causal,
                   const float* alibi_slopes, fa_dtype dtype, int num_splits,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * Bytes of device scratch fa_bwd needs for these sizes: the per-row
 * D_i = dO_i . O_i of Key design 3 and the row statistic rescaled to log2
 * units, both fp32 [B, H, N64] with N64 = N rounded up to a multiple of 64
 * (2 * 4 * B * H * N64 bytes, rounded up to 256). Linear in N. Returns 0 for
 * invalid sizes.
 */
size_t fa_bwd_workspace_size(int B, int H, int Hkv, int N, int d, int causal,
                             int varlen, fa_dtype dtype);

/*
 * Backward pass: dQ, dK, dV of the loss sum(O * dout) by recomputing the score
 * tiles from lse (Key design 3): D_i = dO_i . O_i, dS = P o (dP - D),
 * dV = P^T dO, dQ = scale * dS K, dK = scale * dS^T Q. `o` and `lse` must come
 * from fa_fwd on the same inputs and arguments. dq, dk and dv are overwritten;
 * dk and dv of a kv head hold the sum over its H / Hkv query heads. No atomics
 * are used, so results are bitwise reproducible run to run. ALiBi slopes get no
 * gradient. Only FA_BF16 and FA_FP16 are supported.
 *
 *   workspace, workspace_bytes : caller-owned device scratch of at least
 *                                fa_bwd_workspace_size(...) bytes, 16-byte aligned.
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o,
           const void* dout, const float* lse, void* dq, void* dk, void* dv,
           int B, int H, int Hkv, int N, int d, float scale, int causal,
           const float* alibi_slopes, const int* cu_seqlens, fa_dtype dtype,
           void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward pass of fa_fwd_dropout: the same mask is regenerated from
 * (p_drop, seed, offset), which must equal the forward call's. dV takes the
 * dropped probabilities, dV = (P o M * 256 / K)^T dout, and the gradient
 * reaching P is (dout V^T) o M * 256 / K; D_i = dout_i . O_i still holds with
 * the dropped O. Other arguments, workspace, results and errors as fa_bwd.
 */
int fa_bwd_dropout(const void* q, const void* k, const void* v, const void* o,
                   const void* dout, const float* lse, void* dq, void* dk, void* dv,
                   int B, int H, int Hkv, int N, int d, float scale, int causal,
                   const float* alibi_slopes, const int* cu_seqlens, fa_dtype dtype,
                   float p_drop, unsigned long long seed, unsigned int offset,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward pass of fa_fwd_ext: the same window, softcap and dropout arguments
 * (`o` and `lse` from fa_fwd_ext with the same values). With softcapping the
 * gradient reaching the scaled score is dS * (1 - tanh^2(u / softcap)), so dQ
 * and dK carry that factor. Workspace, errors and guarantees as fa_bwd.
 */
int fa_bwd_ext(const void* q, const void* k, const void* v, const void* o,
               const void* dout, const float* lse, void* dq, void* dk, void* dv,
               int B, int H, int Hkv, int N, int d, float scale, int causal,
               const float* alibi_slopes, const int* cu_seqlens, fa_dtype dtype,
               int window_left, int window_right, float softcap,
               float p_drop, unsigned long long seed, unsigned int offset,
               void* workspace, size_t workspace_bytes, void* stream);

/*
 * The three launches of fa_bwd, selectable one by one, for callers that split
 * them across streams (dK/dV and dQ are independent once D is written) or time
 * them separately. `stages` is a bitwise OR of the fa_bwd_stage values; the
 * selected stages are enqueued on `stream` in the order PREP, DKDV, DQ. DKDV
 * and DQ read the D values that PREP wrote into the same workspace, so the
 * caller orders PREP before them. fa_bwd(...) equals fa_bwd_stages(...,
 * FA_BWD_ALL, ...). Same arguments, checks and errors as fa_bwd; a zero or
 * unknown mask is FA_ERR_INVALID_ARG.
 */
typedef enum fa_bwd_stage {
    FA_BWD_PREP = 1, /* D_i = dO_i . O_i into the workspace (reads o, dout) */
    FA_BWD_DKDV = 2, /* dk, dv (reads q, k, v, dout, lse, D) */
    FA_BWD_DQ = 4,   /* dq (reads q, k, v, dout, lse, D) */
    FA_BWD_ALL = 7
} fa_bwd_stage;

int fa_bwd_stages(const void* q, const void* k, const void* v, const void* o,
                  const void* dout, const float* lse, void* dq, void* dk, void* dv,
                  int B, int H, int Hkv, int N, int d, float scale, int causal,
                  const float* alibi_slopes, const int* cu_seqlens, fa_dtype dtype,
                  void* workspace, size_t workspace_bytes, unsigned stages,
                  void* stream);

/*
 * fa_bwd without the workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc. Same arguments, checks, results and errors as fa_bwd
 * otherwise. The scratch (D and the rescaled row statistic, the same bytes
 * fa_bwd_workspace_size reports) lives in a static device array inside the
 * library: one copy per GPU of fa_bwd_noalloc_max_bytes() = 16 MiB, held until
 * the process ends, i.e. problems with 8 * B * H * N64 <= 16 MiB (N64 = N
 * rounded up to 64); larger ones return FA_ERR_SCRATCH before any launch.
 * The call allocates and frees nothing; the first call on each device looks up
 * that device's copy of the array once (hipGetSymbolAddress, under a lock).
 * Every call on one GPU uses the same array: calls that overlap in time on one
 * GPU (different streams, or several host threads without ordering) race and
 * must be serialised by the caller. Nothing in the array needs to start at
 * zero: each call writes every entry it reads before reading it.
 */
int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                   const void* dout, const float* lse, void* dq, void* dk, void* dv,
                   int B, int H, int Hkv, int N, int d, float scale, int causal,
                   const float* alibi_slopes, const int* cu_seqlens, fa_dtype dtype,
                   void* stream);

/* Size in bytes of fa_bwd_noalloc's per-GPU scratch array. */
size_t fa_bwd_noalloc_max_bytes(void);

/* Static, human-readable text for a status code (never NULL, never freed). */
const char* fa_strerror(int status);

/* Library version as MAJOR * 10000 + MINOR * 100 + PATCH. */
int fa_version(void);

/*
 * FP8 forward: attention computed on e4m3 codes with power-of-two block
 * scales, optionally after a random-sign Walsh-Hadamard rotation of Q and K
 * (page "FlashAttention: Faster Attention Without Dropping a Single
 * Interaction", Method Deep Dive, Key design 4, the FP8 row of the version
 * table: block quantization and incoherent processing; its Limitations
 * section, "Numerical exactness, low precision, and reproducibility", gives
 * the error of FP8 against an exact reference with and without them).
 *
 * Format: OCP e4m3 "fn" (bias 7, largest finite 448, round to nearest even).
 * A block's scale is 2^e, the smallest power of two with amax <= 448 2^e
 * (e >= -127; an all-zero block gets 2^0), so a code is the rounding of
 * x / 2^e alone and x ~ decode(code) * 2^e. Inputs must be finite: a NaN or
 * infinity in a block gives that block undefined codes and scale (not
 * checked; the values are in device memory).
 *
 * Three calls: quantize Q and K (fa_quantize_fp8_qk), quantize V
 * (fa_quantize_fp8_v), then fa_fwd_fp8. Every buffer is caller-owned device
 * memory, 16-byte aligned; calls enqueue on `stream` and return at once.
 * FA_FP16 / FA_BF16 inputs and outputs; d in {64, 128} (other head dims and
 * FA_FP32 are FA_ERR_UNSUPPORTED). No ALiBi, window, packed sequences or
 * backward on this path.
 *
 * fa_quantize_fp8_qk: x [B, N, H, d] (H = Hkv for K) -> codes uint8
 *   [B, N, H, d] and scales float [B, H, ceil(N / 128)]: one scale per
 *   sequence, head and block of 128 tokens. hadamard_signs: NULL, or host
 *   memory holding d / 64 words whose bit i % 64 of word i / 64 set means a
 *   sign of -1 for dim i; each row is then multiplied by those signs and by
 *   the unnormalized d x d Walsh-Hadamard matrix (Sylvester order; fp32
 *   butterflies over strides 1, 2, 4, ...) before quantization. Q and K must
 *   use the same signs. The words are read during the call.
 *
 * fa_quantize_fp8_v: v [B, N, Hkv, d] -> codes_t uint8 [B, Hkv, d, NP] with
 *   NP = fa_fp8_v_keys(N) (N rounded up to a multiple of 128; keys past N are
 *   zero codes), and scales float [B, Hkv, d]: one scale per sequence, kv head
 *   and channel over the whole sequence. Inside each 64-key chunk of a
 *   channel row, key 32 b + 8 i + 4 g + j (b, g in {0, 1}; i, j in 0..3) sits
 *   at byte 32 g + 16 b + 4 i + j, the order the matrix-core operands read.
 *
 * fa_fwd_fp8: O [B, N, H, d] (out_dtype) and lse float [B, H, N] (natural
 *   log) of softmax(scale Q K^T) V on the dequantized inputs, the softmax
 *   probabilities themselves rounded to e4m3 (in [0, 448]) before they
 *   multiply V, and O divided by the sum of those rounded values (lse uses
 *   the unrounded ones). rotated = 1 when Q and K were quantized with
 *   hadamard_signs: the scale is then divided by d (the rotation multiplies
 *   every score by d). causal as fa_fwd; GQA when H > Hkv.
 */
int fa_fp8_v_keys(int N);

int fa_quantize_fp8_qk(const void* x, unsigned char* codes, float* scales,
                       int B, int N, int H, int d,
                       const unsigned long long* hadamard_signs, fa_dtype dtype,
                       void* stream);

int fa_quantize_fp8_v(const void* v, unsigned char* codes_t, float* scales,
                      int B, int N, int Hkv, int d, fa_dtype dtype, void* stream);

int fa_fwd_fp8(const unsigned char* q, const unsigned char* k, const unsigned char* v_t,
               const float* q_scales, const float* k_scales, const float* v_scales,
               void* o, float* lse, int B, int H, int Hkv, int N, int d,
               float scale, int causal, int rotated, fa_dtype out_dtype,
               void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LIBFA_FA_H */
