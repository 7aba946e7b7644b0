"""libfa: exact tiled attention (FlashAttention forward and backward) for MI355X / gfx950.

The compute lives in ``libfa.so`` (hand-written HIP kernels behind the C ABI of
``include/fa.h``); this package is its ctypes binding plus seeded workload
generators.
"""

from ._binding import (  # noqa: F401
    FA_BF16,
    FA_BWD_ALL,
    FA_BWD_DKDV,
    FA_BWD_DQ,
    FA_BWD_PREP,
    FA_FP16,
    FA_FP32,
    FA_OK,
    FaError,
    FlashAttnFn,
    LIB_PATH,
    attention,
    attention_bwd,
    attention_fp8,
    attention_fp8_quantized,
    attention_kvcache,
    fa_bwd,
    fa_bwd_dropout,
    fa_bwd_ext,
    fa_fwd_dropout,
    fa_fwd_ext,
    fa_bwd_noalloc,
    fa_bwd_noalloc_max_bytes,
    fa_bwd_stages,
    fa_bwd_workspace_size,
    fa_fwd,
    fa_fp8_v_keys,
    fa_fwd_fp8,
    fa_fwd_kvcache,
    fa_quantize_fp8_qk,
    fa_quantize_fp8_v,
    hadamard_sign_words,
    fa_kvcache_workspace_size,
    fa_strerror,
    fa_version,
    lib,
    quantize_fp8_qk,
    quantize_fp8_v,
)
