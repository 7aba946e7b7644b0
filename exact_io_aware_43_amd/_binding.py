"""ctypes binding for libfa.so: the C-ABI calls under the same names, plus torch helpers.

Argument marshalling only: every step of attention runs in libfa's HIP kernels.
Torch is used to hand over device pointers, allocate outputs and pick the
current stream. If the library is missing, loading fails loudly; there is no
fallback implementation.
"""

from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfa.so")

FA_FP32, FA_FP16, FA_BF16 = 0, 1, 2
FA_OK = 0
_DTYPE = {torch.float32: FA_FP32, torch.float16: FA_FP16, torch.bfloat16: FA_BF16}

_lib = None


def lib() -> ctypes.CDLL:
    """Load libfa.so once (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libfa.so not found at {LIB_PATH}; build it with "
                               "`python -c 'import __graft_entry__ as g; g.build()'`")
        L = ctypes.CDLL(LIB_PATH)
        vp, ci, cf, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        L.fa_fwd.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, cf, ci, vp, vp, ci, vp]
        L.fa_fwd.restype = ci
        L.fa_bwd_workspace_size.argtypes = [ci, ci, ci, ci, ci, ci, ci, ci]
        L.fa_bwd_workspace_size.restype = sz
        L.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, cf, ci, vp, vp, ci, vp, sz, vp]
        L.fa_bwd.restype = ci
        L.fa_bwd_stages.argtypes = L.fa_bwd.argtypes[:-1] + [ctypes.c_uint, vp]
        L.fa_bwd_stages.restype = ci
        u64, u32 = ctypes.c_ulonglong, ctypes.c_uint
        L.fa_fwd_dropout.argtypes = L.fa_fwd.argtypes[:-1] + [cf, u64, u32, vp]
        L.fa_fwd_dropout.restype = ci
        L.fa_bwd_dropout.argtypes = L.fa_bwd.argtypes[:-3] + [cf, u64, u32, vp, sz, vp]
        L.fa_bwd_dropout.restype = ci
        L.fa_fwd_ext.argtypes = L.fa_fwd.argtypes[:-1] + [ci, ci, cf, cf, u64, u32, vp]
        L.fa_fwd_ext.restype = ci
        L.fa_bwd_ext.argtypes = L.fa_bwd.argtypes[:-3] + [ci, ci, cf, cf, u64, u32, vp, sz, vp]
        L.fa_bwd_ext.restype = ci
        L.fa_kvcache_workspace_size.argtypes = [ci] * 7
        L.fa_kvcache_workspace_size.restype = sz
        L.fa_fwd_kvcache.argtypes = [vp] * 6 + [ci] * 6 + [cf, ci, vp, ci, ci, vp, sz, vp]
        L.fa_fwd_kvcache.restype = ci
        L.fa_bwd_noalloc.argtypes = L.fa_bwd.argtypes[:-3] + [vp]
        L.fa_bwd_noalloc.restype = ci
        L.fa_bwd_noalloc_max_bytes.argtypes = []
        L.fa_bwd_noalloc_max_bytes.restype = sz
        L.fa_fp8_v_keys.argtypes = [ci]
        L.fa_fp8_v_keys.restype = ci
        L.fa_quantize_fp8_qk.argtypes = [vp, vp, vp, ci, ci, ci, ci, vp, ci, vp]
        L.fa_quantize_fp8_qk.restype = ci
        L.fa_quantize_fp8_v.argtypes = [vp, vp, vp, ci, ci, ci, ci, ci, vp]
        L.fa_quantize_fp8_v.restype = ci
        L.fa_fwd_fp8.argtypes = [vp] * 8 + [ci] * 5 + [cf, ci, ci, ci, vp]
        L.fa_fwd_fp8.restype = ci
        L.fa_strerror.argtypes = [ci]
        L.fa_strerror.restype = ctypes.c_char_p
        L.fa_version.argtypes = []
        L.fa_version.restype = ci
        _lib = L
    return _lib


# ----------------------------------------------------------------- raw C-ABI calls

def fa_fwd(q, k, v, o, lse, B, H, Hkv, N, d, scale, causal, alibi_slopes, cu_seqlens, dtype, stream) -> int:
    """``fa_fwd`` with integer device pointers (or None for NULL); returns the status."""
    return lib().fa_fwd(q, k, v, o, lse, B, H, Hkv, N, d, scale, causal, alibi_slopes, cu_seqlens, dtype, stream)


def fa_fwd_dropout(q, k, v, o, lse, B, H, Hkv, N, d, scale, causal, alibi_slopes, cu_seqlens, dtype, p_drop, seed,
                   offset, stream) -> int:
    """``fa_fwd_dropout`` with integer device pointers (or None for NULL); returns the status."""
    return lib().fa_fwd_dropout(q, k, v, o, lse, B, H, Hkv, N, d, scale, causal, alibi_slopes, cu_seqlens, dtype,
                                p_drop, seed, offset, stream)


def fa_bwd_dropout(q, k, v, o, dout, lse, dq, dk, dv, B, H, Hkv, N, d, scale, causal, alibi_slopes, cu_seqlens,
                   dtype, p_drop, seed, offset, workspace, workspace_bytes, stream) -> int:
    """``fa_bwd_dropout`` with integer device pointers (or None for NULL); returns the status."""
    return lib().fa_bwd_dropout(q, k, v, o, dout, lse, dq, dk, dv, B, H, Hkv, N, d, scale, causal, alibi_slopes,
                                cu_seqlens, dtype, p_drop, seed, offset, workspace, workspace_bytes, stream)


def fa_fwd_ext(q, k, v, o, lse, B, H, Hkv, N, d, scale, causal, alibi_slopes, cu_seqlens, dtype, window_left,
               window_right, softcap, p_drop, seed, offset, stream) -> int:
    """``fa_fwd_ext`` with integer device pointers (or None for NULL); returns the status."""
    return lib().fa_fwd_ext(q, k, v, o, lse, B, H, Hkv, N, d, scale, causal, alibi_slopes, cu_seqlens, dtype,
                            window_left, window_right, softcap, p_drop, seed, offset, stream)


def fa_bwd_ext(q, k, v, o, dout, lse, dq, dk, dv, B, H, Hkv, N, d, scale, causal, alibi_slopes, cu_seqlens, dtype,
               window_left, window_right, softcap, p_drop, seed, offset, workspace, workspace_bytes, stream) -> int:
    """``fa_bwd_ext`` with integer device pointers (or None for NULL); returns the status."""
    return lib().fa_bwd_ext(q, k, v, o, dout, lse, dq, dk, dv, B, H, Hkv, N, d, scale, causal, alibi_slopes,
                            cu_seqlens, dtype, window_left, window_right, softcap, p_drop, seed, offset, workspace,
                            workspace_bytes, stream)


def fa_kvcache_workspace_size(B, H, Hkv, Nq, Nk, d, num_splits) -> int:
    return lib().fa_kvcache_workspace_size(B, H, Hkv, Nq, Nk, d, num_splits)


def fa_fwd_kvcache(q, k_cache, v_cache, o, lse, cache_seqlens, B, H, Hkv, Nq, Nk, d, scale, causal, alibi_slopes,
                   dtype, num_splits, workspace, workspace_bytes, stream) -> int:
    """``fa_fwd_kvcache`` with integer device pointers (or None for NULL); returns the status."""
    return lib().fa_fwd_kvcache(q, k_cache, v_cache, o, lse, cache_seqlens, B, H, Hkv, Nq, Nk, d, scale, causal,
                                alibi_slopes, dtype, num_splits, workspace, workspace_bytes, stream)


def fa_bwd_workspace_size(B, H, Hkv, N, d, causal, varlen, dtype) -> int:
    return lib().fa_bwd_workspace_size(B, H, Hkv, N, d, causal, varlen, dtype)


def fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, H, Hkv, N, d, scale, causal, alibi_slopes, cu_seqlens, dtype,
           workspace, workspace_bytes, stream) -> int:
    """``fa_bwd`` with integer device pointers (or None for NULL); returns the status."""
    return lib().fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, H, Hkv, N, d, scale, causal, alibi_slopes,
                        cu_seqlens, dtype, workspace, workspace_bytes, stream)


FA_BWD_PREP, FA_BWD_DKDV, FA_BWD_DQ, FA_BWD_ALL = 1, 2, 4, 7


def fa_bwd_stages(q, k, v, o, dout, lse, dq, dk, dv, B, H, Hkv, N, d, scale, causal, alibi_slopes, cu_seqlens,
                  dtype, workspace, workspace_bytes, stages, stream) -> int:
    """``fa_bwd_stages``: a subset (bitmask of FA_BWD_*) of fa_bwd's launches."""
    return lib().fa_bwd_stages(q, k, v, o, dout, lse, dq, dk, dv, B, H, Hkv, N, d, scale, causal, alibi_slopes,
                               cu_seqlens, dtype, workspace, workspace_bytes, stages, stream)


def fa_bwd_noalloc(q, k, v, o, dout, lse, dq, dk, dv, B, H, Hkv, N, d, scale, causal, alibi_slopes, cu_seqlens,
                   dtype, stream) -> int:
    """``fa_bwd_noalloc``: fa_bwd with the library's static per-GPU scratch instead of a workspace."""
    return lib().fa_bwd_noalloc(q, k, v, o, dout, lse, dq, dk, dv, B, H, Hkv, N, d, scale, causal, alibi_slopes,
                                cu_seqlens, dtype, stream)


def fa_bwd_noalloc_max_bytes() -> int:
    return lib().fa_bwd_noalloc_max_bytes()


def fa_fp8_v_keys(N) -> int:
    return lib().fa_fp8_v_keys(N)


def fa_quantize_fp8_qk(x, codes, scales, B, N, H, d, hadamard_signs, dtype, stream) -> int:
    """``fa_quantize_fp8_qk``; hadamard_signs is a host address of d / 64 uint64 words, or None."""
    return lib().fa_quantize_fp8_qk(x, codes, scales, B, N, H, d, hadamard_signs, dtype, stream)


def fa_quantize_fp8_v(v, codes_t, scales, B, N, Hkv, d, dtype, stream) -> int:
    return lib().fa_quantize_fp8_v(v, codes_t, scales, B, N, Hkv, d, dtype, stream)


def fa_fwd_fp8(q, k, v_t, q_scales, k_scales, v_scales, o, lse, B, H, Hkv, N, d, scale, causal, rotated, out_dtype,
               stream) -> int:
    """``fa_fwd_fp8`` with integer device pointers; returns the status."""
    return lib().fa_fwd_fp8(q, k, v_t, q_scales, k_scales, v_scales, o, lse, B, H, Hkv, N, d, scale, causal, rotated,
                            out_dtype, stream)


def fa_strerror(status: int) -> str:
    return lib().fa_strerror(status).decode()


def fa_version() -> int:
    return lib().fa_version()


# ------------------------------------------------------------------ torch helpers

class FaError(RuntimeError):
    def __init__(self, status: int):
        super().__init__(f"libfa status {status}: {fa_strerror(status)}")
        self.status = status


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream_handle() -> int:
    return torch.cuda.current_stream().cuda_stream


def _shape(q: torch.Tensor, k: torch.Tensor, cu_seqlens, max_seqlen):
    """(B, H, Hkv, N, d) of a call, from q and k (dense) or q, k and cu_seqlens (packed)."""
    if cu_seqlens is None:
        if q.dim() != 4 or k.dim() != 4:
            raise ValueError("dense inputs are q [B, N, H, d], k/v [B, N, Hkv, d]")
        B, N, H, d = q.shape
        Hkv = k.shape[2]
    else:
        if q.dim() != 3 or k.dim() != 3:
            raise ValueError("packed inputs are q [total, H, d], k/v [total, Hkv, d]")
        if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
            raise ValueError("cu_seqlens must be a 1-D tensor of B + 1 offsets")
        if max_seqlen is None:
            raise ValueError("packed inputs need max_seqlen")
        _, H, d = q.shape
        Hkv = k.shape[1]
        B, N = cu_seqlens.numel() - 1, int(max_seqlen)
    return B, H, Hkv, N, d


def _expect(t: Optional[torch.Tensor], name: str, shape, dtype, device) -> None:
    """Raise ValueError unless ``t`` is a contiguous tensor of exactly this shape,
    dtype and device (the layouts the C ABI documents)."""
    if t is None:
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def validate(q, k, v, *, cu_seqlens=None, max_seqlen=None, alibi_slopes=None, q_like=(), lse=None,
             require_device: bool = True):
    """Check every tensor of a call against the sizes (B, H, Hkv, N, d) that q, k and
    cu_seqlens imply, and return those sizes.

    q_like: (name, tensor) pairs that must match q exactly (o, dout, out). Packed
    inputs need int32 cu_seqlens [B + 1]; alibi_slopes is fp32 [H]; lse is fp32
    [B, H, N]. Every tensor must be contiguous and on q's device, which must be a
    GPU unless ``require_device`` is False (host-side tests of this function).
    Lengths inside cu_seqlens live in device memory and are not read here: the
    library treats N as the caller's bound on every length.
    """
    if not isinstance(q, torch.Tensor):
        raise ValueError("q must be a torch.Tensor")
    if require_device and not q.is_cuda:
        raise ValueError("libfa takes device tensors (q is on the host)")
    if q.dtype not in _DTYPE:
        raise ValueError(f"q has dtype {q.dtype}; libfa takes float32, float16 or bfloat16")
    B, H, Hkv, N, d = _shape(q, k, cu_seqlens, max_seqlen)
    dev, dt = q.device, q.dtype
    _expect(q, "q", q.shape, dt, dev)
    if cu_seqlens is None:
        kv_shape = (B, N, Hkv, d)
    else:
        kv_shape = (q.shape[0], Hkv, d)
        _expect(cu_seqlens, "cu_seqlens", (B + 1,), torch.int32, dev)
        if N <= 0:
            raise ValueError("max_seqlen must be positive")
    _expect(k, "k", kv_shape, dt, dev)
    _expect(v, "v", kv_shape, dt, dev)
    if H % Hkv != 0:
        raise ValueError(f"query heads ({H}) must be a multiple of kv heads ({Hkv})")
    if alibi_slopes is not None:
        _expect(alibi_slopes, "alibi_slopes", (H,), torch.float32, dev)
    for name, t in q_like:
        _expect(t, name, q.shape, dt, dev)
    if lse is not None:
        _expect(lse, "lse", (B, H, N), torch.float32, dev)
    return B, H, Hkv, N, d


def attention(q, k, v, causal: bool = False, softmax_scale: Optional[float] = None,
              alibi_slopes: Optional[torch.Tensor] = None, cu_seqlens: Optional[torch.Tensor] = None,
              max_seqlen: Optional[int] = None, out: Optional[torch.Tensor] = None,
              lse: Optional[torch.Tensor] = None, dropout_p: float = 0.0, seed: int = 0, offset: int = 0,
              window_size=(-1, -1), softcap: float = 0.0):
    """Exact attention forward through ``fa_fwd`` (``fa_fwd_dropout`` when
    ``dropout_p`` > 0, ``fa_fwd_ext`` with a window or softcapping): returns
    (o, lse).

    Mirrors ``flash_attn_func(q, k, v, dropout_p, softmax_scale, causal,
    window_size, softcap)``; the dropout mask is the generator's (``seed``,
    ``offset``), which the backward call must repeat. ``lse`` is fp32
    [B, H, N] (N = max_seqlen for packed inputs). Every tensor is validated
    against the layouts of the C ABI.
    """
    B, H, Hkv, N, d = validate(q, k, v, cu_seqlens=cu_seqlens, max_seqlen=max_seqlen, alibi_slopes=alibi_slopes,
                               q_like=(() if out is None else (("out", out),)), lse=lse)
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    o = torch.empty_like(q) if out is None else out
    l = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None else lse
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), l.data_ptr(), B, H, Hkv, N, d, scale,
            int(bool(causal)), _ptr(alibi_slopes), _ptr(cu_seqlens), _DTYPE[q.dtype])
    wl, wr = (int(x) for x in window_size)
    if (wl, wr) != (-1, -1) or softcap:
        st = fa_fwd_ext(*args, wl, wr, float(softcap), float(dropout_p), int(seed), int(offset), _stream_handle())
    elif dropout_p:
        st = fa_fwd_dropout(*args, float(dropout_p), int(seed), int(offset), _stream_handle())
    else:
        st = fa_fwd(*args, _stream_handle())
    if st != FA_OK:
        raise FaError(st)
    return o, l


def attention_bwd(dout, q, k, v, o, lse, causal: bool = False, softmax_scale: Optional[float] = None,
                  alibi_slopes: Optional[torch.Tensor] = None, cu_seqlens: Optional[torch.Tensor] = None,
                  max_seqlen: Optional[int] = None, workspace: Optional[torch.Tensor] = None,
                  dropout_p: float = 0.0, seed: int = 0, offset: int = 0, window_size=(-1, -1),
                  softcap: float = 0.0):
    """Exact attention backward through ``fa_bwd`` (``fa_bwd_dropout`` when
    ``dropout_p`` > 0, with the forward's seed and offset; ``fa_bwd_ext`` with a
    window or softcapping): returns (dq, dk, dv)."""
    B, H, Hkv, N, d = validate(q, k, v, cu_seqlens=cu_seqlens, max_seqlen=max_seqlen, alibi_slopes=alibi_slopes,
                               q_like=(("o", o), ("dout", dout)), lse=lse)
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    dt = _DTYPE[q.dtype]
    ws_bytes = fa_bwd_workspace_size(B, H, Hkv, N, d, int(bool(causal)), int(cu_seqlens is not None), dt)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=q.device)
    elif not (workspace.is_contiguous() and workspace.device == q.device):
        raise ValueError("workspace must be a contiguous tensor on q's device")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(), lse.data_ptr(),
            dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, Hkv, N, d, scale, int(bool(causal)),
            _ptr(alibi_slopes), _ptr(cu_seqlens), dt)
    ws = (workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream_handle())
    wl, wr = (int(x) for x in window_size)
    if (wl, wr) != (-1, -1) or softcap:
        st = fa_bwd_ext(*args, wl, wr, float(softcap), float(dropout_p), int(seed), int(offset), *ws)
    elif dropout_p:
        st = fa_bwd_dropout(*args, float(dropout_p), int(seed), int(offset), *ws)
    else:
        st = fa_bwd(*args, *ws)
    if st != FA_OK:
        raise FaError(st)
    return dq, dk, dv


def attention_kvcache(q, k_cache, v_cache, cache_seqlens, causal: bool = True,
                      softmax_scale: Optional[float] = None, alibi_slopes: Optional[torch.Tensor] = None,
                      num_splits: int = 0, workspace: Optional[torch.Tensor] = None):
    """Decode through ``fa_fwd_kvcache``: q [B, Nq, H, d] against k_cache, v_cache
    [B, Nk, Hkv, d] with int32 cache_seqlens [B]; returns (o [B, Nq, H, d], lse [B, H, Nq])."""
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache)):
        if not isinstance(t, torch.Tensor) or t.dim() != 4:
            raise ValueError(f"{name} must be a 4-d tensor")
    if not q.is_cuda:
        raise ValueError("libfa takes device tensors (q is on the host)")
    B, Nq, H, d = q.shape
    Nk, Hkv = k_cache.shape[1], k_cache.shape[2]
    dev, dt = q.device, q.dtype
    if dt not in (torch.float16, torch.bfloat16):
        raise ValueError("decode takes float16 or bfloat16")
    _expect(q, "q", q.shape, dt, dev)
    _expect(k_cache, "k_cache", (B, Nk, Hkv, d), dt, dev)
    _expect(v_cache, "v_cache", (B, Nk, Hkv, d), dt, dev)
    _expect(cache_seqlens, "cache_seqlens", (B,), torch.int32, dev)
    if alibi_slopes is not None:
        _expect(alibi_slopes, "alibi_slopes", (H,), torch.float32, dev)
    if H % Hkv:
        raise ValueError(f"query heads ({H}) must be a multiple of kv heads ({Hkv})")
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    ws_bytes = fa_kvcache_workspace_size(B, H, Hkv, Nq, Nk, d, num_splits)
    if ws_bytes and workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=dev)
    st = fa_fwd_kvcache(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), o.data_ptr(), lse.data_ptr(),
                        cache_seqlens.data_ptr(), B, H, Hkv, Nq, Nk, d, scale, int(bool(causal)), _ptr(alibi_slopes),
                        _DTYPE[dt], int(num_splits), _ptr(workspace),
                        0 if workspace is None else workspace.numel() * workspace.element_size(), _stream_handle())
    if st != FA_OK:
        raise FaError(st)
    return o, lse


def hadamard_sign_words(signs, d: int):
    """+-1 signs of length d as the d / 64 uint64 words fa_quantize_fp8_qk takes
    (bit i % 64 of word i / 64 set for a sign of -1)."""
    s = torch.as_tensor(signs, dtype=torch.float64).cpu().reshape(-1).tolist()
    if len(s) != d or d % 64 or any(x not in (1.0, -1.0) for x in s):
        raise ValueError(f"hadamard signs must be {d} values of +1 or -1")
    words = (ctypes.c_ulonglong * (d // 64))()
    for i, x in enumerate(s):
        if x < 0:
            words[i // 64] |= 1 << (i % 64)
    return words


def quantize_fp8_qk(x, hadamard_signs=None):
    """Q or K [B, N, H, d] (float16 / bfloat16, device) -> (codes uint8 [B, N, H, d],
    scales float32 [B, H, ceil(N / 128)], powers of two)."""
    if not isinstance(x, torch.Tensor) or x.dim() != 4 or not x.is_cuda:
        raise ValueError("x must be a 4-d device tensor")
    if x.dtype not in (torch.float16, torch.bfloat16):
        raise ValueError("fp8 quantization takes float16 or bfloat16")
    B, N, H, d = x.shape
    _expect(x, "x", x.shape, x.dtype, x.device)
    codes = torch.empty((B, N, H, d), dtype=torch.uint8, device=x.device)
    scales = torch.empty((B, H, (N + 127) // 128), dtype=torch.float32, device=x.device)
    words = None if hadamard_signs is None else hadamard_sign_words(hadamard_signs, d)
    st = fa_quantize_fp8_qk(x.data_ptr(), codes.data_ptr(), scales.data_ptr(), B, N, H, d,
                            None if words is None else ctypes.addressof(words), _DTYPE[x.dtype], _stream_handle())
    if st != FA_OK:
        raise FaError(st)
    return codes, scales


def quantize_fp8_v(v):
    """V [B, N, Hkv, d] (float16 / bfloat16, device) -> (codes_t uint8 [B, Hkv, d, NP]
    in the key order fa_fwd_fp8 reads, scales float32 [B, Hkv, d])."""
    if not isinstance(v, torch.Tensor) or v.dim() != 4 or not v.is_cuda:
        raise ValueError("v must be a 4-d device tensor")
    if v.dtype not in (torch.float16, torch.bfloat16):
        raise ValueError("fp8 quantization takes float16 or bfloat16")
    B, N, Hkv, d = v.shape
    _expect(v, "v", v.shape, v.dtype, v.device)
    npad = fa_fp8_v_keys(N)
    codes = torch.empty((B, Hkv, d, max(npad, 1)), dtype=torch.uint8, device=v.device)
    scales = torch.empty((B, Hkv, d), dtype=torch.float32, device=v.device)
    st = fa_quantize_fp8_v(v.data_ptr(), codes.data_ptr(), scales.data_ptr(), B, N, Hkv, d, _DTYPE[v.dtype],
                           _stream_handle())
    if st != FA_OK:
        raise FaError(st)
    return codes, scales


def attention_fp8_quantized(qc, qs, kc, ks, vc, vs, causal: bool = False, softmax_scale: Optional[float] = None,
                            rotated: bool = False, out_dtype=torch.bfloat16):
    """fa_fwd_fp8 on codes and scales from quantize_fp8_qk / quantize_fp8_v;
    returns (o [B, N, H, d] out_dtype, lse float32 [B, H, N])."""
    for name, t in (("q codes", qc), ("q scales", qs), ("k codes", kc), ("k scales", ks), ("v codes", vc),
                    ("v scales", vs)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
    if qc.dim() != 4 or kc.dim() != 4:
        raise ValueError("q and k codes must be 4-d [B, N, heads, d]")
    B, N, H, d = qc.shape
    Hkv = kc.shape[2]
    dev = qc.device
    _expect(qc, "q codes", (B, N, H, d), torch.uint8, dev)
    _expect(kc, "k codes", (B, N, Hkv, d), torch.uint8, dev)
    _expect(vc, "v codes", (B, Hkv, d, fa_fp8_v_keys(N)), torch.uint8, dev)
    nb = (N + 127) // 128
    _expect(qs, "q scales", (B, H, nb), torch.float32, dev)
    _expect(ks, "k scales", (B, Hkv, nb), torch.float32, dev)
    _expect(vs, "v scales", (B, Hkv, d), torch.float32, dev)
    if out_dtype not in (torch.float16, torch.bfloat16):
        raise ValueError("fp8 attention returns float16 or bfloat16")
    if Hkv == 0 or H % Hkv:
        raise ValueError(f"query heads ({H}) must be a multiple of kv heads ({Hkv})")
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    o = torch.empty((B, N, H, d), dtype=out_dtype, device=dev)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    st = fa_fwd_fp8(qc.data_ptr(), kc.data_ptr(), vc.data_ptr(), qs.data_ptr(), ks.data_ptr(), vs.data_ptr(),
                    o.data_ptr(), lse.data_ptr(), B, H, Hkv, N, d, scale, int(bool(causal)), int(bool(rotated)),
                    _DTYPE[out_dtype], _stream_handle())
    if st != FA_OK:
        raise FaError(st)
    return o, lse


def attention_fp8(q, k, v, causal: bool = False, softmax_scale: Optional[float] = None, hadamard_signs=None,
                  out_dtype=None):
    """FP8 forward from 16-bit Q, K, V: quantize (Q and K rotated when
    hadamard_signs, d values of +-1, are given), then fa_fwd_fp8. Returns (o, lse)."""
    qc, qs = quantize_fp8_qk(q, hadamard_signs)
    kc, ks = quantize_fp8_qk(k, hadamard_signs)
    vc, vs = quantize_fp8_v(v)
    return attention_fp8_quantized(qc, qs, kc, ks, vc, vs, causal=causal, softmax_scale=softmax_scale,
                                   rotated=hadamard_signs is not None, out_dtype=out_dtype or q.dtype)


class FlashAttnFn(torch.autograd.Function):
    """Autograd wrapper: forward saves (q, k, v, o, lse); backward calls fa_bwd."""

    @staticmethod
    def forward(ctx, q, k, v, causal=False, softmax_scale=None, alibi_slopes=None, cu_seqlens=None,
                max_seqlen=None, dropout_p=0.0, seed=0, offset=0, window_size=(-1, -1), softcap=0.0):
        o, lse = attention(q, k, v, causal, softmax_scale, alibi_slopes, cu_seqlens, max_seqlen,
                           dropout_p=dropout_p, seed=seed, offset=offset, window_size=window_size, softcap=softcap)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.args = (causal, softmax_scale, alibi_slopes, cu_seqlens, max_seqlen)
        # the saved generator state and mask variants
        ctx.drop = dict(dropout_p=dropout_p, seed=seed, offset=offset, window_size=window_size, softcap=softcap)
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse = ctx.saved_tensors
        dq, dk, dv = attention_bwd(do.contiguous(), q, k, v, o, lse, *ctx.args, **ctx.drop)
        return dq, dk, dv, None, None, None, None, None, None, None, None, None, None
