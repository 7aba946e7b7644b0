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
    if cu_seqlens is None:
        if q.dim() != 4 or k.dim() != 4:
            raise ValueError("dense inputs are q [B, N, H, d], k/v [B, N, Hkv, d]")
        B, N, H, d = q.shape
        Hkv = k.shape[2]
    else:
        if q.dim() != 3 or k.dim() != 3:
            raise ValueError("packed inputs are q [total, H, d], k/v [total, Hkv, d]")
        if max_seqlen is None:
            raise ValueError("packed inputs need max_seqlen")
        _, H, d = q.shape
        Hkv = k.shape[1]
        B, N = cu_seqlens.numel() - 1, int(max_seqlen)
    return B, H, Hkv, N, d


def _check_tensors(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("libfa takes contiguous device tensors")


def attention(q, k, v, causal: bool = False, softmax_scale: Optional[float] = None,
              alibi_slopes: Optional[torch.Tensor] = None, cu_seqlens: Optional[torch.Tensor] = None,
              max_seqlen: Optional[int] = None, out: Optional[torch.Tensor] = None,
              lse: Optional[torch.Tensor] = None):
    """Exact attention forward through ``fa_fwd``: returns (o, lse).

    Mirrors ``flash_attn_func(q, k, v, softmax_scale=None, causal=...)`` (no
    dropout). ``lse`` is fp32 [B, H, N] (N = max_seqlen for packed inputs).
    """
    _check_tensors(q, k, v, alibi_slopes, cu_seqlens)
    B, H, Hkv, N, d = _shape(q, k, cu_seqlens, max_seqlen)
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    if q.dtype not in _DTYPE or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share one of fp32 / fp16 / bf16")
    o = torch.empty_like(q) if out is None else out
    l = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None else lse
    st = fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), l.data_ptr(), B, H, Hkv, N, d, scale,
                int(bool(causal)), _ptr(alibi_slopes), _ptr(cu_seqlens), _DTYPE[q.dtype], _stream_handle())
    if st != FA_OK:
        raise FaError(st)
    return o, l


def attention_bwd(dout, q, k, v, o, lse, causal: bool = False, softmax_scale: Optional[float] = None,
                  alibi_slopes: Optional[torch.Tensor] = None, cu_seqlens: Optional[torch.Tensor] = None,
                  max_seqlen: Optional[int] = None, workspace: Optional[torch.Tensor] = None):
    """Exact attention backward through ``fa_bwd``: returns (dq, dk, dv)."""
    _check_tensors(dout, q, k, v, o, lse, alibi_slopes, cu_seqlens)
    B, H, Hkv, N, d = _shape(q, k, cu_seqlens, max_seqlen)
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    dt = _DTYPE[q.dtype]
    ws_bytes = fa_bwd_workspace_size(B, H, Hkv, N, d, int(bool(causal)), int(cu_seqlens is not None), dt)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    st = fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(), lse.data_ptr(),
                dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, Hkv, N, d, scale, int(bool(causal)),
                _ptr(alibi_slopes), _ptr(cu_seqlens), dt, workspace.data_ptr(), workspace.numel(),
                _stream_handle())
    if st != FA_OK:
        raise FaError(st)
    return dq, dk, dv


class FlashAttnFn(torch.autograd.Function):
    """Autograd wrapper: forward saves (q, k, v, o, lse); backward calls fa_bwd."""

    @staticmethod
    def forward(ctx, q, k, v, causal=False, softmax_scale=None, alibi_slopes=None, cu_seqlens=None,
                max_seqlen=None):
        o, lse = attention(q, k, v, causal, softmax_scale, alibi_slopes, cu_seqlens, max_seqlen)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.args = (causal, softmax_scale, alibi_slopes, cu_seqlens, max_seqlen)
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse = ctx.saved_tensors
        dq, dk, dv = attention_bwd(do.contiguous(), q, k, v, o, lse, *ctx.args)
        return dq, dk, dv, None, None, None, None, None
