"""Seeded synthetic inputs for the attention workloads, shared by tests, bench and smoke.

This module draws random numbers and rounds them to the storage dtype; it holds
none of the attention arithmetic. Every draw comes from a NumPy
``Generator(PCG64(seed))`` in a fixed order (sequence lengths, then Q, K, V,
dO), as fp32 standard normals times ``std``, then rounded to the storage dtype
with round-to-nearest-even on the host. The same bytes go to the GPU and to the
fp64 checker.

Named workloads (shapes of the pages' attention benchmarks, synthetic values):

* ``fp32_small``   B=1, H=1, N=128, d=64, fp32, non-causal, forward only.
* ``gpt2m``        B=8, H=16, N=1024, d=64, bf16, non-causal (GPT-2-medium shape).
* ``long_causal``  B=1, H=32, N=16384, d=128, bf16, causal, std 1/sqrt(2).
* ``varlen_alibi`` 32 packed sequences, lengths uniform in [64, 8192], H=16,
  d=128, bf16, causal, ALiBi slopes 2^(-8(h+1)/H), forward only.
* ``gqa``          B=2, H=32, Hkv=8, N=8192, d=128, bf16, causal.
* ``DECODE``       one new query per sequence, B=8, H=32, Hkv=8, against key/
  value caches of 8192 .. 16384 keys (capacity 16384), d=128, bf16, causal.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np
import torch

__all__ = ["Workload", "WORKLOADS", "DECODE", "make_inputs", "make_decode_inputs", "alibi_slopes", "flops"]


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str  # "fp32" | "bf16" | "fp16"
    B: int
    H: int
    Hkv: int
    N: int
    d: int
    causal: bool = False
    alibi: bool = False
    std: float = 1.0
    backward: bool = True
    # packed sequences: number of sequences and inclusive length range
    varlen: Optional[tuple] = None
    extra: dict = field(default_factory=dict)

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    "fp32_small": Workload("fp32_small", "fp32", 1, 1, 1, 128, 64, backward=False),
    "gpt2m": Workload("gpt2m", "bf16", 8, 16, 16, 1024, 64),
    "long_causal": Workload("long_causal", "bf16", 1, 32, 32, 16384, 128, causal=True,
                            std=1.0 / math.sqrt(2.0)),
    "varlen_alibi": Workload("varlen_alibi", "bf16", 32, 16, 16, 8192, 128, causal=True,
                             alibi=True, backward=False, varlen=(64, 8192)),
    "gqa": Workload("gqa", "bf16", 2, 32, 8, 8192, 128, causal=True),
    # the long-context shape in fp16 (same draws, rounded to fp16)
    "long_causal_fp16": Workload("long_causal_fp16", "fp16", 1, 32, 32, 16384, 128, causal=True,
                                 std=1.0 / math.sqrt(2.0)),
}

_TORCH_DTYPE = {"fp32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16}


def alibi_slopes(H: int) -> torch.Tensor:
    """Geometric ALiBi slopes 2^(-8 (h+1) / H) for heads h = 0..H-1, fp32."""
    return torch.tensor([2.0 ** (-8.0 * (h + 1) / H) for h in range(H)], dtype=torch.float32)


def _normal(rng: np.random.Generator, shape, std: float, dtype: str) -> torch.Tensor:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return torch.from_numpy(x).to(_TORCH_DTYPE[dtype])


def make_inputs(w: Workload, seed: int = 0, lengths=None, with_grad: Optional[bool] = None) -> dict:
    """Draw one batch of inputs for workload ``w`` on the host.

    Returns a dict with CPU tensors ``q``, ``k``, ``v`` (and ``do`` when the
    workload has a backward), ``cu_seqlens`` (int32 [B+1] or None),
    ``alibi_slopes`` (fp32 [H] or None), ``scale`` (1/sqrt(d)), ``max_seqlen``.
    Dense layouts are q [B, N, H, d], k/v [B, N, Hkv, d]; packed layouts are
    q [T, H, d], k/v [T, Hkv, d]. ``lengths`` overrides the drawn packed lengths.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    with_grad = w.backward if with_grad is None else with_grad
    cu = None
    if w.varlen is not None:
        if lengths is None:
            lo, hi = w.varlen
            lengths = rng.integers(lo, hi + 1, size=w.B)
        lengths = np.asarray(lengths, dtype=np.int64)
        cu = torch.from_numpy(np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32))
        rows = (int(cu[-1]),)
        max_seqlen = int(lengths.max()) if len(lengths) else 0
    else:
        rows = (w.B, w.N)
        max_seqlen = w.N
    out = {
        "q": _normal(rng, rows + (w.H, w.d), w.std, w.dtype),
        "k": _normal(rng, rows + (w.Hkv, w.d), w.std, w.dtype),
        "v": _normal(rng, rows + (w.Hkv, w.d), w.std, w.dtype),
    }
    out["do"] = _normal(rng, rows + (w.H, w.d), w.std, w.dtype) if with_grad else None
    out["cu_seqlens"] = cu
    out["alibi_slopes"] = alibi_slopes(w.H) if w.alibi else None
    out["scale"] = 1.0 / math.sqrt(w.d)
    out["max_seqlen"] = max_seqlen
    return out


# Decode over a key/value cache: one new query per sequence against caches of
# 8192 .. 16384 keys (lengths drawn from the seed), GQA with 4 query heads per
# kv head (the shape of the long-context workloads above).
DECODE = (Workload("decode", "bf16", 8, 32, 8, 16384, 128, causal=True, backward=False), 1, None)


def make_decode_inputs(w: Workload, Nq: int, lengths=None, seed: int = 0) -> dict:
    """Inputs of a decode call: q [B, Nq, H, d], k_cache / v_cache [B, N, Hkv, d]
    (N = w.N, the cache capacity) and int32 cache_seqlens [B]. Draw order:
    lengths (uniform in [N/2, N] unless given), Q, K cache, V cache; values are
    fp32 standard normals times ``std`` rounded to the storage type."""
    rng = np.random.Generator(np.random.PCG64(seed))
    if lengths is None:
        lengths = rng.integers(w.N // 2, w.N + 1, size=w.B)
    lengths = np.asarray(lengths, dtype=np.int64)
    return {
        "q": _normal(rng, (w.B, Nq, w.H, w.d), w.std, w.dtype),
        "k_cache": _normal(rng, (w.B, w.N, w.Hkv, w.d), w.std, w.dtype),
        "v_cache": _normal(rng, (w.B, w.N, w.Hkv, w.d), w.std, w.dtype),
        "cache_seqlens": torch.from_numpy(lengths.astype(np.int32)),
        "alibi_slopes": alibi_slopes(w.H) if w.alibi else None,
        "scale": 1.0 / math.sqrt(w.d),
        "Nq": Nq,
    }


def make_outlier_inputs(w: Workload, seed: int = 0, frac: float = 1e-3, mag: float = 10.0) -> dict:
    """Dense Q, K, V like :func:`make_inputs` (no dO), except that a fraction
    ``frac`` of the entries of each, drawn at random, is multiplied by ``mag``:
    unit-normal features with rare large outliers, the kind of input the FP8
    path's rotation is meant for."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = {}
    for name, heads in (("q", w.H), ("k", w.Hkv), ("v", w.Hkv)):
        x = rng.standard_normal(size=(w.B, w.N, heads, w.d), dtype=np.float32)
        x[rng.random(size=x.shape) < frac] *= np.float32(mag)
        out[name] = torch.from_numpy(x).to(_TORCH_DTYPE[w.dtype])
    out.update(do=None, cu_seqlens=None, alibi_slopes=None, scale=1.0 / math.sqrt(w.d), max_seqlen=w.N)
    return out


def hadamard_signs(d: int, seed: int = 0) -> np.ndarray:
    """d random signs (+1 or -1, float64), the diagonal that precedes the
    Walsh-Hadamard rotation of the FP8 path."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return np.where(rng.random(d) < 0.5, -1.0, 1.0)


def seq_lengths(inputs: dict, w: Workload) -> list:
    """Per-sequence lengths of a drawn batch (all N for dense inputs)."""
    cu = inputs["cu_seqlens"]
    if cu is None:
        return [w.N] * w.B
    c = cu.tolist()
    return [c[i + 1] - c[i] for i in range(len(c) - 1)]


def flops(w: Workload, lengths=None, backward: bool = False) -> float:
    """Dense attention work: 4*H*n^2*d per sequence, halved if causal, x2.5 for backward."""
    if lengths is None:
        lengths = [w.N] * w.B
    f = sum(4.0 * w.H * float(n) * float(n) * w.d for n in lengths)
    if w.causal:
        f *= 0.5
    return f * (2.5 if backward else 1.0)
