"""Plain fp64 CPU oracle for exact scaled-dot-product attention, forward and backward.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything in this
package. The product path (``libfa`` and its Python binding) never calls it,
and it shares no code, table or helper with that path.

Sources, cited by page title and section:

* [PN] "FlashAttention: Faster Attention Without Dropping a Single Interaction"
  (awesome.papernotes.org). Method Deep Dive: Key design 1 (definition of S, P,
  O), Key design 2 (mergeable (m, l, O) state and the saved-state table with
  L = m + log l), Key design 3 (backward by recomputation, D_i and dS).
* [RX] "FlashAttention: The Algorithm That Beat the Memory Wall"
  (repo-explainer.com). "A Tile, a Register File, and a Trick Called Online
  Softmax" (the per-tile loop) and "Varlen Is the Quiet Superpower" (packed
  sequences).
* [GL] "FlashAttention" glossary (inferensys.com): ALiBi and multi-query
  variants are named, without formulas.

What is computed (the plain definition, [PN] Key design 1): for each batch
entry or packed sequence b and query head h, with kv head g = floor(h / G),
G = H / Hkv, and positions i, j in [0, n):

    S_ij = scale * <q_i, k_j> + beta_ij
    P    = row-wise softmax of S          (entries with j > i removed if causal)
    O    = P V,    lse_i = m_i + ln(sum_j exp(S_ij - m_i)),  m_i = max_j S_ij

The method is exact in real arithmetic, so the oracle is that definition:
two-pass softmax over a materialised S, no blocking, every value in fp64.

Readings taken where the pages are silent or garbled (each is also listed in
the design notes of the repository):

1. Scale. The definition divides by sqrt(d); the printed loops omit it. S
   carries an explicit ``scale`` (default 1/sqrt(d)) and, by the chain rule,
   dQ and dK carry the same factor.
2. l is the running sum of exponentials; the statistic kept for backward is
   the natural-log L = m + ln l.
3. Causal masking keeps key j <= query i (query and key lengths are equal).
4. ALiBi (named only): beta_ij = -slope_h * |i - j|, added after scaling and
   before the mask; under causal masking this is -slope_h * (i - j).
5. GQA / MQA (named only): consecutive groups, kv head = floor(h / G); dK and
   dV of a kv head are the sums over its G query heads.
6. Varlen: packed rows [total, heads, d] with ``cu_seqlens`` [B+1]; each
   sequence is an independent attention problem with local positions. The
   statistic ``lse`` is laid out [B, H, Nmax] for both dense and packed
   inputs; entries past a sequence's length are NaN here.
7. A masked score contributes exactly zero; exp(-inf - (-inf)) never occurs in
   the two-pass form because every causal row keeps its diagonal.
8. Dropout ([PN] Key design 1 stage table: the fused operator drops attention
   probabilities and the backward regenerates them from the saved generator
   state, Key design 3): the softmax and lse use every score; the
   probabilities that multiply V are dropped with a counter-based mask and the
   kept ones scaled so their expectation is unchanged. The mask is defined in
   oracle/philox.py.
9. Sliding window (named only: the usage contract's mask row lists sliding
   window next to ALiBi and softcapping): ``window`` = (left, right) keeps key
   j for query i when i - left <= j <= i + right; a negative bound is
   unbounded. Positions are within a sequence, and causal masking applies as
   well (so right is effectively 0 under it).
10. Softcapping (named only, same row): the scaled score u = scale * <q_i, k_j>
   becomes cap * tanh(u / cap) for cap > 0, before the ALiBi bias and the masks;
   by the chain rule the gradient reaching u is dS * (1 - tanh(u / cap)^2).
"""

from __future__ import annotations

import math

import numpy as np

from . import philox as PX

__all__ = [
    "attention_fwd",
    "attention_bwd",
    "head_fwd",
    "head_bwd",
    "head_rows_fwd",
    "online_head_fwd",
    "tile_state",
    "merge_states",
    "decode_fwd",
    "brute_fwd",
]


def _f64(x) -> np.ndarray:
    """Exact fp64 copy of an array (torch CPU tensors, bf16 included, or numpy)."""
    if hasattr(x, "detach"):  # torch tensor; bf16 has no numpy dtype
        import torch  # local: the oracle itself only needs numpy

        return x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def _bias(rows: np.ndarray, n_keys: int, slope: float) -> np.ndarray:
    """ALiBi bias -slope * |i - j| for query positions ``rows`` and keys [0, n_keys) (reading 4)."""
    j = np.arange(n_keys, dtype=np.float64)
    return -slope * np.abs(rows.astype(np.float64)[:, None] - j[None, :])


def _allowed(rows: np.ndarray, n_keys: int, causal: bool, window) -> np.ndarray:
    """Boolean [len(rows), n_keys]: key j visible from query position i (readings 3 and 9)."""
    i = rows.astype(np.int64)[:, None]
    j = np.arange(n_keys, dtype=np.int64)[None, :]
    ok = np.ones((len(rows), n_keys), dtype=bool)
    if causal:
        ok &= j <= i
    if window is not None:
        left, right = window
        if left >= 0:
            ok &= j >= i - left
        if right >= 0:
            ok &= j <= i + right
    return ok


def _scores(qh, kh, scale, causal, slope, rows=None, window=None, softcap=0.0):
    """S = cap(scale * Q K^T) + beta with the masked entries set to -inf ([PN] Key design 1;
    softcapping and the window are readings 10 and 9)."""
    n = kh.shape[0]
    if rows is None:
        rows = np.arange(qh.shape[0])
    s = scale * (qh @ kh.T)
    if softcap > 0.0:
        s = softcap * np.tanh(s / softcap)
    if slope is not None:
        s = s + _bias(rows, n, slope)
    if causal or window is not None:
        s = np.where(_allowed(rows, n, causal, window), s, -np.inf)
    return s


def _softmax_rows(s):
    """Two-pass softmax of each row of S; also returns lse = m + ln(sum exp(S - m)) ([PN] saved-state table)."""
    m = s.max(axis=1)
    e = np.exp(s - m[:, None])
    ell = e.sum(axis=1)
    return e / ell[:, None], m + np.log(ell)


def head_fwd(qh, kh, vh, scale, causal=False, slope=None, keep=None, keep_scale=1.0, window=None, softcap=0.0):
    """One (sequence, head): O = softmax(S) V and lse. Arrays are [n, d] fp64.

    With a dropout mask ``keep`` [n, n] (boolean), O = (P o keep * keep_scale) V:
    the softmax and lse use every score; dropout acts on the probabilities
    that multiply V ([PN] Key design 1 stage table)."""
    p, lse = _softmax_rows(_scores(qh, kh, scale, causal, slope, window=window, softcap=softcap))
    if keep is not None:
        p = np.where(keep, p * keep_scale, 0.0)
    return p @ vh, lse


def head_rows_fwd(qh, kh, vh, rows, scale, causal=False, slope=None, window=None, softcap=0.0):
    """O and lse for the query positions ``rows`` only (the full K and V are used).

    Row i of the output depends only on q_i, K and V, so a sample of rows can be
    checked at sizes where a whole N x N matrix per head would be wasteful.
    """
    rows = np.asarray(rows, dtype=np.int64)
    p, lse = _softmax_rows(_scores(qh[rows], kh, scale, causal, slope, rows=rows, window=window, softcap=softcap))
    return p @ vh, lse


def head_bwd(qh, kh, vh, doh, scale, causal=False, slope=None, keep=None, keep_scale=1.0, window=None,
             softcap=0.0):
    """Gradients of sum(O * dO) for one (sequence, head), by recomputing P ([PN] Key design 3).

    D_i is taken from its definition sum_j P_ij dP_ij; the identity D_i = dO_i . O_i
    stated on the page is checked by the tests, not assumed here. With a dropout
    mask, O = (P o keep * keep_scale) V, so dV uses the dropped probabilities and
    the gradient reaching P is (dO V^T) o keep * keep_scale. With softcapping the
    gradient reaching the scaled score u is dS * (1 - tanh(u / cap)^2) (reading 10).
    """
    p, _ = _softmax_rows(_scores(qh, kh, scale, causal, slope, window=window, softcap=softcap))
    pd = p if keep is None else np.where(keep, p * keep_scale, 0.0)
    dv = pd.T @ doh
    dp = doh @ vh.T
    if keep is not None:
        dp = np.where(keep, dp * keep_scale, 0.0)
    dcorr = (p * dp).sum(axis=1)
    ds = p * (dp - dcorr[:, None])
    if softcap > 0.0:
        ds = ds * (1.0 - np.tanh(scale * (qh @ kh.T) / softcap) ** 2)
    dq = scale * (ds @ kh)
    dk = scale * (ds.T @ qh)
    return dq, dk, dv


def _sequences(q, cu_seqlens):
    """Yield (b, row slice, n) for dense [B, N, H, d] or packed [T, H, d] inputs."""
    if cu_seqlens is None:
        B, N = q.shape[0], q.shape[1]
        for b in range(B):
            yield b, (b, slice(0, N)), N
    else:
        cu = [int(c) for c in np.asarray(cu_seqlens).reshape(-1)]
        for b in range(len(cu) - 1):
            yield b, (slice(cu[b], cu[b + 1]),), cu[b + 1] - cu[b]


def _heads(q, k):
    H, Hkv = q.shape[-2], k.shape[-2]
    if H % Hkv:
        raise ValueError("query heads must be a multiple of kv heads")
    return H, Hkv, H // Hkv


def _dropout(dropout, n, b, h, H):
    """(keep mask, keep scale) of (sequence b, head h) for dropout=(p_drop, seed, offset), or (None, 1)."""
    if dropout is None:
        return None, 1.0
    p_drop, seed, offset = dropout
    K = PX.keep_threshold(p_drop)
    return PX.dropout_keep(n, n, b, h, H, seed, offset, K), 256.0 / K


def attention_fwd(q, k, v, scale=None, causal=False, alibi_slopes=None, cu_seqlens=None, dropout=None,
                  window=None, softcap=0.0):
    """Exact attention forward in fp64.

    Dense: q [B, N, H, d], k and v [B, N, Hkv, d]. Packed (``cu_seqlens`` given):
    q [T, H, d], k and v [T, Hkv, d]. Returns (o, lse): o in q's layout, lse
    [B, H, Nmax] (NaN past each sequence's end). ``dropout`` = (p_drop, seed,
    offset) applies the mask defined in oracle/philox.py; ``window`` = (left,
    right) and ``softcap`` are readings 9 and 10.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    H, Hkv, G = _heads(q, k)
    d = q.shape[-1]
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    slopes = None if alibi_slopes is None else _f64(alibi_slopes).reshape(-1)
    seqs = list(_sequences(q, cu_seqlens))
    nmax = max([n for _, _, n in seqs] + [0])
    o = np.zeros(q.shape[:-1] + v.shape[-1:])
    lse = np.full((len(seqs), H, nmax), np.nan)
    for b, idx, n in seqs:
        if n == 0:
            continue
        for h in range(H):
            g = h // G
            keep, ks = _dropout(dropout, n, b, h, H)
            oh, lh = head_fwd(q[idx][:, h], k[idx][:, g], v[idx][:, g], scale, causal,
                              None if slopes is None else slopes[h], keep, ks, window, softcap)
            o[idx + (h,)] = oh
            lse[b, h, :n] = lh
    return o, lse


def attention_bwd(q, k, v, do, scale=None, causal=False, alibi_slopes=None, cu_seqlens=None, dropout=None,
                  window=None, softcap=0.0):
    """Exact attention backward in fp64: (dq, dk, dv) of the loss sum(O * dO).

    Layouts as in :func:`attention_fwd`. dk and dv of a kv head sum over its
    G query heads (reading 5); ALiBi slopes are constants and get no gradient.
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    H, Hkv, G = _heads(q, k)
    d = q.shape[-1]
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    slopes = None if alibi_slopes is None else _f64(alibi_slopes).reshape(-1)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b, idx, n in _sequences(q, cu_seqlens):
        if n == 0:
            continue
        for h in range(H):
            g = h // G
            keep, ks = _dropout(dropout, n, b, h, H)
            gq, gk, gv = head_bwd(q[idx][:, h], k[idx][:, g], v[idx][:, g], do[idx][:, h], scale,
                                  causal, None if slopes is None else slopes[h], keep, ks, window, softcap)
            dq[idx + (h,)] = gq
            dk[idx + (g,)] += gk
            dv[idx + (g,)] += gv
    return dq, dk, dv


def tile_state(qh, kh, vh, lo, hi, scale, causal=False, slope=None):
    """Softmax state of one query block against the keys [lo, hi) alone ([PN] Key design 2).

    For each query row i the state is (m_i, l_i, U_i): the largest score of the
    row within these keys, the sum of exp(S_ij - m_i) over them, and the
    unnormalised output sum_j exp(S_ij - m_i) V_j. A row that sees none of
    these keys (all masked) has the empty state (-inf, 0, 0).
    """
    n_q = qh.shape[0]
    rows = np.arange(n_q)
    s = _scores(qh, kh[:hi], scale, causal, slope, rows=rows)[:, lo:hi]
    seen = np.isfinite(s).any(axis=1)
    m = np.full(n_q, -np.inf)
    m[seen] = s[seen].max(axis=1)
    w = np.zeros_like(s)
    w[seen] = np.exp(s[seen] - m[seen][:, None])
    return m, w.sum(axis=1), w @ vh[lo:hi]


def merge_states(a, b):
    """State of the union of two disjoint key sets from the states of each ([PN] Key design 2).

    With m = max(m_a, m_b) every term of a is re-referenced by exp(m_a - m) and
    every term of b by exp(m_b - m); an empty side has weight 0.
    """
    (ma, la, ua), (mb, lb, ub) = a, b
    m = np.maximum(ma, mb)
    wa = np.zeros_like(m)
    wb = np.zeros_like(m)
    fa, fb = np.isfinite(ma), np.isfinite(mb)
    wa[fa] = np.exp(ma[fa] - m[fa])
    wb[fb] = np.exp(mb[fb] - m[fb])
    return m, wa * la + wb * lb, wa[:, None] * ua + wb[:, None] * ub


def online_head_fwd(qh, kh, vh, scale, bounds, causal=False, slope=None, order="stream"):
    """O and lse of one (sequence, head) from per-tile states, combined with :func:`merge_states`.

    Keys are split into the tiles [bounds[t], bounds[t+1]). ``order`` is
    "stream" (fold the tiles left to right, the order in which a kernel
    visits them) or "tree" (merge neighbouring pairs until one state is left).
    Normalisation happens once at the end: O = U / l, lse = m + ln l. By the
    page's Theorem 1 this equals :func:`head_fwd` up to rounding for any split
    and any merge order.
    """
    states = [tile_state(qh, kh, vh, lo, hi, scale, causal, slope)
              for lo, hi in zip(bounds[:-1], bounds[1:]) if hi > lo]
    if order == "stream":
        acc = states[0]
        for st in states[1:]:
            acc = merge_states(acc, st)
    elif order == "tree":
        while len(states) > 1:
            states = [merge_states(states[i], states[i + 1]) if i + 1 < len(states) else states[i]
                      for i in range(0, len(states), 2)]
        acc = states[0]
    else:
        raise ValueError(order)
    m, ell, u = acc
    return u / ell[:, None], m + np.log(ell)


def decode_fwd(q, k_cache, v_cache, cache_seqlens, scale=None, causal=True, alibi_slopes=None):
    """Attention of a few new queries over a key/value cache, in fp64 (the decode
    workload; "FlashAttention: Faster Attention Without Dropping a Single
    Interaction", Limitations: long context and inference, and "If the parent
    paper were rewritten in 2026": a separate single-token decode protocol).

    q [B, Nq, H, d]; k_cache, v_cache [B, Nk, Hkv, d]; cache_seqlens [B]: batch
    entry b holds L_b valid keys (positions 0 .. L_b - 1), and its Nq queries are
    the last Nq tokens of that sequence, at positions L_b - Nq + t. Causal keeps
    key j <= L_b - Nq + t (the mask aligned to the end of the cache); ALiBi adds
    -slope_h |position(t) - j|. Returns o [B, Nq, H, d] and lse [B, H, Nq]; a
    query that sees no key (L_b = 0, or causal with L_b - Nq + t < 0) has
    O = 0 and lse = -inf.
    """
    q, k, v = _f64(q), _f64(k_cache), _f64(v_cache)
    B, Nq, H, d = q.shape
    Hkv = k.shape[2]
    G = H // Hkv
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    slopes = None if alibi_slopes is None else _f64(alibi_slopes).reshape(-1)
    lens = [int(x) for x in np.asarray(cache_seqlens).reshape(-1)]
    o = np.zeros((B, Nq, H, d))
    lse = np.full((B, H, Nq), -np.inf)
    for b in range(B):
        L = lens[b]
        pos = L - Nq + np.arange(Nq)
        for h in range(H):
            g = h // G
            s = scale * (q[b, :, h] @ k[b, :L, g].T)
            if slopes is not None:
                s = s - slopes[h] * np.abs(pos[:, None] - np.arange(L)[None, :]).astype(np.float64)
            if causal:
                s = np.where(np.arange(L)[None, :] > pos[:, None], -np.inf, s)
            seen = np.isfinite(s).any(axis=1) if L else np.zeros(Nq, dtype=bool)
            if not seen.any():
                continue
            p, l = _softmax_rows(s[seen])
            o[b, seen, h] = p @ v[b, :L, g]
            lse[b, h, seen] = l
    return o, lse


def brute_fwd(q, k, v, scale=None, causal=False, alibi_slopes=None, cu_seqlens=None, dropout=None,
              window=None, softcap=0.0):
    """Scalar-loop attention with textbook softmax, for tiny inputs (N <= 8).

    Pure Python: nested lists, ``math.exp`` and running sums, no BLAS and no
    max subtraction. Masked keys are left out of the sums instead of being set to
    -inf. Same layouts and return values as :func:`attention_fwd`.
    """
    qa, ka, va = _f64(q), _f64(k), _f64(v)
    H, Hkv = qa.shape[-2], ka.shape[-2]
    G = H // Hkv
    d = qa.shape[-1]
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    slopes = None if alibi_slopes is None else [float(x) for x in _f64(alibi_slopes).reshape(-1)]
    seqs = list(_sequences(qa, cu_seqlens))
    nmax = max([n for _, _, n in seqs] + [0])
    o = np.zeros(qa.shape[:-1] + va.shape[-1:])
    lse = np.full((len(seqs), H, nmax), np.nan)
    for b, idx, n in seqs:
        qs, ks, vs = qa[idx].tolist(), ka[idx].tolist(), va[idx].tolist()
        o_seq = o[idx]  # basic slicing: a view into o
        for h in range(H):
            g = h // G
            keep, kscale = _dropout(dropout, n, b, h, H)
            for i in range(n):
                lo, hi = 0, (i + 1 if causal else n)
                if window is not None:
                    if window[0] >= 0:
                        lo = max(lo, i - window[0])
                    if window[1] >= 0:
                        hi = min(hi, i + window[1] + 1)
                keys = range(lo, hi)
                w = []
                for j in keys:
                    s = 0.0
                    for c in range(d):
                        s += qs[i][h][c] * ks[j][g][c]
                    s *= scale
                    if softcap > 0.0:
                        s = softcap * math.tanh(s / softcap)
                    if slopes is not None:
                        s -= slopes[h] * abs(i - j)
                    w.append(math.exp(s))
                z = sum(w)
                out = [0.0] * len(vs[0][g]) if n else []
                for wj, j in zip(w, keys):
                    f = 1.0 if keep is None else (kscale if keep[i, j] else 0.0)
                    for c in range(len(out)):
                        out[c] += f * wj / z * vs[j][g][c]
                o_seq[i, h] = out
                lse[b, h, i] = math.log(z)
    return o, lse
