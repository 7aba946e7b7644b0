"""Pins for the fp64 oracle: closed forms, invariants, brute force and finite differences.

None of these re-types the oracle's formulas: each checks it against something
the definition fixes independently ("FlashAttention: Faster Attention Without
Dropping a Single Interaction", Method Deep Dive, Key designs 1-3). The
``test_planted_mistakes`` case plants plausible mistakes in the oracle (on the
CPU) and checks that some pin fails for each.
"""

import json
import math
import os
import types

import numpy as np
import pytest

import oracle.attention as OA

HERE = os.path.dirname(os.path.abspath(__file__))
RNG = np.random.default_rng


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _varlen_pack(rng, lengths, H, Hkv, d):
    T = int(sum(lengths))
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    return _rand(rng, T, H, d), _rand(rng, T, Hkv, d), _rand(rng, T, Hkv, d), _rand(rng, T, H, d), cu


VARIANTS = [
    # (causal, alibi, H, Hkv)
    (False, False, 2, 2),
    (True, False, 2, 2),
    (False, True, 2, 2),
    (True, True, 2, 2),
    (True, False, 4, 2),
    (False, True, 3, 1),
]


# --------------------------------------------------------------------------- pins
# Each pin takes the oracle as a namespace so the planted-mistake test can run
# the same checks against a broken copy.

def pin_brute_dense(orc):
    rng = RNG(1)
    for causal, alibi, H, Hkv in VARIANTS:
        for N, d in ((1, 3), (5, 4), (8, 2)):
            q, k, v = _rand(rng, 2, N, H, d), _rand(rng, 2, N, Hkv, d), _rand(rng, 2, N, Hkv, d)
            sl = rng.uniform(0.05, 1.0, size=H) if alibi else None
            o, l = orc.attention_fwd(q, k, v, scale=0.7, causal=causal, alibi_slopes=sl)
            ob, lb = OA.brute_fwd(q, k, v, scale=0.7, causal=causal, alibi_slopes=sl)
            np.testing.assert_allclose(o, ob, rtol=0, atol=1e-13)
            np.testing.assert_allclose(l, lb, rtol=0, atol=1e-13)


def pin_brute_varlen(orc):
    rng = RNG(2)
    for causal, alibi, H, Hkv in VARIANTS:
        lengths = [3, 0, 8, 1, 5]
        q, k, v, _, cu = _varlen_pack(rng, lengths, H, Hkv, 3)
        sl = rng.uniform(0.05, 1.0, size=H) if alibi else None
        o, l = orc.attention_fwd(q, k, v, causal=causal, alibi_slopes=sl, cu_seqlens=cu)
        ob, lb = OA.brute_fwd(q, k, v, causal=causal, alibi_slopes=sl, cu_seqlens=cu)
        np.testing.assert_allclose(o, ob, rtol=0, atol=1e-13)
        np.testing.assert_allclose(l, lb, rtol=0, atol=1e-13, equal_nan=True)


def pin_rows_sum_to_one(orc):
    """With V = 1 every output is 1 because each row of P sums to 1."""
    rng = RNG(3)
    for causal, alibi, H, Hkv in VARIANTS:
        q, k = _rand(rng, 2, 37, H, 5), _rand(rng, 2, 37, Hkv, 5)
        v = np.ones((2, 37, Hkv, 5))
        sl = rng.uniform(0.05, 1.0, size=H) if alibi else None
        o, _ = orc.attention_fwd(q, k, v, causal=causal, alibi_slopes=sl)
        np.testing.assert_allclose(o, 1.0, rtol=0, atol=1e-14)


def pin_identical_keys(orc):
    """All keys equal: P is uniform over the allowed keys, O is the mean of those V, dQ = 0."""
    rng = RNG(4)
    N, d, scale = 9, 4, 0.3
    for causal in (False, True):
        q, v, do = _rand(rng, 1, N, 1, d), _rand(rng, 1, N, 1, d), _rand(rng, 1, N, 1, d)
        k = np.broadcast_to(_rand(rng, 1, 1, 1, d), (1, N, 1, d)).copy()
        o, lse = orc.attention_fwd(q, k, v, scale=scale, causal=causal)
        for i in range(N):
            n_i = i + 1 if causal else N
            np.testing.assert_allclose(o[0, i, 0], v[0, :n_i, 0].mean(axis=0), atol=1e-14)
            s_i = scale * float(q[0, i, 0] @ k[0, 0, 0])
            assert abs(lse[0, 0, i] - (s_i + math.log(n_i))) < 1e-13
        dq, _, _ = orc.attention_bwd(q, k, v, do, scale=scale, causal=causal)
        np.testing.assert_allclose(dq, 0.0, atol=1e-14)


def pin_dominant_score(orc):
    """One score larger than the rest by delta: O copies that V row up to O(e^-delta)."""
    rng = RNG(5)
    N, d = 6, 4
    k = np.zeros((1, N, 1, d))
    for j in range(N):
        k[0, j, 0, j % d] = 1.0 if j < d else -1.0
    q = np.zeros((1, N, 1, d))
    q[0, :, 0, 2] = 40.0  # row i scores key 2 at 40 and every other key at <= 0
    v = _rand(rng, 1, N, 1, d)
    o, lse = orc.attention_fwd(q, k, v, scale=1.0)
    np.testing.assert_allclose(o[0, :, 0], np.broadcast_to(v[0, 2, 0], (N, d)), atol=1e-15)
    np.testing.assert_allclose(lse[0, 0], 40.0, atol=1e-15)


def pin_causal_row0(orc):
    """Causal row 0 sees only key 0: O_0 = V_0 and lse_0 = S_00."""
    rng = RNG(6)
    q, k, v = _rand(rng, 2, 7, 3, 5), _rand(rng, 2, 7, 3, 5), _rand(rng, 2, 7, 3, 5)
    sl = np.array([0.5, 0.25, 0.125])
    o, lse = orc.attention_fwd(q, k, v, scale=0.4, causal=True, alibi_slopes=sl)
    np.testing.assert_allclose(o[:, 0], v[:, 0], atol=1e-15)
    s00 = 0.4 * np.einsum("bhc,bhc->bh", q[:, 0], k[:, 0])
    np.testing.assert_allclose(lse[:, :, 0], s00, atol=1e-15)


def pin_hand_cases(orc):
    """Tiny problems solved by hand (tests/golden/hand_cases.json)."""
    with open(os.path.join(HERE, "golden", "hand_cases.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        q, k, v = (np.array(c[x]) for x in ("q", "k", "v"))
        sl = None if c["alibi_slopes"] is None else np.array(c["alibi_slopes"])
        o, lse = orc.attention_fwd(q, k, v, scale=c["scale"], causal=c["causal"], alibi_slopes=sl)
        np.testing.assert_allclose(o, np.array(c["o"]), rtol=0, atol=1e-15)
        np.testing.assert_allclose(lse, np.array(c["lse"]), rtol=0, atol=1e-15)
        if "do" in c:
            dq, dk, dv = orc.attention_bwd(q, k, v, np.array(c["do"]), scale=c["scale"],
                                           causal=c["causal"], alibi_slopes=sl)
            for got, key in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
                np.testing.assert_allclose(got, np.array(c[key]), rtol=0, atol=1e-15)


def pin_permutation(orc):
    """Non-causal, no bias: permuting keys and values together leaves O and lse unchanged."""
    rng = RNG(7)
    q, k, v = _rand(rng, 2, 11, 4, 6), _rand(rng, 2, 11, 2, 6), _rand(rng, 2, 11, 2, 6)
    perm = rng.permutation(11)
    o1, l1 = orc.attention_fwd(q, k, v)
    o2, l2 = orc.attention_fwd(q, k[:, perm], v[:, perm])
    np.testing.assert_allclose(o1, o2, atol=1e-14)
    np.testing.assert_allclose(l1, l2, atol=1e-14)


def pin_row_shift(orc):
    """k_j -> k_j + u adds scale*<q_i,u> to every score of row i: O unchanged, lse shifted."""
    rng = RNG(8)
    scale = 0.35
    for causal in (False, True):
        q, k, v = _rand(rng, 1, 10, 2, 4), _rand(rng, 1, 10, 2, 4), _rand(rng, 1, 10, 2, 4)
        u = _rand(rng, 4)
        o1, l1 = orc.attention_fwd(q, k, v, scale=scale, causal=causal)
        o2, l2 = orc.attention_fwd(q, k + u, v, scale=scale, causal=causal)
        shift = scale * np.einsum("bnhc,c->bhn", q, u)
        np.testing.assert_allclose(o1, o2, atol=1e-13)
        np.testing.assert_allclose(l2 - l1, shift, atol=1e-13)


def pin_alibi_as_extra_dim(orc):
    """Causal ALiBi -slope*(i-j) = slope*j - slope*i: the slope*j part is one extra head
    dimension (q' = 1, k'_j = slope*j/scale), the -slope*i part a per-row shift of lse."""
    rng = RNG(9)
    N, d, scale = 13, 4, 0.5
    slopes = np.array([0.5, 0.0625])
    q, k, v = _rand(rng, 1, N, 2, d), _rand(rng, 1, N, 2, d), _rand(rng, 1, N, 2, d)
    o, lse = orc.attention_fwd(q, k, v, scale=scale, causal=True, alibi_slopes=slopes)
    for h in range(2):
        qa = np.concatenate([q[:, :, h:h + 1], np.ones((1, N, 1, 1))], axis=-1)
        ka = np.concatenate([k[:, :, h:h + 1], (slopes[h] * np.arange(N) / scale).reshape(1, N, 1, 1)], axis=-1)
        oa, la = orc.attention_fwd(qa, ka, v[:, :, h:h + 1], scale=scale, causal=True)
        np.testing.assert_allclose(o[:, :, h:h + 1], oa, atol=1e-13)
        np.testing.assert_allclose(lse[0, h], la[0, 0] - slopes[h] * np.arange(N), atol=1e-12)
    # slope 0 is no bias at all
    o0, l0 = orc.attention_fwd(q, k, v, scale=scale, causal=True, alibi_slopes=np.zeros(2))
    o1, l1 = orc.attention_fwd(q, k, v, scale=scale, causal=True)
    np.testing.assert_allclose(o0, o1, atol=1e-15)
    np.testing.assert_allclose(l0, l1, atol=1e-15)


def pin_gqa_is_repeated_mha(orc):
    """GQA equals MHA with each kv head repeated for its G consecutive query heads;
    dK and dV are the group sums of the MHA gradients."""
    rng = RNG(10)
    B, N, H, Hkv, d = 2, 9, 6, 2, 3
    G = H // Hkv
    for causal in (False, True):
        q, do = _rand(rng, B, N, H, d), _rand(rng, B, N, H, d)
        k, v = _rand(rng, B, N, Hkv, d), _rand(rng, B, N, Hkv, d)
        kr, vr = np.repeat(k, G, axis=2), np.repeat(v, G, axis=2)
        o1, l1 = orc.attention_fwd(q, k, v, causal=causal)
        o2, l2 = orc.attention_fwd(q, kr, vr, causal=causal)
        np.testing.assert_allclose(o1, o2, atol=1e-14)
        np.testing.assert_allclose(l1, l2, atol=1e-14)
        g1 = orc.attention_bwd(q, k, v, do, causal=causal)
        g2 = orc.attention_bwd(q, kr, vr, do, causal=causal)
        np.testing.assert_allclose(g1[0], g2[0], atol=1e-14)
        np.testing.assert_allclose(g1[1], g2[1].reshape(B, N, Hkv, G, d).sum(axis=3), atol=1e-13)
        np.testing.assert_allclose(g1[2], g2[2].reshape(B, N, Hkv, G, d).sum(axis=3), atol=1e-13)


def pin_varlen_is_independent_dense(orc):
    rng = RNG(11)
    lengths = [4, 1, 9, 0, 6]
    q, k, v, do, cu = _varlen_pack(rng, lengths, 4, 2, 3)
    sl = np.array([0.3, 0.2, 0.1, 0.05])
    o, lse = orc.attention_fwd(q, k, v, causal=True, alibi_slopes=sl, cu_seqlens=cu)
    dq, dk, dv = orc.attention_bwd(q, k, v, do, causal=True, alibi_slopes=sl, cu_seqlens=cu)
    for b, n in enumerate(lengths):
        a, e = cu[b], cu[b + 1]
        if n == 0:
            continue
        ob, lb = orc.attention_fwd(q[None, a:e], k[None, a:e], v[None, a:e], causal=True, alibi_slopes=sl)
        gb = orc.attention_bwd(q[None, a:e], k[None, a:e], v[None, a:e], do[None, a:e], causal=True,
                               alibi_slopes=sl)
        np.testing.assert_allclose(o[a:e], ob[0], atol=1e-14)
        np.testing.assert_allclose(lse[b, :, :n], lb[0], atol=1e-14)
        for g_all, g_b in zip((dq, dk, dv), gb):
            np.testing.assert_allclose(g_all[a:e], g_b[0], atol=1e-14)


def _loss(orc, q, k, v, do, **kw):
    o, _ = orc.attention_fwd(q, k, v, **kw)
    return float((o * do).sum())


def pin_finite_differences(orc):
    """Central differences of sum(O * dO) against every element of Q, K and V."""
    rng = RNG(12)
    h = 1e-6
    cases = [
        dict(causal=False, alibi=False, H=2, Hkv=2, N=4, d=3, lengths=None),
        dict(causal=True, alibi=False, H=2, Hkv=1, N=5, d=2, lengths=None),
        dict(causal=True, alibi=True, H=2, Hkv=2, N=6, d=2, lengths=None),
        dict(causal=False, alibi=True, H=2, Hkv=1, N=4, d=2, lengths=None),
        dict(causal=True, alibi=True, H=2, Hkv=1, N=None, d=2, lengths=[3, 0, 4]),
    ]
    for c in cases:
        if c["lengths"] is None:
            q, k, v = _rand(rng, 1, c["N"], c["H"], c["d"]), _rand(rng, 1, c["N"], c["Hkv"], c["d"]), \
                _rand(rng, 1, c["N"], c["Hkv"], c["d"])
            do = _rand(rng, 1, c["N"], c["H"], c["d"])
            cu = None
        else:
            q, k, v, do, cu = _varlen_pack(rng, c["lengths"], c["H"], c["Hkv"], c["d"])
        kw = dict(scale=0.8, causal=c["causal"], cu_seqlens=cu,
                  alibi_slopes=np.array([0.6, 0.3]) if c["alibi"] else None)
        grads = orc.attention_bwd(q, k, v, do, **kw)
        for which, (x, g) in enumerate(zip((q, k, v), grads)):
            num = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                xp, xm = x.copy(), x.copy()
                xp[idx] += h
                xm[idx] -= h
                args_p = [q, k, v]
                args_m = [q, k, v]
                args_p[which], args_m[which] = xp, xm
                num[idx] = (_loss(orc, *args_p, do, **kw) - _loss(orc, *args_m, do, **kw)) / (2 * h)
            err = np.abs(num - g).max() / max(np.abs(num).max(), 1e-30)
            assert err < 1e-6, (c, which, err)


def pin_backward_identities(orc):
    """D_i = sum_j P_ij dP_ij equals dO_i . O_i; rows of dS sum to 0, hence sum_j dK_j = 0
    per (b, kv head); rows of P sum to 1, hence sum_j dV_j = sum_i dO_i per kv group."""
    rng = RNG(13)
    B, N, H, Hkv, d = 2, 12, 4, 2, 5
    for causal in (False, True):
        q, do = _rand(rng, B, N, H, d), _rand(rng, B, N, H, d)
        k, v = _rand(rng, B, N, Hkv, d), _rand(rng, B, N, Hkv, d)
        o, _ = orc.attention_fwd(q, k, v, causal=causal)
        dq, dk, dv = orc.attention_bwd(q, k, v, do, causal=causal)
        np.testing.assert_allclose(dk.sum(axis=1), 0.0, atol=1e-12)
        grp = do.reshape(B, N, Hkv, H // Hkv, d).sum(axis=(1, 3))
        np.testing.assert_allclose(dv.sum(axis=1), grp, atol=1e-12)
        # D from the definition (head_bwd) vs dO . O: compare via the dQ it implies.
        for b in range(B):
            for hh in range(H):
                g = hh // (H // Hkv)
                s = orc._scores(q[b, :, hh], k[b, :, g], 1 / math.sqrt(d), causal, None)
                p = np.exp(s - s.max(axis=1, keepdims=True))
                p /= p.sum(axis=1, keepdims=True)
                dp = do[b, :, hh] @ v[b, :, g].T
                np.testing.assert_allclose((p * dp).sum(axis=1), (do[b, :, hh] * o[b, :, hh]).sum(axis=1),
                                           atol=1e-12)


def pin_online_equals_two_pass(orc):
    """Blockwise online recurrence with random tile splits equals the two-pass definition."""
    rng = RNG(14)
    for causal, alibi, _, _ in VARIANTS:
        n, d = 23, 6
        q, k, v = _rand(rng, n, d), _rand(rng, n, d), _rand(rng, n, d)
        slope = 0.3 if alibi else None
        o_ref, l_ref = orc.head_fwd(q, k, v, 0.45, causal, slope)
        splits = [list(range(n + 1)),  # B_c = 1
                  [0, n],  # one tile
                  [0, 8, 16, n],  # uneven last tile
                  sorted(set([0, n] + list(rng.integers(1, n, size=5))))]
        for b in splits:
            for order in ("stream", "tree"):
                o, l = OA.online_head_fwd(q, k, v, 0.45, b, causal, slope, order=order)
                np.testing.assert_allclose(o, o_ref, atol=1e-12)
                np.testing.assert_allclose(l, l_ref, atol=1e-12)


def pin_merge_state_by_hand(orc):
    """Two one-key states merged by hand: keys with scores 0 and ln 3 give weights 1/4 and 3/4."""
    a = (np.array([0.0]), np.array([1.0]), np.array([[2.0, -4.0]]))
    b = (np.array([math.log(3.0)]), np.array([1.0]), np.array([[6.0, 8.0]]))
    for x, y in ((a, b), (b, a)):
        m, ell, u = OA.merge_states(x, y)
        np.testing.assert_allclose(m, [math.log(3.0)], atol=1e-15)
        np.testing.assert_allclose(u / ell[:, None], [[0.25 * 2 + 0.75 * 6, 0.25 * -4 + 0.75 * 8]], atol=1e-14)
        np.testing.assert_allclose(m + np.log(ell), [math.log(4.0)], atol=1e-15)
    empty = (np.array([-np.inf]), np.array([0.0]), np.zeros((1, 2)))
    for x, y in ((a, empty), (empty, a)):
        m, ell, u = OA.merge_states(x, y)
        assert m[0] == 0.0 and ell[0] == 1.0 and np.array_equal(u, a[2])


def pin_rows_fwd(orc):
    """The sampled-rows entry gives the same rows as the full computation."""
    rng = RNG(15)
    n, d = 40, 8
    q, k, v = _rand(rng, n, d), _rand(rng, n, d), _rand(rng, n, d)
    rows = np.array([0, 1, 17, 39])
    for causal in (False, True):
        o, l = orc.head_fwd(q, k, v, 0.3, causal, 0.1)
        orow, lrow = orc.head_rows_fwd(q, k, v, rows, 0.3, causal, 0.1)
        np.testing.assert_allclose(orow, o[rows], atol=1e-14)
        np.testing.assert_allclose(lrow, l[rows], atol=1e-14)


PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin(OA)


# ------------------------------------------------------------------ planted mistakes

def _mutant(**overrides):
    """A copy of the oracle namespace whose public functions use mutated helpers."""
    src = {k: getattr(OA, k) for k in dir(OA) if not k.startswith("__")}
    ns = dict(src)
    ns.update(overrides)
    mod = types.ModuleType("oracle_mutant")
    # re-bind the public functions to this namespace so they see the mutated helpers
    for name in ("attention_fwd", "attention_bwd", "head_fwd", "head_bwd", "head_rows_fwd"):
        if name in overrides:
            continue
        f = src[name]
        ns[name] = types.FunctionType(f.__code__, ns, name, f.__defaults__, f.__closure__)
    for k, v in ns.items():
        setattr(mod, k, v)
    return mod


def _m_scores_no_scale(qh, kh, scale, causal, slope, rows=None, window=None, softcap=0.0):
    return OA._scores(qh, kh, 1.0, causal, slope, rows, window, softcap)


def _m_scores_transposed(qh, kh, scale, causal, slope, rows=None, window=None, softcap=0.0):
    n = kh.shape[0]
    rows = np.arange(qh.shape[0]) if rows is None else rows
    s = scale * (kh @ qh.T)[: len(rows)] if kh.shape[0] == qh.shape[0] else scale * (qh @ kh.T)
    if slope is not None:
        s = s + OA._bias(rows, n, slope)
    if causal:
        s = np.where(np.arange(n)[None, :] > rows[:, None], -np.inf, s)
    return s


def _m_scores_alibi_sign(qh, kh, scale, causal, slope, rows=None, window=None, softcap=0.0):
    return OA._scores(qh, kh, scale, causal, None if slope is None else -slope, rows, window, softcap)


def _m_scores_mask_off_by_one(qh, kh, scale, causal, slope, rows=None, window=None, softcap=0.0):
    s = OA._scores(qh, kh, scale, False, slope, rows, window, softcap)
    if causal:
        n = kh.shape[0]
        rows = np.arange(qh.shape[0]) if rows is None else rows
        s = np.where(np.arange(n)[None, :] >= rows[:, None] + 2, -np.inf, s)
    return s


def _m_softmax_no_max_in_lse(s):
    p, lse = OA._softmax_rows(s)
    return p, lse - s.max(axis=1)


def _m_head_bwd_no_scale(qh, kh, vh, doh, scale, causal=False, slope=None, keep=None, keep_scale=1.0, window=None,
                         softcap=0.0):
    dq, dk, dv = OA.head_bwd(qh, kh, vh, doh, scale, causal, slope, keep, keep_scale, window, softcap)
    return dq / scale, dk, dv


def _m_head_bwd_ds_sign(qh, kh, vh, doh, scale, causal=False, slope=None, keep=None, keep_scale=1.0, window=None,
                        softcap=0.0):
    p, _ = OA._softmax_rows(OA._scores(qh, kh, scale, causal, slope))
    dp = doh @ vh.T
    ds = p * (dp + (p * dp).sum(axis=1)[:, None])
    return scale * ds @ kh, scale * ds.T @ qh, p.T @ doh


def _m_head_bwd_dv_untransposed(qh, kh, vh, doh, scale, causal=False, slope=None, keep=None, keep_scale=1.0,
                                window=None, softcap=0.0):
    dq, dk, _ = OA.head_bwd(qh, kh, vh, doh, scale, causal, slope, keep, keep_scale, window, softcap)
    p, _ = OA._softmax_rows(OA._scores(qh, kh, scale, causal, slope))
    return dq, dk, p @ doh


def _m_heads_modulo(q, k):
    H, Hkv = q.shape[-2], k.shape[-2]
    return H, Hkv, 1 if H == Hkv else H // Hkv + 1  # wrong group size


MUTANTS = {
    "score_scale_dropped": dict(_scores=_m_scores_no_scale),
    "scores_transposed": dict(_scores=_m_scores_transposed),
    "alibi_sign_flipped": dict(_scores=_m_scores_alibi_sign),
    "causal_mask_off_by_one": dict(_scores=_m_scores_mask_off_by_one),
    "lse_drops_max": dict(_softmax_rows=_m_softmax_no_max_in_lse),
    "dq_scale_dropped": dict(head_bwd=_m_head_bwd_no_scale),
    "ds_sign_flipped": dict(head_bwd=_m_head_bwd_ds_sign),
    "dv_untransposed": dict(head_bwd=_m_head_bwd_dv_untransposed),
    "gqa_group_wrong": dict(_heads=_m_heads_modulo),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistakes(name):
    """Each planted mistake in a copy of the oracle is caught by at least one pin."""
    mod = _mutant(**MUTANTS[name])
    caught = []
    for pin in PINS:
        try:
            pin(mod)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {name}"


# ------------------------------------------------------------------ decode (KV cache)

def test_decode_is_the_last_rows_of_causal_attention():
    """Causal decode of the last Nq tokens equals those rows of full causal attention
    over the same sequence (with ALiBi and GQA); the cache rows past L_b are ignored."""
    rng = RNG(60)
    B, H, Hkv, d, Nk, Nq = 3, 4, 2, 5, 20, 3
    lens = [20, 7, 3]
    qf = _rand(rng, B, Nk, H, d)
    k, v = _rand(rng, B, Nk, Hkv, d), _rand(rng, B, Nk, Hkv, d)
    sl = np.array([0.5, 0.25, 0.125, 0.0625])
    q = np.stack([qf[b, lens[b] - Nq:lens[b]] for b in range(B)])
    o, lse = OA.decode_fwd(q, k, v, lens, scale=0.6, causal=True, alibi_slopes=sl)
    for b in range(B):
        L = lens[b]
        of, lf = OA.attention_fwd(qf[None, b, :L], k[None, b, :L], v[None, b, :L], scale=0.6, causal=True,
                                  alibi_slopes=sl)
        np.testing.assert_allclose(o[b], of[0, L - Nq:], atol=1e-14)
        np.testing.assert_allclose(lse[b], lf[0, :, L - Nq:], atol=1e-14)
    # garbage in the cache past each length changes nothing
    k2, v2 = k.copy(), v.copy()
    for b in range(B):
        k2[b, lens[b]:] = 1e3
        v2[b, lens[b]:] = -1e3
    o2, l2 = OA.decode_fwd(q, k2, v2, lens, scale=0.6, causal=True, alibi_slopes=sl)
    assert np.array_equal(o, o2) and np.array_equal(lse, l2)


def test_decode_non_causal_and_empty():
    """Non-causal decode is attention of the queries over the valid cache; a query
    that sees no key gives O = 0, lse = -inf."""
    rng = RNG(61)
    q, k, v = _rand(rng, 2, 2, 2, 4), _rand(rng, 2, 9, 1, 4), _rand(rng, 2, 9, 1, 4)
    o, lse = OA.decode_fwd(q, k, v, [9, 0], causal=False)
    ob, lb = OA.brute_fwd(np.concatenate([q[:1], np.zeros((1, 7, 2, 4))], axis=1)[:, :9],
                          k[:1], v[:1], scale=0.5, causal=False)
    np.testing.assert_allclose(o[0], ob[0, :2], atol=1e-13)
    np.testing.assert_allclose(lse[0], lb[0, :, :2], atol=1e-13)
    assert np.all(o[1] == 0) and np.all(lse[1] == -np.inf)
    # causal with fewer keys than queries: the first query of a 1-key cache sees nothing
    o, lse = OA.decode_fwd(q, k, v, [1, 2], causal=True)
    assert lse[0, 0, 0] == -np.inf and np.all(o[0, 0] == 0)
    np.testing.assert_allclose(o[0, 1, :], np.broadcast_to(v[0, 0, 0], (2, 4)), atol=1e-15)


def test_decode_split_merge():
    """States of key splits merged with merge_states give the decode output (the
    split-KV combine of Key design 2)."""
    rng = RNG(62)
    L, d = 37, 6
    q, k, v = _rand(rng, 2, d), _rand(rng, L, d), _rand(rng, L, d)
    ref_o, ref_l = OA.head_fwd(q, k, v, 0.4)
    for splits in ([0, 10, 37], [0, 1, 2, 3, 37], [0, 20, 36, 37]):
        states = [OA.tile_state(q, k, v, lo, hi, 0.4, False) for lo, hi in zip(splits[:-1], splits[1:])]
        acc = states[0]
        for st in states[1:]:
            acc = OA.merge_states(acc, st)
        m, ell, u = acc
        np.testing.assert_allclose(u / ell[:, None], ref_o, atol=1e-13)
        np.testing.assert_allclose(m + np.log(ell), ref_l, atol=1e-13)
