"""Pins of the oracle's sliding-window and softcapping readings (CPU only).

The pages name both variants without formulas ("FlashAttention: Faster
Attention Without Dropping a Single Interaction", Usage contract: the mask row
lists sliding window, ALiBi and softcapping). Readings 9 and 10 of
oracle/attention.py fix them: key j is visible from query i when
i - left <= j <= i + right (negative bound: unbounded; causal applies too), and
the scaled score u becomes cap * tanh(u / cap) before the bias and the masks.

Pins, each independent of the vectorised oracle's own formula:
* brute force: the scalar-loop oracle (its own window bounds and math.tanh)
  on tiny inputs, every variant combined with causal, ALiBi, GQA, varlen;
* reductions: an unbounded window is no window, (left >= n - 1, right = 0) is
  causal, a very large cap is no cap;
* closed forms: window (0, 0) gives O_i = V_i and lse_i = its own score; with
  identical keys the probabilities are uniform over the window, so O_i is the
  mean of V over [i - left, i + right] and lse_i = cap(u) + ln(count);
* central finite differences of sum(O * dO) for the backward with a window
  and with softcapping (the tanh derivative);
* planted mistakes (a window bound off by one, the tanh derivative dropped)
  each fail one of the above.
"""

import math

import numpy as np
import pytest

import oracle.attention as OA

RNG = np.random.default_rng


def _rand(rng, *shape, std=1.0):
    return rng.standard_normal(shape) * std


def _close(a, b, tol):
    a, b = np.asarray(a), np.asarray(b)
    both_nan = np.isnan(a) & np.isnan(b)
    assert np.all(np.abs(np.where(both_nan, 0.0, a - b)) <= tol), np.nanmax(np.abs(a - b))


VARIANTS = [
    dict(window=(2, 1)),
    dict(window=(0, 3), causal=False),
    dict(window=(3, -1)),
    dict(window=(-1, 2)),
    dict(window=(2, 5), causal=True),
    dict(softcap=1.5),
    dict(softcap=0.7, causal=True),
    dict(softcap=2.0, window=(1, 1), alibi=True),
    dict(window=(2, 2), alibi=True, causal=True),
]


@pytest.mark.parametrize("var", VARIANTS, ids=[str(v) for v in VARIANTS])
def test_brute_force_dense(var):
    rng = RNG(80)
    B, N, H, Hkv, d = 2, 7, 4, 2, 3
    q, k, v = _rand(rng, B, N, H, d, std=1.5), _rand(rng, B, N, Hkv, d, std=1.5), _rand(rng, B, N, Hkv, d)
    kw = dict(scale=0.9, causal=var.get("causal", False), window=var.get("window"),
              softcap=var.get("softcap", 0.0),
              alibi_slopes=np.array([0.5, 0.25, 0.125, 0.0625]) if var.get("alibi") else None)
    o, lse = OA.attention_fwd(q, k, v, **kw)
    ob, lb = OA.brute_fwd(q, k, v, **kw)
    _close(o, ob, 1e-13)
    _close(lse, lb, 1e-13)


def test_brute_force_varlen_window_softcap():
    rng = RNG(81)
    lengths, H, Hkv, d = [5, 1, 8, 3], 2, 1, 3
    T = sum(lengths)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    q, k, v = _rand(rng, T, H, d), _rand(rng, T, Hkv, d), _rand(rng, T, Hkv, d)
    kw = dict(cu_seqlens=cu, causal=True, window=(2, 0), softcap=1.2)
    o, lse = OA.attention_fwd(q, k, v, **kw)
    ob, lb = OA.brute_fwd(q, k, v, **kw)
    _close(o, ob, 1e-13)
    _close(lse, lb, 1e-13)


def test_reductions():
    rng = RNG(82)
    B, N, H, d = 1, 9, 2, 4
    q, k, v = _rand(rng, B, N, H, d), _rand(rng, B, N, H, d), _rand(rng, B, N, H, d)
    plain = OA.attention_fwd(q, k, v)
    for w in [(-1, -1), (N - 1, N - 1), (100, -1)]:
        got = OA.attention_fwd(q, k, v, window=w)
        np.testing.assert_array_equal(got[0], plain[0])
        np.testing.assert_array_equal(got[1], plain[1])
    causal = OA.attention_fwd(q, k, v, causal=True)
    for w in [(N - 1, 0), (-1, 0)]:
        got = OA.attention_fwd(q, k, v, window=w)
        np.testing.assert_array_equal(got[0], causal[0])
        np.testing.assert_array_equal(got[1], causal[1])
    # cap * tanh(u / cap) -> u as cap -> inf (the error is about u^3 / (3 cap^2))
    got = OA.attention_fwd(q, k, v, softcap=1e7)
    np.testing.assert_allclose(got[0], plain[0], atol=1e-12)
    np.testing.assert_allclose(got[1], plain[1], atol=1e-12)


def test_window_zero_is_identity():
    rng = RNG(83)
    N, d = 6, 3
    q, k, v = _rand(rng, 1, N, 1, d), _rand(rng, 1, N, 1, d), _rand(rng, 1, N, 1, d)
    o, lse = OA.attention_fwd(q, k, v, scale=0.7, window=(0, 0), softcap=1.3)
    np.testing.assert_allclose(o, v, atol=1e-15)
    own = [1.3 * math.tanh(0.7 * float(q[0, i, 0] @ k[0, i, 0]) / 1.3) for i in range(N)]
    np.testing.assert_allclose(lse[0, 0], own, atol=1e-14)


@pytest.mark.parametrize("window,causal,cap", [((2, 1), False, 0.0), ((3, 0), True, 0.8), ((1, 4), False, 2.5)])
def test_identical_keys_closed_form(window, causal, cap):
    """All keys equal: P is uniform over each row's visible keys."""
    rng = RNG(84)
    N, d = 9, 3
    q = _rand(rng, 1, N, 1, d)
    krow = _rand(rng, d)
    k = np.broadcast_to(krow, (1, N, 1, d)).copy()
    v = _rand(rng, 1, N, 1, d)
    o, lse = OA.attention_fwd(q, k, v, scale=1.1, causal=causal, window=window, softcap=cap)
    for i in range(N):
        lo = max(0, i - window[0]) if window[0] >= 0 else 0
        hi = min(N - 1, i + window[1]) if window[1] >= 0 else N - 1
        if causal:
            hi = min(hi, i)
        u = 1.1 * float(q[0, i, 0] @ krow)
        t = cap * math.tanh(u / cap) if cap > 0 else u
        np.testing.assert_allclose(o[0, i, 0], v[0, lo:hi + 1, 0].mean(axis=0), atol=1e-14)
        assert abs(lse[0, 0, i] - (t + math.log(hi - lo + 1))) < 1e-13


def _loss(q, k, v, do, **kw):
    return float((OA.attention_fwd(q, k, v, **kw)[0] * do).sum())


def _fd_max_rel_err(q, k, v, do, kw, h=1e-6):
    grads = OA.attention_bwd(q, k, v, do, **kw)
    worst = 0.0
    for which, (x, g) in enumerate(zip((q, k, v), grads)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            a_p, a_m = [q, k, v], [q, k, v]
            a_p[which], a_m[which] = xp, xm
            num[idx] = (_loss(*a_p, do, **kw) - _loss(*a_m, do, **kw)) / (2 * h)
        worst = max(worst, np.abs(num - g).max() / max(np.abs(num).max(), 1e-30))
    return worst


def _fd_case(kw, seed=85):
    rng = RNG(seed)
    N, H, Hkv, d = 6, 2, 1, 3
    q, k, v, do = (_rand(rng, 1, N, H, d, std=1.5), _rand(rng, 1, N, Hkv, d, std=1.5), _rand(rng, 1, N, Hkv, d),
                   _rand(rng, 1, N, H, d))
    return q, k, v, do, dict(scale=0.9, **kw)


FD_CASES = [dict(window=(2, 1)), dict(window=(1, 0), causal=True), dict(softcap=0.9),
            dict(softcap=1.4, window=(2, 2), alibi_slopes=np.array([0.3, 0.7]))]


@pytest.mark.parametrize("kw", FD_CASES, ids=[str(sorted(c)) for c in FD_CASES])
def test_finite_differences(kw):
    assert _fd_max_rel_err(*_fd_case(kw)) < 1e-6


def test_planted_mistakes(monkeypatch):
    """A window bound off by one fails the brute-force pin; a backward that drops
    the tanh derivative fails the finite differences."""
    orig_allowed, orig_bwd = OA._allowed, OA.head_bwd

    def allowed_off_by_one(rows, n_keys, causal, window):
        if window is not None and window[0] >= 0:
            window = (window[0] + 1, window[1])
        return orig_allowed(rows, n_keys, causal, window)

    monkeypatch.setattr(OA, "_allowed", allowed_off_by_one)
    with pytest.raises(AssertionError):
        test_brute_force_dense(dict(window=(2, 1)))
    monkeypatch.setattr(OA, "_allowed", orig_allowed)

    def bwd_no_tanh_derivative(qh, kh, vh, doh, scale, causal=False, slope=None, keep=None, keep_scale=1.0,
                               window=None, softcap=0.0):
        # the capped forward, but the gradient of u taken as dS unchanged
        p, _ = OA._softmax_rows(OA._scores(qh, kh, scale, causal, slope, window=window, softcap=softcap))
        dv = p.T @ doh
        dp = doh @ vh.T
        ds = p * (dp - (p * dp).sum(axis=1)[:, None])
        return scale * (ds @ kh), scale * (ds.T @ qh), dv

    monkeypatch.setattr(OA, "head_bwd", bwd_no_tanh_derivative)
    assert _fd_max_rel_err(*_fd_case(dict(softcap=0.9))) > 1e-3
    monkeypatch.setattr(OA, "head_bwd", orig_bwd)
