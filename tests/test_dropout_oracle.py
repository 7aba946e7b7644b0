"""Pins for the dropout parts of the oracle: the Philox-4x32-10 generator and the
mask (oracle/philox.py) and dropout attention forward/backward (oracle/attention.py).

The generator is checked against the known-answer vectors published with it
(tests/golden/philox_kat.json), for its avalanche behaviour, and the mask for
its keep rate; dropout attention against p = 0 (plain attention), a scalar-loop
brute force, its expectation over seeds (the undropped output), central finite
differences of sum(O * dO) at a fixed mask, and the identity D_i = dO_i . O_i.
Sources: "FlashAttention: Faster Attention Without Dropping a Single
Interaction", Method Deep Dive, Key design 1 (stage table: dropout is fused and
its mask regenerated from the saved generator state) and Key design 3.
"""

import json
import os

import numpy as np
import pytest

import oracle.attention as OA
import oracle.philox as PX

HERE = os.path.dirname(os.path.abspath(__file__))
RNG = np.random.default_rng


def _h(x):
    return np.array([int(w, 16) for w in x], dtype=np.uint64)


def test_philox_known_answers():
    with open(os.path.join(HERE, "golden", "philox_kat.json")) as f:
        vecs = json.load(f)["vectors"]
    for v in vecs:
        out = PX.philox4x32(_h(v["counter"]), _h(v["key"]))
        assert [int(x) for x in out] == [int(w, 16) for w in v["out"]]


def test_philox_avalanche():
    """Flipping one counter bit changes about half of the 128 output bits."""
    rng = RNG(40)
    ctr = rng.integers(0, 2 ** 32, size=(64, 4), dtype=np.uint64)
    key = rng.integers(0, 2 ** 32, size=(64, 2), dtype=np.uint64)
    base = PX.philox4x32(ctr, key)
    flips = []
    for bit in range(128):
        c2 = ctr.copy()
        c2[:, bit // 32] ^= np.uint64(1 << (bit % 32))
        diff = PX.philox4x32(c2, key) ^ base
        flips.append(np.unpackbits(diff.view(np.uint8), axis=-1).sum(axis=-1))
    f = np.concatenate(flips).astype(np.float64)
    assert abs(f.mean() - 64.0) < 0.5 and 4.0 < f.std() < 7.0  # binomial(128, 1/2): sd 5.66


def test_mask_element_mapping():
    """The vectorised mask equals the per-element definition, one generator call each."""
    n, H, b, h, seed, offset, K = 70, 3, 1, 2, 0x1234_5678_9ABC_DEF0, 7, 200
    keep = PX.dropout_keep(n, n, b, h, H, seed, offset, K)
    rng = RNG(41)
    for i, j in zip(rng.integers(0, n, 300), rng.integers(0, n, 300)):
        ctr = np.array([2 * (j // 32) + (j // 4) % 2, i, b * H + h, offset], dtype=np.uint64)
        key = np.array([seed & 0xFFFFFFFF, seed >> 32], dtype=np.uint64)
        word = int(PX.philox4x32(ctr, key)[(j % 32) // 8])
        byte = (word >> (8 * (j % 4))) & 0xFF
        assert keep[i, j] == (byte < K)


@pytest.mark.parametrize("p_drop", [0.1, 0.5, 0.9])
def test_mask_keep_rate(p_drop):
    K = PX.keep_threshold(p_drop)
    assert abs(K / 256 - (1 - p_drop)) <= 0.5 / 256
    keep = PX.dropout_keep(512, 512, 0, 0, 1, 99, 0, K)
    n = keep.size
    rate = keep.mean()
    sd = np.sqrt(K / 256 * (1 - K / 256) / n)
    assert abs(rate - K / 256) < 5 * sd
    # different heads, offsets and seeds give different masks; the same give the same
    assert np.array_equal(keep, PX.dropout_keep(512, 512, 0, 0, 1, 99, 0, K))
    assert not np.array_equal(keep, PX.dropout_keep(512, 512, 0, 0, 1, 99, 1, K))
    assert not np.array_equal(keep, PX.dropout_keep(512, 512, 0, 0, 1, 98, 0, K))


def test_keep_threshold_bounds():
    assert PX.keep_threshold(0.0) == 256
    assert PX.keep_threshold(0.5) == 128 and PX.keep_threshold(0.997) == 1
    for bad in (-0.1, 1.0, 1.5, float("nan")):
        with pytest.raises(ValueError):
            PX.keep_threshold(bad)
    with pytest.raises(ValueError):
        PX.keep_threshold(0.9990)  # rounds to K = 0: everything dropped


def _rand(rng, *shape):
    return rng.standard_normal(shape)


@pytest.mark.parametrize("causal,alibi", [(False, False), (True, True)])
def test_dropout_zero_is_plain(causal, alibi):
    rng = RNG(42)
    q, k, v, do = _rand(rng, 2, 40, 4, 8), _rand(rng, 2, 40, 2, 8), _rand(rng, 2, 40, 2, 8), _rand(rng, 2, 40, 4, 8)
    sl = np.array([0.3, 0.2, 0.1, 0.05]) if alibi else None
    o1, l1 = OA.attention_fwd(q, k, v, causal=causal, alibi_slopes=sl)
    o2, l2 = OA.attention_fwd(q, k, v, causal=causal, alibi_slopes=sl, dropout=(0.0, 5, 6))
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    for g1, g2 in zip(OA.attention_bwd(q, k, v, do, causal=causal, alibi_slopes=sl),
                      OA.attention_bwd(q, k, v, do, causal=causal, alibi_slopes=sl, dropout=(0.0, 5, 6))):
        assert np.array_equal(g1, g2)


@pytest.mark.parametrize("causal,alibi,H,Hkv", [(False, False, 2, 2), (True, True, 4, 2), (True, False, 2, 1)])
def test_dropout_brute(causal, alibi, H, Hkv):
    rng = RNG(43)
    for N, d in ((5, 3), (8, 2)):
        q, k, v = _rand(rng, 2, N, H, d), _rand(rng, 2, N, Hkv, d), _rand(rng, 2, N, Hkv, d)
        sl = rng.uniform(0.05, 1.0, size=H) if alibi else None
        kw = dict(scale=0.7, causal=causal, alibi_slopes=sl, dropout=(0.4, 123, 4))
        o, l = OA.attention_fwd(q, k, v, **kw)
        ob, lb = OA.brute_fwd(q, k, v, **kw)
        np.testing.assert_allclose(o, ob, rtol=0, atol=1e-13)
        np.testing.assert_allclose(l, lb, rtol=0, atol=1e-13)
        # lse does not depend on the mask
        np.testing.assert_array_equal(l, OA.attention_fwd(q, k, v, scale=0.7, causal=causal, alibi_slopes=sl)[1])


def test_dropout_expectation():
    """Averaged over seeds, the dropped output is the undropped one (the 256/K scale)."""
    rng = RNG(44)
    q, k, v = _rand(rng, 1, 12, 1, 4), _rand(rng, 1, 12, 1, 4), _rand(rng, 1, 12, 1, 4)
    o_ref, _ = OA.attention_fwd(q, k, v)
    outs = np.stack([OA.attention_fwd(q, k, v, dropout=(0.3, s, 0))[0] for s in range(4000)])
    mean, sd = outs.mean(axis=0), outs.std(axis=0) / np.sqrt(len(outs))
    assert np.all(np.abs(mean - o_ref) < 5 * sd + 1e-12)


def _loss(q, k, v, do, **kw):
    return float((OA.attention_fwd(q, k, v, **kw)[0] * do).sum())


def _fd_max_rel_err(q, k, v, do, kw, h=1e-6):
    """Largest relative gap between attention_bwd and central differences of sum(O * dO)."""
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


def _fd_case(causal, alibi, Hkv, seed=45):
    rng = RNG(seed)
    N, H, d = 6, 2, 3
    q, k, v, do = _rand(rng, 1, N, H, d), _rand(rng, 1, N, Hkv, d), _rand(rng, 1, N, Hkv, d), _rand(rng, 1, N, H, d)
    kw = dict(scale=0.8, causal=causal, alibi_slopes=np.array([0.6, 0.3]) if alibi else None,
              dropout=(0.35, 77, 2))
    return q, k, v, do, kw


@pytest.mark.parametrize("causal,alibi,Hkv", [(False, False, 2), (True, True, 1)])
def test_dropout_finite_differences(causal, alibi, Hkv):
    """At a fixed mask the dropped output is smooth in Q, K, V: central differences."""
    assert _fd_max_rel_err(*_fd_case(causal, alibi, Hkv)) < 1e-6


def test_dropout_d_identity():
    """D_i = sum_j P_ij dP_ij (dP: the gradient reaching the undropped P) equals dO_i . O_i."""
    rng = RNG(46)
    n, d = 30, 5
    q, k, v, do = (_rand(rng, n, d) for _ in range(4))
    keep = PX.dropout_keep(n, n, 0, 0, 1, 9, 3, PX.keep_threshold(0.25))
    ks = 256 / PX.keep_threshold(0.25)
    o, _ = OA.head_fwd(q, k, v, 0.4, False, None, keep, ks)
    s = 0.4 * q @ k.T
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    dp = np.where(keep, (do @ v.T) * ks, 0.0)
    np.testing.assert_allclose((p * dp).sum(axis=1), (do * o).sum(axis=1), atol=1e-12)


# planted mistakes in the dropout code (on the CPU): each must fail a check above
def test_planted_dropout_mistakes(monkeypatch):
    rng = RNG(47)
    q, k, v = _rand(rng, 1, 6, 2, 3), _rand(rng, 1, 6, 2, 3), _rand(rng, 1, 6, 2, 3)
    orig_fwd, orig_bwd = OA.head_fwd, OA.head_bwd

    def fwd_no_scale(qh, kh, vh, scale, causal=False, slope=None, keep=None, keep_scale=1.0, window=None,
                     softcap=0.0):
        return orig_fwd(qh, kh, vh, scale, causal, slope, keep, 1.0, window, softcap)

    def bwd_dp_unmasked(qh, kh, vh, doh, scale, causal=False, slope=None, keep=None, keep_scale=1.0, window=None,
                        softcap=0.0):
        dq, dk, _ = orig_bwd(qh, kh, vh, doh, scale, causal, slope)
        _, _, dv = orig_bwd(qh, kh, vh, doh, scale, causal, slope, keep, keep_scale)
        return dq, dk, dv

    # forward without the 256/K scale: the expectation over seeds is off
    monkeypatch.setattr(OA, "head_fwd", fwd_no_scale)
    outs = np.stack([OA.attention_fwd(q, k, v, dropout=(0.3, s, 0))[0] for s in range(400)])
    monkeypatch.setattr(OA, "head_fwd", orig_fwd)
    o_ref = OA.attention_fwd(q, k, v)[0]
    assert np.abs(outs.mean(axis=0) - o_ref).max() > 5 * (outs.std(axis=0) / 20).max()
    # backward that forgets the mask on dP: central differences disagree
    monkeypatch.setattr(OA, "head_bwd", bwd_dp_unmasked)
    assert _fd_max_rel_err(*_fd_case(False, False, 2)) > 1e-3
