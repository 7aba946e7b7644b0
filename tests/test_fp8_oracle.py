"""Pins of the FP8 oracle (oracle/fp8.py), CPU only.

* e4m3 encoding: agrees with a brute-force nearest-code search over all 256
  codes (ties to the even code) on random and on boundary values, and with
  codes worked out by hand from the OCP e4m3fn layout (sign, 4-bit exponent
  with bias 7, 3-bit mantissa; subnormals m * 2^-9).
* The fp32 Walsh-Hadamard transform equals the product with the explicit
  Sylvester matrix (exactly on small integers, to fp32 rounding otherwise),
  and applying it twice multiplies by d.
* Block exponents are the smallest e with amax <= 448 * 2^e (brute search).
* Quantize / dequantize round trips exactly for representable inputs, keep
  every block maximum in (224, 448] and the relative error within 2^-4.
* The rotation leaves attention unchanged in exact arithmetic, and the FP8
  reference equals exact attention when quantization is exact.
"""

import math

import numpy as np
import pytest

import oracle.attention as OA
import oracle.fp8 as F8

RNG = np.random.default_rng
DEC = F8.e4m3_decode_table()


def _brute_encode(x):
    """Nearest finite code by search, ties to the code with an even mantissa."""
    finite = [c for c in range(256) if np.isfinite(DEC[c])]
    out = []
    for v in np.asarray(x).ravel():
        best = None
        for c in finite:
            dist = abs(DEC[c] - v)
            if best is None or dist < best[0] - 1e-300 or (dist == best[0] and (c & 1) == 0 and (best[1] & 1) == 1):
                best = (dist, c)
        # both +0 and -0 decode to 0: a zero result takes the sign of the input
        c = best[1]
        if DEC[c] == 0.0:
            c = 0x80 if np.signbit(v) else 0x00
        out.append(c)
    return np.array(out, dtype=np.uint8).reshape(np.shape(x))


def test_e4m3_hand_codes():
    # (value, code): 1.0 = 0|0111|000; 1.125 = 0|0111|001; 1.0625 is the tie
    # between 1.0 and 1.125 -> even mantissa 000; 1.1875 ties 1.125 / 1.25 -> 010;
    # 448 = 1.75 * 2^8 = 0|1111|110; 2^-6 = 0|0001|000 (smallest normal);
    # 2^-9 = 0|0000|001 (smallest subnormal); 2^-10 ties 0 / 2^-9 -> 0;
    # 1.5 * 2^-9 ties 1 / 2 units of 2^-9 -> 2; -3.3 ~ -1.65 * 2 -> 1|1000|101;
    # 240 = 1.875 * 2^7 = 0|1110|111; 288 = 1.125 * 2^8 = 0|1111|001.
    cases = [(1.0, 0x38), (1.125, 0x39), (1.0625, 0x38), (1.1875, 0x3A), (448.0, 0x7E), (2.0 ** -6, 0x08),
             (2.0 ** -9, 0x01), (2.0 ** -10, 0x00), (1.5 * 2.0 ** -9, 0x02), (-3.3, 0xC5), (240.0, 0x77),
             (288.0, 0x79), (0.0, 0x00), (0.5, 0x30), (-448.0, 0xFE)]
    vals = np.array([c[0] for c in cases])
    np.testing.assert_array_equal(F8.e4m3_encode(vals), np.array([c[1] for c in cases], dtype=np.uint8))


def test_e4m3_matches_brute_force():
    rng = RNG(100)
    x = np.concatenate([
        rng.uniform(-448, 448, 300),
        rng.standard_normal(300) * 3,
        rng.uniform(-2.0 ** -5, 2.0 ** -5, 200),  # subnormal region and its edge
        (DEC[np.isfinite(DEC)][:200] + DEC[np.isfinite(DEC)][1:201]) / 2,  # midpoints: ties
    ])
    x = x[np.abs(x) <= 448]
    np.testing.assert_array_equal(F8.e4m3_encode(x), _brute_encode(x))


def test_e4m3_round_trip_error():
    rng = RNG(101)
    x = rng.uniform(-448, 448, 2000)
    y = DEC[F8.e4m3_encode(x)]
    big = np.abs(x) >= 2.0 ** -6
    assert np.all(np.abs(y - x)[big] <= np.abs(x[big]) * 2.0 ** -4 + 1e-300)
    assert np.all(np.abs(y - x)[~big] <= 2.0 ** -10)
    g = DEC[np.isfinite(DEC)]
    np.testing.assert_array_equal(DEC[F8.e4m3_encode(g)], g)  # grid points are fixed points
    with pytest.raises(ValueError):
        F8.e4m3_encode(np.array([449.0]))


def _sylvester(d):
    h = np.ones((1, 1))
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


@pytest.mark.parametrize("d", [2, 8, 64, 128])
def test_fwht(d):
    rng = RNG(102)
    xi = rng.integers(-50, 50, size=(5, d)).astype(np.float32)  # sums of small integers: exact in fp32
    np.testing.assert_array_equal(F8.fwht_f32(xi), (xi.astype(np.float64) @ _sylvester(d)).astype(np.float32))
    np.testing.assert_array_equal(F8.fwht_f32(F8.fwht_f32(xi)), d * xi)
    xr = rng.standard_normal((5, d)).astype(np.float32)
    ref = xr.astype(np.float64) @ _sylvester(d)
    assert np.abs(F8.fwht_f32(xr) - ref).max() <= 1e-5 * math.sqrt(d) * np.abs(xr).max() * math.log2(d)


def test_block_exponent():
    rng = RNG(103)
    a = np.concatenate([rng.uniform(0, 1e4, 200), 448.0 * 2.0 ** rng.integers(-20, 20, 50),
                        [448.0, 448.1, 447.9, 1.0, 2.0 ** -12, 3.5, 1.75 * 2 ** 9, 1.7500001 * 2 ** 9]])
    for v in a:
        e = int(F8.block_exponent(v))
        assert v <= 448 * 2.0 ** e and not (v <= 448 * 2.0 ** (e - 1)), (v, e)
    assert int(F8.block_exponent(0.0)) == 0
    # the floor at -127: tinier blocks keep it, 449 * 2^-127 needs -126
    assert int(F8.block_exponent(448.0 * 2.0 ** -127)) == -127
    assert int(F8.block_exponent(449.0 * 2.0 ** -127)) == -126
    for tiny in (448.0 * 2.0 ** -128, 1e-38, 2.0 ** -140, 2.0 ** -149):
        assert int(F8.block_exponent(tiny)) == -127
    # a block of subnormal-range values: scaled by 2^127, still within range and exact
    x = np.zeros((1, 128, 1, 64), dtype=np.float32)
    x[0, :, 0, 0] = 2.0 ** -130
    x[0, 3, 0, 5] = -3 * 2.0 ** -133
    c, e = F8.quantize_qk(x)
    assert int(e[0, 0, 0]) == -127
    np.testing.assert_array_equal(F8.dequantize_qk(c, e), x.astype(np.float64))


def test_quantize_qk_blocks():
    rng = RNG(104)
    x = (rng.standard_normal((2, 300, 3, 64)) * 5).astype(np.float32)
    codes, exps = F8.quantize_qk(x)
    assert exps.shape == (2, 3, 3)
    deq = F8.dequantize_qk(codes, exps)
    for b in range(2):
        for h in range(3):
            for k in range(3):
                blk = x[b, k * 128:(k + 1) * 128, h]
                m = np.abs(blk).max() * 2.0 ** -exps[b, h, k]
                assert 224 < m <= 448
                dq = deq[b, k * 128:(k + 1) * 128, h]
                assert np.all(np.abs(dq - blk) <= np.abs(blk) * 2.0 ** -4 + 2.0 ** (exps[b, h, k] - 10))
    # representable inputs (e4m3 grid values times a common power of two) round trip exactly
    g = DEC[np.isfinite(DEC)]
    xr = (rng.choice(g, size=(1, 128, 1, 32)) * 2.0 ** -3).astype(np.float32)
    xr[0, 0, 0, 0] = 448 * 2.0 ** -3  # pins the block exponent to -3
    c2, e2 = F8.quantize_qk(xr)
    np.testing.assert_array_equal(F8.dequantize_qk(c2, e2), xr.astype(np.float64))


def test_quantize_v_channels():
    rng = RNG(105)
    v = rng.standard_normal((1, 200, 2, 32)) * np.arange(1, 33)  # channel spread grows
    codes, exps = F8.quantize_v(v)
    assert exps.shape == (1, 2, 32)
    deq = F8.dequantize_v(codes, exps)
    m = np.abs(v).max(axis=1) * np.exp2(-exps)
    assert np.all((m > 224) & (m <= 448))
    assert np.all(np.abs(deq - v) <= np.abs(v) * 2.0 ** -4 + np.exp2(exps - 10)[:, None])


def test_rotation_preserves_attention():
    """(Q D H)(K D H)^T = d Q K^T exactly in fp64: attention with scale / d on the
    rotated inputs equals attention on the originals."""
    rng = RNG(106)
    d = 64
    q, k, v = (rng.standard_normal((1, 40, 2, d)) for _ in range(3))
    signs = rng.choice([-1.0, 1.0], size=d)
    hm = _sylvester(d)
    qr, kr = (q * signs) @ hm, (k * signs) @ hm
    o1, l1 = OA.attention_fwd(q, k, v, scale=0.2, causal=True)
    o2, l2 = OA.attention_fwd(qr, kr, v, scale=0.2 / d, causal=True)
    np.testing.assert_allclose(o2, o1, atol=1e-12)
    np.testing.assert_allclose(l2, l1, atol=1e-12)


def test_reference_is_exact_when_quantization_is():
    """Inputs on the e4m3 grid, each block and channel reaching 448 * 2^-2: the
    FP8 reference equals exact attention (no rotation)."""
    rng = RNG(107)
    g = DEC[np.isfinite(DEC) & (np.abs(DEC) <= 64)]
    q, k, v = (rng.choice(g, size=(1, 130, 2, 32)) * 2.0 ** -2 for _ in range(3))
    for t in (q, k, v):
        t[0, 0, :, :] = 448 * 2.0 ** -2  # every block / channel maximum is on the grid
        t[0, 128, :, :] = 448 * 2.0 ** -2
    o, lse, _ = F8.fp8_attention_fwd(q, k, v, scale=0.05, causal=True)
    o_ref, lse_ref = OA.attention_fwd(q, k, v, scale=0.05, causal=True)
    np.testing.assert_allclose(o, o_ref, atol=1e-13)
    np.testing.assert_allclose(lse, lse_ref, atol=1e-13)


def test_rotated_codes_undo_to_the_inputs():
    """Dequantized rotated rows, rotated back (H D / d), recover Q within the
    e4m3 rounding of the rotated values: |error| <= 2^-4 |rotated| summed over
    the row, divided by d (|H| entries are 1)."""
    rng = RNG(108)
    d = 64
    q = rng.standard_normal((1, 200, 2, d)).astype(np.float32)
    q[0, 7, 1, 3] = 40.0  # an outlier the rotation spreads over the row
    signs = rng.choice([-1.0, 1.0], size=d)
    codes, exps = F8.quantize_qk(q, signs)
    rot = F8.dequantize_qk(codes, exps)
    back = (rot @ _sylvester(d)) * signs / d
    rot_exact = ((q.astype(np.float64) * signs) @ _sylvester(d))
    bound = (np.abs(rot_exact) * 2.0 ** -4 + 2.0 ** -10 * 2.0 ** exps.max()).sum(axis=-1, keepdims=True) / d
    assert np.all(np.abs(back - q) <= bound + 1e-6)
