"""FP8 (e4m3) forward attention with block scales and a Hadamard rotation: the
plain CPU definition of what the quantized path computes.

TEST INFRASTRUCTURE: imported only by tests/, the smoke check and bench.py's
CPU baseline; the library never calls it and shares no code with it.

Source: "FlashAttention: Faster Attention Without Dropping a Single
Interaction", Method Deep Dive, Key design 4 (the FlashAttention-3 row: FP8
with block quantization and incoherent processing) and Limitations,
"Numerical exactness, low precision, and reproducibility" (FP8 error against an
exact reference: 2.4e-2 without, 9.1e-3 with those two techniques). The pages
name the techniques without fixing their details; the readings taken here:

1. Format: e4m3 with the OCP "fn" encoding (bias 7, largest finite 448, no
   infinities, 0x7F / 0xFF NaN), round to nearest, ties to even, including the
   subnormal range (smallest 2^-9). Inputs are scaled into range first, so
   nothing saturates.
2. Block scales are powers of two: the scale exponent of a block is the
   smallest e with amax <= 448 * 2^e, so x * 2^-e is exact and the code of an
   element depends on x alone; e is at least -127, so that the scale and its
   reciprocal are finite fp32 numbers (only blocks with amax below
   448 * 2^-128, about 1.3e-36, are affected). Q and K: one exponent per (sequence, head,
   block of 128 tokens). V: one exponent per (sequence, kv head, channel) over
   the whole sequence, which folds into the output exactly
   (O[:, c] = 2^e_c * sum_j P_j V8[j, c]).
3. Incoherent processing: Q and K rows are multiplied elementwise by caller
   given signs (+-1) and by the unnormalized Walsh-Hadamard matrix H_d
   (Sylvester order), so (Q D H)(K D H)^T = d Q K^T; the softmax scale is then
   divided by d. Computed in fp32 with the butterfly order of :func:`fwht_f32`,
   the order the quantizer uses, so that both sides round identically.
4. The reference of the quantized path is exact attention (fp64, two-pass
   softmax) of the dequantized Q, K, V. The kernel also rounds P to e4m3 for
   the second product; that error is covered by the RMSE contract, not by this
   reference.
"""

from __future__ import annotations

import math

import numpy as np

from . import attention as OA

__all__ = ["E4M3_MAX", "e4m3_decode_table", "e4m3_encode", "fwht_f32", "block_exponent", "quantize_qk",
           "quantize_v", "dequantize_qk", "dequantize_v", "fp8_attention_fwd"]

E4M3_MAX = 448.0
QK_BLOCK = 128


def e4m3_decode_table() -> np.ndarray:
    """fp64 value of every e4m3fn code 0..255 (NaN for 0x7F and 0xFF)."""
    out = np.empty(256)
    for c in range(256):
        s = -1.0 if c & 0x80 else 1.0
        e = (c >> 3) & 0xF
        m = c & 0x7
        if e == 0xF and m == 0x7:
            out[c] = np.nan
        elif e == 0:
            out[c] = s * m * 2.0 ** -9  # subnormal: m / 8 * 2^-6
        else:
            out[c] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return out


_DECODE = e4m3_decode_table()


def e4m3_encode(x) -> np.ndarray:
    """Codes of x (|x| <= 448, finite) rounded to nearest e4m3fn, ties to the even
    code, the sign bit that of x (so a negative value that rounds to zero is
    -0, 0x80). Works from the binary exponent of each value: the spacing of the
    grid at |x| is 2^(E - 3) for E = floor(log2 |x|) >= -6 and 2^-9 below."""
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)) or np.any(np.abs(x) > E4M3_MAX):
        raise ValueError("e4m3_encode takes finite values in [-448, 448]")
    a = np.abs(x)
    E = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    E = np.maximum(E, -6.0)
    step = 2.0 ** (E - 3)
    q = a / step  # exact: step is a power of two
    n = np.floor(q)
    frac = q - n
    up = (frac > 0.5) | ((frac == 0.5) & (n % 2 == 1))
    n = n + up
    mag = n * step  # the rounded magnitude
    # mag -> code
    code = np.zeros(x.shape, dtype=np.int64)
    nz = mag > 0
    Em = np.floor(np.log2(np.where(nz, mag, 1.0)))
    sub = nz & (Em < -6)
    norm = nz & ~sub
    code[sub] = (mag[sub] / 2.0 ** -9).astype(np.int64)
    code[norm] = ((Em[norm] + 7).astype(np.int64) << 3) | ((mag[norm] / 2.0 ** Em[norm] - 1.0) * 8).astype(np.int64)
    code = code | np.where(np.signbit(x), 0x80, 0)  # the sign is kept, also on a result of zero
    return code.astype(np.uint8)


def fwht_f32(x: np.ndarray) -> np.ndarray:
    """Unnormalized Walsh-Hadamard transform of the last axis (length a power of
    two) in fp32: stages h = 1, 2, 4, ..., each replacing the pair (a, b) at
    positions (i, i + h) of every 2h-block by (a + b, a - b). Equals x @ H_d
    with H_d the Sylvester-order Hadamard matrix, up to fp32 rounding."""
    y = np.array(x, dtype=np.float32, copy=True)
    d = y.shape[-1]
    h = 1
    while h < d:
        z = y.reshape(y.shape[:-1] + (d // (2 * h), 2, h))
        a, b = z[..., 0, :].copy(), z[..., 1, :].copy()
        z[..., 0, :] = a + b
        z[..., 1, :] = a - b
        y = z.reshape(y.shape)
        h *= 2
    return y


E_MIN = -127


def block_exponent(amax) -> np.ndarray:
    """Smallest integer e >= -127 with amax <= 448 * 2^e (0 where amax = 0).
    Exact: with amax = m 2^E, m in [1, 2), it is E - 8 if m <= 1.75 and E - 7
    otherwise, raised to -127 if lower (reading 2)."""
    a = np.asarray(amax, dtype=np.float64)
    m, E = np.frexp(np.where(a > 0, a, 1.0))  # a = m 2^E, m in [0.5, 1)
    m, E = 2 * m, E - 1
    e = np.maximum(np.where(m <= 1.75, E - 8, E - 7), E_MIN)
    return np.where(a > 0, e, 0).astype(np.int64)


def quantize_qk(x, signs=None, block: int = QK_BLOCK):
    """Q or K [B, N, H, d] (values as given, any float type) -> (codes uint8
    [B, N, H, d], exponents int [B, H, ceil(N / block)]). With ``signs`` [d],
    each row is first multiplied by the signs and transformed by
    :func:`fwht_f32` (reading 3), in fp32."""
    xf = OA._f64(x).astype(np.float32)  # exact: the inputs are 16-bit
    if signs is not None:
        xf = fwht_f32(xf * np.asarray(signs, dtype=np.float32))
    B, N, H, d = xf.shape
    nb = (N + block - 1) // block
    codes = np.zeros((B, N, H, d), dtype=np.uint8)
    exps = np.zeros((B, H, nb), dtype=np.int64)
    for b in range(B):
        for h in range(H):
            for k in range(nb):
                blk = xf[b, k * block:(k + 1) * block, h].astype(np.float64)
                e = int(block_exponent(np.abs(blk).max() if blk.size else 0.0))
                exps[b, h, k] = e
                codes[b, k * block:(k + 1) * block, h] = e4m3_encode(blk * 2.0 ** -e)
    return codes, exps


def quantize_v(v):
    """V [B, N, Hkv, d] -> (codes uint8 [B, N, Hkv, d], exponents int [B, Hkv, d]):
    one scale per channel over the whole sequence (reading 2)."""
    vf = OA._f64(v)
    e = block_exponent(np.abs(vf).max(axis=1))  # [B, Hkv, d]
    codes = e4m3_encode(vf * np.exp2(-e)[:, None, :, :])
    return codes, e


def dequantize_qk(codes, exps, block: int = QK_BLOCK) -> np.ndarray:
    vals = _DECODE[np.asarray(codes)]
    scale = np.exp2(np.repeat(np.asarray(exps), block, axis=2)[:, :, : vals.shape[1]])  # [B, H, N]
    return vals * scale.transpose(0, 2, 1)[..., None]


def dequantize_v(codes, exps) -> np.ndarray:
    return _DECODE[np.asarray(codes)] * np.exp2(np.asarray(exps))[:, None, :, :]


def fp8_attention_fwd(q, k, v, scale=None, causal=False, signs=None):
    """Reference of the FP8 path (reading 4): quantize Q, K (with the rotation when
    ``signs`` is given) and V, dequantize, and run exact fp64 attention with the
    softmax scale divided by d under the rotation. Returns (o, lse, parts) with
    parts = (q codes, q exps, k codes, k exps, v codes, v exps)."""
    d = np.asarray(OA._f64(q)).shape[-1]
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    qc, qe = quantize_qk(q, signs)
    kc, ke = quantize_qk(k, signs)
    vc, ve = quantize_v(v)
    s_eff = scale / d if signs is not None else scale
    o, lse = OA.attention_fwd(dequantize_qk(qc, qe), dequantize_qk(kc, ke), dequantize_v(vc, ve), scale=s_eff,
                              causal=causal)
    return o, lse, (qc, qe, kc, ke, vc, ve)
