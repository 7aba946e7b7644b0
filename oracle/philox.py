"""Philox4x32-10 counter-based generator and the attention-dropout mask, in plain numpy.

TEST INFRASTRUCTURE (see oracle/attention.py for who may import it).

Generator: J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw, "Parallel Random
Numbers: As Easy as 1, 2, 3", SC'11, the Philox-4x32 bijection with 10 rounds.
State is a 128-bit counter (four 32-bit words c0..c3) and a 64-bit key (k0, k1).
One round multiplies c0 and c2 by the constants M0 = 0xD2511F53 and
M1 = 0xCD9E8D57 into 64-bit products (hi, lo) and forms the new counter

    (hi(M1 c2) ^ c1 ^ k0,  lo(M1 c2),  hi(M0 c0) ^ c3 ^ k1,  lo(M0 c0)),

after which the key is bumped by the Weyl constants W0 = 0x9E3779B9 and
W1 = 0xBB67AE85 (mod 2^32). The output is the counter after ten rounds, the
first round using the key as given.

Dropout mask (the fused operator's dropout, "FlashAttention: Faster Attention
Without Dropping a Single Interaction", Method Deep Dive, Key design 1 stage
table and Key design 3: the backward regenerates the mask from the saved
generator state instead of storing it). For sequence b, query head h, query
position i and key position j (positions local to the sequence):

    counter = (2 * (j // 32) + (j // 4) % 2,  i,  b * H + h,  offset)
    key     = (seed mod 2^32,  seed // 2^32)
    byte    = byte (j % 4) (little-endian) of output word (j % 32) // 8
    keep    = byte < K,   K = round(256 * (1 - p_drop)),   1 <= K <= 256

and a kept probability is scaled by 256 / K, so the expectation of every
dropped weight equals the undropped one. The counter layout gives the 16
elements of one query row and one half of a 32-key block to one generator
call. This is the library's definition of which random number goes to which
element; nothing on the pages fixes it (parity is against this definition).
"""

from __future__ import annotations

import numpy as np

M0 = 0xD2511F53
M1 = 0xCD9E8D57
W0 = 0x9E3779B9
W1 = 0xBB67AE85
MASK32 = 0xFFFFFFFF


def philox4x32(counter, key, rounds: int = 10):
    """Philox-4x32 of uint32 arrays: counter (..., 4), key (..., 2); returns (..., 4) uint32.

    Products use uint64 arithmetic (exact for 32 x 32 bits)."""
    c = np.array(counter, dtype=np.uint64) & MASK32
    k = np.array(key, dtype=np.uint64) & MASK32
    c0, c1, c2, c3 = (c[..., t].copy() for t in range(4))
    k0, k1 = k[..., 0].copy(), k[..., 1].copy()
    for _ in range(rounds):
        p0 = np.uint64(M0) * c0
        p1 = np.uint64(M1) * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & np.uint64(MASK32)
        hi1, lo1 = p1 >> np.uint64(32), p1 & np.uint64(MASK32)
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
        k0 = (k0 + np.uint64(W0)) & np.uint64(MASK32)
        k1 = (k1 + np.uint64(W1)) & np.uint64(MASK32)
    return np.stack([c0, c1, c2, c3], axis=-1).astype(np.uint32)


def keep_threshold(p_drop: float) -> int:
    """K = round(256 (1 - p_drop)); a weight is kept when its random byte is below K."""
    if not (0.0 <= p_drop < 1.0):
        raise ValueError("p_drop must lie in [0, 1)")
    K = int(np.rint(256.0 * (1.0 - p_drop)))
    if K < 1:
        raise ValueError("p_drop rounds to dropping everything")
    return K


def dropout_keep(n_q: int, n_k: int, b: int, h: int, H: int, seed: int, offset: int, K: int) -> np.ndarray:
    """Boolean keep mask [n_q, n_k] of (sequence b, query head h), from the definition above."""
    i = np.arange(n_q, dtype=np.uint64)[:, None]
    j = np.arange(n_k, dtype=np.uint64)[None, :]
    ctr = np.stack(np.broadcast_arrays(2 * (j // 32) + (j // 4) % 2, i,
                                       np.uint64(b * H + h), np.uint64(offset & MASK32)), axis=-1)
    key = np.array([seed & MASK32, (seed >> 32) & MASK32], dtype=np.uint64)
    words = philox4x32(ctr, np.broadcast_to(key, ctr.shape[:-1] + (2,)))
    w = np.take_along_axis(words, ((j % 32) // 8).astype(np.int64)[..., None].repeat(n_q, axis=0), axis=-1)[..., 0]
    byte = (w >> ((j % 4) * 8).astype(np.uint32)) & np.uint32(0xFF)
    return byte < K
