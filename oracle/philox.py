"""Philox4x32-10 counter-based generator (Salmon, Moraes, Dror, Shaw, "Parallel
random numbers: as easy as 1, 2, 3", SC'11), written from its published definition.

The pages ask for "stochastic rounding" and a "random Hadamard transform" (Four Over
Six documentation page, §Four Over Six) without naming a generator; Philox4x32-10 is
the reading taken, seeded by a 64-bit key.

One round maps counter (c0, c1, c2, c3) under key (k0, k1) to
    (hi(M1*c2) ^ c1 ^ k0,  lo(M1*c2),  hi(M0*c0) ^ c3 ^ k1,  lo(M0*c0))
with 64-bit products split into 32-bit halves; the key is bumped by the Weyl
constants (W0, W1) between rounds.  Ten rounds.
"""
from __future__ import annotations

import numpy as np

M0 = 0xD2511F53
M1 = 0xCD9E8D57
W0 = 0x9E3779B9
W1 = 0xBB67AE85
MASK32 = 0xFFFFFFFF


def philox4x32_10(counter: np.ndarray, key) -> np.ndarray:
    """counter: (..., 4) integers < 2^32; key: (k0, k1) or an (..., 2) array.
    Returns (..., 4) uint32 output words."""
    c = np.asarray(counter, dtype=np.uint64) & np.uint64(MASK32)
    c0, c1, c2, c3 = c[..., 0], c[..., 1], c[..., 2], c[..., 3]
    k = np.asarray(key, dtype=np.uint64) & np.uint64(MASK32)
    k0 = np.broadcast_to(k[..., 0], c0.shape).copy()
    k1 = np.broadcast_to(k[..., 1], c0.shape).copy()
    m0, m1 = np.uint64(M0), np.uint64(M1)
    w0, w1 = np.uint64(W0), np.uint64(W1)
    mask = np.uint64(MASK32)
    sh = np.uint64(32)
    for rnd in range(10):
        if rnd > 0:
            k0 = (k0 + w0) & mask
            k1 = (k1 + w1) & mask
        p0 = m0 * c0                       # < 2^64, exact in uint64
        p1 = m1 * c2
        n0 = ((p1 >> sh) ^ c1 ^ k0) & mask
        n1 = p1 & mask
        n2 = ((p0 >> sh) ^ c3 ^ k1) & mask
        n3 = p0 & mask
        c0, c1, c2, c3 = n0, n1, n2, n3
    return np.stack([c0, c1, c2, c3], axis=-1).astype(np.uint32)


def split_seed(seed: int):
    """64-bit seed -> key words (low 32 bits, high 32 bits)."""
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    return (seed & MASK32, seed >> 32)
