"""Philox4x32-10 and the dropout keep rule (oracle side, numpy).

Philox4x32-10 is the counter-based generator of Salmon, Moraes, Dror and Shaw,
"Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11): a 128-bit counter
(four 32-bit words) and a 64-bit key (two words) go through ten rounds. A round
multiplies counter words 0 and 2 by two fixed odd 32-bit multipliers, keeps the
high and low halves of both 64-bit products, and recombines them with the other
two words and the key by XOR; between rounds the key words are bumped by two
Weyl constants (the golden ratio and sqrt(3)-1, each scaled to 2^32).

The pages ask for dropout fused into the attention kernel (anthology-of-the-sota
practice SOTA-114, "The general form of the practice above it": the chain is
matmul, scale, mask, softmax, dropout, matmul). They leave the random source
open; the reading taken here makes the keep decision a pure function of
(seed, b, h, i, j) so that the forward, the backward and this oracle all draw
the same bits without storing a mask:

    key     = (seed mod 2^32, seed >> 32)
    counter = (j >> 2, i, h, b)
    u       = Philox4x32-10(counter, key)[j & 3]
    keep    = u >= T,    T = floor(p32 * 2^32)

p32 is the dropout probability rounded to float32; T is exact in float64.
"""
from __future__ import annotations

import numpy as np

# SC'11 constants: round multipliers and Weyl key increments.
PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85
_MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(counter, key) -> np.ndarray:
    """Philox4x32-10 block function.

    counter: integer array (..., 4) of 32-bit words; key: array (..., 2).
    Returns uint32 (..., 4). Broadcasts over leading dimensions.
    """
    counter = np.asarray(counter, dtype=np.uint64)
    key = np.asarray(key, dtype=np.uint64)
    c0, c1, c2, c3 = (counter[..., t] & _MASK32 for t in range(4))
    k0 = key[..., 0] & _MASK32
    k1 = key[..., 1] & _MASK32
    m0 = np.uint64(PHILOX_M0)
    m1 = np.uint64(PHILOX_M1)
    for rnd in range(10):
        if rnd > 0:
            k0 = (k0 + np.uint64(PHILOX_W0)) & _MASK32
            k1 = (k1 + np.uint64(PHILOX_W1)) & _MASK32
        prod0 = m0 * c0          # < 2^64: exact in uint64
        prod1 = m1 * c2
        hi0, lo0 = prod0 >> np.uint64(32), prod0 & _MASK32
        hi1, lo1 = prod1 >> np.uint64(32), prod1 & _MASK32
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    out = np.stack(np.broadcast_arrays(c0, c1, c2, c3), axis=-1)
    return out.astype(np.uint32)


def seed_key(seed: int) -> tuple[int, int]:
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    return seed & 0xFFFFFFFF, seed >> 32


def drop_threshold(p: float) -> int:
    """T = floor(p32 * 2^32) with p32 the float32 rounding of p (exact in fp64)."""
    p32 = float(np.float32(p))
    if not (0.0 <= p32 < 1.0):
        raise ValueError("dropout probability must satisfy 0 <= p < 1")
    return int(np.floor(p32 * 4294967296.0))


def keep_scale(p: float) -> float:
    """Factor applied to kept values: 1 / (1 - p32) in float64."""
    p32 = float(np.float32(p))
    return 1.0 / (1.0 - p32)


def uniform_bits(seed: int, b: int, h: int, i, j) -> np.ndarray:
    """The 32-bit draw u(seed, b, h, i, j); i and j broadcast."""
    i = np.asarray(i, dtype=np.uint64)
    j = np.asarray(j, dtype=np.uint64)
    i, j = np.broadcast_arrays(i, j)
    ctr = np.stack([j >> np.uint64(2), i,
                    np.full_like(i, h), np.full_like(i, b)], axis=-1)
    k0, k1 = seed_key(seed)
    r = philox4x32_10(ctr, np.array([k0, k1], dtype=np.uint64))
    word = (j & np.uint64(3)).astype(np.int64)
    return np.take_along_axis(r, word[..., None], axis=-1)[..., 0]


def keep_mask(seed: int, b: int, h: int, n_q: int, n_k: int, p: float,
              rows=None) -> np.ndarray:
    """Boolean keep-mask [len(rows), n_k] for head (b, h); rows default to all.

    One Philox call per (i, j >> 2) yields the four draws of keys 4t..4t+3.
    """
    rows = np.arange(n_q) if rows is None else np.asarray(rows)
    if p == 0.0:
        return np.ones((rows.size, n_k), dtype=bool)
    T = drop_threshold(p)
    groups = (n_k + 3) // 4
    t = np.arange(groups, dtype=np.uint64)
    ii = rows.astype(np.uint64)
    ctr = np.empty((rows.size, groups, 4), dtype=np.uint64)
    ctr[..., 0] = t[None, :]
    ctr[..., 1] = ii[:, None]
    ctr[..., 2] = h
    ctr[..., 3] = b
    k0, k1 = seed_key(seed)
    r = philox4x32_10(ctr, np.array([k0, k1], dtype=np.uint64))
    u = r.reshape(rows.size, groups * 4)[:, :n_k]
    return u >= np.uint32(T)
