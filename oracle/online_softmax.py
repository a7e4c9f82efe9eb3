"""fp64 model of the tiled online-softmax recurrence (oracle, test infrastructure).

"Why FlashAttention Is a Kernel Story", section "Tiling: fitting the work inside
SRAM", gives the per-tile update for a block of scores s (one block of keys):

    m_new = max(m_old, rowmax(s))
    l_new = exp(m_old - m_new) * l_old + rowsum(exp(s - m_new))
    O_new = diag(exp(m_old - m_new)) * O_old + exp(s - m_new) * V_block

and, after the last block, O = O / l; the same section says the result is
identical to full attention. This module walks the keys in blocks of ``block``
columns exactly in that order (no other reordering), with masked scores set to
-inf, dropout applied to the O update only (keep / (1 - p32) from the Philox
rule), and the statistic saved as lse = m + ln l (one natural-log value per row,
instead of the page's separate l and m). It exists to show, in tests, that this
recurrence reproduces the definition in ``attention.py`` for any block size,
which pins the algorithm the GPU kernels implement.
"""
from __future__ import annotations

import numpy as np

from . import attention


def forward_head(q, k, v, *, scale, block, causal=False, kv_len=None,
                 dropout_p=0.0, seed=0, b=0, h=0):
    """One head with the tiled recurrence. q, k, v: [N, d]. Returns (O, lse)."""
    q = attention._f64(q)
    k = attention._f64(k)
    v = attention._f64(v)
    N, d = q.shape
    s = attention.scale64(scale)
    kvl = None
    if kv_len is not None:
        kvl = np.zeros(b + 1, dtype=np.int64)
        kvl[b] = int(kv_len)
    valid = attention.valid_mask(N, b, causal, kvl)
    Z = attention.dropout_factor(seed, b, h, N, dropout_p)

    m = np.full(N, -np.inf)
    l = np.zeros(N)
    O = np.zeros((N, d))
    for j0 in range(0, N, block):
        j1 = min(N, j0 + block)
        sblk = s * (q @ k[j0:j1].T)
        sblk = np.where(valid[:, j0:j1], sblk, -np.inf)
        m_new = np.maximum(m, sblk.max(axis=1))
        # Rows whose scores are all -inf so far have nothing to rescale: use 0
        # as the reference so exp(-inf - ref) = 0 instead of NaN.
        ref = np.where(np.isfinite(m_new), m_new, 0.0)
        alpha = np.exp(m - ref)
        p = np.exp(sblk - ref[:, None])
        l = alpha * l + p.sum(axis=1)
        O = alpha[:, None] * O + (p * Z[:, j0:j1]) @ v[j0:j1]
        m = m_new
    has = l > 0
    O = np.where(has[:, None], O / np.where(has, l, 1.0)[:, None], 0.0)
    with np.errstate(divide="ignore"):
        lse = np.where(has, m + np.log(np.where(has, l, 1.0)), -np.inf)
    return O, lse
