"""fp8 (e4m3) attention: the format and the error of rounding P (oracle side).

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``.

"Why FlashAttention Is a Kernel Story", section "When it falls down", names
low-precision score tiles (BF16 or FP8) as a variant that needs care with
precision. The variant built here reads Q, K and V stored as OCP FP8 E4M3
("e4m3fn": 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits, no
infinities, the all-ones pattern is NaN, largest finite value 448) and forms
both products on fp8 tensor-core operands. Two readings:

1. The result it is checked against is exact attention of the stored values:
   Q, K and V decoded exactly (every e4m3 value is exact in float64), then the
   plain definition of ``oracle.attention.forward``. Products of two e4m3
   values are exact in fp32 and the scores are accumulated in fp32, so the
   scores carry no fp8 error.

2. The one approximation is the rounding of the probabilities to e4m3 before
   the product with V. They are rounded relative to the running reference
   maximum of the online softmax (the kernel cannot know the row maximum
   before it has seen every key), so the value rounded for key j of row i is
   x_ij = sigma * exp(S_ij - m_i), with m_i the row maximum and sigma >= 1
   (the reference never exceeds the row maximum; sigma <= 2^8 by the lazy
   update, so x <= 256 < 448 never overflows). O is then normalised by the
   fp32 sum of the unrounded x. Writing L_i = sum_j exp(S_ij - m_i) >= 1 and
   P_ij = exp(S_ij - m_i) / L_i, the e4m3 rounding error of x is at most
   2^-4 x for x >= 2^-6 (half an ulp, 3 mantissa bits) and at most 2^-10 below
   (half the subnormal spacing 2^-9), so after normalisation each term carries
   at most max(2^-4 P_ij, 2^-10 / (sigma L_i)) <= max(2^-4 P_ij, 2^-10 / L_i):

       |O_fp8_ic - O_ic| <= sum_j max(2^-4 P_ij, 2^-10 / L_i) |V_jc|

   A term rounded against an older, lower reference and rescaled later has
   an even smaller error in final units (the rescale factor is <= 1).

   The bound is loose when P is spread over many keys, so the tests add an
   aggregate check: to first order the error of O_ic is a sum of independent
   rounding errors, each uniform within +-half an ulp, whose variance is at
   most max(2^-8 P_ij^2, 2^-20 / L_i^2) / 3; the summed squared error over many
   entries concentrates near its expectation, which this upper model exceeds.

Functions here are pinned in ``tests/test_oracle_fp8.py``: the format against
its definition and torch's float8_e4m3fn cast, the rounding bounds
exhaustively, and the O bound and variance model against an emulation of a
tiled online softmax that rounds to e4m3.
"""
from __future__ import annotations

import numpy as np

from .attention import _f64, head_probs, scale64, valid_mask

E4M3_MAX = 448.0
E4M3_MIN_NORMAL = 2.0 ** -6
E4M3_SUBNORMAL_STEP = 2.0 ** -9


def decode_e4m3(code) -> np.ndarray:
    """Value of each 8-bit OCP E4M3 code (float64; NaN for the two NaN codes)."""
    c = np.asarray(code, dtype=np.int64) & 0xFF
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e - 7.0))
    val = np.where((e == 0xF) & (m == 0x7), np.nan, val)
    return sign * val


def e4m3_values() -> np.ndarray:
    """All finite non-negative e4m3 values, ascending (0, subnormals, normals)."""
    v = decode_e4m3(np.arange(0x80))
    return np.unique(v[np.isfinite(v)])


def round_e4m3(x) -> np.ndarray:
    """Round to the nearest e4m3 value, ties to the one with an even mantissa
    (|x| <= 448 + 16; larger magnitudes are not used here and raise)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    if np.any(a >= E4M3_MAX + 16.0):
        raise ValueError("outside the e4m3 rounding range")
    grid = e4m3_values()                          # 0 .. 448
    hi = np.clip(np.searchsorted(grid, a, side="left"), 1, grid.size - 1)
    lo = hi - 1
    glo, ghi = grid[lo], grid[hi]
    dlo, dhi = a - glo, ghi - a
    # Mantissa parity of a grid entry: its index among the finite codes is
    # the code itself (codes 0..0x7E are increasing), so even index = even m.
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    r = np.where(a >= grid[-1], grid[-1], np.where(pick_hi, ghi, glo))
    r = np.where(a == 0, 0.0, r)
    return np.sign(x) * r


def to_e4m3_exact(t) -> np.ndarray:
    """float64 array of tensor values stored as e4m3 (exact decoding)."""
    return _f64(t)


def row_stats(q, k, *, scale, causal=False, kv_len=None, window=None, b=0, h=0,
              rows=None):
    """For one head: P (rows x N_k), L_i = sum_j exp(S_ij - m_i) and the
    validity mask, by definition (fp64)."""
    q, k = _f64(q), _f64(k)
    N, Nk = q.shape[2], k.shape[2]
    rsel = np.arange(N) if rows is None else np.asarray(rows)
    s = scale64(scale)
    valid = valid_mask(N, b, causal, None if kv_len is None else np.asarray(_f64(kv_len)),
                       rows=rsel, n_k=Nk, window=window)
    S, lse, P = head_probs(q[b, h, rsel], k[b, h], s, valid)
    with np.errstate(invalid="ignore"):
        m = np.where(np.isfinite(lse), S.max(axis=1, initial=-np.inf), 0.0)
        L = np.where(np.isfinite(lse), np.exp(lse - m), 1.0)
    return P, L, valid


def p_rounding_bound(P, L, v, Z=None) -> np.ndarray:
    """Per-element bound on |O_fp8 - O| from rounding P to e4m3 (reading 2
    above): sum_j max(2^-4 P_ij, 2^-10 / L_i) Z_ij |V_jc|, over valid keys only
    (P_ij = 0 elsewhere, and an invalid key contributes nothing). Z is the
    dropout factor keep / (1 - p) (rows x keys; 1 when None): a dropped term is
    an exact zero, a kept one is rounded and then scaled."""
    v = np.abs(_f64(v))
    w = np.maximum(2.0 ** -4 * P, np.where(P > 0, 2.0 ** -10 / L[:, None], 0.0))
    if Z is not None:
        w = w * Z
    return w @ v


def p_rounding_variance(P, L, v, Z=None) -> np.ndarray:
    """Upper model of the variance of each element's error from rounding P:
    sum_j max(2^-8 P_ij^2, 2^-20 / L_i^2) / 3 * Z_ij^2 V_jc^2 (independent
    errors, each uniform within +-half an ulp)."""
    v = _f64(v)
    var = np.maximum(2.0 ** -8 * P * P, np.where(P > 0, 2.0 ** -20 / (L[:, None] ** 2), 0.0))
    if Z is not None:
        var = var * Z * Z
    return (var / 3.0) @ (v * v)
