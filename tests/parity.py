"""Tolerances and comparison helpers for GPU-vs-oracle parity tests.

The bar (exact attention in fp16/bf16 with fp32 accumulation):
  * O:    max |O_gpu - O_ref| <= 1e-2 when O is written in float32; when O is
          written in the input dtype, the storage rounding of O_ref itself is
          added: <= 1e-2 + ulp(O_ref)/2 per element.
  * lse:  |lse_gpu - lse_ref| <= 1e-3 * max(1, |lse_ref|); rows with no visible
          key must be exactly -inf.
  * dQ, dK, dV: max-abs <= 2e-2 (plus half an ulp of the reference when
          written in the input dtype).
The mean signed error is reported next to the max (a rounding-bias check).
"""
from __future__ import annotations

import numpy as np
import torch

O_ATOL = 1e-2
LSE_RTOL = 1e-3
GRAD_ATOL = 2e-2


def half_ulp(ref: np.ndarray, dtype: torch.dtype) -> np.ndarray:
    """Half a unit in the last place of ref in the storage dtype (0 for float32)."""
    if dtype == torch.float32:
        return np.zeros_like(ref)
    mant = {torch.float16: 10, torch.bfloat16: 7}[dtype]
    a = np.abs(ref)
    e = np.floor(np.log2(np.maximum(a, 1e-30)))
    if dtype == torch.float16:
        e = np.maximum(e, -14)
    return 0.5 * np.exp2(e - mant)


def to64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def check_close(name: str, got, ref: np.ndarray, atol, out_dtype: torch.dtype):
    """atol may be a scalar or an array broadcastable to ref."""
    g = to64(got) if isinstance(got, torch.Tensor) else np.asarray(got, np.float64)
    err = g - ref
    bound = atol + half_ulp(ref, out_dtype)
    bad = ~(np.abs(err) <= bound)
    if bad.any():
        idx = np.argwhere(bad)[0]
        raise AssertionError(
            f"{name}: {bad.sum()} of {bad.size} elements beyond bound; first at "
            f"{tuple(idx)}: got {g[tuple(idx)]!r} ref {ref[tuple(idx)]!r}; "
            f"max|err| {np.nanmax(np.abs(err)):.3e}")
    return float(np.abs(err).max()) if err.size else 0.0, float(err.mean()) if err.size else 0.0


def d_rounding_bounds(q, k, do, O_ref, P, scale, out_dtype):
    """First-order effect on dQ and dK of storing O in out_dtype.

    The backward takes O as the forward stored it; D_i = dO_i . O_i then
    carries O's rounding, |dD_i| <= sum_c |dO_ic| ulp(O_ic)/2, and since
    dS_ij = P_ij (dP_ij - D_i):
        |d dQ_ic| <= s * dD_i * sum_j P_ij |K_jc|
        |d dK_jc| <= s * sum_i P_ij dD_i |Q_ic|
    All inputs are oracle-side (fp64 reference O and P, the seeded inputs).
    Returns (bound_dq, bound_dk) shaped like q.
    """
    if out_dtype == torch.float32:
        return 0.0, 0.0
    s = float(np.float32(scale))
    dD = (np.abs(to64(do)) * half_ulp(O_ref, out_dtype)).sum(-1)      # [B,H,N]
    qa, ka = np.abs(to64(q)), np.abs(to64(k))
    bdq = s * dD[..., None] * (P @ ka)
    bdk = s * np.swapaxes(P, -1, -2) @ (dD[..., None] * qa)
    return bdq, bdk


def check_lse(got, ref: np.ndarray):
    g = to64(got) if isinstance(got, torch.Tensor) else np.asarray(got, np.float64)
    empty = np.isneginf(ref)
    assert np.all(np.isneginf(g[empty])), "rows with no visible key must have lse = -inf"
    f = ~empty
    err = np.abs(g[f] - ref[f])
    bound = LSE_RTOL * np.maximum(1.0, np.abs(ref[f]))
    bad = ~(err <= bound)
    if bad.any():
        raise AssertionError(f"lse: {bad.sum()} rows beyond bound; max err {err.max():.3e}")
    return float(err.max()) if err.size else 0.0


def plain_excess(name: str, got, ref: np.ndarray, atol: float) -> int:
    """Number of elements beyond the plain bound |err| <= atol (no storage
    half-ulp added), printed for the record; not an assertion."""
    g = to64(got) if isinstance(got, torch.Tensor) else np.asarray(got, np.float64)
    n = int((~(np.abs(g - ref) <= atol)).sum())
    print(f"  {name}: {n} of {g.size} elements beyond plain {atol:g}")
    return n
