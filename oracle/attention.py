"""Exact softmax attention by definition, fp64 numpy (oracle, test infrastructure).

What it computes follows the op chain that the fused kernel replaces
(anthology-of-the-sota practice SOTA-114, "The general form of the practice
above it": matmul, scale, mask, softmax, dropout, matmul) and the standard
forward of "Why FlashAttention Is a Kernel Story", section "The real bottleneck:
memory bandwidth, not FLOPs" (S = QK^T, P = softmax(S), O = PV). The same page,
section "Tiling", states that the tiled result is identical to full attention,
so the plain definition is the expected result. The backward is the gradient of
that definition; the page's "When it falls down" section (backward pass) says
the kernel recomputes S and P from the saved output and log-sum-exp, which is
the same mathematics.

Per head (b, h), with s = float64(float32(scale)), N_q query rows, N_k key rows
and the diagonal offset off = N_k - N_q:

    valid(i, j) = (not causal or j <= i + off)
                  and (W_left  < 0 or j >= i + off - W_left)
                  and (W_right < 0 or j <= i + off + W_right)
                  and (kv_len is None or j < kv_len[b])
    S_ij  = s * Q_i . K_j          where valid, -inf elsewhere
    lse_i = log sum_j exp(S_ij)    (-inf for a row with no valid key)
    P_ij  = exp(S_ij - lse_i)      (0 for such a row)
    Z_ij  = keep(seed,b,h,i,j) / (1 - p32)   (Z = 1 when p = 0)
    O_i   = sum_j P_ij Z_ij V_j

Backward, given dO:
    dV_j  = sum_i P_ij Z_ij dO_i
    dP_ij = Z_ij (dO_i . V_j)
    D_i   = sum_j P_ij dP_ij              (equals dO_i . O_i)
    dS_ij = P_ij (dP_ij - D_i)
    dQ_i  = s sum_j dS_ij K_j ;  dK_j = s sum_i dS_ij Q_i

Readings taken where the pages are silent: layout (B, H, N, d); mask applied
before the softmax as -inf; dropout after normalisation, before the product with
V (so lse is over undropped scores); causal keeps j <= i on square N x N; key
padding masks keys j >= kv_len[b] for every query row; a row with no valid key
gives O = 0, lse = -inf and zero gradients.

Sliding-window and non-square (cross-attention) variants: the same page,
section "When it falls down", names sliding-window attention (Longformer- and
Mistral-style) and cross-attention with non-square K, V grids as the variants
that need changes to the tiling. Readings: K and V may have N_k != N_q rows;
query i lines up with key i + (N_k - N_q) (the last query with the last key),
and the causal mask and the window are taken relative to that key; the window
(W_left, W_right) keeps keys within W_left before and W_right after it,
inclusive, -1 meaning unbounded on that side (Mistral-style: causal with
W_left = w - 1; Longformer-style: W_left = W_right = w). kv_len is clamped to
[0, N_k].

Inputs are any real arrays: q (B, H, N_q, d), k and v (B, H, N_k, d), dO like q;
they are upcast to float64 exactly.
"""
from __future__ import annotations

import numpy as np

from . import philox


def _f64(x) -> np.ndarray:
    try:  # torch tensors (any dtype, including bfloat16) -> exact float64
        import torch
        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.float64)


def scale64(scale: float) -> float:
    """The caller passes the scale as float32; the oracle uses that value exactly."""
    return float(np.float32(scale))


def valid_mask(n: int, b: int, causal: bool, kv_len, rows=None, *, n_k=None,
               window=None) -> np.ndarray:
    """Boolean [len(rows), n_k]: which keys each query row may attend to.

    n is the number of query rows N_q, n_k the number of keys (default n);
    window is None or (W_left, W_right) with -1 for an unbounded side.
    """
    n_k = n if n_k is None else int(n_k)
    rows = np.arange(n) if rows is None else np.asarray(rows)
    j = np.arange(n_k)[None, :]
    at = rows[:, None] + (n_k - n)          # the key each query row lines up with
    m = np.ones((rows.size, n_k), dtype=bool)
    if causal:
        m &= j <= at
    if window is not None:
        wl, wr = int(window[0]), int(window[1])
        if wl >= 0:
            m &= j >= at - wl
        if wr >= 0:
            m &= j <= at + wr
    if kv_len is not None:
        L = int(min(max(int(kv_len[b]), 0), n_k))
        m &= j < L
    return m


def dropout_factor(seed, b, h, n, p, rows=None, *, n_k=None) -> np.ndarray:
    """Z restricted to the given rows: keep / (1 - p32), or all ones when p = 0."""
    n_k = n if n_k is None else int(n_k)
    rows = np.arange(n) if rows is None else np.asarray(rows)
    if p == 0.0:
        return np.ones((rows.size, n_k))
    keep = philox.keep_mask(seed, b, h, n, n_k, p, rows=rows)
    return keep.astype(np.float64) * philox.keep_scale(p)


def head_probs(q, k, s, valid):
    """Scores, log-sum-exp and probabilities for one head (rows of q given)."""
    S = s * (q @ k.T)
    S = np.where(valid, S, -np.inf)
    m = S.max(axis=1, initial=-np.inf)
    has = np.isfinite(m)
    m_safe = np.where(has, m, 0.0)
    with np.errstate(invalid="ignore"):
        E = np.exp(S - m_safe[:, None])
    E = np.where(valid, E, 0.0)
    l = E.sum(axis=1)
    with np.errstate(divide="ignore"):
        lse = np.where(has, m_safe + np.log(np.where(has, l, 1.0)), -np.inf)
    P = np.where(has[:, None], E / np.where(has, l, 1.0)[:, None], 0.0)
    return S, lse, P


def probabilities(q, k, *, scale, causal=False, kv_len=None, window=None):
    """P for every head, [B, H, N_q, N_k] (small inputs only)."""
    q, k = _f64(q), _f64(k)
    B, H, N, _ = q.shape
    Nk = k.shape[2]
    s = scale64(scale)
    out = np.empty((B, H, N, Nk))
    for b in range(B):
        valid = valid_mask(N, b, causal, kv_len, n_k=Nk, window=window)
        for h in range(H):
            out[b, h] = head_probs(q[b, h], k[b, h], s, valid)[2]
    return out


def forward(q, k, v, *, scale, causal=False, kv_len=None, dropout_p=0.0,
            seed=0, heads=None, rows=None, window=None):
    """O and lse by definition.

    heads: optional list of (b, h) to evaluate (others are left as NaN);
    rows:  optional query-row subset (each row is independent by definition).
    Returns (O [B,H,N,d] or [B,H,R,d], lse [B,H,N] or [B,H,R]) in float64.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    kv_len = None if kv_len is None else np.asarray(_f64(kv_len), dtype=np.int64)
    B, H, N, d = q.shape
    Nk = k.shape[2]
    s = scale64(scale)
    rsel = np.arange(N) if rows is None else np.asarray(rows)
    R = rsel.size
    O = np.full((B, H, R, d), np.nan)
    lse = np.full((B, H, R), np.nan)
    todo = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    for (b, h) in todo:
        valid = valid_mask(N, b, causal, kv_len, rows=rsel, n_k=Nk, window=window)
        _, lse_bh, P = head_probs(q[b, h, rsel], k[b, h], s, valid)
        Z = dropout_factor(seed, b, h, N, dropout_p, rows=rsel, n_k=Nk)
        O[b, h] = (P * Z) @ v[b, h]
        lse[b, h] = lse_bh
    return O, lse


def backward(q, k, v, do, *, scale, causal=False, kv_len=None, dropout_p=0.0,
             seed=0, heads=None, window=None):
    """dQ, dK, dV by definition (float64), full N_q x N_k per head."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    kv_len = None if kv_len is None else np.asarray(_f64(kv_len), dtype=np.int64)
    B, H, N, d = q.shape
    Nk = k.shape[2]
    s = scale64(scale)
    dq = np.full_like(q, np.nan)
    dk = np.full_like(k, np.nan)
    dv = np.full_like(v, np.nan)
    todo = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    for (b, h) in todo:
        valid = valid_mask(N, b, causal, kv_len, n_k=Nk, window=window)
        _, _, P = head_probs(q[b, h], k[b, h], s, valid)
        Z = dropout_factor(seed, b, h, N, dropout_p, n_k=Nk)
        PZ = P * Z
        dv[b, h] = PZ.T @ do[b, h]
        dP = Z * (do[b, h] @ v[b, h].T)
        D = (P * dP).sum(axis=1)
        dS = P * (dP - D[:, None])
        dq[b, h] = s * (dS @ k[b, h])
        dk[b, h] = s * (dS.T @ q[b, h])
    return dq, dk, dv


def backward_sampled(q, k, v, do, *, scale, causal=False, kv_len=None,
                     dropout_p=0.0, seed=0, heads, rows, cols, row_chunk=1024,
                     window=None):
    """dQ on sampled query rows and dK, dV on sampled key columns, by definition.

    Used at sizes where a full N x N matrix per head is too large to hold with
    its gradient companions. D_i and lse_i need every row's full softmax, so the
    rows are visited in chunks (each row's terms are independent); the sampled
    columns of dK and dV are sums over all rows i of the same definitions.
    Returns dicts keyed by (b, h): dq [R, d], dk [C, d], dv [C, d].
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    kv_len = None if kv_len is None else np.asarray(_f64(kv_len), dtype=np.int64)
    B, H, N, d = q.shape
    Nk = k.shape[2]
    s = scale64(scale)
    rows = np.asarray(rows)
    cols = np.asarray(cols)
    out_dq, out_dk, out_dv = {}, {}, {}
    for (b, h) in heads:
        dk_acc = np.zeros((cols.size, d))
        dv_acc = np.zeros((cols.size, d))
        dq_rows = np.zeros((rows.size, d))
        for r0 in range(0, N, row_chunk):
            rr = np.arange(r0, min(N, r0 + row_chunk))
            valid = valid_mask(N, b, causal, kv_len, rows=rr, n_k=Nk, window=window)
            _, _, P = head_probs(q[b, h, rr], k[b, h], s, valid)
            Z = dropout_factor(seed, b, h, N, dropout_p, rows=rr, n_k=Nk)
            dP = Z * (do[b, h, rr] @ v[b, h].T)
            D = (P * dP).sum(axis=1)
            dS = P * (dP - D[:, None])
            dv_acc += (P[:, cols] * Z[:, cols]).T @ do[b, h, rr]
            dk_acc += s * (dS[:, cols].T @ q[b, h, rr])
            sel = np.nonzero((rows >= r0) & (rows < r0 + rr.size))[0]
            if sel.size:
                dq_rows[sel] = s * (dS[rows[sel] - r0] @ k[b, h])
        out_dq[(b, h)] = dq_rows
        out_dk[(b, h)] = dk_acc
        out_dv[(b, h)] = dv_acc
    return out_dq, out_dk, out_dv
