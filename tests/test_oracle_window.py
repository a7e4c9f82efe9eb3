"""Pins for the oracle's sliding-window and non-square (cross-attention) masks.

"Why FlashAttention Is a Kernel Story", section "When it falls down", names
sliding-window attention and cross-attention with non-square K, V grids as the
variants that need changes to the tiling. The oracle reads them as: K and V have
N_k rows, query i lines up with key i + (N_k - N_q), causal keeps keys up to that
key, and a window (W_left, W_right) keeps keys at most W_left before and W_right
after it (-1: unbounded). Each test ties that reading to something that is not
the oracle's own mask code:
  * a pure-Python triple loop (no numpy) on tiny shapes;
  * PyTorch's CPU scaled-dot-product attention in float64 with its own causal
    flag (top-left aligned) on an equivalent square problem, for the
    bottom-right causal mask, and its autograd for the gradients;
  * closed forms: a zero-width window selects one value row; equal scores give
    the mean of the values inside the window;
  * invariants: a window wider than the keys changes nothing; causal equals a
    zero right window; shifting the whole sequence shifts the result for rows
    whose window lies inside it; central finite differences of the backward.
"""
import itertools
import math

import numpy as np
import pytest
import torch

import attn_workloads as W
from oracle import attention as A
from oracle import philox

# (N_q, N_k, causal, window)
SHAPES = [
    (5, 8, True, None),
    (8, 5, True, None),
    (6, 6, False, (2, 1)),
    (7, 4, False, (1, 0)),
    (4, 7, True, (2, -1)),
    (8, 8, True, (3, -1)),
    (3, 8, False, (-1, 2)),
    (6, 3, False, None),
]


def _brute_head(q, k, v, s, causal, window, L, Z):
    nq, nk, d = len(q), len(k), len(q[0])
    O = [[0.0] * d for _ in range(nq)]
    lse = [0.0] * nq
    for i in range(nq):
        centre = i + nk - nq
        sc = []
        for j in range(nk):
            ok = not causal or j <= centre
            if window is not None:
                if window[0] >= 0 and j < centre - window[0]:
                    ok = False
                if window[1] >= 0 and j > centre + window[1]:
                    ok = False
            if L is not None and j >= L:
                ok = False
            if ok:
                sc.append((j, s * sum(q[i][t] * k[j][t] for t in range(d))))
        if not sc:
            lse[i] = -math.inf
            continue
        m = max(x for _, x in sc)
        lse[i] = m + math.log(sum(math.exp(x - m) for _, x in sc))
        for j, x in sc:
            pij = math.exp(x - lse[i]) * Z[i][j]
            for t in range(d):
                O[i][t] += pij * v[j][t]
    return O, lse


@pytest.mark.parametrize("nq,nk,causal,window", SHAPES)
@pytest.mark.parametrize("p", [0.0, 0.3])
@pytest.mark.parametrize("pad", [False, True])
def test_forward_matches_pure_python_brute_force(nq, nk, causal, window, p, pad):
    kv = [max(1, nk - 2), nk] if pad else None
    inp = W.random_case(2, 2, nq, 4, "fp16", seed=nq * 13 + nk, kv_len=kv, n_k=nk)
    scale = 0.41
    O, lse = A.forward(inp.q, inp.k, inp.v, scale=scale, causal=causal, kv_len=inp.kv_len,
                       dropout_p=p, seed=inp.seed, window=window)
    s = float(np.float32(scale))
    q, k, v = (t.double().tolist() for t in (inp.q, inp.k, inp.v))
    for b, h in itertools.product(range(2), range(2)):
        keep = philox.keep_mask(inp.seed, b, h, nq, nk, p)
        Z = [[(philox.keep_scale(p) if keep[i][j] else 0.0) if p else 1.0
              for j in range(nk)] for i in range(nq)]
        L = None if kv is None else kv[b]
        Ob, lb = _brute_head(q[b][h], k[b][h], v[b][h], s, causal, window, L, Z)
        assert np.allclose(O[b, h], np.array(Ob), atol=1e-12, rtol=0)
        assert np.allclose(lse[b, h], np.array(lb), atol=1e-12, rtol=0)


@pytest.mark.parametrize("nq,nk", [(17, 40), (64, 130), (40, 17), (100, 64), (33, 33)])
def test_bottom_right_causal_matches_torch_sdpa_fp64(nq, nk):
    """torch's is_causal aligns top-left (key j visible to row r iff j <= r).
    Bottom-right alignment is the top-left mask of the square problem whose
    N_k - N_q leading query rows come first (N_k >= N_q), or of the last N_k
    query rows alone (N_k < N_q, where the earlier rows see no key)."""
    d = 32
    inp = W.random_case(2, 2, nq, d, "bf16", seed=nq + nk, std=2.0, with_do=True, n_k=nk)
    scale = 1.0 / math.sqrt(d)
    s = float(np.float32(scale))
    O, lse = A.forward(inp.q, inp.k, inp.v, scale=scale, causal=True)
    dq, dk, dv = A.backward(inp.q, inp.k, inp.v, inp.do, scale=scale, causal=True)
    q, k, v, do = (t.double() for t in (inp.q, inp.k, inp.v, inp.do))
    if nk >= nq:
        lead = torch.zeros(2, 2, nk - nq, d, dtype=torch.float64)
        qs = torch.cat([lead, q], dim=2).requires_grad_(True)
        dos = torch.cat([lead, do], dim=2)
        sel = slice(nk - nq, nk)
        first = 0
    else:
        qs = q[:, :, nq - nk:].clone().requires_grad_(True)
        dos = do[:, :, nq - nk:]
        sel = slice(0, nk)
        first = nq - nk
    ks, vs = k.clone().requires_grad_(True), v.clone().requires_grad_(True)
    ref = torch.nn.functional.scaled_dot_product_attention(qs, ks, vs, is_causal=True, scale=s)
    ref.backward(dos)
    _, ref_lse = torch.ops.aten._scaled_dot_product_flash_attention_for_cpu(
        qs.detach(), ks.detach(), vs.detach(), 0.0, True, scale=s)
    assert np.abs(O[:, :, first:] - ref.detach()[:, :, sel].numpy()).max() < 1e-10
    assert np.abs(lse[:, :, first:] - ref_lse[:, :, sel].numpy()).max() < 1e-10
    assert np.abs(dq[:, :, first:] - qs.grad[:, :, sel].numpy()).max() < 1e-10
    assert np.abs(dk - ks.grad.numpy()).max() < 1e-10
    assert np.abs(dv - vs.grad.numpy()).max() < 1e-10
    if first:
        assert np.all(O[:, :, :first] == 0) and np.all(np.isneginf(lse[:, :, :first]))
        assert np.all(dq[:, :, :first] == 0)


@pytest.mark.parametrize("nq,nk,causal", [(9, 9, False), (6, 11, True), (11, 6, False)])
@pytest.mark.parametrize("p", [0.0, 0.4])
def test_zero_width_window_selects_one_value(nq, nk, causal, p):
    inp = W.random_case(2, 2, nq, 16, "bf16", seed=3 + nq, n_k=nk)
    O, lse = A.forward(inp.q, inp.k, inp.v, scale=0.3, causal=causal, window=(0, 0),
                       dropout_p=p, seed=inp.seed)
    q, k, v = (t.double().numpy() for t in (inp.q, inp.k, inp.v))
    s = float(np.float32(0.3))
    for b, h in itertools.product(range(2), range(2)):
        keep = philox.keep_mask(inp.seed, b, h, nq, nk, p)
        for i in range(nq):
            j = i + nk - nq
            if 0 <= j < nk:
                z = (keep[i, j] * philox.keep_scale(p)) if p else 1.0
                assert np.allclose(O[b, h, i], z * v[b, h, j], atol=1e-14, rtol=0)
                assert abs(lse[b, h, i] - s * q[b, h, i] @ k[b, h, j]) < 1e-13
            else:
                assert np.all(O[b, h, i] == 0) and np.isneginf(lse[b, h, i])


@pytest.mark.parametrize("window", [(3, 2), (5, -1), (-1, 4), (0, 6)])
@pytest.mark.parametrize("nk", [19, 26])
def test_equal_scores_give_mean_inside_window(window, nk):
    nq = 19
    inp = W.random_case(1, 2, nq, 8, "fp16", seed=nk, n_k=nk)
    q = torch.zeros_like(inp.q)
    O, lse = A.forward(q, inp.k, inp.v, scale=0.5, window=window)
    v = inp.v.double().numpy()
    for h in range(2):
        for i in range(nq):
            c = i + nk - nq
            lo = 0 if window[0] < 0 else max(0, c - window[0])
            hi = nk - 1 if window[1] < 0 else min(nk - 1, c + window[1])
            assert np.allclose(O[0, h, i], v[0, h, lo:hi + 1].mean(0), atol=1e-13, rtol=0)
            assert abs(lse[0, h, i] - math.log(hi - lo + 1)) < 1e-13


@pytest.mark.parametrize("causal", [False, True])
def test_window_wider_than_keys_changes_nothing(causal):
    inp = W.random_case(2, 2, 30, 16, "bf16", seed=8, with_do=True, kv_len=[25, 30], n_k=45)
    kw = dict(scale=0.25, causal=causal, kv_len=inp.kv_len, dropout_p=0.2, seed=inp.seed)
    O1, l1 = A.forward(inp.q, inp.k, inp.v, **kw)
    O2, l2 = A.forward(inp.q, inp.k, inp.v, window=(75, 75), **kw)
    assert np.array_equal(O1, O2) and np.array_equal(l1, l2)
    g1 = A.backward(inp.q, inp.k, inp.v, inp.do, **kw)
    g2 = A.backward(inp.q, inp.k, inp.v, inp.do, window=(75, -1), **kw)
    for a, b in zip(g1, g2):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("nq,nk", [(20, 20), (12, 31), (31, 12)])
def test_causal_equals_zero_right_window(nq, nk):
    inp = W.random_case(1, 2, nq, 8, "fp16", seed=nq * nk, with_do=True, n_k=nk)
    kw = dict(scale=0.35, dropout_p=0.25, seed=inp.seed)
    for wl in (-1, 4):
        O1, l1 = A.forward(inp.q, inp.k, inp.v, causal=True, window=(wl, -1), **kw)
        O2, l2 = A.forward(inp.q, inp.k, inp.v, causal=False, window=(wl, 0), **kw)
        assert np.array_equal(O1, O2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("window,causal", [((4, 3), False), ((6, -1), True)])
def test_window_is_relative_to_the_row(window, causal):
    """Dropping the first t positions of Q, K, V shifts every row whose window
    lies inside the remaining keys by t (square, no padding, no dropout)."""
    N, t = 40, 9
    inp = W.random_case(1, 2, N, 16, "bf16", seed=17)
    O, lse = A.forward(inp.q, inp.k, inp.v, scale=0.3, causal=causal, window=window)
    Os, ls = A.forward(inp.q[:, :, t:], inp.k[:, :, t:], inp.v[:, :, t:], scale=0.3,
                       causal=causal, window=window)
    rows = np.arange(t + window[0], N)
    assert np.abs(Os[:, :, rows - t] - O[:, :, rows]).max() < 1e-13
    assert np.abs(ls[:, :, rows - t] - lse[:, :, rows]).max() < 1e-13
    # rows whose window is cut by the shift see fewer keys
    assert np.abs(ls[:, :, 0] - lse[:, :, t]).max() > 1e-6


@pytest.mark.parametrize("nq,nk,causal,window", [(5, 7, True, (3, -1)), (6, 4, False, (1, 1)),
                                                 (6, 6, False, (2, 0))])
@pytest.mark.parametrize("p", [0.0, 0.3])
def test_backward_central_finite_differences(nq, nk, causal, window, p):
    d = 4
    inp = W.random_case(2, 1, nq, d, "fp16", seed=61 + nq, with_do=True,
                        kv_len=[nk - 1, nk], n_k=nk)
    q, k, v, do = (t.double().numpy() for t in (inp.q, inp.k, inp.v, inp.do))
    kw = dict(scale=0.7, causal=causal, kv_len=inp.kv_len, dropout_p=p, seed=inp.seed,
              window=window)
    dq, dk, dv = A.backward(q, k, v, do, **kw)
    assert dk.shape == k.shape and dq.shape == q.shape

    def loss(qq, kk, vv):
        O, _ = A.forward(qq, kk, vv, **kw)
        return float((O * do).sum())

    h = 1e-6
    for pos, (x, g) in enumerate(((q, dq), (k, dk), (v, dv))):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            args_p = [q, k, v]
            args_m = [q, k, v]
            xp = x.copy()
            xm = x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p[pos] = xp
            args_m[pos] = xm
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        assert np.abs(num - g).max() < 1e-7, "qkv"[pos]


def test_sampled_forms_equal_full_forms_non_square():
    nq, nk, d = 70, 150, 16
    inp = W.random_case(2, 2, nq, d, "bf16", seed=71, with_do=True, kv_len=[140, 150], n_k=nk)
    kw = dict(scale=0.2, causal=True, kv_len=inp.kv_len, dropout_p=0.15, seed=inp.seed,
              window=(40, -1))
    O, lse = A.forward(inp.q, inp.k, inp.v, **kw)
    rows = np.array([0, 3, 50, 69])
    Or, lr = A.forward(inp.q, inp.k, inp.v, rows=rows, heads=[(1, 0)], **kw)
    assert np.abs(Or[1, 0] - O[1, 0, rows]).max() < 1e-14
    assert np.abs(lr[1, 0] - lse[1, 0, rows]).max() < 1e-14
    dq, dk, dv = A.backward(inp.q, inp.k, inp.v, inp.do, **kw)
    cols = np.array([1, 100, 139, 149])
    sq, sk, sv = A.backward_sampled(inp.q, inp.k, inp.v, inp.do, heads=[(1, 1)],
                                    rows=rows, cols=cols, row_chunk=32, **kw)
    assert np.abs(sq[(1, 1)] - dq[1, 1, rows]).max() < 1e-13
    assert np.abs(sk[(1, 1)] - dk[1, 1, cols]).max() < 1e-13
    assert np.abs(sv[(1, 1)] - dv[1, 1, cols]).max() < 1e-13


def test_single_row_and_tail_forms_equal_the_full_backward():
    """Under a causal mask, query row r alone against keys 0..r (a non-square
    grid, bottom-right aligned) gives row r's dQ, and the last t rows against
    all keys give the last t key columns' dK and dV: the forms the 2^20-token
    GPU test evaluates."""
    g = torch.Generator().manual_seed(0)
    N, d = 300, 16
    q, k, v, do = (torch.randn(1, 1, N, d, generator=g, dtype=torch.float64) for _ in range(4))
    kw = dict(scale=0.25, causal=True)
    dq, dk, dv = A.backward(q, k, v, do, **kw)
    for r in (0, 1, 137, N - 1):
        dq_r, _, _ = A.backward_sampled(q[:, :, r:r + 1], k[:, :, :r + 1], v[:, :, :r + 1],
                                        do[:, :, r:r + 1], heads=[(0, 0)], rows=[0],
                                        cols=np.zeros(0, dtype=np.int64), row_chunk=1, **kw)
        assert np.abs(dq_r[(0, 0)] - dq[0, 0, r:r + 1]).max() < 1e-12
    lo = N - 40
    _, dk_r, dv_r = A.backward_sampled(q[:, :, lo:], k, v, do[:, :, lo:], heads=[(0, 0)],
                                       rows=np.zeros(0, dtype=np.int64),
                                       cols=np.arange(lo, N), row_chunk=8, **kw)
    assert np.abs(dk_r[(0, 0)] - dk[0, 0, lo:]).max() < 1e-12
    assert np.abs(dv_r[(0, 0)] - dv[0, 0, lo:]).max() < 1e-12
