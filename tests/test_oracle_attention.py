"""Pins for the attention oracle (CPU only).

Each test ties the fp64 oracle to something that is not the oracle itself:
  * a pure-Python triple loop (no numpy) on N <= 8 for every mask and dropout;
  * PyTorch's CPU scaled-dot-product attention in float64, and its autograd,
    for dropout 0 (a library routine, called);
  * closed forms: equal scores give the mean of the valid values and
    lse = ln(#valid); a dominant score selects one value row; causal row 0 sees
    only key 0;
  * the tiled online-softmax recurrence of the pages for several block sizes;
  * invariants: rows of P sum to 1, shift and permutation invariance,
    central finite differences of the backward, gradient sum rules.
"""
import itertools
import math

import numpy as np
import pytest
import torch

import attn_workloads as W
from oracle import attention as A
from oracle import online_softmax as OS
from oracle import philox

MASKS = ["none", "causal", "pad", "causal_pad"]


def _case(N, d, mask, *, B=2, H=2, seed=0, dtype="fp16", std=1.0, with_do=False):
    kv = None
    if "pad" in mask:
        kv = [max(1, N - 3), max(1, N // 2)][:B] + [N] * max(0, B - 2)
    inp = W.random_case(B, H, N, d, dtype, seed=seed, std=std, with_do=with_do,
                        kv_len=kv)
    return inp, ("causal" in mask), inp.kv_len


# --------------------------------------------------------------------------
# pure-Python brute force (no numpy in the arithmetic)

def _brute_head(q, k, v, s, causal, L, Z):
    n = len(q)
    d = len(q[0])
    O = [[0.0] * d for _ in range(n)]
    lse = [0.0] * n
    for i in range(n):
        sc = []
        for j in range(n):
            ok = (not causal or j <= i) and (L is None or j < L)
            if ok:
                sc.append((j, s * sum(q[i][t] * k[j][t] for t in range(d))))
        if not sc:
            lse[i] = -math.inf
            continue
        m = max(x for _, x in sc)
        tot = sum(math.exp(x - m) for _, x in sc)
        lse[i] = m + math.log(tot)
        for j, x in sc:
            pij = math.exp(x - lse[i]) * Z[i][j]
            for t in range(d):
                O[i][t] += pij * v[j][t]
    return O, lse


@pytest.mark.parametrize("mask", MASKS)
@pytest.mark.parametrize("p", [0.0, 0.3])
@pytest.mark.parametrize("N", [1, 2, 5, 8])
def test_forward_matches_pure_python_brute_force(mask, p, N):
    inp, causal, kv = _case(N, 4, mask, seed=N * 7 + len(mask))
    scale = 0.37
    O, lse = A.forward(inp.q, inp.k, inp.v, scale=scale, causal=causal, kv_len=kv,
                       dropout_p=p, seed=inp.seed)
    s = float(np.float32(scale))
    q = inp.q.double().tolist()
    k = inp.k.double().tolist()
    v = inp.v.double().tolist()
    B, H = inp.q.shape[:2]
    for b, h in itertools.product(range(B), range(H)):
        keep = philox.keep_mask(inp.seed, b, h, N, N, p)
        Z = [[(1.0 / (1.0 - float(np.float32(p))) if keep[i][j] else 0.0) if p else 1.0
              for j in range(N)] for i in range(N)]
        L = None if kv is None else int(kv[b])
        Ob, lb = _brute_head(q[b][h], k[b][h], v[b][h], s, causal, L, Z)
        assert np.allclose(O[b, h], np.array(Ob), atol=1e-12, rtol=0)
        assert np.allclose(lse[b, h], np.array(lb), atol=1e-12, rtol=0)


# --------------------------------------------------------------------------
# library routine: torch CPU SDPA in float64 (dropout 0)

def _sdpa_mask(N, B, causal, kv):
    m = torch.ones(B, 1, N, N, dtype=torch.bool)
    if causal:
        m &= torch.ones(N, N, dtype=torch.bool).tril()
    if kv is not None:
        for b in range(B):
            m[b, :, :, int(kv[b]):] = False
    return m


@pytest.mark.parametrize("mask", MASKS)
@pytest.mark.parametrize("N,d", [(7, 16), (64, 32), (100, 64), (130, 128)])
def test_forward_backward_match_torch_sdpa_fp64(mask, N, d):
    inp, causal, kv = _case(N, d, mask, seed=N + d, with_do=True, std=2.0)
    scale = 1.0 / math.sqrt(d)
    s = float(np.float32(scale))
    q, k, v, do = (t.double().requires_grad_(True) for t in (inp.q, inp.k, inp.v, inp.do))
    am = _sdpa_mask(N, q.shape[0], causal, kv)
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=am, scale=s)
    ref.backward(do)
    _, ref_lse = torch.ops.aten._scaled_dot_product_flash_attention_for_cpu(
        q.detach(), k.detach(), v.detach(), 0.0, False, attn_mask=torch.where(
            am, 0.0, -math.inf).double(), scale=s)
    O, lse = A.forward(inp.q, inp.k, inp.v, scale=scale, causal=causal, kv_len=kv)
    dq, dk, dv = A.backward(inp.q, inp.k, inp.v, inp.do, scale=scale, causal=causal,
                            kv_len=kv)
    assert np.abs(O - ref.detach().numpy()).max() < 1e-10
    assert np.abs(lse - ref_lse.numpy()).max() < 1e-10
    assert np.abs(dq - q.grad.numpy()).max() < 1e-10
    assert np.abs(dk - k.grad.numpy()).max() < 1e-10
    assert np.abs(dv - v.grad.numpy()).max() < 1e-10


# --------------------------------------------------------------------------
# closed forms

@pytest.mark.parametrize("mask", MASKS)
@pytest.mark.parametrize("p", [0.0, 0.25])
def test_equal_scores_give_mean_of_valid_values(mask, p):
    N = 23
    inp, causal, kv = _case(N, 8, mask, seed=5)
    q = torch.zeros_like(inp.q)
    O, lse = A.forward(q, inp.k, inp.v, scale=0.5, causal=causal, kv_len=kv,
                       dropout_p=p, seed=inp.seed)
    v = inp.v.double().numpy()
    B, H = q.shape[:2]
    for b, h in itertools.product(range(B), range(H)):
        keep = philox.keep_mask(inp.seed, b, h, N, N, p)
        for i in range(N):
            js = [j for j in range(N) if (not causal or j <= i)
                  and (kv is None or j < int(kv[b]))]
            z = np.array([(keep[i, j] * philox.keep_scale(p)) if p else 1.0 for j in js])
            exp_o = (z[:, None] * v[b, h, js]).sum(0) / len(js)
            assert np.allclose(O[b, h, i], exp_o, atol=1e-13, rtol=0)
            assert abs(lse[b, h, i] - math.log(len(js))) < 1e-13


def test_row_without_valid_key():
    inp, _, _ = _case(6, 8, "pad", seed=2)
    kv = torch.tensor([0, 3], dtype=torch.int32)
    O, lse = A.forward(inp.q, inp.k, inp.v, scale=0.3, kv_len=kv)
    assert np.all(O[0] == 0) and np.all(np.isneginf(lse[0]))
    assert np.all(np.isfinite(lse[1]))
    do = torch.randn(inp.q.shape, dtype=torch.float64)
    dq, dk, dv = A.backward(inp.q, inp.k, inp.v, do, scale=0.3, kv_len=kv)
    assert np.all(dq[0] == 0) and np.all(dk[0] == 0) and np.all(dv[0] == 0)
    assert np.all(dk[1, :, 3:] == 0) and np.all(dv[1, :, 3:] == 0)


@pytest.mark.parametrize("p", [0.0, 0.4])
def test_dominant_score_selects_one_value(p):
    N, d = 16, 16
    g = torch.Generator().manual_seed(11)
    k = torch.randn(1, 1, N, d, generator=g, dtype=torch.float64)
    jstar = torch.randint(0, N, (N,), generator=g)
    # q_i = 40 * k_{j*} / |k_{j*}|^2 * ... chosen so S_ij* - S_ij >= 30 for j != j*.
    k = k / k.norm(dim=-1, keepdim=True)
    k[0, 0] = torch.eye(N, d, dtype=torch.float64)[:N]
    q = torch.zeros(1, 1, N, d, dtype=torch.float64)
    for i in range(N):
        q[0, 0, i] = 200.0 * k[0, 0, jstar[i]]
    v = torch.randn(1, 1, N, d, generator=g, dtype=torch.float64)
    S = (q[0, 0] @ k[0, 0].T).numpy()
    for i in range(N):
        others = np.delete(S[i], jstar[i])
        assert S[i, jstar[i]] - others.max() >= 30
    seed = 77
    O, lse = A.forward(q, k, v, scale=1.0, dropout_p=p, seed=seed)
    keep = philox.keep_mask(seed, 0, 0, N, N, p)
    for i in range(N):
        z = (keep[i, jstar[i]] * philox.keep_scale(p)) if p else 1.0
        assert np.allclose(O[0, 0, i], z * v[0, 0, jstar[i]].numpy(), atol=1e-10, rtol=0)
        assert abs(lse[0, 0, i] - S[i, jstar[i]]) < 1e-10


@pytest.mark.parametrize("p", [0.0, 0.5])
def test_causal_first_row_is_first_value(p):
    inp, _, _ = _case(9, 16, "causal", seed=4)
    O, lse = A.forward(inp.q, inp.k, inp.v, scale=0.25, causal=True, dropout_p=p,
                       seed=inp.seed)
    q, k, v = (t.double().numpy() for t in (inp.q, inp.k, inp.v))
    for b, h in itertools.product(range(2), range(2)):
        keep = philox.keep_mask(inp.seed, b, h, 9, 9, p)
        z = (keep[0, 0] * philox.keep_scale(p)) if p else 1.0
        assert np.allclose(O[b, h, 0], z * v[b, h, 0], atol=1e-14, rtol=0)
        assert abs(lse[b, h, 0] - 0.25 * q[b, h, 0] @ k[b, h, 0]) < 1e-13


# --------------------------------------------------------------------------
# invariants

@pytest.mark.parametrize("mask", MASKS)
def test_probability_rows_sum_to_one(mask):
    inp, causal, kv = _case(50, 32, mask, seed=9, std=3.0)
    P = A.probabilities(inp.q, inp.k, scale=0.2, causal=causal, kv_len=kv)
    sums = P.sum(-1)
    assert np.abs(sums - 1.0).max() < 1e-13
    assert (P >= 0).all()
    if causal:
        assert np.all(np.triu(P[..., :, :], 1) == 0)


@pytest.mark.parametrize("mask", MASKS)
@pytest.mark.parametrize("p", [0.0, 0.2])
@pytest.mark.parametrize("block", [1, 3, 64, None])
def test_online_softmax_recurrence_equals_definition(mask, p, block):
    N = 97
    inp, causal, kv = _case(N, 16, mask, seed=13, std=3.0)
    O, lse = A.forward(inp.q, inp.k, inp.v, scale=0.3, causal=causal, kv_len=kv,
                       dropout_p=p, seed=inp.seed)
    for b, h in itertools.product(range(2), range(2)):
        Ot, lt = OS.forward_head(inp.q[b, h], inp.k[b, h], inp.v[b, h], scale=0.3,
                                 block=block or N, causal=causal,
                                 kv_len=None if kv is None else int(kv[b]),
                                 dropout_p=p, seed=inp.seed, b=b, h=h)
        assert np.abs(Ot - O[b, h]).max() <= 1e-13
        assert np.abs(lt - lse[b, h]).max() <= 1e-13


@pytest.mark.parametrize("mask", ["none", "causal", "pad"])
def test_key_shift_invariance(mask):
    inp, causal, kv = _case(40, 16, mask, seed=21)
    q, k, v = (t.double() for t in (inp.q, inp.k, inp.v))
    u = torch.randn(16, dtype=torch.float64)
    s = float(np.float32(0.25))
    O1, l1 = A.forward(q, k, v, scale=0.25, causal=causal, kv_len=kv)
    O2, l2 = A.forward(q, k + u, v, scale=0.25, causal=causal, kv_len=kv)
    assert np.abs(O1 - O2).max() < 1e-12
    assert np.abs((l2 - l1) - s * (q.numpy() @ u.numpy())).max() < 1e-11


def test_key_value_permutation_invariance():
    inp, _, _ = _case(40, 16, "none", seed=22)
    perm = torch.randperm(40, generator=torch.Generator().manual_seed(1))
    O1, l1 = A.forward(inp.q, inp.k, inp.v, scale=0.25)
    O2, l2 = A.forward(inp.q, inp.k[:, :, perm], inp.v[:, :, perm], scale=0.25)
    assert np.abs(O1 - O2).max() < 1e-13
    assert np.abs(l1 - l2).max() < 1e-13


@pytest.mark.parametrize("mask", MASKS)
@pytest.mark.parametrize("p", [0.0, 0.3])
def test_backward_central_finite_differences(mask, p):
    N, d = 6, 4
    inp, causal, kv = _case(N, d, mask, B=2, H=1, seed=31, with_do=True)
    q, k, v, do = (t.double().numpy() for t in (inp.q, inp.k, inp.v, inp.do))
    kw = dict(scale=0.7, causal=causal, kv_len=kv, dropout_p=p, seed=inp.seed)
    dq, dk, dv = A.backward(q, k, v, do, **kw)

    def loss(qq, kk, vv):
        O, _ = A.forward(qq, kk, vv, **kw)
        return float((O * do).sum())

    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp = x.copy()
            xm = x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = [q, k, v]
            args_m = [q, k, v]
            pos = "qkv".index(name)
            args_p[pos] = xp
            args_m[pos] = xm
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        assert np.abs(num - g).max() < 1e-7, name


@pytest.mark.parametrize("mask", MASKS)
def test_gradient_sum_rules(mask):
    N, d = 33, 16
    inp, causal, kv = _case(N, d, mask, seed=41, with_do=True)
    dq, dk, dv = A.backward(inp.q, inp.k, inp.v, inp.do, scale=0.3, causal=causal,
                            kv_len=kv)
    # sum_j dS_ij = 0 for every i  =>  sum_j dK_j = s * sum_i (sum_j dS_ij) Q_i = 0
    assert np.abs(dk.sum(axis=2)).max() < 1e-12
    # without dropout, sum_j P_ij = 1 for rows with a valid key => sum_j dV_j = sum_i dO_i
    do = inp.do.double().numpy()
    assert np.abs(dv.sum(axis=2) - do.sum(axis=2)).max() < 1e-11
    # equal keys: S_ij is constant in j on the valid set, dS rows sum to 0 => dQ = 0
    k_eq = inp.k.clone()
    k_eq[:] = inp.k[:, :, :1]
    dq2, _, _ = A.backward(inp.q, k_eq, inp.v, inp.do, scale=0.3, causal=causal,
                           kv_len=kv)
    assert np.abs(dq2).max() < 1e-12


def test_sampled_forms_equal_full_forms():
    N, d = 150, 32
    inp, causal, kv = _case(N, d, "causal_pad", seed=51, with_do=True)
    kw = dict(scale=0.2, causal=causal, kv_len=kv, dropout_p=0.15, seed=inp.seed)
    O, lse = A.forward(inp.q, inp.k, inp.v, **kw)
    rows = np.array([0, 3, 77, 149])
    Or, lr = A.forward(inp.q, inp.k, inp.v, rows=rows, heads=[(1, 0)], **kw)
    assert np.abs(Or[1, 0] - O[1, 0, rows]).max() < 1e-14
    assert np.abs(lr[1, 0] - lse[1, 0, rows]).max() < 1e-14
    dq, dk, dv = A.backward(inp.q, inp.k, inp.v, inp.do, **kw)
    cols = np.array([1, 70, 148])
    sq, sk, sv = A.backward_sampled(inp.q, inp.k, inp.v, inp.do, heads=[(1, 1)],
                                    rows=rows, cols=cols, row_chunk=40, **kw)
    assert np.abs(sq[(1, 1)] - dq[1, 1, rows]).max() < 1e-13
    assert np.abs(sk[(1, 1)] - dk[1, 1, cols]).max() < 1e-13
    assert np.abs(sv[(1, 1)] - dv[1, 1, cols]).max() < 1e-13
