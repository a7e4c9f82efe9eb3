"""GPU parity at extreme sizes: one causal head of 2^20 tokens (d = 128) and a
batch of 4096 short heads. The long head exercises the index arithmetic far
beyond the benchmark's sizes. The oracle checks it on sampled query rows (O,
lse, dQ) and on the last 300 key columns (dK, dV), each from the definition:
under the causal mask query row r sees keys 0..r only, which is the
non-square problem of that one row against those keys (bottom-right
alignment puts it on key r); and key columns j >= N - 300 receive gradient
only from rows i >= j, which is the problem of those 300 rows against all N
keys. The gradients are also checked through properties that hold at any size
(sum_j dK_j = 0; sum_j dV_j = sum_i dO_i without dropout)."""
import sys

import numpy as np
import pytest
import torch

import attn_workloads as W
import exact_tiled_attention_20_amd as attn
from oracle import attention as A
from parity import GRAD_ATOL, O_ATOL, check_close, check_lse

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _say(msg):
    print(msg)
    sys.stdout.flush()


def test_one_head_of_a_million_tokens():
    N, d = 1 << 20, 128
    g = torch.Generator().manual_seed(77)
    q, k, v, do = (torch.randn(1, 1, N, d, generator=g).to(torch.bfloat16) for _ in range(4))
    scale = d ** -0.5
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    _say("2^20-token head: gpu forward + backward")
    o, lse = attn.fwd(qd, kd, vd, causal=True, scale=scale, out_dtype=torch.float32)
    dq, dk, dv = attn.bwd(qd, kd, vd, o, lse, dod, causal=True, scale=scale,
                          out_dtype=torch.float32)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 127, 128, 4095, 65536, 500001, N - 129, N - 2, N - 1])
    _say("2^20-token head: oracle on sampled rows")
    O_r, l_r = A.forward(q, k, v, rows=rows, scale=scale, causal=True)
    check_close("O", o[:, :, rows].cpu(), O_r, O_ATOL, torch.float32)
    check_lse(lse[:, :, rows].cpu(), l_r)
    kw = dict(scale=scale, causal=True)
    _say("2^20-token head: oracle dQ on sampled rows")
    for r in rows:
        dq_r, _, _ = A.backward_sampled(q[:, :, r:r + 1], k[:, :, :r + 1], v[:, :, :r + 1],
                                        do[:, :, r:r + 1], heads=[(0, 0)], rows=[0],
                                        cols=np.zeros(0, dtype=np.int64), row_chunk=1, **kw)
        check_close(f"dQ row {r}", dq[0, 0, r:r + 1].cpu(), dq_r[(0, 0)], GRAD_ATOL,
                    torch.float32)
    lo = N - 300
    cols = np.arange(lo, N)
    _say("2^20-token head: oracle dK, dV on the last 300 key columns")
    _, dk_r, dv_r = A.backward_sampled(q[:, :, lo:], k, v, do[:, :, lo:], heads=[(0, 0)],
                                       rows=np.zeros(0, dtype=np.int64), cols=cols,
                                       row_chunk=8, **kw)
    ek, _ = check_close("dK tail", dk[0, 0, lo:].cpu(), dk_r[(0, 0)], GRAD_ATOL, torch.float32)
    ev, _ = check_close("dV tail", dv[0, 0, lo:].cpu(), dv_r[(0, 0)], GRAD_ATOL, torch.float32)
    sk = dk.double().sum(dim=2).abs().max().item()
    dsv = (dv.double().sum(dim=2) - dod.double().sum(dim=2)).abs().max().item()
    _say(f"2^20-token head: dK/dV tail max|err| {ek:.2e} / {ev:.2e}; max|sum dK| {sk:.3e}, "
         f"max|sum dV - sum dO| {dsv:.3e}")
    assert sk < 0.5 and dsv < 0.5
    assert torch.isfinite(dq).all() and torch.isfinite(dk).all() and torch.isfinite(dv).all()


def test_four_thousand_short_heads():
    B, H, N, d = 64, 64, 64, 64
    inp = W.random_case(B, H, N, d, "fp16", seed=5, with_do=True)
    q, k, v, do = (t.to(DEV) for t in (inp.q, inp.k, inp.v, inp.do))
    o, lse = attn.fwd(q, k, v, causal=True, scale=0.125, out_dtype=torch.float32)
    dq, dk, dv = attn.bwd(q, k, v, o, lse, do, causal=True, scale=0.125,
                          out_dtype=torch.float32)
    torch.cuda.synchronize()
    heads = [(0, 0), (B - 1, H - 1), (17, 42), (40, 3)]
    O_ref, lse_ref = A.forward(inp.q, inp.k, inp.v, scale=0.125, causal=True, heads=heads)
    g_ref = A.backward(inp.q, inp.k, inp.v, inp.do, scale=0.125, causal=True, heads=heads)
    for (b, h) in heads:
        check_close("O", o[b, h].cpu(), O_ref[b, h], O_ATOL, torch.float32)
        check_lse(lse[b, h].cpu(), lse_ref[b, h])
        for name, got, ref in zip(("dQ", "dK", "dV"), (dq, dk, dv), g_ref):
            check_close(name, got[b, h].cpu(), ref[b, h], GRAD_ATOL, torch.float32)
