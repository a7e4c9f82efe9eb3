"""GPU parity at the full sizes of the variants the benchmark times: a
Mistral-style sliding window of 4096 keys over a 16K-token causal layer (B=1,
H=32, N=16384, d=128, bf16), a 2048-query chunk attending causally,
bottom-right aligned, to a 16384-key context (B=4, H=16, d=128, bf16), and
head dimension 256 (B=1, H=16, N=16384, causal, bf16), each forward +
backward in the launch configuration the benchmark uses (outputs in the input
dtype) and in the float32-output mode.

The oracle checks sampled heads: on sampled query rows (O, lse, dQ) and key
columns (dK, dV), each evaluated from the definition ("Why FlashAttention Is
a Kernel Story", section "When it falls down", names both variants)."""
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


# The variants with a backward (the fp8 forward variants have their own tests
# in test_gpu_fp8.py).
@pytest.fixture(scope="module", params=[n for n, w in W.VARIANTS.items() if w.backward])
def variant_gpu(request):
    w = W.VARIANTS[request.param]
    inp = W.make_inputs(w)
    q, k, v, do = (t.to(DEV) for t in (inp.q, inp.k, inp.v, inp.do))
    res = {}
    for odt in (inp.q.dtype, torch.float32):
        _say(f"[{w.name}] gpu fwd+bwd out={odt}")
        o, lse = attn.fwd(q, k, v, causal=w.causal, window=w.window, scale=w.scale,
                          out_dtype=odt)
        dq, dk, dv = attn.bwd(q, k, v, o, lse, do, causal=w.causal, window=w.window,
                              scale=w.scale, out_dtype=odt)
        torch.cuda.synchronize()
        res[odt] = tuple(t.cpu() for t in (o, lse, dq, dk, dv))
    del q, k, v, do
    return w, inp, res


def test_variant_fwd_bwd_sampled(variant_gpu):
    w, inp, res = variant_gpu
    rng = np.random.default_rng(w.seed)
    heads = [(0, 0), (w.B - 1, w.H - 1), (int(rng.integers(w.B)), int(rng.integers(w.H)))]
    edge_rows = [0, 1, 63, 64, 4095, 4096, w.N // 2, w.N - 1]
    rows = np.unique(np.concatenate([[r for r in edge_rows if r < w.N],
                                     rng.integers(0, w.N, 90)]))
    edge_cols = [0, 1, 127, 128, 4095, 4096, 8191, w.Nk - 2, w.Nk - 1]
    cols = np.unique(np.concatenate([[c for c in edge_cols if c < w.Nk],
                                     rng.integers(0, w.Nk, 90)]))
    kw = dict(scale=w.scale, causal=w.causal, window=w.window)
    for head in heads:
        b, h = head
        _say(f"[{w.name}] head {head}: oracle on {rows.size} rows / {cols.size} columns")
        O_r, l_r = A.forward(inp.q, inp.k, inp.v, rows=rows, heads=[head], **kw)
        dq_r, dk_r, dv_r = A.backward_sampled(inp.q, inp.k, inp.v, inp.do, heads=[head],
                                              rows=rows, cols=cols, **kw)
        for odt, (o, lse, dq, dk, dv) in res.items():
            eo, _ = check_close("O", o[b, h, rows], O_r[b, h], O_ATOL, odt)
            check_lse(lse[b, h, rows], l_r[b, h])
            eq, _ = check_close("dQ", dq[b, h, rows], dq_r[head], GRAD_ATOL, odt)
            ek, _ = check_close("dK", dk[b, h, cols], dk_r[head], GRAD_ATOL, odt)
            ev, _ = check_close("dV", dv[b, h, cols], dv_r[head], GRAD_ATOL, odt)
            _say(f"[{w.name}] head {head} out={odt}: max|err| O {eo:.2e} dQ {eq:.2e} "
                 f"dK {ek:.2e} dV {ev:.2e}")


def test_variant_gradient_invariants(variant_gpu):
    """Hold at any size (float32 mode, no dropout): sum_j dK_j = 0 per head;
    sum_j dV_j = sum_i dO_i over the rows that see at least one key (all rows
    here: the window and the bottom-right diagonal always keep key c_i)."""
    w, inp, res = variant_gpu
    o, lse, dq, dk, dv = res[torch.float32]
    sk = dk.double().sum(dim=2).abs().max().item()
    dsv = (dv.double().sum(dim=2) - inp.do.double().sum(dim=2)).abs().max().item()
    _say(f"[{w.name}] max|sum_j dK_j| {sk:.3e}, max|sum_j dV_j - sum_i dO_i| {dsv:.3e}")
    assert sk < 1.0 and dsv < 1.0

