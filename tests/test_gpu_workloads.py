"""GPU parity at the full sizes of the five named workloads, in the launch
configuration the benchmark times (outputs in the input dtype), plus the
float32-output mode as the strict gate.

Where the oracle cannot materialise every head in seconds, it checks sampled
heads and, inside a head, sampled query rows (forward, dQ) and key columns
(dK, dV) -- each evaluated one by one from the definition."""
import sys

import numpy as np
import pytest
import torch

import attn_workloads as W
import exact_tiled_attention_20_amd as attn
from oracle import attention as A
from oracle import philox
from parity import GRAD_ATOL, O_ATOL, check_close, check_lse, plain_excess, to64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _say(msg):
    print(msg)
    sys.stdout.flush()


def _gpu_forward(w, inp, out_dtype):
    q, k, v = (t.to(DEV) for t in (inp.q, inp.k, inp.v))
    kv = None if inp.kv_len is None else inp.kv_len.to(DEV)
    o, lse = attn.fwd(q, k, v, causal=w.causal, kv_len=kv, dropout_p=w.dropout_p,
                      seed=inp.seed, scale=w.scale, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def _sampled_heads(w, n, seed):
    rng = np.random.default_rng(seed)
    heads = [(0, 0), (w.B - 1, w.H - 1)]
    while len(heads) < n:
        hd = (int(rng.integers(w.B)), int(rng.integers(w.H)))
        if hd not in heads:
            heads.append(hd)
    return heads


@pytest.fixture(scope="module")
def inputs_cache():
    return {}


def _inputs(cache, name):
    if name not in cache:
        cache[name] = W.make_inputs(W.WORKLOADS[name])
    return cache[name]


@pytest.mark.parametrize("name", ["tiny_b1h2n256d64_fp16", "decoder_b8h12n1024d64_fp16_causal",
                                  "bert_b16h16n512d64_fp16_pad_drop"])
def test_forward_every_head(name, inputs_cache):
    w = W.WORKLOADS[name]
    inp = _inputs(inputs_cache, name)
    _say(f"[{name}] oracle forward, all {w.B * w.H} heads")
    O_ref, lse_ref = A.forward(inp.q, inp.k, inp.v, scale=w.scale, causal=w.causal,
                               kv_len=inp.kv_len, dropout_p=w.dropout_p, seed=inp.seed)
    for odt in (inp.q.dtype, torch.float32):
        _say(f"[{name}] gpu forward out={odt}")
        o, lse = _gpu_forward(w, inp, odt)
        err, bias = check_close("O", o, O_ref, O_ATOL, odt)
        check_lse(lse, lse_ref)
        _say(f"[{name}] out={odt}: max|err| {err:.3e}, mean signed err {bias:.2e}")


def test_dropout_mask_of_padded_workload(inputs_cache):
    name = "bert_b16h16n512d64_fp16_pad_drop"
    w = W.WORKLOADS[name]
    inp = _inputs(inputs_cache, name)
    keep = attn.dropout_mask(w.B, w.H, w.N, w.dropout_p, inp.seed, DEV).cpu().numpy()
    for b, h in _sampled_heads(w, 6, 3):
        assert np.array_equal(keep[b, h].astype(bool),
                              philox.keep_mask(inp.seed, b, h, w.N, w.N, w.dropout_p))
    drop_rate = 1.0 - keep.mean()
    assert abs(drop_rate - w.dropout_p) < 5 * np.sqrt(0.09 / keep.size)


LONG = "long_b4h16n4096d128_bf16_causal"


@pytest.fixture(scope="module")
def long_gpu(inputs_cache):
    w = W.WORKLOADS[LONG]
    inp = _inputs(inputs_cache, LONG)
    return w, inp, {odt: _gpu_forward(w, inp, odt) for odt in (inp.q.dtype, torch.float32)}


@pytest.mark.parametrize("b", range(4))
def test_long_forward_every_head(long_gpu, b):
    """4 x 16 heads, N = 4096, d = 128, causal, Q and K ~ 3 N(0,1): every head on
    every row, in both output modes (one batch entry per test)."""
    w, inp, gpu = long_gpu
    kw = dict(scale=w.scale, causal=w.causal)
    worst = {odt: (0.0, 0) for odt in gpu}
    for h in range(w.H):
        O_h, l_h = A.forward(*(t[b:b + 1, h:h + 1] for t in (inp.q, inp.k, inp.v)), **kw)
        O_h, l_h = O_h[0, 0], l_h[0, 0]
        for odt, (o, lse) in gpu.items():
            err, _ = check_close(f"O[{b},{h}] out={odt}", o[b, h], O_h, O_ATOL, odt)
            check_lse(lse[b, h], l_h)
            n = int((~(np.abs(to64(o[b, h]) - O_h) <= O_ATOL)).sum())
            worst[odt] = (max(worst[odt][0], err), worst[odt][1] + n)
    for odt, (err, n) in worst.items():
        _say(f"[{LONG}] batch {b} out={odt}: max|err| {err:.3e}; {n} of {w.H * w.N * w.d} "
             f"elements beyond plain {O_ATOL:g}")


CTX = "ctx16k_b1h32n16384d128_bf16_causal_bwd"


@pytest.fixture(scope="module")
def ctx_gpu(inputs_cache):
    """Forward + backward at B=1, H=32, N=16384, d=128 on the GPU, both output modes."""
    w = W.WORKLOADS[CTX]
    inp = _inputs(inputs_cache, CTX)
    q, k, v, do = (t.to(DEV) for t in (inp.q, inp.k, inp.v, inp.do))
    res = {}
    for odt in (inp.q.dtype, torch.float32):
        _say(f"[{CTX}] gpu fwd+bwd out={odt}")
        o, lse = attn.fwd(q, k, v, causal=True, scale=w.scale, out_dtype=odt)
        dq, dk, dv = attn.bwd(q, k, v, o, lse, do, causal=True, scale=w.scale, out_dtype=odt)
        torch.cuda.synchronize()
        res[odt] = tuple(t.cpu() for t in (o, lse, dq, dk, dv))
    return w, inp, res


CTX_HEADS = [(0, 0), (0, 31), (0, 11), (0, 22)]


@pytest.mark.parametrize("head", CTX_HEADS)
def test_ctx16k_fwd_bwd_full_head(ctx_gpu, head):
    """Every one of the 16384 rows (O, lse, dQ) and of the 16384 key columns
    (dK, dV) of the sampled head, against the oracle evaluated in row chunks
    (each chunk forms its full rows of P and dS)."""
    w, inp, res = ctx_gpu
    b, h = head
    rows = np.arange(w.N)
    kw = dict(scale=w.scale, causal=True)
    # The oracle sees only this head (each head is independent by definition).
    qh, kh, vh, doh = (t[b:b + 1, h:h + 1] for t in (inp.q, inp.k, inp.v, inp.do))
    _say(f"[{CTX}] head {head}: oracle forward, all {w.N} rows")
    O_r = np.empty((w.N, w.d))
    l_r = np.empty(w.N)
    for r0 in range(0, w.N, 1024):
        rr = rows[r0:r0 + 1024]
        O_c, l_c = A.forward(qh, kh, vh, rows=rr, **kw)
        O_r[rr] = O_c[0, 0]
        l_r[rr] = l_c[0, 0]
    _say(f"[{CTX}] head {head}: oracle backward, all rows and key columns")
    dq_r, dk_r, dv_r = (x[(0, 0)] for x in A.backward_sampled(
        qh, kh, vh, doh, heads=[(0, 0)], rows=rows, cols=rows, **kw))
    for odt, (o, lse, dq, dk, dv) in res.items():
        eo, _ = check_close("O", o[b, h], O_r, O_ATOL, odt)
        check_lse(lse[b, h], l_r)
        eq, bq = check_close("dQ", dq[b, h], dq_r, GRAD_ATOL, odt)
        ek, bk = check_close("dK", dk[b, h], dk_r, GRAD_ATOL, odt)
        ev, bv = check_close("dV", dv[b, h], dv_r, GRAD_ATOL, odt)
        _say(f"[{CTX}] head {head} out={odt}: max|err| O {eo:.2e} dQ {eq:.2e} "
             f"dK {ek:.2e} dV {ev:.2e}; mean signed dQ {bq:.1e} dK {bk:.1e} dV {bv:.1e}")
        plain_excess("O", o[b, h], O_r, O_ATOL)
        for name, g, r in (("dQ", dq[b, h], dq_r), ("dK", dk[b, h], dk_r),
                           ("dV", dv[b, h], dv_r)):
            plain_excess(name, g, r, GRAD_ATOL)
        sys.stdout.flush()


def test_ctx16k_gradient_invariants(ctx_gpu):
    """Properties of the exact gradients that hold at any size (float32 mode):
    sum_j dK_j = 0 per head, and sum_j dV_j = sum_i dO_i (no dropout, every row
    has a visible key)."""
    w, inp, res = ctx_gpu
    o, lse, dq, dk, dv = res[torch.float32]
    do = inp.do.double()
    sk = dk.double().sum(dim=2)
    assert sk.abs().max().item() < 1.0, sk.abs().max().item()
    dsv = (dv.double().sum(dim=2) - do.sum(dim=2)).abs().max().item()
    assert dsv < 1.0, dsv
    _say(f"[{CTX}] max|sum_j dK_j| {sk.abs().max().item():.3e}, "
         f"max|sum_j dV_j - sum_i dO_i| {dsv:.3e}")
