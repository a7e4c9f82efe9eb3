"""GPU parity of the fp8 (e4m3) forward against the oracle.

Q, K and V are e4m3; the oracle evaluates exact attention of the stored values
(decoded exactly to float64). The kernel's one approximation, rounding P to
e4m3 before the product with V, is bounded per element by
oracle.fp8.p_rounding_bound (at most 2^-4 relative per term, 2^-10 / L below
2^-6, dropout factor included); the bound here adds 2e-3 for the fp32
arithmetic (exp2, accumulation) and half an ulp of O when O is stored in
bfloat16. Because that bound is loose when P is spread over many keys, each
case also checks that the summed squared error stays below the upper variance
model of independent rounding errors (oracle.fp8.p_rounding_variance), which an
index mistake would exceed many times over. lse is fp32 and exact-path:
|dlse| <= 1e-3 max(1, |lse|)."""
import sys

import numpy as np
import pytest
import torch

import attn_workloads as W
import exact_tiled_attention_20_amd as attn
from oracle import attention as A
from oracle import fp8 as F8
from parity import check_lse, half_ulp, to64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
FP32_SLACK = 2e-3


def _say(msg):
    print(msg)
    sys.stdout.flush()


def _check(o, lse, inp, kw, heads=None, rows=None, out_dtype=torch.bfloat16):
    """Element bound and aggregate variance check on the given heads/rows.
    Returns (max |err|, sum err^2, sum of the variance model)."""
    q, k, v = inp.q, inp.k, inp.v
    B, H, N, _ = q.shape
    Nk = k.shape[2]
    heads = heads or [(b, h) for b in range(B) for h in range(H)]
    rsel = np.arange(N) if rows is None else np.asarray(rows)
    O_ref, lse_ref = A.forward(q, k, v, heads=heads, rows=rsel, **kw)
    og = to64(o)
    lg = to64(lse)
    vv = to64(v)
    emax, se, sv = 0.0, 0.0, 0.0
    for (b, h) in heads:
        P, L, valid = F8.row_stats(q, k, scale=kw["scale"], causal=kw.get("causal", False),
                                   kv_len=kw.get("kv_len"), window=kw.get("window"), b=b, h=h,
                                   rows=rsel)
        Z = None
        if kw.get("dropout_p", 0.0) > 0:
            Z = A.dropout_factor(kw["seed"], b, h, N, kw["dropout_p"], rows=rsel, n_k=Nk)
        ref = O_ref[b, h]
        got = og[b, h][rsel] if rows is not None else og[b, h]
        st = half_ulp(ref, out_dtype)
        bound = F8.p_rounding_bound(P, L, vv[b, h], Z) + FP32_SLACK + st
        err = got - ref
        bad = ~(np.abs(err) <= bound)
        if bad.any():
            i, c = np.argwhere(bad)[0]
            raise AssertionError(
                f"O[{b},{h}]: {bad.sum()} elements beyond the fp8 bound; first row "
                f"{rsel[i]} col {c}: got {got[i, c]!r} ref {ref[i, c]!r} bound {bound[i, c]:.3e}")
        emax = max(emax, float(np.abs(err).max()) if err.size else 0.0)
        se += float((err ** 2).sum())
        sv += float(F8.p_rounding_variance(P, L, vv[b, h], Z).sum() + (st ** 2 / 3).sum())
        lrow = lg[b, h][rsel] if rows is not None else lg[b, h]
        check_lse(lrow, lse_ref[b, h])
    return emax, se, sv


def _run(inp, kw, out_dtype):
    q, k, v = (t.to(DEV) for t in (inp.q, inp.k, inp.v))
    gkw = dict(kw)
    if gkw.get("kv_len") is not None:
        gkw["kv_len"] = gkw["kv_len"].to(DEV)
    o, lse = attn.fwd(q, k, v, out_dtype=out_dtype, **gkw)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


SWEEP = [
    # (N, Nk, mask, kv_len, window, p, qk_std, out)
    (1, 1, "none", None, None, 0.0, 1.0, torch.float32),
    (63, 63, "causal", None, None, 0.0, 1.0, torch.bfloat16),
    (64, 64, "none", None, None, 0.0, 3.0, torch.float32),
    (65, 65, "causal", None, None, 0.1, 1.0, torch.float32),
    (129, 129, "none", [100, 129], None, 0.0, 1.0, torch.bfloat16),
    (200, 200, "causal", [150, 1], None, 0.1, 3.0, torch.float32),
    (300, 700, "causal", None, (120, -1), 0.0, 1.0, torch.bfloat16),
    (700, 300, "causal", None, None, 0.0, 1.0, torch.float32),
    (257, 257, "none", None, (30, 40), 0.0, 3.0, torch.bfloat16),
    (1000, 1000, "causal", None, None, 0.0, 1.0, torch.bfloat16),
    (1000, 1000, "none", [1000, 537], None, 0.1, 1.0, torch.float32),
    (1024, 1024, "causal", None, None, 0.0, 3.0, torch.float32),
]


@pytest.mark.parametrize("case", SWEEP, ids=lambda c: f"N{c[0]}_Nk{c[1]}_{c[2]}_kv{c[3]}_w{c[4]}_p{c[5]}_s{c[6]}")
def test_fp8_forward_sweep(case):
    N, Nk, mask, kv, window, p, std, odt = case
    inp = W.random_case(2, 2, N, 128, "e4m3", seed=N * 7 + Nk, std=std, kv_len=kv, n_k=Nk)
    kw = dict(scale=1.0 / np.sqrt(128), causal=mask == "causal", kv_len=inp.kv_len,
              window=window, dropout_p=p, seed=inp.seed)
    _say(f"[fp8] case {case}")
    o, lse = _run(inp, kw, odt)
    emax, se, sv = _check(o, lse, inp, kw, out_dtype=odt)
    n = o.numel()
    _say(f"[fp8] max|err| {emax:.3e}; sum err^2 / variance model = {se / max(sv, 1e-300):.3f} "
         f"over {n} elements")
    if n >= 8192:
        assert se <= sv, (se, sv)


def test_fp8_rejected_for_the_backward_and_other_head_dims():
    inp = W.random_case(1, 1, 64, 128, "e4m3", seed=3, with_do=False)
    q, k, v = (t.to(DEV) for t in (inp.q, inp.k, inp.v))
    o, lse = attn.fwd(q, k, v)
    assert o.dtype == torch.bfloat16
    with pytest.raises(attn.AttnError) as e:
        attn.bwd(q, k, v, o, lse, torch.zeros(q.shape, dtype=torch.bfloat16, device=DEV).to(
            torch.float8_e4m3fn))
    assert e.value.status in (1, 2)
    q64 = torch.zeros(1, 1, 64, 64, dtype=torch.float8_e4m3fn, device=DEV)
    with pytest.raises(attn.AttnError) as e:
        attn.fwd(q64, q64, q64)
    assert e.value.status == 2
    torch.cuda.synchronize()


def test_fp8_long_layer_sampled():
    """B=4 H=16 N=4096 d=128, causal, Q and K ~ 3 N(0,1) (wide score range):
    two heads on every row, every head on 48 sampled rows."""
    w = W.VARIANTS["fp8_b4h16n4096d128_causal"]
    inp = W.make_inputs(w)
    kw = dict(scale=w.scale, causal=True)
    _say("[fp8 long] gpu forward")
    o, lse = _run(inp, kw, torch.bfloat16)
    e1, se1, sv1 = _check(o, lse, inp, kw, heads=[(0, 0), (3, 15)])
    rows = np.unique(np.concatenate([[0, 1, 63, 64, 4095],
                                     np.random.default_rng(9).integers(0, w.N, 43)]))
    e2, se2, sv2 = _check(o, lse, inp, kw, rows=rows)
    _say(f"[fp8 long] max|err| {max(e1, e2):.3e}; sum err^2 / variance model "
         f"{(se1 + se2) / (sv1 + sv2):.3f}")
    assert se1 + se2 <= sv1 + sv2


def test_fp8_ctx16k_sampled_rows():
    """B=1 H=32 N=16384 d=128 causal, Q, K, V ~ N(0,1): 64 sampled rows of
    three heads (flat probabilities: the aggregate check carries the weight)."""
    w = W.VARIANTS["fp8_b1h32n16384d128_causal"]
    inp = W.make_inputs(w)
    kw = dict(scale=w.scale, causal=True)
    _say("[fp8 16K] gpu forward")
    o, lse = _run(inp, kw, torch.float32)
    rows = np.unique(np.concatenate([[0, 1, 8191, 16383],
                                     np.random.default_rng(10).integers(0, w.N, 60)]))
    e, se, sv = _check(o, lse, inp, kw, heads=[(0, 0), (0, 17), (0, 31)], rows=rows,
                       out_dtype=torch.float32)
    _say(f"[fp8 16K] max|err| {e:.3e}; sum err^2 / variance model {se / sv:.3f}")
    assert se <= sv
