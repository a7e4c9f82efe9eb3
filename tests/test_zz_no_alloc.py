"""attn_bwd_noalloc (the backward with the library's fixed per-GPU scratch in
place of a caller workspace) against attn_bwd on the same inputs, through the
C ABI: two calls in a row, the second on a smaller problem, so that what the
first call left in the shared scratch cannot leak into the second. Both entry
points run the same kernels on the same inputs, so their outputs must agree
bit for bit (which is within the parity bar by construction)."""
import sys

import numpy as np
import pytest
import torch

import attn_workloads as W
import exact_tiled_attention_20_amd as attn

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _say(msg):
    print(msg)
    sys.stdout.flush()


CASES = [
    # (B, H, N, Nk, d, dtype, kw, out_dtype): the larger problem first.
    (2, 3, 1000, 1000, 128, "bf16", dict(causal=True), None),
    (1, 2, 300, 270, 64, "fp16",
     dict(causal=True, window=(100, -1), kv_len=[250], dropout_p=0.1, seed=77), torch.float32),
]


def _run(case, noalloc):
    B, H, N, Nk, d, dt, kw, odt = case
    kw = dict(kw)
    kv = kw.pop("kv_len", None)
    inp = W.random_case(B, H, N, d, dt, seed=N + d, with_do=True, n_k=Nk, kv_len=kv)
    q, k, v, do = (t.to(DEV) for t in (inp.q, inp.k, inp.v, inp.do))
    kvd = None if inp.kv_len is None else inp.kv_len.to(DEV)
    kw.update(kv_len=kvd, scale=1.0 / np.sqrt(d), out_dtype=odt)
    o, lse = attn.fwd(q, k, v, **kw)
    fn = attn.bwd_noalloc if noalloc else attn.bwd
    grads = fn(q, k, v, o, lse, do, **kw)
    torch.cuda.synchronize()
    return [g.cpu() for g in grads]


def test_noalloc_matches_the_workspace_entry_point_twice():
    assert attn.noalloc_max_workspace_bytes() == 16 << 20
    for case in CASES:
        _say(f"[noalloc] case B,H,N,Nk,d,dtype = {case[:6]} {case[6]}")
        ref = _run(case, noalloc=False)
        got = _run(case, noalloc=True)
        for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
            assert g.shape == r.shape and g.dtype == r.dtype, name
            assert torch.equal(g, r), f"{name}: max diff {(g.double() - r.double()).abs().max()}"
        _say(f"[noalloc] case {case[:6]}: dQ, dK, dV bit-identical to attn_bwd")


def test_noalloc_refuses_a_problem_beyond_its_scratch():
    """B*H*N rows whose workspace exceeds the scratch: refused before any launch."""
    q = torch.zeros(1, 64, (1 << 15) + 64, 64, dtype=torch.float16, device=DEV)
    o = torch.zeros_like(q)
    lse = torch.zeros(q.shape[:3], dtype=torch.float32, device=DEV)
    with pytest.raises(attn.AttnError) as e:
        attn.bwd_noalloc(q, q, q, o, lse, q)
    assert e.value.status == 5
    torch.cuda.synchronize()
