"""GPU parity for head dimension 256 (forward and backward), against the
fp64 oracle.

"Why FlashAttention Is a Kernel Story", section "When it falls down", notes
that head dimensions like 256 need smaller tiles or spill on parts with small
on-chip memory. On gfx950 a 64-key K tile and V tile at d = 256 take 32 KiB
each, so the double-buffered pair fits the 160 KiB LDS at one workgroup of
four waves per CU; the kernel is the same tiled forward at one wave per SIMD.
The dK/dV kernel keeps 128 keys of K and V resident (128 KiB) with single
16 KiB Q and dO tiles; dQ has the forward's shape."""
import sys

import numpy as np
import pytest
import torch

import attn_workloads as W
import exact_tiled_attention_20_amd as attn
from oracle import attention as A
from parity import O_ATOL, check_close, check_lse

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a device"
    attn.load_library()
    yield


CASES = [(N, dt, mask, p)
         for N in (1, 63, 64, 65, 200, 700)
         for dt in ("fp16", "bf16")
         for mask in ("none", "causal", "pad", "window")
         for p in (0.0, 0.1)
         if p == 0.0 or N in (65, 200)]


@pytest.mark.parametrize("N,dt,mask,p", CASES)
def test_fwd_d256(N, dt, mask, p):
    B, H, d = 2, 2, 256
    kv = [max(1, N - 9), N] if mask == "pad" else None
    nk = N + 37 if mask == "window" else None
    inp = W.random_case(B, H, N, d, dt, seed=N + len(mask) * 5, std=1.5, kv_len=kv, n_k=nk)
    causal = mask in ("causal", "window")
    window = (50, -1) if mask == "window" else None
    scale = 1.0 / np.sqrt(d)
    O_ref, lse_ref = A.forward(inp.q, inp.k, inp.v, scale=scale, causal=causal,
                               kv_len=inp.kv_len, dropout_p=p, seed=inp.seed, window=window)
    q, k, v = (t.to(DEV) for t in (inp.q, inp.k, inp.v))
    kvd = None if inp.kv_len is None else inp.kv_len.to(DEV)
    print(f"d256 fwd N={N} {dt} {mask} p={p}")
    sys.stdout.flush()
    for odt in (torch.float32, inp.q.dtype):
        o, lse = attn.fwd(q, k, v, causal=causal, kv_len=kvd, dropout_p=p, seed=inp.seed,
                          scale=scale, out_dtype=odt, window=window)
        torch.cuda.synchronize()
        check_close("O", o, O_ref, O_ATOL, odt)
        check_lse(lse, lse_ref)


def test_fwd_d256_wide_scores_long():
    """Q, K ~ 3 N(0,1) at N = 2500, causal: the running maximum moves often."""
    inp = W.random_case(1, 2, 2500, 256, "bf16", seed=77, std=3.0)
    scale = 1.0 / 16.0
    O_ref, lse_ref = A.forward(inp.q, inp.k, inp.v, scale=scale, causal=True)
    q, k, v = (t.to(DEV) for t in (inp.q, inp.k, inp.v))
    o, lse = attn.fwd(q, k, v, causal=True, scale=scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    check_close("O", o, O_ref, O_ATOL, torch.float32)
    check_lse(lse, lse_ref)


BWD_CASES = [(N, dt, mask, p)
             for N in (1, 63, 65, 200, 300)
             for dt in ("fp16", "bf16")
             for mask in ("none", "causal", "pad", "window")
             for p in (0.0, 0.2)
             if p == 0.0 or N in (65, 200)]



@pytest.mark.parametrize("N,dt,mask,p", BWD_CASES)
def test_bwd_d256(N, dt, mask, p):
    from parity import GRAD_ATOL, d_rounding_bounds
    B, H, d = 2, 2, 256
    kv = [max(1, N - 9), N] if mask == "pad" else None
    nk = N + 37 if mask == "window" else None
    inp = W.random_case(B, H, N, d, dt, seed=N * 3 + len(mask), with_do=True, kv_len=kv,
                        n_k=nk)
    causal = mask in ("causal", "window")
    window = (50, -1) if mask == "window" else None
    scale = 1.0 / np.sqrt(d)
    kw = dict(scale=scale, causal=causal, kv_len=inp.kv_len, dropout_p=p, seed=inp.seed,
              window=window)
    dq_ref, dk_ref, dv_ref = A.backward(inp.q, inp.k, inp.v, inp.do, **kw)
    O_ref, _ = A.forward(inp.q, inp.k, inp.v, **kw)
    P = A.probabilities(inp.q, inp.k, scale=scale, causal=causal, kv_len=inp.kv_len,
                        window=window)
    q, k, v, do = (t.to(DEV) for t in (inp.q, inp.k, inp.v, inp.do))
    kvd = None if inp.kv_len is None else inp.kv_len.to(DEV)
    print(f"d256 bwd N={N} {dt} {mask} p={p}")
    sys.stdout.flush()
    for odt in (torch.float32, inp.q.dtype):
        o, lse = attn.fwd(q, k, v, causal=causal, kv_len=kvd, dropout_p=p, seed=inp.seed,
                          scale=scale, out_dtype=odt, window=window)
        dq, dk, dv = attn.bwd(q, k, v, o, lse, do, causal=causal, kv_len=kvd, dropout_p=p,
                              seed=inp.seed, scale=scale, out_dtype=odt, window=window)
        torch.cuda.synchronize()
        bdq, bdk = d_rounding_bounds(inp.q, inp.k, inp.do, O_ref, P, scale, odt)
        check_close("dQ", dq, dq_ref, GRAD_ATOL + bdq, odt)
        check_close("dK", dk, dk_ref, GRAD_ATOL + bdk, odt)
        check_close("dV", dv, dv_ref, GRAD_ATOL, odt)
