"""GPU check of the backward's first step (B0, preprocess) through the stage
entry point, on its workspace: D_i = dO_i . O_i in fp32 and lse_i in log2
units, in two float32 arrays of Np rows per head (N rounded up to a multiple
of 4), the rows past N holding D = 0 and lse = +inf so that the dK/dV kernel's
four-row loads read finite values ("Why FlashAttention Is a Kernel Story",
section "When it falls down": the backward rebuilds its statistics from the
stored output and log-sum-exp).

O and lse here are seeded inputs of their own, not a forward's output: the
preprocess only combines what it is given, and the expected values come from
those inputs in fp64."""
import math
import sys

import numpy as np
import pytest
import torch

import exact_tiled_attention_20_amd as attn

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
LOG2E = 1.4426950408889634

CASES = [  # B, H, N, d, dtype, out_dtype
    (2, 3, 101, 64, torch.float16, torch.float16),
    (1, 2, 7, 128, torch.bfloat16, torch.bfloat16),
    (1, 1, 1, 64, torch.float16, torch.float32),
    (2, 2, 130, 128, torch.bfloat16, torch.float32),
    (1, 1, 256, 256, torch.bfloat16, torch.bfloat16),
]


@pytest.mark.parametrize("B,H,N,d,dt,odt", CASES)
def test_preprocess_fills_padded_workspace(B, H, N, d, dt, odt):
    print(f"preprocess workspace B={B} H={H} N={N} d={d} {dt} -> {odt}")
    sys.stdout.flush()
    g = torch.Generator().manual_seed(1000 + N + d)
    q, k, v, do = (torch.randn(B, H, N, d, generator=g).to(dt) for _ in range(4))
    o = torch.randn(B, H, N, d, generator=g).to(odt)
    lse = (torch.randn(B, H, N, generator=g) * 4).float()
    lse[..., ::5] = -math.inf  # rows without a visible key
    qd, kd, vd, dod, od, lsed = (t.to(DEV) for t in (q, k, v, do, o, lse))
    need = attn.bwd_workspace_bytes(qd, k=kd, causal=True, out_dtype=odt)
    n_pad = (N + 3) // 4 * 4
    arr = (B * H * n_pad * 4 + 255) // 256 * 256
    assert need == 2 * arr
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device=DEV)  # NaN everywhere
    outs = (torch.empty(B, H, N, d, dtype=odt, device=DEV),
            torch.empty(B, H, N, d, dtype=odt, device=DEV),
            torch.empty(B, H, N, d, dtype=odt, device=DEV))
    attn.bwd(qd, kd, vd, od, lsed, dod, causal=True, out_dtype=odt, workspace=ws, out=outs,
             stage=attn.BWD_STAGE_PREPROCESS)
    torch.cuda.synchronize()
    wsh = ws.cpu()
    delta = wsh[:B * H * n_pad * 4].view(torch.float32).reshape(B, H, n_pad).numpy()
    lse2 = wsh[arr:arr + B * H * n_pad * 4].view(torch.float32).reshape(B, H, n_pad).numpy()
    # Padding rows: exactly D = 0 and lse = +inf.
    assert np.all(delta[..., N:] == 0.0)
    assert np.all(np.isposinf(lse2[..., N:]))
    # D_i = dO_i . O_i: the fp32 sum of d products is within d ulps of the fp64 value.
    prod = do.double().numpy() * o.double().numpy()
    want = prod.sum(-1)
    bound = d * np.finfo(np.float32).eps * np.abs(prod).sum(-1) + 1e-30
    err = np.abs(delta[..., :N] - want)
    print(f"  max |D - D_ref| {err.max():.3e}")
    assert np.all(err <= bound)
    # lse in log2 units: lse * log2(e) rounded once in fp32; +inf where lse = -inf.
    l_ref = lse.numpy().astype(np.float64)
    dead = np.isneginf(l_ref)
    assert np.all(np.isposinf(lse2[..., :N][dead]))
    live = ~dead
    ref2 = l_ref[live] * LOG2E
    assert np.all(np.abs(lse2[..., :N][live] - ref2) <= 2 * np.spacing(np.abs(ref2).astype(np.float32)))
