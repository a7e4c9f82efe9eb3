"""GPU parity for the sliding-window and non-square (cross-attention) masks:
the HIP kernels (through the C ABI) against the fp64 oracle.

"Why FlashAttention Is a Kernel Story", section "When it falls down", names
sliding-window attention and cross-attention with non-square K, V grids as the
variants that need tiling changes. Query i lines up with key i + Nk - N; the
causal mask and the window (left, right; -1 unbounded) are taken from that
key. The cases span several tiles with ragged tails on both axes, windows that
start and end inside a tile, rows that see no key at all, key padding and
dropout, both dtypes and both head dimensions."""
import itertools
import sys

import numpy as np
import pytest
import torch

import attn_workloads as W
import exact_tiled_attention_20_amd as attn
from oracle import attention as A
from oracle import philox
from parity import GRAD_ATOL, O_ATOL, check_close, check_lse, d_rounding_bounds

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a device"
    attn.load_library()
    yield


# (N, Nk, causal, window)
FWD_SHAPES = [
    (200, 64, False, None), (64, 200, False, None), (129, 1000, False, None),
    (1000, 129, True, None), (129, 1000, True, None), (300, 300, True, (100, -1)),
    (300, 300, False, (37, 37)), (513, 513, False, (0, 0)), (513, 700, True, (64, -1)),
    (700, 513, True, (200, -1)), (257, 257, False, (-1, 50)), (1, 300, True, None),
    (300, 1, True, None), (190, 190, False, (5, 130)), (1000, 1000, True, (511, -1)),
    (64, 64, True, (63, -1)), (77, 400, False, (20, 3)),
]


def _kv(Nk, B, pad):
    if not pad:
        return None
    vals = [Nk, max(1, Nk // 2), max(1, Nk - 70), 0]
    return [vals[b % len(vals)] for b in range(B)]


@pytest.mark.parametrize("N,Nk,causal,window", FWD_SHAPES)
@pytest.mark.parametrize("d,dt", [(64, "fp16"), (128, "bf16")])
@pytest.mark.parametrize("pad,p", [(False, 0.0), (True, 0.1)])
def test_fwd_band_and_non_square(N, Nk, causal, window, d, dt, pad, p):
    B, H = (4, 2) if pad else (1, 3)
    inp = W.random_case(B, H, N, d, dt, seed=N * 7 + Nk + d, std=1.5, kv_len=_kv(Nk, B, pad),
                        n_k=Nk)
    scale = 1.0 / np.sqrt(d)
    kw = dict(scale=scale, causal=causal, kv_len=inp.kv_len, dropout_p=p, seed=inp.seed,
              window=window)
    O_ref, lse_ref = A.forward(inp.q, inp.k, inp.v, **kw)
    q, k, v = (t.to(DEV) for t in (inp.q, inp.k, inp.v))
    kv = None if inp.kv_len is None else inp.kv_len.to(DEV)
    print(f"fwd N={N} Nk={Nk} causal={causal} window={window} d={d} {dt} pad={pad} p={p}")
    sys.stdout.flush()
    for odt in (torch.float32, inp.q.dtype):
        o, lse = attn.fwd(q, k, v, causal=causal, kv_len=kv, dropout_p=p, seed=inp.seed,
                          scale=scale, out_dtype=odt, window=window)
        torch.cuda.synchronize()
        check_close("O", o, O_ref, O_ATOL, odt)
        check_lse(lse, lse_ref)


BWD_SHAPES = [
    (200, 64, False, None), (64, 300, True, None), (300, 129, True, None),
    (300, 300, True, (100, -1)), (257, 257, False, (40, 40)), (129, 129, False, (0, 0)),
    (400, 650, True, (150, -1)), (650, 400, False, (-1, 30)), (100, 520, False, (60, 10)),
]


@pytest.mark.parametrize("N,Nk,causal,window", BWD_SHAPES)
@pytest.mark.parametrize("d,dt", [(64, "fp16"), (128, "bf16")])
@pytest.mark.parametrize("pad,p", [(False, 0.0), (True, 0.2)])
def test_bwd_band_and_non_square(N, Nk, causal, window, d, dt, pad, p):
    B, H = (4, 2) if pad else (1, 2)
    inp = W.random_case(B, H, N, d, dt, seed=N * 3 + Nk + d, with_do=True,
                        kv_len=_kv(Nk, B, pad), n_k=Nk)
    scale = 1.0 / np.sqrt(d)
    kw = dict(scale=scale, causal=causal, kv_len=inp.kv_len, dropout_p=p, seed=inp.seed,
              window=window)
    dq_ref, dk_ref, dv_ref = A.backward(inp.q, inp.k, inp.v, inp.do, **kw)
    O_ref, _ = A.forward(inp.q, inp.k, inp.v, **kw)
    P = A.probabilities(inp.q, inp.k, scale=scale, causal=causal, kv_len=inp.kv_len,
                        window=window)
    q, k, v, do = (t.to(DEV) for t in (inp.q, inp.k, inp.v, inp.do))
    kv = None if inp.kv_len is None else inp.kv_len.to(DEV)
    print(f"bwd N={N} Nk={Nk} causal={causal} window={window} d={d} {dt} pad={pad} p={p}")
    sys.stdout.flush()
    for odt in (torch.float32, inp.q.dtype):
        o, lse = attn.fwd(q, k, v, causal=causal, kv_len=kv, dropout_p=p, seed=inp.seed,
                          scale=scale, out_dtype=odt, window=window)
        dq, dk, dv = attn.bwd(q, k, v, o, lse, do, causal=causal, kv_len=kv, dropout_p=p,
                              seed=inp.seed, scale=scale, out_dtype=odt, window=window)
        torch.cuda.synchronize()
        assert dk.shape == k.shape and dq.shape == q.shape
        bdq, bdk = d_rounding_bounds(inp.q, inp.k, inp.do, O_ref, P, scale, odt)
        check_close("dQ", dq, dq_ref, GRAD_ATOL + bdq, odt)
        check_close("dK", dk, dk_ref, GRAD_ATOL + bdk, odt)
        check_close("dV", dv, dv_ref, GRAD_ATOL, odt)


def test_rows_without_keys_under_a_band():
    """Nk < N with the causal mask: the first N - Nk rows see no key (O = 0,
    lse = -inf, dQ = 0); a zero-width window past the last key does the same."""
    N, Nk, d = 300, 100, 64
    inp = W.random_case(1, 2, N, d, "bf16", seed=9, with_do=True, n_k=Nk)
    q, k, v, do = (t.to(DEV) for t in (inp.q, inp.k, inp.v, inp.do))
    o, lse = attn.fwd(q, k, v, causal=True, scale=0.125, out_dtype=torch.float32)
    dq, dk, dv = attn.bwd(q, k, v, o, lse, do, causal=True, scale=0.125,
                          out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.all(o[:, :, :N - Nk] == 0) and torch.all(torch.isneginf(lse[:, :, :N - Nk]))
    assert torch.all(dq[:, :, :N - Nk] == 0)
    O_ref, lse_ref = A.forward(inp.q, inp.k, inp.v, scale=0.125, causal=True)
    check_close("O", o, O_ref, O_ATOL, torch.float32)
    check_lse(lse, lse_ref)
    # window (0, 0) with Nk > N: row i sees exactly key i + Nk - N
    inp2 = W.random_case(1, 2, 90, d, "fp16", seed=10, n_k=250)
    q2, k2, v2 = (t.to(DEV) for t in (inp2.q, inp2.k, inp2.v))
    o2, lse2 = attn.fwd(q2, k2, v2, window=(0, 0), scale=0.125, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o2.cpu(), inp2.v[:, :, 160:].float())


@pytest.mark.parametrize("N,Nk,p", [(5, 9, 0.1), (130, 61, 0.1), (64, 513, 0.3)])
def test_dropout_mask_non_square_bit_exact(N, Nk, p):
    B, H, seed = 2, 2, 0x5851F42D4C957F2D ^ Nk
    keep = attn.dropout_mask(B, H, N, p, seed, DEV, n_k=Nk).cpu().numpy().astype(bool)
    for b, h in itertools.product(range(B), range(H)):
        assert np.array_equal(keep[b, h], philox.keep_mask(seed, b, h, N, Nk, p)), (b, h)


def test_band_fwd_bitwise_deterministic():
    inp = W.random_case(1, 4, 1500, 128, "bf16", seed=15, n_k=2100)
    q, k, v = (t.to(DEV) for t in (inp.q, inp.k, inp.v))
    a = attn.fwd(q, k, v, causal=True, window=(333, -1), scale=0.09)
    b = attn.fwd(q, k, v, causal=True, window=(333, -1), scale=0.09)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_window_wider_than_int_range_equals_no_window():
    """Window sides up to 2^31 - 1 are legal; the host clamps the band edges
    to +-2^30 (beyond every index of a valid shape), so the result equals the
    unmasked / causal one."""
    big = 2**31 - 1
    inp = W.random_case(1, 2, 333, 128, "bf16", seed=21, with_do=True, n_k=401)
    q, k, v, do = (t.to(DEV) for t in (inp.q, inp.k, inp.v, inp.do))
    for causal in (False, True):
        O_ref, lse_ref = A.forward(inp.q, inp.k, inp.v, scale=0.09, causal=causal)
        o, lse = attn.fwd(q, k, v, causal=causal, scale=0.09, window=(big, big),
                          out_dtype=torch.float32)
        g = attn.bwd(q, k, v, o, lse, do, causal=causal, scale=0.09, window=(big, big),
                     out_dtype=torch.float32)
        torch.cuda.synchronize()
        check_close("O", o, O_ref, O_ATOL, torch.float32)
        check_lse(lse, lse_ref)
        g_ref = A.backward(inp.q, inp.k, inp.v, inp.do, scale=0.09, causal=causal)
        for name, got, ref in zip(("dQ", "dK", "dV"), g, g_ref):
            check_close(name, got, ref, GRAD_ATOL, torch.float32)


@pytest.mark.parametrize("causal,window,p", [(True, None, 0.0), (False, (300, 40), 0.1)])
def test_bwd_bitwise_deterministic(causal, window, p):
    """dQ has its own kernel (no atomics): two backward passes on the same
    inputs give identical bits."""
    inp = W.random_case(2, 3, 900, 128, "bf16", seed=33, with_do=True, n_k=1100)
    q, k, v, do = (t.to(DEV) for t in (inp.q, inp.k, inp.v, inp.do))
    kw = dict(causal=causal, window=window, dropout_p=p, seed=inp.seed, scale=0.09)
    o, lse = attn.fwd(q, k, v, **kw)
    g1 = attn.bwd(q, k, v, o, lse, do, **kw)
    g2 = attn.bwd(q, k, v, o, lse, do, **kw)
    torch.cuda.synchronize()
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


@pytest.mark.parametrize("causal,window,nk", [(True, None, None), (True, (200, -1), 700),
                                              (False, (40, 60), 450)])
def test_bwd_stages_equal_bwd(causal, window, nk):
    """attn_bwd_stage called for preprocess, dK/dV and dQ in that order on one
    stream runs the same kernels as attn_bwd: identical bits."""
    inp = W.random_case(2, 2, 500, 128, "bf16", seed=44, with_do=True, n_k=nk)
    q, k, v, do = (t.to(DEV) for t in (inp.q, inp.k, inp.v, inp.do))
    kw = dict(causal=causal, window=window, scale=0.09)
    o, lse = attn.fwd(q, k, v, **kw)
    g_all = attn.bwd(q, k, v, o, lse, do, **kw)
    ws = torch.empty(attn.bwd_workspace_bytes(q, k=k, **kw), dtype=torch.uint8, device=DEV)
    out = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    for st in (attn.BWD_STAGE_PREPROCESS, attn.BWD_STAGE_DKDV, attn.BWD_STAGE_DQ):
        attn.bwd(q, k, v, o, lse, do, out=out, workspace=ws, stage=st, **kw)
    torch.cuda.synchronize()
    for a, b in zip(g_all, out):
        assert torch.equal(a, b)
