"""Empty problems through the torch binding on the device: B, H or N = 0 give
empty outputs and enqueue no kernel, and zero key rows against a non-empty
query block is refused before the library is called (Nk = 0 in the C struct
stands for Nk = N, so passing it on would make the kernels read N rows of an
empty K)."""
import pytest
import torch

import exact_tiled_attention_20_amd as attn

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a device"
    attn.load_library()
    yield


def _qkv(B, H, N, Nk, d=64, dt=torch.float16):
    g = torch.Generator().manual_seed(5)
    mk = lambda n: torch.randn(B, H, n, d, generator=g).to(dt).to(DEV)  # noqa: E731
    return mk(N), mk(Nk), mk(Nk)


@pytest.mark.parametrize("B,H,N", [(0, 3, 100), (2, 0, 100), (2, 3, 0), (0, 0, 0)])
@pytest.mark.parametrize("causal", [False, True])
def test_empty_forward_and_backward(B, H, N, causal):
    q, k, v = _qkv(B, H, N, N)
    kw = dict(causal=causal, dropout_p=0.2, seed=3, window=(7, -1))
    o, lse = attn.fwd(q, k, v, **kw)
    assert o.shape == q.shape and lse.shape == q.shape[:3]
    dq, dk, dv = attn.bwd(q, k, v, o, lse, torch.zeros_like(q), **kw)
    assert dq.shape == q.shape and dk.shape == k.shape and dv.shape == v.shape
    keep = attn.dropout_mask(B, H, N, 0.2, 3, DEV)
    assert keep.shape == (B, H, N, N)
    torch.cuda.synchronize()


def test_no_query_rows_with_keys():
    q, k, v = _qkv(2, 3, 0, 40)
    o, lse = attn.fwd(q, k, v)
    assert o.numel() == 0 and lse.numel() == 0
    with pytest.raises(attn.AttnError):
        attn.bwd(q, k, v, o, lse, torch.zeros_like(q))


def test_zero_key_rows_with_queries_is_refused():
    q, k, v = _qkv(2, 3, 50, 0)
    with pytest.raises(ValueError):
        attn.fwd(q, k, v)
    with pytest.raises(ValueError):
        attn.dropout_mask(2, 3, 50, 0.1, 1, DEV, n_k=0)
