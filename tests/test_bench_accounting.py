"""CPU checks of the benchmark's FLOP accounting: the number of visible
query-key pairs it charges a masked workload equals the count of the oracle's
mask, and closed forms for the named variants."""
import types

import pytest

import attn_workloads as W
import bench
from oracle import attention as A


@pytest.mark.parametrize("N,Nk", [(1, 1), (7, 7), (50, 13), (13, 50), (64, 200), (129, 129)])
@pytest.mark.parametrize("causal", [False, True])
def test_visible_pairs_match_the_oracle_mask(N, Nk, causal):
    for window in [None, (0, 0), (3, -1), (-1, 5), (10, 2), (1000, -1)]:
        w = types.SimpleNamespace(N=N, Nk=Nk, causal=causal, window=window)
        mask = A.valid_mask(N, 0, causal, None, n_k=Nk, window=window)
        assert bench.visible_pairs(w) == float(mask.sum()), (N, Nk, causal, window)


def test_variant_pair_counts_in_closed_form():
    swa = W.VARIANTS["swa4096_b1h32n16384d128_bf16_bwd"]
    n, left = swa.N, swa.window[0]
    # row i sees min(i, left) + 1 keys
    assert bench.visible_pairs(swa) == (left + 1) * (left + 2) / 2 + (n - left - 1) * (left + 1)
    chunk = W.VARIANTS["chunk_b4h16n2048nk16384d128_bf16_causal_bwd"]
    # bottom-right causal: query i sees keys 0 .. i + Nk - N
    assert bench.visible_pairs(chunk) == sum(i + chunk.Nk - chunk.N + 1 for i in range(chunk.N))
    d256 = W.VARIANTS["d256_b1h16n16384_bf16_causal_bwd"]
    assert bench.visible_pairs(d256) == d256.N * (d256.N + 1) / 2
