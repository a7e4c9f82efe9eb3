"""Pins for the oracle's Philox4x32-10 and dropout keep rule (CPU only).

The oracle's generator is written from the SC'11 definition. It is pinned to
something other than itself by:
  * rocRAND's Philox4x32-10 engine, called (not copied) through a small host
    wrapper built here with hipcc, on random counters and keys;
  * the threshold rule's exact values;
  * the statistics of the keep decision (drop rate within 5 sigma of p, no
    lag-1 correlation along queries or keys).
"""
import ctypes
import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle import philox

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def rocrand_lib(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available to build the rocRAND wrapper")
    out = tmp_path_factory.mktemp("rocrand") / "rocrand_philox_host.so"
    src = os.path.join(HERE, "helpers", "rocrand_philox_host.cpp")
    subprocess.run([hipcc, "-O1", "-fPIC", "-shared", "-x", "hip",
                    "--offload-arch=gfx950", "-o", str(out), src],
                   check=True, capture_output=True)
    return ctypes.CDLL(str(out))


def _rocrand_blocks(lib, ctr: np.ndarray, seed: int) -> np.ndarray:
    ctr = np.ascontiguousarray(ctr, dtype=np.uint32)
    out = np.zeros_like(ctr)
    lib.rocrand_philox_blocks(ctr.ctypes.data_as(ctypes.c_void_p),
                              ctypes.c_uint64(seed),
                              out.ctypes.data_as(ctypes.c_void_p),
                              ctypes.c_int(ctr.shape[0]))
    return out


@pytest.mark.parametrize("seed", [0, 1, 0x0123456789ABCDEF, 0xFFFFFFFFFFFFFFFF,
                                  0x243F6A8885A308D3])
def test_block_function_matches_rocrand(rocrand_lib, seed):
    rng = np.random.default_rng(seed & 0xFFFF)
    ctr = rng.integers(0, 2**32, size=(4096, 4), dtype=np.uint64).astype(np.uint32)
    ctr[:, 1] &= (1 << 30) - 1     # the wrapper passes words 0..1 as offset*4
    ctr[:8] = 0                    # plus a few structured counters
    ctr[1, 0] = 1
    ctr[2, 2] = 1
    ctr[3, 3] = 0xFFFFFFFF
    ctr[4] = [7, 5, 3, 1]
    ref = _rocrand_blocks(rocrand_lib, ctr, seed)
    got = philox.philox4x32_10(ctr, np.array(philox.seed_key(seed), dtype=np.uint64))
    assert np.array_equal(got, ref)


def test_keep_rule_uses_declared_counter_layout(rocrand_lib):
    """keep(seed,b,h,i,j) reads word j&3 of Philox((j>>2, i, h, b), seed)."""
    seed, b, h, n = 0xDEADBEEF12345678, 3, 5, 37
    i = np.arange(n)
    ctr = np.zeros((n * ((n + 3) // 4), 4), dtype=np.uint32)
    idx = 0
    for ii in range(n):
        for t in range((n + 3) // 4):
            ctr[idx] = [t, ii, h, b]
            idx += 1
    words = _rocrand_blocks(rocrand_lib, ctr, seed).reshape(n, -1)[:, :n]
    T = philox.drop_threshold(0.3)
    assert np.array_equal(philox.keep_mask(seed, b, h, n, n, 0.3), words >= T)
    u = philox.uniform_bits(seed, b, h, i[:, None], i[None, :])
    assert np.array_equal(u, words)


def test_threshold_values():
    assert philox.drop_threshold(0.0) == 0
    assert philox.drop_threshold(0.5) == 2**31
    # 0.1 rounds to 13421773 * 2^-27 in float32, so T = 13421773 * 32.
    assert philox.drop_threshold(0.1) == 429496736
    assert philox.drop_threshold(np.nextafter(np.float32(1), np.float32(0))) == 2**32 - 256
    for bad in (1.0, -0.1, 2.0, float("nan")):
        with pytest.raises(ValueError):
            philox.drop_threshold(bad)
    assert philox.keep_scale(0.5) == 2.0


def test_p_zero_keeps_everything():
    assert philox.keep_mask(123, 0, 0, 9, 9, 0.0).all()


@pytest.mark.parametrize("p", [0.1, 0.5, 0.9])
def test_drop_rate_and_lag1(p):
    n = 4096      # 4096 x 4096 = 1.7e7 draws for one head
    keep = philox.keep_mask(0x9E3779B97F4A7C15, 2, 7, n, n, p)
    draws = keep.size
    drop_rate = 1.0 - keep.mean()
    sigma = np.sqrt(p * (1 - p) / draws)
    assert abs(drop_rate - p) < 5 * sigma
    x = keep.astype(np.float64) - keep.mean()
    var = (x * x).mean()
    for lag_axis in (0, 1):
        a = x[1:, :] if lag_axis == 0 else x[:, 1:]
        b = x[:-1, :] if lag_axis == 0 else x[:, :-1]
        corr = (a * b).mean() / var
        assert abs(corr) < 5 / np.sqrt(a.size)


def test_distinct_heads_and_batches_decorrelated():
    n, p = 256, 0.5
    base = philox.keep_mask(42, 0, 0, n, n, p)
    for (b, h) in [(0, 1), (1, 0), (1, 1)]:
        other = philox.keep_mask(42, b, h, n, n, p)
        agree = (base == other).mean()
        assert abs(agree - 0.5) < 5 * 0.5 / n
