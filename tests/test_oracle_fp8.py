"""Pins for oracle/fp8.py (CPU only).

  * the e4m3 format: hand-decoded codes from the format's definition, every
    code against torch's float8_e4m3fn (a library routine, called), and the
    oracle's own round-to-nearest-even against torch's cast on a dense grid,
    every tie and the subnormal range;
  * the rounding bounds the O bound rests on, checked exhaustively: half an ulp
    is at most 2^-4 x for normal x and 2^-10 below 2^-6;
  * the O bound and the variance model against an independent emulation of a
    tiled online softmax that rounds the probabilities to e4m3 against a lazily
    raised reference (tiles of 64 keys, references raised by more than 2^8 in
    probability, earlier terms rescaled); with a planted index mistake (value
    rows swapped inside a tile) the aggregate check fails, so it would catch
    such a mistake in a kernel.
"""
import numpy as np
import pytest
import torch

from oracle import fp8 as F8


def test_decode_hand_values():
    cases = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6,
             0x38: 1.0, 0x39: 1.125, 0x40: 2.0, 0x7E: 448.0, 0x77: 240.0,
             0x80: -0.0, 0xB8: -1.0, 0xFE: -448.0}
    for c, v in cases.items():
        assert F8.decode_e4m3(c) == v, hex(c)
    assert np.isnan(F8.decode_e4m3(0x7F)) and np.isnan(F8.decode_e4m3(0xFF))
    vals = F8.e4m3_values()
    assert vals.size == 127 and vals[0] == 0.0 and vals[-1] == 448.0
    assert np.all(np.diff(vals) > 0)


def test_decode_matches_torch_for_every_code():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = F8.decode_e4m3(np.arange(256))
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])


def test_round_matches_torch_cast():
    rng = np.random.default_rng(0)
    vals = F8.e4m3_values()
    mids = (vals[1:] + vals[:-1]) / 2                       # every tie
    x = np.concatenate([rng.uniform(-460, 460, 200000),
                        rng.uniform(-2 ** -5, 2 ** -5, 200000),
                        np.exp2(rng.uniform(-12, 8.8, 100000)),
                        mids, -mids, vals, -vals, [0.0, 463.9, -463.9]])
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(F8.round_e4m3(x), ref)


def test_rounding_error_bounds_are_exhaustive_and_tight():
    vals = F8.e4m3_values()
    # every binade / subnormal interval sampled densely, ends included
    x = np.unique(np.concatenate([np.linspace(a, b, 2001) for a, b in zip(vals[:-1], vals[1:])]))
    err = np.abs(F8.round_e4m3(x) - x)
    normal = x >= F8.E4M3_MIN_NORMAL
    assert np.all(err[normal] <= 2.0 ** -4 * x[normal] * (1 + 1e-15))
    assert np.all(err[~normal] <= 2.0 ** -10 * (1 + 1e-15))
    # nearly tight: the worst relative error, 1/17, sits just above a power of
    # two (x = 2^e (1 + 1/16) rounds down to 2^e)
    assert np.isclose(np.max(err[normal] / x[normal]), 1.0 / 17.0, rtol=1e-3)
    assert np.max(err[~normal]) >= 0.99 * 2.0 ** -10


def _emulate_row(S, V, tile=64, thr=8.0, swap_in_tile=False):
    """Tiled online softmax over one row of scores S (natural-log units),
    rounding exp(S_j - ref) to e4m3 before the product with V; the reference
    is raised only when a tile's maximum exceeds it by more than thr in log2
    units (probability 2^thr). O is normalised by the unrounded sum."""
    ref = -np.inf
    acc = np.zeros(V.shape[1])
    l = 0.0
    for t0 in range(0, S.size, tile):
        s = S[t0:t0 + tile]
        vt = V[t0:t0 + tile].copy()
        if swap_in_tile and vt.shape[0] > 1:
            vt[[0, 1]] = vt[[1, 0]]
        mx = s.max()
        if mx > ref + thr * np.log(2.0):
            alpha = 0.0 if ref == -np.inf else np.exp(ref - mx)
            acc *= alpha
            l *= alpha
            ref = mx
        x = np.exp(s - ref)
        l += x.sum()
        acc += F8.round_e4m3(x) @ vt
    return acc / l


def _exact_row(S, V):
    p = np.exp(S - S.max())
    return (p / p.sum()) @ V


@pytest.mark.parametrize("spread", [0.3, 1.0, 3.0, 9.0])
def test_o_bound_and_variance_model_hold_for_a_tiled_emulation(spread):
    """Rows of 64..3000 keys with scores of several spreads (flat to one
    dominant key), V drawn as e4m3 N(0,1): every element within the bound and
    the summed squared error below the upper variance model; for flat and
    moderate rows not vacuously (above a fifth of it). With a dominant key the
    error is far below the model: that key's x is often exactly 1."""
    rng = np.random.default_rng(int(spread * 10))
    se, sv = 0.0, 0.0
    for n in (64, 65, 300, 3000):
        for _ in range(6):
            # scores that rise and fall so that the reference is raised mid-row
            S = rng.normal(0, spread, n) + np.linspace(-spread, spread, n) * rng.choice([-1, 1])
            V = F8.round_e4m3(np.clip(rng.normal(0, 1, (n, 16)), -400, 400))
            got = _emulate_row(S, V)
            ref = _exact_row(S, V)
            p = np.exp(S - S.max())
            L = np.array([p.sum()])
            P = (p / p.sum())[None, :]
            bound = F8.p_rounding_bound(P, L, V)[0]
            err = got - ref
            assert np.all(np.abs(err) <= bound + 1e-12)
            se += float((err ** 2).sum())
            sv += float(F8.p_rounding_variance(P, L, V)[0].sum())
    assert se <= sv, (se, sv)
    if spread <= 1.0:
        assert se >= 0.2 * sv, (se, sv)


def test_aggregate_check_catches_a_swapped_value_row():
    """The planted mistake (two value rows exchanged inside every tile) passes
    the loose per-element bound on flat rows but fails the aggregate check."""
    rng = np.random.default_rng(7)
    se, sv = 0.0, 0.0
    for _ in range(40):
        n = 1024
        S = rng.normal(0, 0.3, n)
        V = F8.round_e4m3(rng.normal(0, 1, (n, 16)))
        got = _emulate_row(S, V, swap_in_tile=True)
        ref = _exact_row(S, V)
        p = np.exp(S - S.max())
        L = np.array([p.sum()])
        P = (p / p.sum())[None, :]
        se += float(((got - ref) ** 2).sum())
        sv += float(F8.p_rounding_variance(P, L, V)[0].sum())
    assert se > 3 * sv, (se, sv)


def test_row_stats_match_the_definition():
    rng = np.random.default_rng(3)
    q = torch.from_numpy(rng.normal(0, 1, (1, 1, 5, 8)))
    k = torch.from_numpy(rng.normal(0, 1, (1, 1, 7, 8)))
    P, L, valid = F8.row_stats(q, k, scale=0.25, causal=True)
    S = 0.25 * (q[0, 0].numpy() @ k[0, 0].numpy().T)
    for i in range(5):
        vis = np.arange(7) <= i + 2
        e = np.exp(S[i, vis] - S[i, vis].max())
        assert np.allclose(P[i, vis], e / e.sum(), rtol=0, atol=1e-15)
        assert np.all(P[i, ~vis] == 0)
        assert np.isclose(L[i], e.sum(), rtol=1e-15)


def test_bound_with_dropout_factor():
    """Z = keep / (1 - p): dropped terms are exact zeros, kept ones are rounded
    then scaled; the bound weighted by Z holds on the emulation."""
    rng = np.random.default_rng(11)
    for _ in range(20):
        n = 500
        S = rng.normal(0, 1.0, n)
        V = F8.round_e4m3(rng.normal(0, 1, (n, 8)))
        keep = rng.random(n) >= 0.2
        Z = keep / 0.8
        p = np.exp(S - S.max())
        L = np.array([p.sum()])
        P = (p / p.sum())[None, :]
        # emulation: zero the dropped keys' x before rounding, scale by 1/(1-p)
        got = _emulate_row(S, V * Z[:, None])       # rounding x, then times Z V
        ref = (P[0] * Z) @ V
        bound = F8.p_rounding_bound(P, L, V, Z=Z[None, :])[0]
        assert np.all(np.abs(got - ref) <= bound + 1e-12)
