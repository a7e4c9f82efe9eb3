"""C-ABI tests that need no GPU: the library loads, exports every entry point
declared in include/attn.h, rejects every invalid argument on the host
before anything is enqueued, and accepts empty problems without enqueueing
anything (so these calls never touch a device)."""
import ctypes
import os
import re

import pytest

import exact_tiled_attention_20_amd as attn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(attn.LIB_PATH):
        from exact_tiled_attention_20_amd import build
        build.build(verbose=False)
    return attn.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*[A-Za-z_][\w\s\*]*?\b(attn_\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_binding_exports():
    assert declared_functions() == sorted(attn.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_version_and_status_strings(lib):
    assert lib.attn_version() == 500
    for code, name in attn.STATUS_NAMES.items():
        assert attn.status_string(code).startswith(name)
    assert "unknown" in attn.status_string(99)


def test_struct_layout_matches_header():
    # int32 x 6, float, int32, pointer (8-aligned), float, uint64, int32 x 3
    assert ctypes.sizeof(attn.AttnParams) == 72
    assert attn.AttnParams.kv_len.offset == 32
    assert attn.AttnParams.seed.offset == 48
    assert attn.AttnParams.Nk.offset == 56
    assert attn.AttnParams.window_left.offset == 60
    assert attn.AttnParams.window_right.offset == 64


FAKE = 0x10000   # 16-byte aligned, never dereferenced: validation fails first
SIZE = 1 << 40   # distinct ranges so no aliasing is reported


def _ptrs(n):
    return [FAKE + i * SIZE for i in range(n)]


def _params(**kw):
    base = dict(B=2, H=3, N=100, d=64, dtype=attn.ATTN_F16, out_dtype=attn.ATTN_F16,
                scale=0.125, causal=False, dropout_p=0.0, seed=1)
    raw_causal = kw.pop("causal", None)
    base.update(kw)
    B, H, N, d = base.pop("B"), base.pop("H"), base.pop("N"), base.pop("d")
    p = attn.make_params(B, H, N, d, **base)
    if raw_causal is not None:
        p.causal = raw_causal
    return p


INVALID = [
    dict(B=-1), dict(H=-1), dict(N=-1), dict(d=0),
    dict(dtype=7), dict(out_dtype=-1), dict(causal=2),
    dict(scale=0.0), dict(scale=-0.125), dict(scale=float("inf")), dict(scale=float("nan")),
    dict(dropout_p=1.0), dict(dropout_p=-0.1), dict(dropout_p=float("nan")),
    dict(N=1 << 24, d=128),           # N*d per head overflows int32 indexing
    dict(N=8, n_k=1 << 24, d=128),    # Nk*d per head overflows int32 indexing
    dict(B=1 << 16, H=1 << 15),       # B*H overflows
    dict(n_k=-1), dict(window=(-2, 0)), dict(window=(0, -7)),
]
UNSUPPORTED = [
    dict(d=96), dict(d=512), dict(d=32),
    dict(dtype=attn.ATTN_F32, out_dtype=attn.ATTN_F32),
    dict(dtype=attn.ATTN_F16, out_dtype=attn.ATTN_BF16),
]


def _fwd(lib, p, ptrs=None, stream=None):
    q, k, v, o, lse = ptrs or _ptrs(5)
    return lib.attn_fwd(ctypes.byref(p), q, k, v, o, lse, stream)


def _bwd(lib, p, ptrs=None, ws_bytes=1 << 30):
    q, k, v, o, lse, do, dq, dk, dv, ws = ptrs or _ptrs(10)
    return lib.attn_bwd(ctypes.byref(p), q, k, v, o, lse, do, dq, dk, dv, ws, ws_bytes, None)


@pytest.mark.parametrize("kw", INVALID)
def test_invalid_params_rejected(lib, kw):
    p = _params(**kw)
    assert _fwd(lib, p) == 1
    assert _bwd(lib, p) == 1
    assert lib.attn_bwd_workspace_bytes(ctypes.byref(p)) == 0
    assert lib.attn_dropout_mask(ctypes.byref(p), FAKE, None) == 1


@pytest.mark.parametrize("kw", UNSUPPORTED)
def test_unsupported_combinations_never_fall_back(lib, kw):
    p = _params(**kw)
    assert _fwd(lib, p) == 2
    assert _bwd(lib, p) == 2


def test_null_params_pointer(lib):
    assert lib.attn_fwd(None, *_ptrs(5), None) == 1
    assert lib.attn_bwd_workspace_bytes(None) == 0


@pytest.mark.parametrize("slot", range(5))
def test_fwd_null_or_misaligned_pointer(lib, slot):
    for bad in (0, FAKE + 8 + slot * SIZE):
        ptrs = _ptrs(5)
        ptrs[slot] = bad
        assert _fwd(lib, _params(), ptrs) == 1


@pytest.mark.parametrize("slot", range(9))
def test_bwd_null_or_misaligned_pointer(lib, slot):
    for bad in (0, FAKE + 4 + slot * SIZE):
        ptrs = _ptrs(10)
        ptrs[slot] = bad
        assert _bwd(lib, _params(), ptrs) == 1


def test_fwd_rejects_aliasing(lib):
    q, k, v, o, lse = _ptrs(5)
    assert _fwd(lib, _params(), [q, k, v, q, lse]) == 1          # o aliases q
    assert _fwd(lib, _params(), [q, k, v, o, o + 1024]) == 1     # lse inside o


def test_bwd_workspace_checks(lib):
    p = _params()
    need = lib.attn_bwd_workspace_bytes(ctypes.byref(p))
    # two fp32 (B, H, N) arrays (D and lse in log2 units), each 256-byte rounded
    assert need == 2 * (((2 * 3 * 100 * 4 + 255) // 256) * 256)
    ptrs = _ptrs(10)
    assert _bwd(lib, p, ptrs, ws_bytes=need - 1) == 3
    bad = list(ptrs)
    bad[9] = 0
    assert _bwd(lib, p, bad, ws_bytes=need) == 3
    bad[9] = FAKE + 9 * SIZE + 128           # not 256-byte aligned
    assert _bwd(lib, p, bad, ws_bytes=need) == 3


def test_bwd_stage_validation(lib):
    q, k, v, o, lse, do, dq, dk, dv, ws = _ptrs(10)
    p = _params()
    for bad_stage in (-1, 3, 100):
        assert lib.attn_bwd_stage(ctypes.byref(p), bad_stage, q, k, v, o, lse, do, dq, dk, dv,
                                  ws, 1 << 30, None) == 1
    p = _params(d=96)
    assert lib.attn_bwd_stage(ctypes.byref(p), 1, q, k, v, o, lse, do, dq, dk, dv,
                              ws, 1 << 30, None) == 2


def test_bwd_rejects_output_aliasing(lib):
    ptrs = _ptrs(10)
    ptrs[7] = ptrs[6]                        # dk aliases dq
    assert _bwd(lib, _params(), ptrs) == 1
    ptrs = _ptrs(10)
    ptrs[8] = ptrs[0]                        # dv aliases q
    assert _bwd(lib, _params(), ptrs) == 1


def test_misaligned_kv_len(lib):
    p = _params()
    p.kv_len = ctypes.c_void_p(FAKE + 2)
    assert _fwd(lib, p) == 1


def test_dropout_mask_pointer_checks(lib):
    p = _params(dropout_p=0.1)
    assert lib.attn_dropout_mask(ctypes.byref(p), None, None) == 1
    assert lib.attn_dropout_mask(ctypes.byref(p), FAKE + 1, None) == 1


def test_aliasing_checks_cover_the_key_rows(lib):
    """K and V span (B, H, Nk, d): an output placed past their first N rows but
    inside their Nk rows still aliases them."""
    p = _params(N=100, n_k=1000)
    q, k, v, o, lse = _ptrs(5)
    inside_k = k + 2 * 3 * 100 * 64 * 2 + 4096
    assert _fwd(lib, p, [q, k, v, inside_k, lse]) == 1
    ptrs = _ptrs(10)
    ptrs[7] = ptrs[1] + 2 * 3 * 500 * 64 * 2          # dk inside k's key rows
    assert _bwd(lib, p, ptrs) == 1


def test_workspace_rows_are_padded_to_four(lib):
    """The backward workspace holds two fp32 arrays of B x H x Np rows, Np = N
    rounded up to a multiple of 4, each rounded up to 256 bytes."""
    for n, n_pad in ((1, 4), (3, 4), (4, 4), (101, 104), (1000, 1000), (1001, 1004)):
        p = _params(N=n)
        want = 2 * (((2 * 3 * n_pad * 4 + 255) // 256) * 256)
        assert lib.attn_bwd_workspace_bytes(ctypes.byref(p)) == want, n


def test_head_dim_256_is_supported(lib):
    """d = 256 passes validation for forward and backward: with the fake
    pointers every check passes up to aliasing, which is then reported."""
    p = _params(d=256)
    assert lib.attn_bwd_workspace_bytes(ctypes.byref(p)) == 2 * (((2 * 3 * 100 * 4 + 255) // 256) * 256)
    q, k, v, o, lse = _ptrs(5)
    assert _fwd(lib, p, [q, k, v, q, lse]) == 1      # o aliases q: rejected, not unsupported
    bad = _params(d=256, scale=0.0)
    assert _fwd(lib, bad) == 1 and _bwd(lib, bad) == 1
    drop = _params(d=256, dropout_p=0.1)
    assert lib.attn_bwd_workspace_bytes(ctypes.byref(drop)) > 0


@pytest.mark.parametrize("kw", [dict(B=0), dict(H=0), dict(N=0), dict(B=0, N=0, H=0),
                                dict(N=0, causal=True, dropout_p=0.3, window=(5, -1))])
def test_empty_problem_is_a_no_op(lib, kw):
    """B, H or N = 0: every entry point accepts the call without reading a
    pointer (all NULL here) and enqueues nothing (no stream, no device)."""
    p = _params(**kw)
    assert _fwd(lib, p, [None] * 5) == 0
    assert lib.attn_bwd_workspace_bytes(ctypes.byref(p)) == 0
    assert _bwd(lib, p, [None] * 10, ws_bytes=0) == 0
    for stage in (0, 1, 2):
        assert lib.attn_bwd_stage(ctypes.byref(p), stage, *([None] * 10), 0, None) == 0
    assert lib.attn_dropout_mask(ctypes.byref(p), None, None) == 0


def test_empty_problem_still_validates_the_other_fields(lib):
    assert _fwd(lib, _params(N=0, scale=0.0), [None] * 5) == 1
    assert _fwd(lib, _params(B=0, d=96), [None] * 5) == 2
    assert _bwd(lib, _params(H=0, dropout_p=1.0), [None] * 10, ws_bytes=0) == 1
    assert lib.attn_dropout_mask(ctypes.byref(_params(N=0, window=(0, -3))), None, None) == 1


def test_no_query_rows_with_keys_needs_the_key_tensors(lib):
    """N = 0 with Nk > 0: the forward has nothing to write; the backward writes
    dK = dV = 0, so the (non-empty) key tensors need real pointers. With NULL
    ones it is rejected before anything is enqueued."""
    p = _params(N=0, n_k=50)
    assert _fwd(lib, p, [None] * 5) == 0
    assert lib.attn_bwd_workspace_bytes(ctypes.byref(p)) == 0
    assert _bwd(lib, p, [None] * 10, ws_bytes=0) == 1
    assert lib.attn_bwd_stage(ctypes.byref(p), 1, *([None] * 10), 0, None) == 1
    assert _bwd(lib, _params(B=0, N=0, n_k=50), [None] * 10, ws_bytes=0) == 0


def test_zero_key_rows_need_only_the_query_side(lib):
    """Nk = 0 with N > 0 is a valid problem (every row sees no key). The key
    tensors are empty, so their pointers may be NULL, but the query-side ones
    may not (checked here with NULL q, which fails before any launch)."""
    p = _params(N=40, n_k=0)
    q, k, v, o, lse = _ptrs(5)
    assert _fwd(lib, p, [None, None, None, o, lse]) == 1
    ptrs = _ptrs(10)
    for slot in (0, 1, 2, 7, 8):            # q, and the empty k, v, dk, dv
        ptrs[slot] = None
    assert _bwd(lib, p, ptrs, ws_bytes=1 << 20) == 1
    assert lib.attn_dropout_mask(ctypes.byref(p), None, None) == 0   # no cells


def test_empty_ranges_do_not_alias(lib):
    """A tensor with no elements overlaps nothing, even where its (unused)
    pointer falls inside another tensor. Checked on a problem that fails later
    for a reason the aliasing check cannot hide: d = 96 is reported as
    unsupported, not as invalid."""
    p = _params(N=40, n_k=0, d=96)
    q, k, v, o, lse = _ptrs(5)
    assert _fwd(lib, p, [q, q + 64, q + 64, o, lse]) == 2


def test_window_sides_beyond_int32_are_clamped():
    p = attn.make_params(1, 1, 8, 64, dtype=attn.ATTN_F16, out_dtype=attn.ATTN_F16,
                         scale=0.125, window=(2 ** 32 + 5, 2 ** 40))
    assert p.window_left == 2 ** 31 - 1 and p.window_right == 2 ** 31 - 1
    p = attn.make_params(1, 1, 8, 64, dtype=attn.ATTN_F16, out_dtype=attn.ATTN_F16,
                         scale=0.125, window=(3, -1))
    assert (p.window_left, p.window_right, p.Nk) == (3, -1, 8)


def test_noalloc_rejects_before_touching_a_device(lib):
    """attn_bwd_noalloc validates like attn_bwd and checks its scratch limit
    before any HIP call: invalid parameters, NULL pointers and problems whose
    workspace exceeds the fixed scratch all fail on a machine with no GPU."""
    cap = lib.attn_bwd_noalloc_max_workspace_bytes()
    assert cap == 16 << 20
    ptrs = _ptrs(9)
    assert lib.attn_bwd_noalloc(ctypes.byref(_params(scale=0.0)), *ptrs, None) == 1
    assert lib.attn_bwd_noalloc(ctypes.byref(_params(d=96)), *ptrs, None) == 2
    bad = list(ptrs)
    bad[3] = 0
    assert lib.attn_bwd_noalloc(ctypes.byref(_params()), *bad, None) == 1
    # 2^21 rows need two 8 MiB arrays plus nothing else: exactly at the limit
    # would fit, one row-block more does not.
    big = _params(B=1, H=64, N=1 << 15, d=64)
    assert lib.attn_bwd_workspace_bytes(ctypes.byref(big)) == cap
    bigger = _params(B=1, H=64, N=(1 << 15) + 64, d=64)
    assert lib.attn_bwd_workspace_bytes(ctypes.byref(bigger)) > cap
    assert lib.attn_bwd_noalloc(ctypes.byref(bigger), *ptrs, None) == 5
    assert "scratch" in attn.status_string(5)
    # Empty problems need no scratch and enqueue nothing.
    assert lib.attn_bwd_noalloc(ctypes.byref(_params(B=0)), *([None] * 9), None) == 0


def test_fp8_forward_validation(lib):
    """e4m3 inputs: d = 128 with bf16 or float O is accepted (checked up to the
    aliasing test, which fails on purpose here); other head dimensions and
    output dtypes, and the backward, are unsupported."""
    base = dict(dtype=attn.ATTN_E4M3, out_dtype=attn.ATTN_BF16, d=128)
    q, k, v, o, lse = _ptrs(5)
    assert _fwd(lib, _params(**base), [q, k, v, q, lse]) == 1           # o aliases q
    assert _fwd(lib, _params(**dict(base, d=64))) == 2
    assert _fwd(lib, _params(**dict(base, out_dtype=attn.ATTN_F16))) == 2
    assert _fwd(lib, _params(**dict(base, out_dtype=attn.ATTN_E4M3))) == 2
    assert _bwd(lib, _params(**base)) == 2
    assert lib.attn_bwd_workspace_bytes(ctypes.byref(_params(**base))) == 0
    assert _fwd(lib, _params(dtype=attn.ATTN_F16, out_dtype=attn.ATTN_E4M3)) == 2
