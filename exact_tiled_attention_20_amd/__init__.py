"""Exact tiled (fused) softmax attention for MI355X (gfx950).

A thin ctypes binding over ``libattn.so`` (C ABI in ``include/attn.h``). This
module only marshals arguments: it checks tensor shapes, dtypes and devices,
allocates outputs with torch on the current device, and passes raw device
pointers and the current HIP stream to the library. Every step of the
computation runs in the library's HIP kernels; there is no fallback path, and
the module raises if the library is missing or a call fails.

    o, lse = fwd(q, k, v, causal=False, kv_len=None, dropout_p=0.0, seed=0,
                 scale=None, out_dtype=None, window=None)
    dq, dk, dv = bwd(q, k, v, o, lse, do, <same keyword arguments>)
    dq, dk, dv = bwd_noalloc(q, k, v, o, lse, do, <same keyword arguments>)
    keep = dropout_mask(B, H, N, dropout_p, seed, device, n_k=None)

q and dO are (B, H, N, d); k and v are (B, H, Nk, d) (Nk = N for
self-attention; Nk = 0 is allowed: every row then sees no key), contiguous,
float16 or bfloat16, d in {64, 128, 256}; the forward also takes
float8_e4m3fn q, k, v at d = 128 (O in bfloat16 by default, or float32). Every tensor argument, including
caller-supplied outputs and the workspace, must be on q's device. Query i lines
up with key i + Nk - N. window = (left, right) keeps keys at most `left` before
and `right` after that key (-1: unbounded side; sides above 2^31 - 1, wider
than any sequence, are clamped to it).
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libattn.so")

ATTN_F16, ATTN_BF16, ATTN_F32, ATTN_E4M3 = 0, 1, 2, 3
STATUS_NAMES = {0: "ATTN_OK", 1: "ATTN_ERR_INVALID_ARG", 2: "ATTN_ERR_UNSUPPORTED",
                3: "ATTN_ERR_WORKSPACE", 4: "ATTN_ERR_LAUNCH", 5: "ATTN_ERR_TOO_LARGE"}

# Entry points declared in include/attn.h (checked by the ABI tests).
EXPORTS = ("attn_fwd", "attn_bwd", "attn_bwd_stage", "attn_bwd_workspace_bytes",
           "attn_bwd_noalloc", "attn_bwd_noalloc_max_workspace_bytes",
           "attn_dropout_mask", "attn_status_string", "attn_version")
BWD_STAGE_PREPROCESS, BWD_STAGE_DKDV, BWD_STAGE_DQ = 0, 1, 2


class AttnParams(ctypes.Structure):
    """Mirror of attn_params in include/attn.h."""
    _fields_ = [
        ("B", ctypes.c_int32), ("H", ctypes.c_int32), ("N", ctypes.c_int32),
        ("d", ctypes.c_int32),
        ("dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("causal", ctypes.c_int32),
        ("kv_len", ctypes.c_void_p),
        ("dropout_p", ctypes.c_float),
        ("seed", ctypes.c_uint64),
        ("Nk", ctypes.c_int32),
        ("window_left", ctypes.c_int32), ("window_right", ctypes.c_int32),
    ]


class AttnError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)}")


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libattn.so and declare its signatures. Raises if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build it with `python -m exact_tiled_attention_20_amd.build` "
            "(the library has no fallback implementation)")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER(AttnParams)
    vp = ctypes.c_void_p
    lib.attn_fwd.argtypes = [P, vp, vp, vp, vp, vp, vp]
    lib.attn_fwd.restype = ctypes.c_int
    lib.attn_bwd.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.attn_bwd.restype = ctypes.c_int
    lib.attn_bwd_stage.argtypes = [P, ctypes.c_int32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                   ctypes.c_size_t, vp]
    lib.attn_bwd_stage.restype = ctypes.c_int
    lib.attn_bwd_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.attn_bwd_noalloc.restype = ctypes.c_int
    lib.attn_bwd_noalloc_max_workspace_bytes.argtypes = []
    lib.attn_bwd_noalloc_max_workspace_bytes.restype = ctypes.c_size_t
    lib.attn_bwd_workspace_bytes.argtypes = [P]
    lib.attn_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.attn_dropout_mask.argtypes = [P, vp, vp]
    lib.attn_dropout_mask.restype = ctypes.c_int
    lib.attn_status_string.argtypes = [ctypes.c_int]
    lib.attn_status_string.restype = ctypes.c_char_p
    lib.attn_version.argtypes = []
    lib.attn_version.restype = ctypes.c_int32
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().attn_status_string(int(status)).decode()


INT32_MAX = (1 << 31) - 1


def make_params(B: int, H: int, N: int, d: int, *, dtype: int, out_dtype: int,
                scale: float, causal: bool = False, kv_len_ptr: int = 0,
                dropout_p: float = 0.0, seed: int = 0, n_k: Optional[int] = None,
                window=None) -> AttnParams:
    """Fill attn_params. n_k defaults to N (self-attention). Window sides above
    INT32_MAX are clamped to it: the library treats that as wider than any
    sequence, which is what such a side means (a silent int32 wrap-around
    would give a different mask)."""
    wl, wr = (-1, -1) if window is None else (int(window[0]), int(window[1]))
    wl, wr = min(wl, INT32_MAX), min(wr, INT32_MAX)
    nk = N if n_k is None else int(n_k)
    return AttnParams(int(B), int(H), int(N), int(d), int(dtype), int(out_dtype),
                      float(scale), 1 if causal else 0,
                      ctypes.c_void_p(kv_len_ptr or None), float(dropout_p),
                      int(seed) & 0xFFFFFFFFFFFFFFFF, nk, wl, wr)


# --------------------------------------------------------------------------
# torch-facing wrappers (torch provides device memory and the stream)

def _torch():
    import torch
    return torch


def _code(dt) -> int:
    torch = _torch()
    if dt == torch.float16:
        return ATTN_F16
    if dt == torch.bfloat16:
        return ATTN_BF16
    if dt == torch.float32:
        return ATTN_F32
    if dt == torch.float8_e4m3fn:
        return ATTN_E4M3
    raise TypeError(f"unsupported dtype {dt}")


def _stream_ptr(device) -> int:
    torch = _torch()
    return int(torch.cuda.current_stream(device).cuda_stream)


def _check_qkv(q, k, v):
    torch = _torch()
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
            raise ValueError(f"{name} must be a device tensor")
        if t.dim() != 4 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous (B, H, N, d) tensor")
    if not (k.shape == v.shape and q.shape[:2] == k.shape[:2] and q.shape[3] == k.shape[3]):
        raise ValueError("q must be (B, H, N, d) and k, v (B, H, Nk, d)")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must have the same dtype")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k, v must be on the same device")


def _params_from(q, k, *, causal, kv_len, dropout_p, seed, scale, out_dtype, window):
    torch = _torch()
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    # e4m3 inputs write O in bfloat16 unless float32 is asked for.
    default_out = torch.bfloat16 if q.dtype == torch.float8_e4m3fn else q.dtype
    odt = default_out if out_dtype is None else out_dtype
    kv_ptr = 0
    if kv_len is not None:
        if kv_len.dtype != torch.int32 or kv_len.device != q.device or kv_len.numel() != B \
                or not kv_len.is_contiguous():
            raise ValueError("kv_len must be a contiguous int32 device tensor of B entries")
        kv_ptr = kv_len.data_ptr()
    if window is not None and (len(window) != 2 or min(int(w) for w in window) < -1):
        raise ValueError("window must be (left, right) with each side >= -1")
    # make_params clamps sides above INT32_MAX (wider than any sequence).
    p = make_params(B, H, N, d, dtype=_code(q.dtype), out_dtype=_code(odt), scale=scale,
                    causal=causal, kv_len_ptr=kv_ptr, dropout_p=dropout_p, seed=seed,
                    n_k=k.shape[2], window=window)
    return p, odt


def _check_like(name, t, shape, dtype, device):
    """A tensor argument the kernels read or write: its shape, dtype, device
    and layout must be exactly what the launch assumes (a wrong-sized or host
    buffer would be read or written out of bounds on the device)."""
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a tensor")
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError(f"{name} must be {tuple(shape)} {dtype}, got {tuple(t.shape)} {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def fwd(q, k, v, *, causal: bool = False, kv_len=None, dropout_p: float = 0.0,
        seed: int = 0, scale: Optional[float] = None, out_dtype=None, window=None,
        out=None, lse=None) -> Tuple["torch.Tensor", "torch.Tensor"]:
    """Fused forward: returns (O, lse). O has out_dtype (default q.dtype).
    out and lse, if given, must be a contiguous (B, H, N, d) tensor in out_dtype
    and a contiguous float32 (B, H, N) tensor on q's device."""
    torch = _torch()
    lib = load_library()
    _check_qkv(q, k, v)
    p, odt = _params_from(q, k, causal=causal, kv_len=kv_len, dropout_p=dropout_p, seed=seed,
                          scale=scale, out_dtype=out_dtype, window=window)
    B, H, N, d = q.shape
    if out is None:
        out = torch.empty((B, H, N, d), dtype=odt, device=q.device)
    else:
        _check_like("out", out, (B, H, N, d), odt, q.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    else:
        _check_like("lse", lse, (B, H, N), torch.float32, q.device)
    st = lib.attn_fwd(ctypes.byref(p), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                      out.data_ptr(), lse.data_ptr(), _stream_ptr(q.device))
    if st != 0:
        raise AttnError(st, "attn_fwd")
    return out, lse


def bwd_workspace_bytes(q, *, causal=False, kv_len=None, dropout_p=0.0, seed=0,
                        scale=None, out_dtype=None, window=None, k=None) -> int:
    p, _ = _params_from(q, q if k is None else k, causal=causal, kv_len=kv_len,
                        dropout_p=dropout_p, seed=seed, scale=scale, out_dtype=out_dtype,
                        window=window)
    return int(load_library().attn_bwd_workspace_bytes(ctypes.byref(p)))


def bwd(q, k, v, o, lse, do, *, causal: bool = False, kv_len=None, dropout_p: float = 0.0,
        seed: int = 0, scale: Optional[float] = None, out_dtype=None, window=None,
        workspace=None, out=None, stage: Optional[int] = None):
    """Fused backward with recomputation: returns (dQ, dK, dV) in out_dtype.

    out: optional preallocated (dq, dk, dv); workspace: optional uint8 device
    buffer of at least bwd_workspace_bytes(...) bytes; stage: None runs all
    three kernels, else one of BWD_STAGE_* (see attn_bwd_stage)."""
    torch = _torch()
    lib = load_library()
    _check_qkv(q, k, v)
    _check_like("do", do, q.shape, q.dtype, q.device)
    p, odt = _params_from(q, k, causal=causal, kv_len=kv_len, dropout_p=dropout_p, seed=seed,
                          scale=scale, out_dtype=out_dtype, window=window)
    _check_like("o (the forward output)", o, q.shape, odt, q.device)
    _check_like("lse (the forward's statistic)", lse, q.shape[:3], torch.float32, q.device)
    need = int(lib.attn_bwd_workspace_bytes(ctypes.byref(p)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    elif not isinstance(workspace, torch.Tensor) or workspace.device != q.device \
            or not workspace.is_contiguous():
        raise ValueError(f"workspace must be a contiguous tensor on {q.device}")
    if out is None:
        out = (torch.empty(q.shape, dtype=odt, device=q.device),
               torch.empty(k.shape, dtype=odt, device=q.device),
               torch.empty(k.shape, dtype=odt, device=q.device))
    dq, dk, dv = out
    for name, t, like in zip(("dq", "dk", "dv"), out, (q, k, v)):
        _check_like(name, t, like.shape, odt, q.device)
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
            do.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
            workspace.data_ptr(), workspace.numel() * workspace.element_size(),
            _stream_ptr(q.device))
    if stage is None:
        st = lib.attn_bwd(ctypes.byref(p), *args)
    else:
        st = lib.attn_bwd_stage(ctypes.byref(p), int(stage), *args)
    if st != 0:
        raise AttnError(st, "attn_bwd" if stage is None else "attn_bwd_stage")
    return dq, dk, dv


def bwd_noalloc(q, k, v, o, lse, do, *, causal: bool = False, kv_len=None,
                dropout_p: float = 0.0, seed: int = 0, scale: Optional[float] = None,
                out_dtype=None, window=None, out=None):
    """attn_bwd_noalloc: the backward with the library's fixed per-GPU scratch
    in place of a workspace (bit-identical to bwd). The library allocates
    nothing; pass `out` = (dq, dk, dv) to allocate nothing here either.
    Problems whose workspace would exceed the scratch raise AttnError
    (ATTN_ERR_TOO_LARGE)."""
    torch = _torch()
    lib = load_library()
    _check_qkv(q, k, v)
    _check_like("do", do, q.shape, q.dtype, q.device)
    p, odt = _params_from(q, k, causal=causal, kv_len=kv_len, dropout_p=dropout_p, seed=seed,
                          scale=scale, out_dtype=out_dtype, window=window)
    _check_like("o (the forward output)", o, q.shape, odt, q.device)
    _check_like("lse (the forward's statistic)", lse, q.shape[:3], torch.float32, q.device)
    if out is None:
        out = (torch.empty(q.shape, dtype=odt, device=q.device),
               torch.empty(k.shape, dtype=odt, device=q.device),
               torch.empty(k.shape, dtype=odt, device=q.device))
    dq, dk, dv = out
    for name, t, like in zip(("dq", "dk", "dv"), out, (q, k, v)):
        _check_like(name, t, like.shape, odt, q.device)
    st = lib.attn_bwd_noalloc(ctypes.byref(p), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                              o.data_ptr(), lse.data_ptr(), do.data_ptr(), dq.data_ptr(),
                              dk.data_ptr(), dv.data_ptr(), _stream_ptr(q.device))
    if st != 0:
        raise AttnError(st, "attn_bwd_noalloc")
    return dq, dk, dv


def noalloc_max_workspace_bytes() -> int:
    return int(load_library().attn_bwd_noalloc_max_workspace_bytes())


def dropout_mask(B: int, H: int, N: int, dropout_p: float, seed: int, device,
                 d: int = 64, n_k: Optional[int] = None) -> "torch.Tensor":
    """The raw Philox keep decisions, uint8 (B, H, N, Nk), as the kernels draw them."""
    torch = _torch()
    lib = load_library()
    nk = N if n_k is None else int(n_k)
    keep = torch.empty((B, H, N, nk), dtype=torch.uint8, device=device)
    p = make_params(B, H, N, d, dtype=ATTN_F16, out_dtype=ATTN_F16, scale=1.0,
                    dropout_p=dropout_p, seed=seed, n_k=nk)
    st = lib.attn_dropout_mask(ctypes.byref(p), keep.data_ptr(), _stream_ptr(device))
    if st != 0:
        raise AttnError(st, "attn_dropout_mask")
    return keep
