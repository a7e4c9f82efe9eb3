"""Seeded synthetic workloads for exact tiled attention.

This module only draws inputs. It holds none of the attention arithmetic, so the
CPU oracle (``oracle/``), the tests and ``bench.py`` can all use it without the
oracle and the HIP path sharing any code.

Shapes follow the workloads named for the method: a tiny sanity head, a
small-decoder layer, a long causal bf16 layer with a wide score range, a
BERT-style padded layer with dropout, and a 16K-token causal layer with a
backward pass. All tensors are (B, H, N, d), d innermost, drawn in float32 on the
CPU from ``torch.Generator().manual_seed(seed)`` and rounded to nearest-even into
the storage dtype, so every consumer sees identical bits.
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Tuple

import torch

DTYPES = {"fp16": torch.float16, "bf16": torch.bfloat16, "e4m3": torch.float8_e4m3fn}

# Fixed 64-bit dropout seed used by the padded+dropout workload.
DROPOUT_SEED = 0x243F6A8885A308D3


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str               # "fp16" | "bf16"
    causal: bool = False
    pad: bool = False        # key padding with per-batch valid length
    pad_lo: int = 0          # valid length drawn uniformly from [pad_lo, pad_hi]
    pad_hi: int = 0
    dropout_p: float = 0.0
    qk_std: float = 1.0      # Q and K drawn as qk_std * N(0, 1)
    backward: bool = False   # the workload includes dO and the backward pass
    seed: int = 0
    n_k: int = 0             # rows of K and V (0: N, self-attention)
    window: Optional[Tuple[int, int]] = None   # (left, right), -1 unbounded

    @property
    def Nk(self) -> int:
        return self.n_k or self.N

    @property
    def scale(self) -> float:
        return 1.0 / (self.d ** 0.5)

    @property
    def torch_dtype(self) -> torch.dtype:
        return DTYPES[self.dtype]

    def flops_fwd(self) -> float:
        """4*B*H*N^2*d, halved under a causal mask (the plain convention)."""
        f = 4.0 * self.B * self.H * self.N * self.N * self.d
        return f / 2 if self.causal else f

    def flops_bwd(self) -> float:
        """Five N^2*d contractions instead of the forward's two: 2.5x forward."""
        return 2.5 * self.flops_fwd()


WORKLOADS = {
    "tiny_b1h2n256d64_fp16": Workload(
        "tiny_b1h2n256d64_fp16", B=1, H=2, N=256, d=64, dtype="fp16", seed=1001),
    "decoder_b8h12n1024d64_fp16_causal": Workload(
        "decoder_b8h12n1024d64_fp16_causal", B=8, H=12, N=1024, d=64, dtype="fp16",
        causal=True, seed=1002),
    "long_b4h16n4096d128_bf16_causal": Workload(
        "long_b4h16n4096d128_bf16_causal", B=4, H=16, N=4096, d=128, dtype="bf16",
        causal=True, qk_std=3.0, seed=1003),
    "bert_b16h16n512d64_fp16_pad_drop": Workload(
        "bert_b16h16n512d64_fp16_pad_drop", B=16, H=16, N=512, d=64, dtype="fp16",
        pad=True, pad_lo=256, pad_hi=512, dropout_p=0.1, seed=1004),
    "ctx16k_b1h32n16384d128_bf16_causal_bwd": Workload(
        "ctx16k_b1h32n16384d128_bf16_causal_bwd", B=1, H=32, N=16384, d=128,
        dtype="bf16", causal=True, backward=True, seed=1005),
}

# Order matters: the first is the small case, the third is the headline forward.
WORKLOAD_ORDER = list(WORKLOADS)

# The variants the method's description names as needing tiling changes
# (sliding-window attention, cross-attention on a non-square grid, head
# dimension 256), at the sizes of the 16K-context layer: a Mistral-style causal
# window of 4096 keys, a 2048-query chunk attending causally (bottom-right) to
# a 16384-key context, as in chunked prefill against a key/value cache, and
# d = 256.
VARIANTS = {
    "swa4096_b1h32n16384d128_bf16_bwd": Workload(
        "swa4096_b1h32n16384d128_bf16_bwd", B=1, H=32, N=16384, d=128, dtype="bf16",
        causal=True, window=(4095, -1), backward=True, seed=1006),
    "chunk_b4h16n2048nk16384d128_bf16_causal_bwd": Workload(
        "chunk_b4h16n2048nk16384d128_bf16_causal_bwd", B=4, H=16, N=2048, d=128,
        dtype="bf16", causal=True, n_k=16384, backward=True, seed=1007),
    # fp8 (e4m3) forward at the sizes of the long layer (wide score range) and
    # of the 16K-context layer: Q, K, V drawn as for those layers in float32
    # and rounded to nearest-even e4m3.
    "fp8_b4h16n4096d128_causal": Workload(
        "fp8_b4h16n4096d128_causal", B=4, H=16, N=4096, d=128, dtype="e4m3",
        causal=True, qk_std=3.0, seed=1009),
    "fp8_b1h32n16384d128_causal": Workload(
        "fp8_b1h32n16384d128_causal", B=1, H=32, N=16384, d=128, dtype="e4m3",
        causal=True, seed=1010),
    # Head dimension 256: the same tokens and FLOP per layer as the 16K-context
    # layer with half the heads.
    "d256_b1h16n16384_bf16_causal_bwd": Workload(
        "d256_b1h16n16384_bf16_causal_bwd", B=1, H=16, N=16384, d=256, dtype="bf16",
        causal=True, backward=True, seed=1008),
}


@dataclasses.dataclass
class Inputs:
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    do: Optional[torch.Tensor]
    kv_len: Optional[torch.Tensor]   # int32 [B] or None
    seed: int                        # dropout seed (64-bit)


def make_inputs(w: Workload, *, seed: Optional[int] = None) -> Inputs:
    """Draw the workload's tensors on the CPU in storage dtype."""
    g = torch.Generator().manual_seed(w.seed if seed is None else seed)
    shape = (w.B, w.H, w.N, w.d)
    dt = w.torch_dtype

    def draw(std: float) -> torch.Tensor:
        x = torch.randn(shape, generator=g, dtype=torch.float32)
        if std != 1.0:
            x = x * std
        return x.to(dt)

    kshape = (w.B, w.H, w.Nk, w.d)

    def draw_k(std: float) -> torch.Tensor:
        x = torch.randn(kshape, generator=g, dtype=torch.float32)
        if std != 1.0:
            x = x * std
        return x.to(dt)

    q = draw(w.qk_std)
    k = draw_k(w.qk_std)
    v = draw_k(1.0)
    do = draw(1.0) if w.backward else None
    kv_len = None
    if w.pad:
        kv_len = torch.randint(w.pad_lo, w.pad_hi + 1, (w.B,), generator=g,
                               dtype=torch.int64).to(torch.int32)
    return Inputs(q, k, v, do, kv_len, DROPOUT_SEED if w.dropout_p > 0 else 0)


def random_case(B: int, H: int, N: int, d: int, dtype: str, *, seed: int,
                std: float = 1.0, with_do: bool = False,
                kv_len: Optional[list] = None, n_k: Optional[int] = None) -> Inputs:
    """Small seeded case for sweeps: same recipe as the named workloads.

    n_k: number of key/value rows (default N); Q and dO keep N rows.
    """
    g = torch.Generator().manual_seed(seed)
    shape = (B, H, N, d)
    kshape = (B, H, N if n_k is None else n_k, d)
    dt = DTYPES[dtype]
    q = (torch.randn(shape, generator=g) * std).to(dt)
    k = (torch.randn(kshape, generator=g) * std).to(dt)
    v = torch.randn(kshape, generator=g).to(dt)
    do = torch.randn(shape, generator=g).to(dt) if with_do else None
    kl = None if kv_len is None else torch.tensor(kv_len, dtype=torch.int32)
    return Inputs(q, k, v, do, kl, 0x9E3779B97F4A7C15 ^ seed)
