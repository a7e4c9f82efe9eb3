"""Build libattn.so (gfx950) in-tree with hipcc.

Usage: python -m exact_tiled_attention_20_amd.build [--jobs N]

Each source in csrc/ is compiled to its own object in parallel and linked into
exact_tiled_attention_20_amd/libattn.so. Always rebuilds (it is the "does it
build" check as well as the build).
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libattn.so")
SOURCES = ["attn_api.cpp", "attn_fwd.hip", "attn_fwd_fp8.hip", "attn_bwd.hip",
           "attn_bwd_dq256.hip", "attn_dropout_mask.hip", "attn_noalloc.hip"]

ARCH = "gfx950"
# Packed fp32 VALU forms are disabled: only scalar/vector fp32 ops are emitted.
COMMON_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
]
# MFMA results placed in VGPRs rather than AGPRs, so the softmax arithmetic
# that consumes score tiles needs no accumulator-register copies. Every source
# but the d = 256 dQ kernel's, whose Q and dO operands the flag would push into
# the accumulation registers (copied back before every MFMA).
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
NO_VGPR_FORM = {"attn_bwd_dq256.hip"}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the ROCm toolchain is required to build libattn.so")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    flags = COMMON_FLAGS + ([] if src in NO_VGPR_FORM else VGPR_FORM)
    cmd = [hipcc(), *flags, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    noise = [ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    if noise:
        sys.stderr.write("\n".join(noise) + "\n")
    return obj


def build(jobs: int | None = None, verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 4, 16)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    args = ap.parse_args()
    build(args.jobs)


if __name__ == "__main__":
    main()
