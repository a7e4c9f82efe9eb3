#!/usr/bin/env python
"""Benchmark of the fused exact-attention path on one MI355X.

One step = one pass of the whole path over one batch: attn_fwd (the fused tiled
forward, O and lse) followed by the three backward kernels (D = rowsum(dO*O),
dK/dV with recomputation, dQ with recomputation), on the 16K-token causal bf16
workload B=1, H=32, N=16384, d=128 with dO ~ N(0,1). Inputs are resident on the
device before timing starts; outputs and the workspace are preallocated.

FLOP convention: forward 4*B*H*N^2*d, halved under the causal mask; backward
2.5x forward (five N^2*d contractions against two). Throughput is reported in
TFLOP/s and as a fraction of MI355X's dense bf16 MFMA peak (2516.6 TFLOP/s).

Prints ONE JSON line. Options:
  --gpus N      only 1 is supported (the path runs on one GPU)
  --steps K     timed steps (default 10)
  --warmup W    untimed steps first (default 3)
  --no-cpu-baseline   skip timing the CPU oracle on its bounded samples (every
                      named workload; the headline entry is the backward
                      workload's, with the host's CPU model, core count and
                      BLAS library)
  --no-per-config     skip the forward timings on each named workload (the
                      `forward_per_config` field: median and minimum per
                      launch, roofline fractions, one cold launch at N=4096)
  --no-variants       skip the variants (the `variants` field: a sliding
                      window of 4096 keys at N=16384 and a 2048-query chunk
                      against 16384 keys, each forward and forward +
                      backward, TFLOP/s over the visible query-key pairs; and
                      the forward at head dimension 256)
  --no-unfused        skip timing standard attention as separate torch ops
                      (matmul, mask, softmax, dropout, matmul; the backward
                      by hand for the backward workloads) against the fused
                      kernels on every workload, with the extra device memory
                      each allocates and the largest |O difference| (the
                      `unfused_comparison` field, on by default)
  --only WORKLOAD     only --steps passes of one workload (forward and
                      backward), for hardware-counter runs
  --inputs KIND       with --only: `drawn` (the workload's own inputs, the
                      default), `zeros` (Q, K, V and dO all zero) or `signs`
                      (each drawn value replaced by its sign). The kernels
                      execute the same instructions on all three; the chip's
                      clock does not stay the same.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "fused attention TFLOP/s + % of fp16/bf16 MFMA peak, fwd and fwd+bwd"
PEAK_BF16_TFLOPS = 2516.6          # 256 CU x 4096 flop/clk x 2.4 GHz, dense
PEAK_FP8_TFLOPS = 5000.0           # MI355X dense fp8 (e4m3) MFMA peak
PEAK_HBM_GBS = 8000.0
WORKLOAD = "ctx16k_b1h32n16384d128_bf16_causal_bwd"
FWD_WORKLOAD = "long_b4h16n4096d128_bf16_causal"
KERNEL_NAMES = ("attn_fwd_kernel", "attn_bwd_preprocess_kernel", "attn_bwd_dkdv_kernel",
                "attn_bwd_dq_kernel")


def _csrc_digest() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "exact_tiled_attention_20_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def _traffic_for(kernel: str, workload: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel sources; otherwise None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        table = json.load(f)
    rec = table.get(f"{kernel}@{workload}")
    if not rec or rec.get("csrc_digest") != _csrc_digest():
        return None
    return rec.get("bytes_per_launch")


def _clock_for(kernel: str, workload: str):
    """Average shader clock (MHz) while the kernel ran, from committed rocprofv3
    counter runs (active cycles over the same dispatches' durations), if they
    were taken on the current kernel sources; otherwise None."""
    path = os.path.join(ROOT, "profiles", "clock.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        table = json.load(f)
    rec = table.get(f"{kernel}@{workload}")
    if not rec or rec.get("csrc_digest") != _csrc_digest():
        return None
    return rec.get("avg_clock_mhz")


def _at_clock(tflops: float, mhz):
    """The dense bf16 peak scales with the clock: the datasheet figure is
    quoted at 2400 MHz."""
    if mhz is None:
        return None
    peak = PEAK_BF16_TFLOPS * mhz / 2400.0
    return {"avg_clock_mhz": mhz, "peak_tflops_at_clock": round(peak, 1),
            "pct_of_clock_peak": round(100 * tflops / peak, 2)}


def _host_info() -> dict:
    """The host the oracle runs on: logical CPUs, CPU model, the BLAS library
    numpy calls and the threads it uses."""
    info = {"os_cpu_count": os.cpu_count(), "cpu_model": None, "blas": None,
            "blas_threads": None}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    info["cpu_model"] = line.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass
    try:
        from threadpoolctl import threadpool_info
        blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if blas:
            info["blas"] = f"{blas[0].get('internal_api')} {blas[0].get('version')}"
            info["blas_threads"] = int(max(i.get("num_threads", 1) for i in blas))
    except Exception:  # pragma: no cover
        pass
    return info


# Bounded oracle samples per named workload (heads of batch 0 upward, all
# rows unless a causal prefix is named); the rest of each workload is the same
# computation on other heads, so its time is extrapolated by the head count.
CPU_SAMPLES = {
    "tiny_b1h2n256d64_fp16": dict(heads=2),
    "decoder_b8h12n1024d64_fp16_causal": dict(heads=96),
    "long_b4h16n4096d128_bf16_causal": dict(heads=64),
    "bert_b16h16n512d64_fp16_pad_drop": dict(heads=256),
    "ctx16k_b1h32n16384d128_bf16_causal_bwd": dict(heads=4),
}


def _oracle_sample(w, inputs, heads: int) -> dict:
    """Time the fp64 oracle (as it stands) on the first `heads` heads of the
    workload (row-major over (b, h)), forward, plus the backward when the
    workload has one."""
    from oracle import attention as A
    nh = min(heads, w.B * w.H)
    todo = [(i // w.H, i % w.H) for i in range(nh)]
    kw = dict(scale=w.scale, causal=w.causal, kv_len=inputs.kv_len, dropout_p=w.dropout_p,
              seed=inputs.seed, heads=todo)
    t0 = time.perf_counter()
    A.forward(inputs.q, inputs.k, inputs.v, **kw)
    if inputs.do is not None:
        A.backward(inputs.q, inputs.k, inputs.v, inputs.do, **kw)
    dt = time.perf_counter() - t0
    flops = w.flops_fwd() * (3.5 if inputs.do is not None else 1.0) * nh / (w.B * w.H)
    total_heads = w.B * w.H
    return {"heads": nh, "of_heads": total_heads, "pass": "fwd+bwd" if inputs.do is not None
            else "fwd", "seconds": round(dt, 3), "tflops": round(flops / dt / 1e12, 6),
            "full_workload_seconds": round(dt * total_heads / nh, 1),
            "full_workload_is_extrapolated": nh < total_heads}


def cpu_baseline(W, cache: dict, headline: str) -> dict:
    """The fp64 oracle timed on the host on a bounded sample of every named
    workload (CPU_SAMPLES); the headline entry (value, unit, sample) is the
    backward workload's, the others are listed per workload with the host's
    description. Inputs are the same seeded tensors the GPU runs use."""
    host = _host_info()
    per = {}
    for name, spec in CPU_SAMPLES.items():
        w = W.WORKLOADS[name]
        inputs = cache.get(name) or W.make_inputs(w)
        per[name] = _oracle_sample(w, inputs, spec["heads"])
        print(f"bench: cpu oracle {name}: {per[name]['seconds']} s", file=sys.stderr, flush=True)
    h = per[headline]
    return {"value": h["tflops"], "unit": "TFLOP/s",
            "cores": host["blas_threads"] or host["os_cpu_count"], "kind": "oracle",
            "sample": f"{h['heads']} of the {h['of_heads']} heads of {headline}, every row, "
                      f"fp64 numpy {h['pass']} ({h['seconds']} s; the whole workload "
                      f"extrapolates to {h['full_workload_seconds']} s)",
            "seconds": h["seconds"], "host": host, "per_config": per}


def per_config_forward(attn, W, dev, reuse=None, min_iters=50, min_ms=200.0) -> dict:
    """Forward alone on every named workload: 10 warm-up launches, then at
    least min_iters launches and min_ms of GPU time, each bracketed by its own
    HIP events on the launch stream; median and minimum per launch. Reports
    nominal TFLOP/s (4BHN^2d, half under causal), for the padded workload also
    the effective rate over visible pairs, the fraction of the dense bf16/fp16
    peak, and the attainable roofline min(peak, AI x 8 TB/s) with AI the
    algorithmic flop per byte (Q, K, V read once; O and lse written once).
    For the N=4096 workload also one cold launch, after 512 MiB of device
    writes have displaced it from the caches."""
    import torch
    out = {}
    for name, w in W.WORKLOADS.items():
        if reuse is not None and name in reuse:
            q, k, v, kv = reuse[name]
        else:
            inp = W.make_inputs(w)
            q, k, v = (t.to(dev) for t in (inp.q, inp.k, inp.v))
            kv = None if inp.kv_len is None else inp.kv_len.to(dev)
        seed = W.DROPOUT_SEED if w.dropout_p > 0 else 0
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)

        def launch():
            attn.fwd(q, k, v, causal=w.causal, kv_len=kv, dropout_p=w.dropout_p, seed=seed,
                     scale=w.scale, out=o, lse=lse)

        for _ in range(10):
            launch()
        torch.cuda.synchronize()
        times = []
        while len(times) < min_iters or sum(times) < min_ms:
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(min_iters)]
            for e0, e1 in evs:
                e0.record()
                launch()
                e1.record()
            torch.cuda.synchronize()
            times += [e0.elapsed_time(e1) for e0, e1 in evs]
        times.sort()
        med, mn = times[len(times) // 2], times[0]
        flops = w.flops_fwd()
        elt = 2
        nbytes = 4 * w.B * w.H * w.N * w.d * elt + 4 * w.B * w.H * w.N
        ai = flops / nbytes
        attainable = min(PEAK_BF16_TFLOPS, ai * PEAK_HBM_GBS / 1000.0)
        tf = flops / (med * 1e-3) / 1e12
        rec = {"launches": len(times), "median_ms": round(med, 5), "min_ms": round(mn, 5),
               "tflops": round(tf, 2), "pct_of_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2),
               "ai_flop_per_byte": round(ai, 1), "attainable_tflops": round(attainable, 1),
               "frac_of_attainable": round(tf / attainable, 4)}
        if kv is not None:
            vis = float(kv.double().clamp(0, w.N).sum().item()) / (w.B * w.N)
            rec["effective_tflops"] = round(tf * vis, 2)
            rec["visible_key_fraction"] = round(vis, 4)
        if name == "long_b4h16n4096d128_bf16_causal":
            scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
            scratch.fill_(1)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            launch()
            e1.record()
            torch.cuda.synchronize()
            rec["cold_ms"] = round(e0.elapsed_time(e1), 5)
            del scratch
        out[name] = rec
        del o, lse
    return out


def visible_pairs(w) -> float:
    """Query-key pairs a masked variant computes per head: row i sees keys
    [max(0, c - left), min(Nk - 1, c, c + right)] with c = i + Nk - N (causal
    caps at c; -1 leaves a window side open)."""
    import numpy as np
    i = np.arange(w.N, dtype=np.int64)
    c = i + (w.Nk - w.N)
    lo = np.zeros_like(i)
    hi = np.full_like(i, w.Nk - 1)
    if w.causal:
        hi = np.minimum(hi, c)
    if w.window is not None:
        if w.window[0] >= 0:
            lo = np.maximum(lo, c - w.window[0])
        if w.window[1] >= 0:
            hi = np.minimum(hi, c + w.window[1])
    return float(np.maximum(0, hi - lo + 1).sum())


def variant_timings(attn, W, dev, reps: int = 30) -> dict:
    """The variants (sliding window; non-square grid; d = 256): forward alone
    and, where the workload has one, forward + the three backward kernels,
    each bracketed by HIP events on the launch stream after 5 warm-up passes;
    medians. FLOP count the pairs actually visible: forward 4*d per pair,
    backward 2.5x that."""
    import torch
    out = {}
    for name, w in W.VARIANTS.items():
        inp = W.make_inputs(w)
        q, k, v = (t.to(dev) for t in (inp.q, inp.k, inp.v))
        do = inp.do.to(dev) if w.backward else None
        o = torch.empty(q.shape, dtype=torch.bfloat16 if w.dtype == "e4m3" else q.dtype,
                        device=dev)
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
        kw = dict(causal=w.causal, window=w.window, scale=w.scale)
        grads = ws = None
        if w.backward:
            grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
            ws = torch.empty(attn.bwd_workspace_bytes(q, k=k, **kw), dtype=torch.uint8,
                             device=dev)

        def fwd():
            attn.fwd(q, k, v, out=o, lse=lse, **kw)

        def bwd():
            if w.backward:
                attn.bwd(q, k, v, o, lse, do, out=grads, workspace=ws, **kw)

        for _ in range(5):
            fwd()
            bwd()
        torch.cuda.synchronize()
        tf, tb = [], []
        for _ in range(reps):
            e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            e[0].record()
            fwd()
            e[1].record()
            bwd()
            e[2].record()
            torch.cuda.synchronize()
            tf.append(e[0].elapsed_time(e[1]))
            tb.append(e[1].elapsed_time(e[2]))
        tf.sort()
        tb.sort()
        fm, bm = tf[len(tf) // 2], tb[len(tb) // 2]
        pairs = visible_pairs(w) * w.B * w.H
        f_fwd = 4.0 * w.d * pairs
        fwd_tf = f_fwd / (fm * 1e-3) / 1e12
        step_tf = 3.5 * f_fwd / ((fm + bm) * 1e-3) / 1e12 if w.backward else None
        peak = PEAK_FP8_TFLOPS if w.dtype == "e4m3" else PEAK_BF16_TFLOPS
        out[name] = {
            "B": w.B, "H": w.H, "N": w.N, "Nk": w.Nk, "d": w.d, "causal": w.causal,
            "dtype": w.dtype, "window": list(w.window) if w.window else None,
            "visible_pairs_per_head": int(pairs / (w.B * w.H)),
            "fwd_ms": round(fm, 4),
            "fwd_tflops": round(fwd_tf, 1),
            "peak_tflops": peak,
            "fwd_pct_of_peak": round(100 * fwd_tf / peak, 2),
        }
        if w.backward:
            out[name].update({
                "bwd_ms": round(bm, 4), "fwd_bwd_tflops": round(step_tf, 1),
                "fwd_bwd_pct_of_peak": round(100 * step_tf / PEAK_BF16_TFLOPS, 2)})
        del q, k, v, do, o, lse, grads, ws
        torch.cuda.empty_cache()
    return out


def unfused_attention(q, k, v, *, scale, dead=None, dropout_p=0.0, do=None):
    """Standard (unfused) attention as separate torch ops, the chain the fused
    kernel replaces: S = scale Q K^T materialised in the input dtype, -inf where
    `dead` (a boolean mask broadcastable to S) is set, softmax, dropout (torch's
    own RNG), O = P V. With dO also the backward written out by hand:
    dV = P^T dO, dP = dO V^T, D = rowsum(dO * O), dS = P (dP - D),
    dQ = scale dS K, dK = scale dS^T Q. Every right-hand matmul operand is made
    contiguous first. Returns (O, (dQ, dK, dV) or None)."""
    import torch
    import torch.nn.functional as F
    kt = k.transpose(-1, -2).contiguous()
    s = torch.matmul(q, kt)
    s.mul_(scale)
    if dead is not None:
        s.masked_fill_(dead, float("-inf"))
    p = torch.softmax(s, dim=-1)
    del s
    pd = F.dropout(p, dropout_p) if dropout_p > 0 else p
    o = torch.matmul(pd, v)
    if do is None:
        return o, None
    vt = v.transpose(-1, -2).contiguous()
    dv = torch.matmul(pd.transpose(-1, -2).contiguous(), do)
    dp = torch.matmul(do, vt)
    dd = (do.float() * o.float()).sum(-1, keepdim=True).to(q.dtype)
    ds = p * (dp - dd)
    del dp
    dq = torch.matmul(ds, k).mul_(scale)
    dk = torch.matmul(ds.transpose(-1, -2).contiguous(), q).mul_(scale)
    return o, (dq, dk, dv)


def unfused_comparison(attn, W, dev, reps_small: int = 20, reps_large: int = 5) -> dict:
    """Standard attention as separate torch ops against the fused kernels, on
    every named workload and variant: S = scale*Q K^T materialised in the input dtype,
    mask by -inf, softmax, dropout (torch's own RNG: same work, different
    mask), O = P V; for the backward workload also dV = P^T dO,
    dP = dO V^T, D = rowsum(dO*O), dS = P*(dP - D), dQ = scale*dS K,
    dK = scale*dS^T Q. Every right-hand matmul operand is made contiguous
    first, and those transposed copies are timed separately (the copy share).
    Reports median times, the device memory each path needs beyond its inputs
    (outputs, workspace and temporaries), and the largest |O_unfused - O_fused|."""
    import torch

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        ts.sort()
        return ts[len(ts) // 2]

    def peak_extra(fn):
        torch.cuda.synchronize()
        base = torch.cuda.memory_allocated()
        torch.cuda.reset_peak_memory_stats()
        fn()
        torch.cuda.synchronize()
        return torch.cuda.max_memory_allocated() - base

    out = {}
    for name, w in dict(W.WORKLOADS, **W.VARIANTS).items():
        if w.dtype == "e4m3":
            continue    # no fp8 path among torch's standard attention ops
        inp = W.make_inputs(w)
        q, k, v = (t.to(dev) for t in (inp.q, inp.k, inp.v))
        kv = None if inp.kv_len is None else inp.kv_len.to(dev)
        do = None if inp.do is None else inp.do.to(dev)
        seed = W.DROPOUT_SEED if w.dropout_p > 0 else 0
        reps = reps_large if w.N >= 4096 or w.Nk >= 4096 else reps_small
        # Keys each query row may not see: past its causal or window bound
        # (query i lines up with key i + Nk - N), or past the padding length.
        i_idx = torch.arange(w.N, device=dev)[:, None] + (w.Nk - w.N)
        j_idx = torch.arange(w.Nk, device=dev)[None, :]
        dead = None
        if w.causal:
            dead = (j_idx > i_idx)[None, None]
        if w.window is not None:
            if w.window[0] >= 0:
                lo = (j_idx < i_idx - w.window[0])[None, None]
                dead = lo if dead is None else (dead | lo)
            if w.window[1] >= 0:
                hi = (j_idx > i_idx + w.window[1])[None, None]
                dead = hi if dead is None else (dead | hi)
        if kv is not None:
            pad = (j_idx >= kv[:, None].long())[:, None, None, :]
            dead = pad if dead is None else (dead | pad)
        o_f = torch.empty_like(q)
        lse_f = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
        grads_f = None
        if do is not None:
            grads_f = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
        ws = None
        if do is not None:
            ws = torch.empty(attn.bwd_workspace_bytes(q, k=k, causal=w.causal, scale=w.scale,
                                                      window=w.window),
                             dtype=torch.uint8, device=dev)
        state = {}

        def fused():
            attn.fwd(q, k, v, causal=w.causal, kv_len=kv, dropout_p=w.dropout_p, seed=seed,
                     scale=w.scale, out=o_f, lse=lse_f, window=w.window)
            if do is not None:
                attn.bwd(q, k, v, o_f, lse_f, do, causal=w.causal, kv_len=kv,
                         dropout_p=w.dropout_p, seed=seed, scale=w.scale, out=grads_f,
                         workspace=ws, window=w.window)

        def transposes():
            kt = k.transpose(-1, -2).contiguous()
            if do is None:
                return kt, None
            return kt, v.transpose(-1, -2).contiguous()

        def unfused():
            o, g = unfused_attention(q, k, v, scale=w.scale, dead=dead,
                                     dropout_p=w.dropout_p, do=do)
            state["o"] = o
            if g is not None:
                state["g"] = g

        def transposes_bwd():
            # The two N x Nk transposed copies of the backward, on tensors of
            # the same shape and dtype as P and dS.
            t = torch.empty(w.B, w.H, w.N, w.Nk, dtype=q.dtype, device=dev)
            t.transpose(-1, -2).contiguous()
            t.transpose(-1, -2).contiguous()

        t_fused = timed(fused, reps)
        # The fused path's footprint: its preallocated outputs (and workspace)
        # plus anything allocated during the call.
        owned = o_f.nbytes + lse_f.nbytes
        if do is not None:
            owned += sum(g.nbytes for g in grads_f) + ws.nbytes
        m_fused = owned + peak_extra(fused)
        t_unf = timed(unfused, reps)
        state.clear()
        m_unf = peak_extra(unfused)
        fused()
        torch.cuda.synchronize()
        err = float((state["o"].float() - o_f.float()).abs().max().item())
        state.clear()
        t_copy = timed(transposes, reps)
        if do is not None:
            t_copy += timed(transposes_bwd, reps)
        if name in W.VARIANTS:
            f_fwd = 4.0 * w.d * visible_pairs(w) * w.B * w.H
            flops = f_fwd * (3.5 if do is not None else 1.0)
        else:
            flops = w.flops_fwd() + (w.flops_bwd() if do is not None else 0.0)
        out[name] = {
            "pass": "fwd+bwd" if do is not None else "fwd",
            "fused_ms": round(t_fused, 4), "unfused_ms": round(t_unf, 4),
            "unfused_transposed_copies_ms": round(t_copy, 4),
            "speedup": round(t_unf / t_fused, 2),
            "speedup_without_copies": round((t_unf - t_copy) / t_fused, 2),
            "fused_tflops": round(flops / (t_fused * 1e-3) / 1e12, 1),
            "fused_bytes": int(m_fused), "unfused_bytes": int(m_unf),
            "memory_ratio": round(m_unf / m_fused, 1),
            "max_abs_o_diff": round(err, 5) if w.dropout_p == 0 else None,
        }
        del q, k, v, do, kv, o_f, lse_f, grads_f, ws, dead
        torch.cuda.empty_cache()
    return out


def only_workload(attn, W, dev, name: str, steps: int, warmup: int, inputs: str = "drawn") -> int:
    """--only: passes of one workload (forward, then the backward wherever the
    input dtype has one: e4m3 is forward-only), timed with HIP events on the
    launch stream. A workload without its own dO gets one drawn from N(0, 1)
    with its seed + 1, so that counter runs cover every backward instance."""
    import torch
    w = W.WORKLOADS.get(name) or W.VARIANTS.get(name)
    if w is None:
        print(f"bench.py: unknown workload {name}", file=sys.stderr)
        return 2
    inp = W.make_inputs(w)
    q, k, v = (t.to(dev) for t in (inp.q, inp.k, inp.v))
    do = None if inp.do is None else inp.do.to(dev)
    if do is None and w.dtype != "e4m3":
        g = torch.Generator().manual_seed(w.seed + 1)
        do = torch.randn(q.shape, generator=g).to(q.dtype).to(dev)
    if inputs != "drawn":
        # Same shapes and dtypes, other bit patterns: all zero, or +-1.
        def recast(x):
            if x is None:
                return None
            y = torch.zeros_like(x.float()) if inputs == "zeros" else torch.sign(x.float())
            return y.to(x.dtype)
        q, k, v, do = recast(q), recast(k), recast(v), recast(do)
    kv = None if inp.kv_len is None else inp.kv_len.to(dev)
    kw = dict(causal=w.causal, window=w.window, scale=w.scale, kv_len=kv,
              dropout_p=w.dropout_p, seed=inp.seed)
    o, lse = attn.fwd(q, k, v, **kw)
    grads = ws = None
    if do is not None:
        grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
        ws = torch.empty(max(1, attn.bwd_workspace_bytes(q, k=k, **kw)), dtype=torch.uint8,
                         device=dev)

    def one():
        attn.fwd(q, k, v, out=o, lse=lse, **kw)
        if do is not None:
            attn.bwd(q, k, v, o, lse, do, out=grads, workspace=ws, **kw)

    for _ in range(warmup):
        one()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        one()
    e1.record()
    torch.cuda.synchronize()
    print(json.dumps({"workload": name, "inputs": inputs, "steps": steps,
                      "ms_per_pass": round(e0.elapsed_time(e1) / max(steps, 1), 4),
                      "pass": "fwd+bwd" if do is not None else "fwd"}))
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-unfused", action="store_true",
                    help="skip the unfused torch comparison on every workload")
    ap.add_argument("--no-per-config", action="store_true",
                    help="skip timing the forward on each named workload")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip timing the sliding-window and non-square variants")
    ap.add_argument("--fwd-only", action="store_true",
                    help="time only the forward headline workload (for profiling)")
    ap.add_argument("--only", default=None, metavar="WORKLOAD",
                    help="run only --steps passes (after --warmup) of the named workload or "
                         "variant, forward and backward (forward only for e4m3), and print "
                         "their times: the entry point for hardware-counter runs")
    ap.add_argument("--inputs", default="drawn", choices=("drawn", "zeros", "signs"),
                    help="with --only: the workload's drawn inputs, all zeros, or their signs")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run only a plain 1 GiB device-to-device copy (reference for "
                         "hardware byte counters)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: this path runs on one GPU; --gpus {args.gpus} (WORLD_SIZE={world}) "
              "is not supported. Heads are independent, so a multi-GPU run would shard "
              "(b, h) across GPUs with no communication; run one process per GPU instead.",
              file=sys.stderr)
        return 2

    import torch
    import attn_workloads as W
    import exact_tiled_attention_20_amd as attn

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    attn.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.calibrate_copy:
        # 1 GiB read + 1 GiB written per launch: the known traffic against
        # which FETCH_SIZE / WRITE_SIZE counter readings are scaled.
        src = torch.empty(1 << 29, dtype=torch.bfloat16, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": src.numel() * 2, "launches": 3}))
        return 0

    if args.only is not None:
        return only_workload(attn, W, dev, args.only, args.steps, args.warmup, args.inputs)

    # -- forward headline workload (4 x 16 heads, N = 4096, d = 128, causal) --
    wf = W.WORKLOADS[FWD_WORKLOAD]
    fi = W.make_inputs(wf)
    fq, fk, fv = (t.to(dev) for t in (fi.q, fi.k, fi.v))
    fo = torch.empty_like(fq)
    flse = torch.empty(fq.shape[:3], dtype=torch.float32, device=dev)

    def fwd_long():
        attn.fwd(fq, fk, fv, causal=wf.causal, scale=wf.scale, out=fo, lse=flse)

    # One launch takes well under a millisecond, so the clocks need a few dozen
    # launches to settle before the timed repetitions.
    for _ in range(max(args.warmup, 1) * 20):
        fwd_long()
    torch.cuda.synchronize()
    reps = 100
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fwd_long()
    e1.record()
    torch.cuda.synchronize()
    fwd_long_ms = e0.elapsed_time(e1) / reps
    fwd_long_tflops = wf.flops_fwd() / (fwd_long_ms * 1e-3) / 1e12
    del fq, fk, fv, fo, flse
    if args.fwd_only:
        print(json.dumps({"workload": FWD_WORKLOAD, "fwd_ms": fwd_long_ms,
                          "fwd_tflops": fwd_long_tflops}))
        return 0

    # -- the step workload: forward + backward at B=1, H=32, N=16384, d=128 --
    w = W.WORKLOADS[WORKLOAD]
    inputs = W.make_inputs(w)
    q, k, v, do = (t.to(dev) for t in (inputs.q, inputs.k, inputs.v, inputs.do))
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    grads = tuple(torch.empty_like(q) for _ in range(3))
    ws = torch.empty(attn.bwd_workspace_bytes(q, causal=w.causal, scale=w.scale),
                     dtype=torch.uint8, device=dev)
    kw = dict(causal=w.causal, scale=w.scale)
    stages = (attn.BWD_STAGE_PREPROCESS, attn.BWD_STAGE_DKDV, attn.BWD_STAGE_DQ)

    def step(events=None):
        if events is not None:
            events[0].record()
        attn.fwd(q, k, v, out=o, lse=lse, **kw)
        for i, s in enumerate(stages):
            if events is not None:
                events[i + 1].record()
            attn.bwd(q, k, v, o, lse, do, out=grads, workspace=ws, stage=s, **kw)
        if events is not None:
            events[4].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    K = args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_kernel = [0.0] * 4
    step_ms = 0.0
    for ev in evs:
        for j in range(4):
            per_kernel[j] += ev[j].elapsed_time(ev[j + 1]) / K
        step_ms += ev[0].elapsed_time(ev[4]) / K
    ms_per_step = wall * 1e3 / K

    f_fwd = w.flops_fwd()
    f_total = f_fwd + w.flops_bwd()
    value = f_total / (ms_per_step * 1e-3) / 1e12
    # Algorithmic FLOP per launch: the forward's two contractions; the dK/dV
    # kernel's four (S, dP, dV, dK); the dQ kernel's one (dQ) -- its second
    # evaluation of S and dP is recomputation beyond the algorithm's count.
    alg = {"attn_fwd_kernel": f_fwd, "attn_bwd_preprocess_kernel": 0.0,
           "attn_bwd_dkdv_kernel": 2.0 * f_fwd, "attn_bwd_dq_kernel": 0.5 * f_fwd}
    kernels = {}
    for name, ms in zip(KERNEL_NAMES, per_kernel):
        kernels[name] = {"avg_ms": round(ms, 4),
                         "alg_tflops": round(alg[name] / (ms * 1e-3) / 1e12, 2) if alg[name] else None}
    # The preprocess kernel is HBM-bound: it reads dO, O and lse, and writes D
    # and lse in log2 units.
    pre_bytes = 2 * q.numel() * 2 + lse.numel() * 12
    kernels["attn_bwd_preprocess_kernel"]["gbs"] = round(pre_bytes / (per_kernel[1] * 1e-3) / 1e9, 1)
    dom = max(range(4), key=lambda j: per_kernel[j])
    dom_name = KERNEL_NAMES[dom]
    if alg[dom_name] > 0:
        achieved = alg[dom_name] / (per_kernel[dom] * 1e-3) / 1e12
        roof = {"kernel": dom_name, "bound": "mfma", "achieved": round(achieved, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4)}
    else:
        achieved = pre_bytes / (per_kernel[dom] * 1e-3) / 1e9
        roof = {"kernel": dom_name, "bound": "hbm", "achieved": round(achieved, 1),
                "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4)}
    roof["traffic"] = _traffic_for(dom_name, WORKLOAD)
    fwd_tflops = f_fwd / (per_kernel[0] * 1e-3) / 1e12
    # The same figures against the peak at the clock the chip actually ran.
    clock = {"source": "profiles/clock.json (rocprofv3 counters on these kernel sources)",
             "fwd": _at_clock(fwd_tflops, _clock_for("attn_fwd_kernel", WORKLOAD)),
             "fwd_long": _at_clock(fwd_long_tflops, _clock_for("attn_fwd_kernel", FWD_WORKLOAD))}
    if roof["unit"] == "TFLOP/s":
        clock[dom_name] = _at_clock(roof["achieved"], _clock_for(dom_name, WORKLOAD))

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": WORKLOAD, "B": w.B, "H": w.H, "N": w.N, "d": w.d,
                   "causal": w.causal, "pass": "fwd+bwd"},
        "pct_of_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "fwd": {"tflops": round(fwd_tflops, 2),
                "pct_of_peak": round(100 * fwd_tflops / PEAK_BF16_TFLOPS, 2),
                "ms": round(per_kernel[0], 4)},
        "fwd_long": {"workload": FWD_WORKLOAD, "ms": round(fwd_long_ms, 4),
                     "tflops": round(fwd_long_tflops, 2),
                     "pct_of_peak": round(100 * fwd_long_tflops / PEAK_BF16_TFLOPS, 2)},
        "kernels": kernels,
        "event_ms_per_step": round(step_ms, 4),
        "roofline": roof,
        "clock": clock,
        "csrc_digest": _csrc_digest(),
    }
    print(f"bench: step {ms_per_step:.3f} ms ({value:.1f} TFLOP/s)", file=sys.stderr, flush=True)
    if not args.no_per_config:
        out["forward_per_config"] = per_config_forward(
            attn, W, dev, reuse={WORKLOAD: (q, k, v, None)})
    if not args.no_variants:
        print("bench: variants", file=sys.stderr, flush=True)
        out["variants"] = variant_timings(attn, W, dev)
    if not args.no_unfused:
        print("bench: unfused comparison", file=sys.stderr, flush=True)
        out["unfused_comparison"] = unfused_comparison(attn, W, dev)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(W, {WORKLOAD: inputs}, WORKLOAD)
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
