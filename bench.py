#!/usr/bin/env python3
"""Benchmark of the RoPE-scaled tiled attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload yarn_32k_bf16]

Prints ONE JSON line.  The headline ``value`` is causal prefill TFLOP/s on the
YaRN 32K workload (B=1, 32 query / 8 KV heads, D=128, N=32768, bf16, base
1e4, L=2048, s=16, alpha=1, beta=32); a step is one pass of the prefill path
over that input: the cos/sin table for the 32768 positions, K rotated once
(rope_apply into a scratch buffer), then the fused kernel that rotates q on
load and runs the tiled online softmax (--rotate-k-on-load rotates K inside
the kernel instead).  Inputs are resident in HBM before timing starts.  The
same line carries:

  * ``roofline``: the prefill kernel's algorithmic flops / its mean launch
    time (HIP events on the launch stream; the median and the fastest launch
    beside it) against the bf16 dense MFMA peak,
    plus HBM traffic from committed rocprofv3 counters when they were taken
    on the current kernel source (else null);
  * ``decode``: 128K split-K decode (B=16, GQA 32/8, PI s=16, 64 splits):
    algorithmic bytes / time against the 8 TB/s HBM peak;
  * ``ring``: the 128K NTK prefill as Ring Attention over 8 devices run on
    this GPU (contiguous, zig-zag and striped shards): TFLOP/s of the whole
    ring and each device's share timed alone;
  * ``merge``: attn_merge_states on two fp32 states the size of one 128K
    ring device's query run, against the 8 TB/s HBM peak;
  * ``window``: the same prefill with a 4096-key sliding window and 4 sink
    tokens (flops of the kept pairs only), and its time against full causal;
  * ``half_pairs``: the same prefill with half-split pairs (x_i, x_i+D/2)
    for K's rotation and q's rotation on load, and its time against the
    interleaved pairs of the headline;
  * ``backward``: dq, dk, dv of the same prefill, TFLOP/s of the five
    backward products;
  * ``gqa_8k``: the GQA 8K prefill (B=1, 32/8 heads, D=128, N=8192, base
    5e5, unscaled), same launch, against the bf16 peak;
  * ``cpu_baseline`` (top level for the headline, and inside each leg): the
    fp64 oracle on the host cores, on a bounded sample of that leg's
    workload, run in a pool of single-threaded worker processes before the
    GPU is touched;
  * ``library``: path and SHA-256 of the libsrt.so that was loaded.

FLOPs count only (query, key) pairs the causal mask keeps, 4*D per pair per
query head.  Decode bytes count K and V once plus q, out, lse and the split-K
workspace written and read back.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "causal prefill attn TFLOP/s + 128K decode GB/s, % of MI355X roofline"
PEAK_BF16_TFLOPS = 2516.6       # 256 CU x 2.4 GHz x 4096 flop/clk/CU, dense
PEAK_HBM_GBS = 8000.0
# rocprofv3 counters of the prefill kernel, one file per workload; a file is
# used only for the workload, launch flags and kernel source it was taken on
COUNTER_FILES = {"yarn_32k_bf16": os.path.join(ROOT, "profiles", "prefill_bf16_yarn32k_counters.json"),
                 "gqa_8k_bf16": os.path.join(ROOT, "profiles", "prefill_bf16_gqa8k_counters.json")}
BENCH_ROPE_FLAGS = 1            # the timed launch: q rotated on load, K rotated once by rope_apply
LIB_PATH = os.path.join(ROOT, "scaled_rope_tiled_amd", "libsrt.so")
PREFILL_SRC = os.path.join(ROOT, "scaled_rope_tiled_amd", "csrc", "prefill_bf16.hip")


def causal_pairs(Nq: int, Nk: int, q_pos0: int = 0, k_pos0: int = 0) -> int:
    """Number of (query, key) pairs with k_pos0 + c <= q_pos0 + r (exact integer count)."""
    total = 0
    # row r sees clamp(q_pos0 - k_pos0 + r + 1, 0, Nk) keys
    off = q_pos0 - k_pos0 + 1
    r_lo = max(0, -off)                 # first row with a positive count
    r_full = max(0, Nk - off)           # first row that sees all Nk keys
    a, b = min(r_lo, Nq), min(max(r_full, r_lo), Nq)
    if b > a:                           # ramp rows: off + r keys
        total += (b - a) * off + (a + b - 1) * (b - a) // 2
    if Nq > b:
        total += (Nq - b) * Nk
    return total


def prefill_flops(B, Hq, Nq, Nk, D, q_pos0=0, k_pos0=0, causal=True) -> float:
    pairs = causal_pairs(Nq, Nk, q_pos0, k_pos0) if causal else Nq * Nk
    return 4.0 * D * B * Hq * pairs


def window_pairs(N: int, window: int, sink: int) -> int:
    """(query, key) pairs a causal sliding window of W keys plus S sinks keeps."""
    import numpy as np
    i = np.arange(N, dtype=np.int64)
    return int(np.sum(np.minimum(i + 1, window) + np.minimum(sink, np.maximum(0, i - window + 1))))


def _sha(path: str) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def _ensure_built():
    """Build libsrt.so only when it is absent (a built library is used as is)."""
    if not os.path.exists(LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()


class Timer:
    """HIP events on the current stream around a callable, averaged over calls."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = []

    def run(self, fn):
        t = self.torch
        e0, e1 = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        e0.record()
        r = fn()
        e1.record()
        self.pairs.append((e0, e1))
        return r

    def times_ms(self):
        return sorted(a.elapsed_time(b) for a, b in self.pairs)

    def mean_ms(self):
        return sum(a.elapsed_time(b) for a, b in self.pairs) / max(1, len(self.pairs))

    def median_min_ms(self):
        t = self.times_ms()
        if not t:
            return None, None
        med = t[len(t) // 2] if len(t) % 2 else 0.5 * (t[len(t) // 2 - 1] + t[len(t) // 2])
        return med, t[0]


# ----------------------------------------------------------------------------- prefill (headline)

def bench_prefill(srt, torch, w, steps, warmup, prerotate_k=False):
    import synth
    D = w.D
    q = synth.randn((w.B, w.Hq, w.N, D), torch.bfloat16, w.seed, synth.Q_ID, "cuda")
    k = synth.randn((w.B, w.Hkv, w.N, D), torch.bfloat16, w.seed, synth.K_ID, "cuda")
    v = synth.randn((w.B, w.Hkv, w.N, D), torch.bfloat16, w.seed, synth.V_ID, "cuda")
    rp = w.rope
    th, ms, _ = srt.rope_inv_freq(rp.method, rp.base, rp.s, rp.L, rp.alpha, rp.beta, D)
    out = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.N), dtype=torch.float32, device="cuda")
    table = torch.empty((w.N, D // 2, 2), dtype=torch.float32, device="cuda")
    krot = torch.empty_like(k) if prerotate_k else None
    kt = Timer(torch)

    import ctypes as C
    import numpy as np
    thc = np.ascontiguousarray(th)
    lib = srt.lib()
    stream = torch.cuda.current_stream().cuda_stream

    def step(timed):
        from scaled_rope_tiled_amd import _lib as L
        L.check(lib.srt_rope_cos_sin(thc.ctypes.data_as(C.POINTER(C.c_double)), D, ms, w.N,
                                     C.c_void_p(table.data_ptr()), stream), "rope_cos_sin")
        if prerotate_k:
            srt.rope_apply(k, table, out=krot)
            fn = lambda: srt.attn_prefill(q, krot, v, table=table, rope_flags=srt.ROTATE_Q, out=out, lse=lse)
        else:
            fn = lambda: srt.attn_prefill(q, k, v, table=table, out=out, lse=lse)
        if timed:
            kt.run(fn)
        else:
            fn()

    for _ in range(warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step(True)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / steps
    flops = prefill_flops(w.B, w.Hq, w.N, w.N, D)
    kernel_ms = kt.mean_ms()
    med, mn = kt.median_min_ms()
    return {"flops": flops, "ms_per_step": ms_step, "kernel_ms": kernel_ms, "kernel_ms_median": med,
            "kernel_ms_min": mn,
            "tflops_step": flops / (ms_step * 1e-3) / 1e12, "tflops_kernel": flops / (kernel_ms * 1e-3) / 1e12}


def traffic_from_counters(workload: str, rope_flags: int):
    """HBM bytes per launch and MFMA busy fraction of the prefill kernel from
    committed rocprofv3 counters, if they were taken on this workload, with
    these launch flags, on this kernel source."""
    path = COUNTER_FILES.get(workload)
    if path is None or not os.path.exists(path):
        return None, None, "no counter file for this workload"
    with open(path) as f:
        c = json.load(f)
    if c.get("workload") != workload or c.get("rope_flags") != rope_flags:
        return None, None, "counter file taken on another workload or launch"
    if c.get("source_sha256") != _sha(PREFILL_SRC):
        return None, None, "kernel changed since the counters were taken"
    fetch = c["fetch_kib_per_dispatch"] * 1024.0 * c["fetch_scale"]
    write = c["write_kib_per_dispatch"] * 1024.0 * c["write_scale"]
    return fetch + write, c.get("mfma_util"), "rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated"


# ----------------------------------------------------------------------------- sliding window

def bench_window(srt, torch, w, window, sink, steps, warmup, full_kernel_ms):
    """The prefill workload with a sliding window and sinks: O(N W) work."""
    import synth
    D = w.D
    q = synth.randn((w.B, w.Hq, w.N, D), torch.bfloat16, w.seed, synth.Q_ID, "cuda")
    k = synth.randn((w.B, w.Hkv, w.N, D), torch.bfloat16, w.seed, synth.K_ID, "cuda")
    v = synth.randn((w.B, w.Hkv, w.N, D), torch.bfloat16, w.seed, synth.V_ID, "cuda")
    rp = w.rope
    th, ms, _ = srt.rope_inv_freq(rp.method, rp.base, rp.s, rp.L, rp.alpha, rp.beta, D)
    table = srt.rope_cos_sin(th, D, ms, w.N, "cuda")
    krot = srt.rope_apply(k, table)
    out = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.N), dtype=torch.float32, device="cuda")
    kt = Timer(torch)
    fn = lambda: srt.attn_prefill(q, krot, v, table=table, rope_flags=srt.ROTATE_Q, out=out, lse=lse,
                                  window=window, sink=sink)
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    for _ in range(steps):
        kt.run(fn)
    torch.cuda.synchronize()
    kernel_ms = kt.mean_ms()
    pairs = window_pairs(w.N, window, sink)
    flops = 4.0 * D * w.B * w.Hq * pairs
    tf = flops / (kernel_ms * 1e-3) / 1e12
    return {"workload": f"{w.name} with window {window}, {sink} sinks", "unit": "TFLOP/s", "value": round(tf, 2),
            "kernel_ms": round(kernel_ms, 4), "alg_flops_per_launch": flops,
            "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
            "work_vs_full_causal": round(pairs / causal_pairs(w.N, w.N), 4),
            "time_vs_full_causal": round(kernel_ms / full_kernel_ms, 4) if full_kernel_ms else None}


def bench_half_pairs(srt, torch, w, steps, warmup, full_kernel_ms):
    """The prefill workload with half-split pairs (x_i, x_i+D/2): K rotated once with that pairing and q
    rotated on load with it.  The other frequency-step variants (Dynamic NTK, per-pair factor tables) only
    change the host-built table, not what the kernels do."""
    import synth
    D = w.D
    q = synth.randn((w.B, w.Hq, w.N, D), torch.bfloat16, w.seed, synth.Q_ID, "cuda")
    k = synth.randn((w.B, w.Hkv, w.N, D), torch.bfloat16, w.seed, synth.K_ID, "cuda")
    v = synth.randn((w.B, w.Hkv, w.N, D), torch.bfloat16, w.seed, synth.V_ID, "cuda")
    rp = w.rope
    th, ms, _ = srt.rope_inv_freq(rp.method, rp.base, rp.s, rp.L, rp.alpha, rp.beta, D)
    table = srt.rope_cos_sin(th, D, ms, w.N, "cuda")
    krot = srt.rope_apply(k, table, pairing="half")
    out = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.N), dtype=torch.float32, device="cuda")
    kt = Timer(torch)
    fn = lambda: srt.attn_prefill(q, krot, v, table=table, rope_flags=srt.ROTATE_Q | srt.PAIR_HALF, out=out,
                                  lse=lse)
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    for _ in range(steps):
        kt.run(fn)
    torch.cuda.synchronize()
    kernel_ms = kt.mean_ms()
    flops = 4.0 * D * w.B * w.Hq * causal_pairs(w.N, w.N)
    tf = flops / (kernel_ms * 1e-3) / 1e12
    return {"workload": f"{w.name} with half-split pairs", "unit": "TFLOP/s", "value": round(tf, 2),
            "kernel_ms": round(kernel_ms, 4), "alg_flops_per_launch": flops,
            "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
            "time_vs_interleaved": round(kernel_ms / full_kernel_ms, 4) if full_kernel_ms else None}


# ----------------------------------------------------------------------------- backward

def bench_backward(srt, torch, w, steps, warmup):
    """Gradients of the prefill workload (dq, dk, dv from out, lse and dO):
    delta, dk/dv and dq launches.  Algorithmic flops: the five products of
    the backward pass (S, dP, dV, dK, dQ), 10 D per kept pair per query head;
    the kernels recompute S and dP in both the dk/dv and the dq kernel (14 D).
    The timed call includes rotating q and k once into the workspace."""
    import synth
    D = w.D
    q = synth.randn((w.B, w.Hq, w.N, D), torch.bfloat16, w.seed, synth.Q_ID, "cuda")
    k = synth.randn((w.B, w.Hkv, w.N, D), torch.bfloat16, w.seed, synth.K_ID, "cuda")
    v = synth.randn((w.B, w.Hkv, w.N, D), torch.bfloat16, w.seed, synth.V_ID, "cuda")
    do = synth.randn((w.B, w.Hq, w.N, D), torch.bfloat16, w.seed, synth.DO_ID, "cuda")
    rp = w.rope
    th, ms, _ = srt.rope_inv_freq(rp.method, rp.base, rp.s, rp.L, rp.alpha, rp.beta, D)
    table = srt.rope_cos_sin(th, D, ms, w.N, "cuda")
    out, lse = srt.attn_prefill(q, k, v, table=table)
    dq = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    dk = torch.empty(k.shape, dtype=torch.float32, device="cuda")
    dv = torch.empty(v.shape, dtype=torch.float32, device="cuda")
    ws = torch.empty(srt.attn_backward_workspace_size(torch.bfloat16, w.B, w.Hq, w.Hkv, w.N, w.N, D,
                                                      srt.ROTATE_Q | srt.ROTATE_K), dtype=torch.uint8, device="cuda")
    fn = lambda: srt.attn_backward(q, k, v, out, do, lse, table=table, workspace=ws, dq=dq, dk=dk, dv=dv)
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    kt = Timer(torch)
    for _ in range(steps):
        kt.run(fn)
    torch.cuda.synchronize()
    ms_ = kt.mean_ms()
    flops = 2.5 * prefill_flops(w.B, w.Hq, w.N, w.N, D)
    tf = flops / (ms_ * 1e-3) / 1e12
    return {"workload": f"{w.name} backward (dq, dk, dv)", "unit": "TFLOP/s", "value": round(tf, 2),
            "ms_per_step": round(ms_, 4), "alg_flops_per_step": flops,
            "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
            "note": "three launches (delta, dk/dv, dq) timed together with HIP events; 10 D flops per kept pair"}


# ----------------------------------------------------------------------------- decode

def bench_decode(srt, torch, w, steps, warmup):
    import synth
    D = w.D
    N = w.N
    q = synth.randn((w.B, w.Hq, D), torch.bfloat16, w.seed, synth.Q_ID, "cuda")
    k = synth.randn((w.B, w.Hkv, N, D), torch.bfloat16, w.seed, synth.K_ID, "cuda")
    v = synth.randn((w.B, w.Hkv, N, D), torch.bfloat16, w.seed, synth.V_ID, "cuda")
    rp = w.rope
    th, ms, _ = srt.rope_inv_freq(rp.method, rp.base, rp.s, rp.L, rp.alpha, rp.beta, D)
    table = srt.rope_cos_sin(th, D, ms, N, "cuda")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    srt.rope_apply(k, table, out=k)                 # rotated cache, in place (setup, not timed in the step)
    torch.cuda.synchronize()
    cache_ms = (time.perf_counter() - t0) * 1e3
    ws = torch.empty(srt.attn_decode_workspace_size(w.B, w.Hq, D, w.splits), dtype=torch.uint8, device="cuda")
    out = torch.empty((w.B, w.Hq, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.B, w.Hq), dtype=torch.float32, device="cuda")
    kt = Timer(torch)
    fn = lambda: srt.attn_decode_splitk(q, k, v, num_splits=w.splits, table=table, workspace=ws, out=out, lse=lse)
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        kt.run(fn)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / steps
    kv = 2.0 * w.B * w.Hkv * N * D * 2
    ws_bytes = w.B * w.Hq * w.splits * (D + 1) * 4.0
    alg = kv + w.B * w.Hq * D * 2 * 2 + w.B * w.Hq * 4 + 2 * ws_bytes
    kernel_ms = kt.mean_ms()
    med, mn = kt.median_min_ms()
    gbs = alg / (kernel_ms * 1e-3) / 1e9
    del k, v
    return {"workload": w.name, "unit": "GB/s", "value": round(gbs, 1), "ms_per_step": round(ms_step, 4),
            "kernel_ms": round(kernel_ms, 4), "kernel_ms_median": round(med, 4), "kernel_ms_min": round(mn, 4),
            "alg_bytes": alg,
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4)},
            "cache_build_ms": round(cache_ms, 3)}


# ----------------------------------------------------------------------------- merge

def bench_merge(srt, torch, w, steps, warmup):
    """attn_merge_states on two fp32 partial states of one 128K ring device's
    query run (B=1, 32 heads, C = N / chunks rows, D=128), in place into the
    first, as a separate ring step would merge them.  HBM-bound: per row it
    reads two D-vectors and two lse values and writes one D-vector and one
    lse (algorithmic bytes)."""
    import synth
    C = w.N // w.chunks
    shape = (w.B, w.Hq, C, w.D)
    oa = synth.randn(shape, torch.float32, w.seed, synth.Q_ID, "cuda")
    ob = synth.randn(shape, torch.float32, w.seed, synth.K_ID, "cuda")
    la = synth.randn(shape[:3], torch.float32, w.seed, synth.V_ID, "cuda")
    lb = synth.randn(shape[:3], torch.float32, w.seed, synth.DO_ID, "cuda")
    fn = lambda: srt.attn_merge_states(oa, la, ob, lb, out=oa, lse_out=la)
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    kt = Timer(torch)
    for _ in range(steps):
        kt.run(fn)
    torch.cuda.synchronize()
    ms_ = kt.mean_ms()
    rows = w.B * w.Hq * C
    alg = rows * (3 * w.D * 4 + 3 * 4)
    gbs = alg / (ms_ * 1e-3) / 1e9
    return {"workload": f"attn_merge_states, two fp32 states of {w.Hq} heads x {C} rows x {w.D}", "unit": "GB/s",
            "value": round(gbs, 1), "kernel_ms": round(ms_, 4), "alg_bytes": alg,
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4)}}


# ----------------------------------------------------------------------------- ring step on one GPU

def bench_ring(srt, torch, w, steps, warmup):
    """One device's ring step, for all P = w.chunks devices of a ring, run on
    this GPU with srt_attn_ring_prefill (K rotated once into the workspace, q
    on load); once per partition.  The whole ring gives the job's TFLOP/s;
    each device's share, timed alone, gives the per-device balance (the step
    time of a real P-GPU ring is its slowest device, transfers aside)."""
    import numpy as np
    import synth
    D, N, P = w.D, w.N, w.chunks
    q = synth.randn((w.B, w.Hq, N, D), torch.bfloat16, w.seed, synth.Q_ID, "cuda")
    k = synth.randn((w.B, w.Hkv, N, D), torch.bfloat16, w.seed, synth.K_ID, "cuda")
    v = synth.randn((w.B, w.Hkv, N, D), torch.bfloat16, w.seed, synth.V_ID, "cuda")
    rp = w.rope
    th, ms, _ = srt.rope_inv_freq(rp.method, rp.base, rp.s, rp.L, rp.alpha, rp.beta, D)
    flops = prefill_flops(w.B, w.Hq, N, N, D)
    out = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, N), dtype=torch.float32, device="cuda")
    res = {}
    for part in ("contiguous", "zigzag", "striped"):
        if part == "contiguous":
            qs, ks, vs = q, k, v
        else:
            C = N // P
            if part == "striped":
                pos = (np.arange(P)[:, None] + P * np.arange(C)[None, :]).reshape(-1)
            else:
                h = C // 2
                pos = np.concatenate([np.concatenate([r * h + np.arange(h), (2 * P - 1 - r) * h + np.arange(h)])
                                      for r in range(P)])
            ip = torch.from_numpy(pos).cuda()
            qs, ks, vs = (t.index_select(2, ip).contiguous() for t in (q, k, v))
        ws = torch.empty(srt.attn_ring_workspace_size(w.B, w.Hq, w.Hkv, N, D, torch.bfloat16, P, part),
                         dtype=torch.uint8, device="cuda")

        def ring(device=-1):
            table = srt.rope_cos_sin(th, D, ms, N, "cuda")
            srt.attn_ring_prefill(qs, ks, vs, num_devices=P, partition=part, device=device, table=table,
                                  workspace=ws, out=out, lse=lse)

        for _ in range(warmup):
            ring()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            ring()
        torch.cuda.synchronize()
        ms_step = (time.perf_counter() - t0) * 1e3 / steps
        dev_ms = []
        for r in range(P):
            t = Timer(torch)
            for _ in range(2):
                t.run(lambda: ring(r))
            torch.cuda.synchronize()
            dev_ms.append(t.mean_ms())
        tf = flops / (ms_step * 1e-3) / 1e12
        res[part] = {"ms_per_step": round(ms_step, 3), "tflops": round(tf, 2),
                     "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                     "device_ms": [round(x, 3) for x in dev_ms],
                     "slowest_device_ms": round(max(dev_ms), 3),
                     "slowest_over_mean": round(max(dev_ms) / (sum(dev_ms) / P), 3)}
        if part != "contiguous":
            del qs, ks, vs
        del ws
        torch.cuda.empty_cache()
    c = res["contiguous"]
    return {"workload": w.name, "unit": "TFLOP/s", "value": c["tflops"], "ms_per_step": c["ms_per_step"],
            "devices": P, "frac_of_bf16_peak": c["frac_of_bf16_peak"], "partitions": res,
            "note": "all devices' shares run on this GPU; device_ms times each share alone (compute only)"}


# ----------------------------------------------------------------------------- CPU baseline (oracle)
#
# The oracle (fp64 numpy, unchanged) timed on the host cores, in a pool of
# single-threaded worker processes, one (query-row block, KV group) or one
# decode (sequence, KV group) per task.  Each task draws its own N(0,1) inputs
# (fp64; values differ from the GPU draw, and the oracle's time does not
# depend on them) and times only the oracle call.  The rate is the work done
# over the workers' busy time shared among them: work / (sum of task times /
# workers).  The pool is started from a process that has not touched the GPU
# and is shut down before any GPU work.

def _oracle_worker_init(*_):
    """One BLAS thread per worker process (set before numpy is first imported)."""
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS", "BLIS_NUM_THREADS"):
        os.environ[var] = "1"
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:
        pass


def _oracle_rows_task(t):
    """Query rows [r0, r1) of G heads of one KV group, each against all its
    visible keys (keys [0, r1), causal)."""
    import numpy as np
    from oracle import attention as OA
    seed, D, G, r0, r1, theta, mscale, sm = t
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((1, 1, r1, D))
    v = rng.standard_normal((1, 1, r1, D))
    q = rng.standard_normal((1, G, r1 - r0, D))
    t0 = time.perf_counter()
    OA.attention(q, k, v, sm_scale=sm, causal=True, q_pos0=r0, k_pos0=0, theta=theta, mscale=mscale)
    dt = time.perf_counter() - t0
    pairs = G * ((r0 + 1 + r1) * (r1 - r0) // 2)
    return dt, 4.0 * D * pairs, G * (r1 - r0)


def _oracle_decode_task(t):
    """One sequence's query heads of one KV group against its whole rotated cache."""
    import numpy as np
    from oracle import attention as OA
    seed, N, D, G, theta, mscale, sm = t
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((1, 1, N, D))
    v = rng.standard_normal((1, 1, N, D))
    q = rng.standard_normal((1, G, D))
    t0 = time.perf_counter()
    OA.decode(q, k, v, sm_scale=sm, theta=theta, mscale=mscale)
    dt = time.perf_counter() - t0
    return dt, 2.0 * N * D * 2, 1          # bytes: the group's bf16 K and V rows, read once


def _run_pool(pool, workers, tasks, fn, budget_s):
    """Run tasks (in the given order) with `workers` in flight until the time
    budget is spent; returns (busy seconds, work, units, tasks done, wall)."""
    import concurrent.futures as cf
    t0 = time.perf_counter()
    it = iter(tasks)
    inflight = set()
    busy = work = units = 0.0
    done = 0
    for _ in range(workers):
        t = next(it, None)
        if t is None:
            break
        inflight.add(pool.submit(fn, t))
    while inflight:
        fin, inflight = cf.wait(inflight, return_when=cf.FIRST_COMPLETED)
        for f in fin:
            dt, wk, un = f.result()
            busy += dt
            work += wk
            units += un
            done += 1
            if time.perf_counter() - t0 < budget_s:
                t = next(it, None)
                if t is not None:
                    inflight.add(pool.submit(fn, t))
    return busy, work, units, done, time.perf_counter() - t0


def _row_block_tasks(w, th, ms, block, seed):
    """Row blocks of one KV group spread evenly over the whole sequence, in a
    seeded random order, so that a budget cut keeps the row-length mix."""
    import numpy as np
    G = w.Hq // w.Hkv
    starts = np.arange(0, w.N, block)
    order = np.random.default_rng(seed).permutation(len(starts))
    return [(seed * 7919 + int(i), w.D, G, int(starts[i]), int(min(w.N, starts[i] + block)), th, ms, w.sm_scale)
            for i in order]


def cpu_baselines(legs, budget_s):
    """Oracle rates of the prefill, ring and decode legs, in one worker pool."""
    import concurrent.futures as cf
    import multiprocessing as mp
    import numpy as np
    import synth
    from oracle import rope as OR
    from oracle import attention as OA
    workers = max(1, min(16, os.cpu_count() or 1))
    res = {}
    ctx = mp.get_context("spawn")
    with cf.ProcessPoolExecutor(max_workers=workers, mp_context=ctx, initializer=_oracle_worker_init) as pool:
        # start the workers (interpreter start-up is not the oracle's time)
        list(pool.map(_oracle_worker_init, range(workers)))
        for leg, (wname, share) in legs.items():
            w = synth.WORKLOADS[wname]
            rp = w.rope
            th, ms, _ = OR.inv_freq(rp.method, rp.base, rp.s, rp.L, rp.alpha, rp.beta, w.D)
            b = budget_s * share
            G = w.Hq // w.Hkv
            if w.kind == "decode":
                tasks = [(w.seed * 7919 + i, w.N, w.D, G, th, ms, w.sm_scale) for i in range(w.B * w.Hkv)]
                busy, work, units, done, wall = _run_pool(pool, workers, tasks, _oracle_decode_task, b)
                rate = work / (busy / workers) / 1e9
                total = 2.0 * w.B * w.Hkv * w.N * w.D * 2
                res[leg] = {"value": round(rate, 4), "unit": "GB/s", "cores": workers, "kind": "oracle",
                            "sample": f"{int(done)} of the {w.B * w.Hkv} (sequence, KV group) decode problems of "
                                      f"{w.name} ({G} query heads against {w.N} cached keys each), fp64 numpy, "
                                      f"{workers} single-threaded worker processes, {wall:.1f} s wall",
                            "full_config_s_extrapolated": round(total / (rate * 1e9), 2)}
            else:
                tasks = _row_block_tasks(w, th, ms, 256, w.seed)
                busy, work, units, done, wall = _run_pool(pool, workers, tasks, _oracle_rows_task, b)
                rate = work / (busy / workers) / 1e12
                total = 4.0 * w.D * w.B * w.Hq * (w.N * (w.N + 1) // 2)
                res[leg] = {"value": round(rate, 6), "unit": "TFLOP/s", "cores": workers, "kind": "oracle",
                            "sample": f"{int(units)} query rows ({int(done)} blocks of 256 rows x {G} heads of one "
                                      f"KV group, spread over all {w.N} positions, each row against all its "
                                      f"visible keys) of {w.name}, fp64 numpy, {workers} single-threaded worker "
                                      f"processes, {wall:.1f} s wall",
                            "full_config_s_extrapolated": round(total / (rate * 1e12), 1)}
    return res


# ----------------------------------------------------------------------------- copy calibration

def copy_calibration(torch, nbytes: int, reps: int):
    """A plain device copy of known size, for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE."""
    x = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    y = torch.empty_like(x)
    for _ in range(reps):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "reps": reps}))


def prefill_leg(p, w, traffic=None, mfma_util=None, traffic_note=None):
    """Roofline fields of one prefill measurement (kernel time from HIP events)."""
    return {"bound": "mfma", "achieved": round(p["tflops_kernel"], 2), "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": round(p["tflops_kernel"] / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic, "traffic_note": traffic_note,
            "mfma_busy_from_counters": None if mfma_util is None else round(mfma_util, 4),
            "kernel": "prefill_bf16_kernel", "kernel_ms": round(p["kernel_ms"], 4),
            "kernel_ms_median": round(p["kernel_ms_median"], 4), "kernel_ms_min": round(p["kernel_ms_min"], 4),
            "alg_flops_per_launch": p["flops"]}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="yarn_32k_bf16", choices=["gqa_8k_bf16", "yarn_32k_bf16"])
    ap.add_argument("--rotate-k-on-load", action="store_true",
                    help="rotate K inside the prefill kernel at every tile load (default: once, with rope_apply)")
    ap.add_argument("--no-extras", action="store_true", help="skip the decode, ring, window, backward and 8K legs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=24.0,
                    help="seconds of oracle time over all legs (split among them)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES")
    ap.add_argument("--only", choices=["decode", "ring", "window", "half_pairs", "backward", "gqa_8k", "merge"],
                    default=None,
                    help="run one extra leg alone and print its JSON (for profiling that leg's kernels)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(json.dumps({"error": "this benchmark runs on one GPU; --gpus must be 1 (the multi-GPU ring is "
                                   "not built: its per-device share is the ring leg's device_ms)"}))
        sys.exit(2)
    if "SRT_LIB" in os.environ:
        print(json.dumps({"error": "SRT_LIB is set: the benchmark measures only the in-tree library "
                                   "scaled_rope_tiled_amd/libsrt.so"}))
        sys.exit(2)

    # oracle baselines first: their worker processes start before this process touches the GPU
    cpu = {}
    if not args.no_cpu_baseline and not args.only and not args.copy_calibration:
        legs = {"headline": (args.workload, 0.3)}
        if not args.no_extras:
            legs.update({"gqa_8k": ("gqa_8k_bf16", 0.2), "ring": ("ntk_128k_ring_bf16", 0.25),
                         "decode": ("decode_128k_bf16", 0.25)})
            if args.workload == "gqa_8k_bf16":
                del legs["gqa_8k"]
        cpu = cpu_baselines(legs, args.cpu_budget)

    import torch
    if args.copy_calibration:
        copy_calibration(torch, args.copy_calibration, 5)
        return
    _ensure_built()
    import scaled_rope_tiled_amd as srt
    from scaled_rope_tiled_amd import _lib
    import synth
    library = {"path": os.path.relpath(_lib.LIB_PATH, ROOT), "sha256": _sha(_lib.LIB_PATH)}

    w = synth.WORKLOADS[args.workload]
    if args.only:
        if args.only == "decode":
            r = bench_decode(srt, torch, synth.WORKLOADS["decode_128k_bf16"], args.steps, args.warmup)
        elif args.only == "ring":
            r = bench_ring(srt, torch, synth.WORKLOADS["ntk_128k_ring_bf16"], args.steps, args.warmup)
        elif args.only == "window":
            r = bench_window(srt, torch, w, 4096, 4, args.steps, args.warmup, None)
        elif args.only == "half_pairs":
            r = bench_half_pairs(srt, torch, w, args.steps, args.warmup, None)
        elif args.only == "merge":
            r = bench_merge(srt, torch, synth.WORKLOADS["ntk_128k_ring_bf16"], args.steps, args.warmup)
        elif args.only == "gqa_8k":
            w8 = synth.WORKLOADS["gqa_8k_bf16"]
            r = prefill_leg(bench_prefill(srt, torch, w8, args.steps, args.warmup, True), w8)
        else:
            r = bench_backward(srt, torch, w, args.steps, args.warmup)
        print(json.dumps({args.only: r, "library": library}), flush=True)
        return
    p = bench_prefill(srt, torch, w, args.steps, args.warmup, not args.rotate_k_on_load)
    flags = 3 if args.rotate_k_on_load else BENCH_ROPE_FLAGS
    roof = prefill_leg(p, w, *traffic_from_counters(w.name, flags))
    line = {"metric": METRIC, "value": round(p["tflops_step"], 2), "unit": "TFLOP/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(p["ms_per_step"], 4),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic",
            "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "N": w.N, "D": w.D,
                       "causal": True, "rope": w.note, "step": ("cos/sin table + prefill rotating q and k on load"
                                                               if args.rotate_k_on_load else
                                                               "cos/sin table + rope_apply(k) + prefill rotating q on load")},
            "roofline": roof}
    if not args.no_extras:
        if args.workload != "gqa_8k_bf16":
            torch.cuda.empty_cache()
            w8 = synth.WORKLOADS["gqa_8k_bf16"]
            p8 = bench_prefill(srt, torch, w8, 5 * args.steps, args.warmup, True)
            line["gqa_8k"] = {"workload": w8.name, "unit": "TFLOP/s", "value": round(p8["tflops_kernel"], 2),
                              "ms_per_step": round(p8["ms_per_step"], 4),
                              "roofline": prefill_leg(p8, w8, *traffic_from_counters(w8.name, BENCH_ROPE_FLAGS))}
            if "gqa_8k" in cpu:
                line["gqa_8k"]["cpu_baseline"] = cpu["gqa_8k"]
        torch.cuda.empty_cache()
        line["decode"] = bench_decode(srt, torch, synth.WORKLOADS["decode_128k_bf16"], max(5, args.steps), args.warmup)
        if "decode" in cpu:
            line["decode"]["cpu_baseline"] = cpu["decode"]
        torch.cuda.empty_cache()
        line["ring"] = bench_ring(srt, torch, synth.WORKLOADS["ntk_128k_ring_bf16"], max(2, args.steps // 5), 1)
        if "ring" in cpu:
            line["ring"]["cpu_baseline"] = cpu["ring"]
        torch.cuda.empty_cache()
        line["merge"] = bench_merge(srt, torch, synth.WORKLOADS["ntk_128k_ring_bf16"], args.steps, args.warmup)
        torch.cuda.empty_cache()
        line["window"] = bench_window(srt, torch, w, 4096, 4, args.steps, args.warmup, p["kernel_ms"])
        torch.cuda.empty_cache()
        line["half_pairs"] = bench_half_pairs(srt, torch, w, args.steps, args.warmup, p["kernel_ms"])
        torch.cuda.empty_cache()
        line["backward"] = bench_backward(srt, torch, w, max(3, args.steps // 4), 1)
        torch.cuda.empty_cache()
    if "headline" in cpu:
        line["cpu_baseline"] = cpu["headline"]
    line["library"] = library
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
