#!/usr/bin/env python3
"""Benchmark of the fused quantize -> int8 GEMM -> dequant linear layer on one MI355X.

One step = one pass of the hot path over one batch: per-token activation
quantization (fp16 x -> int8 x_q + fp32 s_x) followed by the int8 GEMM with the
per-channel dequantization fused into its store (fp16 y). Default workload: M=4096
tokens, N=10240 output channels, K=2560 input channels, seeded synthetic inputs
(weights quantized once, offline, outside the timed region). Inputs are resident in HBM
before timing starts. For M <= 16 the step is one w8a8_linear call (quantization inside
the GEMV kernel); for M <= 128 the weights rotate over copies totalling more than
512 MB, so that no step finds them in the 256 MB Infinity Cache.

Prints ONE JSON line: metric/value (INT8 TOPS = 2*M*N*K / step time), a roofline
object for the dominant kernel (the GEMM; its launch duration is timed with HIP events
on its stream around as many back-to-back launches as there are timed steps, right after
them, with no event between launches) and a cpu_baseline object (the CPU oracle timed on a bounded
sample of the same workload on the host cores).

The defaults (1000 warmup steps, 2000 timed steps: about 0.3 s of GEMM work at the
headline) time the chip in its steady state under load. Over the first few ms of load the
same graph runs up to 20 % slower per step (clocks still ramping), so a short run measures
that transient rather than the kernels.

Usage: python bench.py [--gpus 1] [--steps 2000] [--warmup 1000] [--no-cpu-baseline]
       [--workload pc|pg64|pg128|w4|w4pc|m1|m1w4|m1w4pc|qwen3|mv|mvg128|sdpa|rmsnorm] [--copy-ref-mb MB]
       [--no-graph] [--no-m1]

roofline.traffic (HBM bytes per GEMM launch) comes from the rocprofv3 FETCH_SIZE and
WRITE_SIZE summary committed under profiles/ for this workload, scaled by the same
counters measured on a plain copy of known size; it is reported only while the kernel's
source file (named in the summary) still has the hash recorded there, else null.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

PEAK_INT8_TOPS = 5000.0  # MI355X dense INT8 MFMA, 5.0 POP/s
PEAK_HBM_GBS = 8000.0    # MI355X HBM3E, 8 TB/s
ROOT = os.path.dirname(os.path.abspath(__file__))

# name -> (M, N, K, weight bits, group size)
WORKLOADS = {
    "pc": (4096, 10240, 2560, 8, 0),
    "pg128": (4096, 10240, 2560, 8, 128),
    "pg64": (4096, 10240, 2560, 8, 64),
    "w4": (4096, 10240, 2560, 4, 128),
    "m1": (1, 10240, 2560, 8, 0),
    "m1w4": (1, 10240, 2560, 4, 128),
    "w4pc": (4096, 10240, 2560, 4, 0),
    "m1w4pc": (1, 10240, 2560, 4, 0),
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=1000)
    ap.add_argument("--workload", default="pc", choices=sorted(WORKLOADS) + ["qwen3", "mv", "mvg128", "sdpa", "rmsnorm"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-m1", action="store_true", help="leave the fused M=1 results out of the default line")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="time budget of the CPU-oracle sample")
    ap.add_argument("--copy-ref-mb", type=int, default=0,
                    help="first run one plain device copy of this many MiB (a counter reference)")
    ap.add_argument("--no-graph", action="store_true",
                    help="issue the steps one by one instead of as a graph replay (for counter "
                         "collection; the timing then includes the host's issue time)")
    return ap.parse_args()


def source_sha(rel_paths):
    """sha256 of the named source files' bytes, concatenated in order ('a+b+c': a kernel's
    translation unit and the local headers it includes)."""
    h = hashlib.sha256()
    for rel in rel_paths.split("+"):
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload):
    """HBM bytes per launch of the dominant kernel from the committed counter summary, if the
    kernel's source files still have the hash recorded there."""
    path = os.path.join(ROOT, "profiles", f"traffic_gemm_{workload}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    fields = dict(re.findall(r"^\s*-?\s*(\w+)\s*=\s*(\S+)\s*$", text, flags=re.M))
    src = fields.get("kernel_source")
    if not src or not all(os.path.exists(os.path.join(ROOT, p)) for p in src.split("+")):
        return None
    if fields.get("kernel_source_sha256") != source_sha(src):
        return None
    try:
        return float(fields["fetch_bytes_per_launch"]) + float(fields["write_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(x, W, bits, gs, budget_s):
    """Time the CPU oracle on a bounded row sample of the same workload."""
    import oracle

    oracle.build(force=False)
    N, K = W.shape
    if bits == 8:
        wq, sw = oracle.quantize_weight(W, 8, gs)
    else:
        wq, sw = oracle.quantize_weight(W, 4, gs)
    rows_done, chunk = 0, 64
    t0 = time.perf_counter()
    while rows_done < x.shape[0]:
        xs = x[rows_done:rows_done + chunk]
        if bits == 4:
            oracle.linear_w4(xs, wq, sw, gs)
        elif gs:
            oracle.linear_pg(xs, wq, sw, gs)
        else:
            oracle.linear_pc(xs, wq, sw)
        rows_done += xs.shape[0]
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    ops = 2.0 * rows_done * N * K
    return {"value": ops / dt / 1e12, "unit": "TOPS", "cores": _omp_threads(), "kind": "oracle",
            "host": _cpu_model(),
            "sample": f"first {rows_done} of {x.shape[0]} token rows (full N={N}, K={K}); "
                      f"per-token quantize + int GEMM + fp64 dequant; {dt:.2f} s"}


def _gomp():
    """The OpenMP runtime the oracle library links (gcc's libgomp), or None."""
    import ctypes
    try:
        return ctypes.CDLL("libgomp.so.1")
    except OSError:
        return None


def _omp_threads():
    g = _gomp()
    if g is not None:
        return int(g.omp_get_max_threads())
    return int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_single_thread():
    """The oracle on one thread, on the small per-channel workload (M=128, N=10240, K=2560)."""
    import oracle
    from synth_inputs import linear_inputs

    g = _gomp()
    if g is None:
        return None
    M, N, K = 128, 10240, 2560
    x, W = linear_inputs(M, N, K, seed=0)
    oracle.build(force=False)
    wq, sw = oracle.quantize_weight(W, 8, 0)
    before = int(g.omp_get_max_threads())
    g.omp_set_num_threads(1)
    try:
        t0 = time.perf_counter()
        oracle.linear_pc(x, wq, sw)
        dt = time.perf_counter() - t0
    finally:
        g.omp_set_num_threads(before)
    return {"value": 2.0 * M * N * K / dt / 1e12, "unit": "TOPS", "cores": 1,
            "sample": f"M={M} N={N} K={K} per channel, whole; {dt:.2f} s"}


def mv_decode(args, torch, w8a8, gs):
    """The decode path without activation quantization (int8_mv) at M=1, N=10240, K=2560:
    one step is one int8_mv call on fp16 activations, weights streamed from HBM (rotated over
    copies larger than the Infinity Cache)."""
    import oracle
    from synth_inputs import linear_inputs

    M, N, K = 1, 10240, 2560
    x_np, W_np = linear_inputs(M, N, K, seed=0)
    x = torch.from_numpy(x_np).cuda()
    wq, sw = w8a8.quantize_weight(torch.from_numpy(W_np).cuda(), 8, gs)  # offline: not timed
    wbytes = wq.numel()
    copies = [wq] + [wq.clone() for _ in range((512 << 20) // wbytes)]
    y = torch.empty((M, N), dtype=torch.float16, device="cuda")

    def step(i):
        w8a8.int8_mv(x, copies[i % len(copies)], sw, gs, y=y, stream=torch.cuda.current_stream())

    for i in range(len(copies)):
        step(i)
    ms_per_step, event_ms = timed_steps(args, torch, step)
    kernel_ms = event_ms if event_ms is not None else ms_per_step
    ops = 2.0 * M * N * K
    alg_bytes = wbytes + sw.numel() * 4 + M * K * 2 + M * N * 2  # weights + scales, x in, y out
    achieved = alg_bytes / (kernel_ms * 1e-3) / 1e9
    result = {
        "metric": f"decode matrix-vector (int8 weights x fp16 activations, no activation quantization), "
                  f"M={M} N={N} K={K}",
        "value": ops / (ms_per_step * 1e-3) / 1e12, "unit": "TOPS", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"int8_mv ({args.workload}): weights dequantized on the fly, fp32 products and sums",
                   "M": M, "N": N, "K": K, "weight_bits": 8, "group_size": gs, "out": "fp16",
                   "parallelism": "single GPU"},
        "step_event_ms": event_ms, "weight_copies": len(copies),
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": measured_traffic(args.workload),
                     "kernel": "int8_mv (mv_kernel)", "launch_ms": kernel_ms, "alg_bytes": alg_bytes},
    }
    if not args.no_cpu_baseline:
        oracle.build(force=False)
        owq, osw = oracle.quantize_weight(W_np, 8, gs)
        reps, t0 = 0, time.perf_counter()
        while reps == 0 or time.perf_counter() - t0 < min(args.cpu_seconds, 2.0):
            oracle.linear_mv(x_np, owq, osw, gs)
            reps += 1
        dt = time.perf_counter() - t0
        cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
        result["cpu_baseline"] = {"value": reps * ops / dt / 1e12, "unit": "TOPS", "cores": cores, "kind": "oracle",
                                  "sample": f"{reps} full calls (M=1, N={N}, K={K}); fp64 sum of x * q * s; "
                                            f"{dt:.2f} s"}
    return result


def sdpa_bench(args, torch, w8a8):
    """Decode-step attention (sdpa_decode) for GQA8 (32 query heads over 4 KV heads), D = 128, a
    32768-token fp16 cache, batch 1: one step is one call; the cache (67 MB) is read once per
    step, so the roofline is HBM."""
    import oracle

    B, Hq, Hkv, N, D = 1, 32, 4, 32768, 128
    rng = np.random.default_rng(0)
    q = (rng.standard_normal((B, Hq, D)) * 1.5).astype(np.float16)
    k = rng.standard_normal((B, Hkv, N, D)).astype(np.float16)
    v = rng.standard_normal((B, Hkv, N, D)).astype(np.float16)
    qd, kd, vd = (torch.from_numpy(a).cuda() for a in (q, k, v))
    ws = torch.empty(max(w8a8.sdpa_decode_workspace(B, Hq, Hkv, N, D), 16) // 4, dtype=torch.int32, device="cuda")
    o = torch.empty((B, Hq, D), dtype=torch.float16, device="cuda")

    # the pages' AutoTune: time the candidate slice counts once, then every step uses the fastest
    tuned = w8a8.sdpa_decode_autotune(qd, kd, vd, o=o, workspace=ws)

    def step(i):
        w8a8.sdpa_decode(qd, kd, vd, o=o, workspace=ws, stream=torch.cuda.current_stream())

    ms_per_step, event_ms = timed_steps(args, torch, step)
    kernel_ms = event_ms if event_ms is not None else ms_per_step
    alg_bytes = 2 * B * Hkv * N * D * 2 + 2 * B * Hq * D * 2  # K and V once, q in, o out
    achieved = alg_bytes / (kernel_ms * 1e-3) / 1e9
    result = {
        "metric": f"decode attention (sdpa_decode), GQA {Hq}/{Hkv} heads, D={D}, N={N} fp16 cache, batch {B}",
        "value": alg_bytes / (ms_per_step * 1e-3) / 1e9, "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "sdpa_decode: one query token per head, grouped KV heads, split-KV + merge",
                   "B": B, "Hq": Hq, "Hkv": Hkv, "N": N, "D": D, "in": "fp16", "out": "fp16",
                   "slices_per_kv_head": tuned, "parallelism": "single GPU"},
        "step_event_ms": event_ms,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": measured_traffic(args.workload),
                     "kernel": "sdpa_kernel + sdpa_combine_kernel", "launch_ms": kernel_ms, "alg_bytes": alg_bytes},
    }
    if not args.no_cpu_baseline:
        oracle.build(force=False)
        heads, t0 = 0, time.perf_counter()
        while heads < Hq and time.perf_counter() - t0 < min(args.cpu_seconds, 5.0):
            # query heads of one KV head at a time (each reads that KV head's cache once)
            g = Hq // Hkv
            kv = heads // g
            oracle.sdpa_decode(q[:, heads:heads + g], k[:, kv:kv + 1], v[:, kv:kv + 1])
            heads += g
        dt = time.perf_counter() - t0
        cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
        done = alg_bytes * heads / Hq
        result["cpu_baseline"] = {"value": done / dt / 1e9, "unit": "GB/s", "cores": cores, "kind": "oracle",
                                  "sample": f"{heads} of {Hq} query heads ({heads * Hkv // Hq} KV heads), fp64; "
                                            f"{dt:.2f} s"}
    return result


def rmsnorm_bench(args, torch, w8a8):
    """RMSNorm producer writing the int8 codes and per-token scale of the next linear layer
    (rmsnorm_quantize) at M = 4096 token rows of K = 10240, the long-K layer input: one step
    is one call; x is read once and the codes written once, so the roofline is HBM. x rotates
    over copies larger than the Infinity Cache, as a producer's output would arrive."""
    import oracle
    from synth_inputs import rmsnorm_inputs

    M, K, eps = 4096, 10240, 1e-6
    x, g = rmsnorm_inputs(M, K, seed=0)
    copies = max(1, -(-(320 << 20) // x.nbytes))
    xs = [torch.from_numpy(x).cuda() for _ in range(copies)]
    gd = torch.from_numpy(g).cuda()
    xq = torch.empty((M, K), dtype=torch.int8, device="cuda")
    sx = torch.empty((M,), dtype=torch.float32, device="cuda")

    def step(i):
        w8a8.rmsnorm_quantize(xs[i % copies], gd, eps, xq, sx, stream=torch.cuda.current_stream())

    ms_per_step, event_ms = timed_steps(args, torch, step)
    kernel_ms = event_ms if event_ms is not None else ms_per_step
    alg_bytes = M * K * 2 + K * 2 + M * K + M * 4  # x and g in, codes and scales out
    achieved = alg_bytes / (kernel_ms * 1e-3) / 1e9
    result = {
        "metric": f"RMSNorm -> int8 codes + per-token scale (rmsnorm_quantize), M={M} K={K} fp16",
        "value": alg_bytes / (ms_per_step * 1e-3) / 1e9, "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "rmsnorm_quantize: the norm in front of a linear layer writes its int8 input",
                   "M": M, "K": K, "in": "fp16", "gamma": "fp16", "x_copies": copies, "parallelism": "single GPU"},
        "step_event_ms": event_ms,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": measured_traffic(args.workload),
                     "kernel": "rmsnorm_quantize_kernel", "launch_ms": kernel_ms, "alg_bytes": alg_bytes},
    }
    if not args.no_cpu_baseline:
        oracle.build(force=False)
        rows, t0 = 0, time.perf_counter()
        while rows < M and time.perf_counter() - t0 < args.cpu_seconds:
            oracle.rmsnorm_quantize(x[rows:rows + 256], g, eps)
            rows += 256
        dt = time.perf_counter() - t0
        cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
        result["cpu_baseline"] = {"value": alg_bytes * rows / M / dt / 1e9, "unit": "GB/s", "cores": cores,
                                  "kind": "oracle", "sample": f"first {rows} of {M} rows; {dt:.2f} s"}
    return result


CLOCK = {}  # engine clock over the last timed region (clock_record), for the JSON line


def clock_record(torch, before, after):
    """Mean engine clock (MHz) between two clock probes, per compute unit that both probes
    visited (both counters of a pair read on one compute unit): 100 MHz times the ratio of the
    shader-clock and 100 MHz counter differences; median, p10 and p90 over those units."""
    def firsts(t):
        a = t.cpu().numpy().reshape(-1, 4)
        d = {}
        for loc, sclk, ref, _ in a:
            # XCC id and the HW_ID fields that name a compute unit (CU, shader array, engine)
            key = (int(loc) >> 32, (int(loc) >> 8) & 0xFF)
            d.setdefault(key, (int(sclk), int(ref)))
        return d
    b, a = firsts(before), firsts(after)
    mhz = [100.0 * (a[k][0] - b[k][0]) / (a[k][1] - b[k][1]) for k in b if k in a and a[k][1] > b[k][1]]
    if not mhz:
        return None
    return {"median_mhz": float(np.median(mhz)), "p10_mhz": float(np.percentile(mhz, 10)),
            "p90_mhz": float(np.percentile(mhz, 90)), "units": len(mhz),
            "interval_us": float(np.median([a[k][1] - b[k][1] for k in b if k in a])) / 100.0,
            "how": "s_memtime against s_memrealtime on each compute unit, probes right before and after "
                   "the host-timed replay"}


def step_distribution(torch, step, n, first):
    """Per-step times (ms) of n steps issued one by one, an event recorded after each: p10,
    median and p90. A second pass after the timed replay, not the timed steps themselves."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    torch.cuda.synchronize()
    ev[0].record()
    for i in range(n):
        step(first + i)
        ev[i + 1].record()
    torch.cuda.synchronize()
    d = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(n)])
    return {"p10_ms": float(np.percentile(d, 10)), "p50_ms": float(np.percentile(d, 50)),
            "p90_ms": float(np.percentile(d, 90)), "n": n,
            "how": "events between eagerly issued steps, after the timed replay"}


def timed_steps(args, torch, step, w8a8=None):
    """Warmup, then args.steps steps replayed as one captured graph (or issued one by one
    with --no-graph). Returns (ms per step by the host clock, ms per step by events or
    None). The graph is captured after the first few warmup steps (the rest run right
    before the timed replay, so the GPU does not sit idle during the capture between the
    warmup and the timed steps). With w8a8 given, clock probes on the replay's stream
    bracket the timed region and CLOCK holds the engine clock over it."""
    CLOCK.clear()
    if args.no_graph:
        for i in range(args.warmup):
            step(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            step(args.warmup + i)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / args.steps, None
    first = min(args.warmup, 3)
    for i in range(first):
        step(i)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        for i in range(args.steps):
            step(args.warmup + i)
    for i in range(first, args.warmup):
        step(i)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    probes = [torch.zeros(4096, dtype=torch.int64, device="cuda") for _ in range(2)] if w8a8 else None
    if probes:
        w8a8.w8a8_debug_clock_probe(probes[1], stream=side)  # first launch (code load) outside the timing
    torch.cuda.synchronize()
    if probes:
        w8a8.w8a8_debug_clock_probe(probes[0], stream=side)  # enqueued before the host clock starts
    t0 = time.perf_counter()
    with torch.cuda.stream(side):
        e0.record()
        graph.replay()
        e1.record()
    torch.cuda.synchronize()
    host_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    if probes:
        w8a8.w8a8_debug_clock_probe(probes[1], stream=side)  # after the host clock stopped
        torch.cuda.synchronize()
        rec = clock_record(torch, probes[0], probes[1])
        if rec:
            CLOCK.update(rec)
    return host_ms, e0.elapsed_time(e1) / args.steps


def qwen3_block(args, torch, w8a8):
    """One Qwen3-8B-shaped decoder block's seven linears at prefill (M=2048 tokens), W8A8
    per-channel, bf16 out: each of the four block inputs is quantized once per step; q, k,
    v share one GEMM over their concatenated weights (N = 6144) and gate, up another
    (N = 24576): exact, since per-channel weight scales belong to output rows.

    A second chain times the same GEMMs with the producers writing their int8 inputs: the
    RMSNorm in front of q/k/v and of gate/up (rmsnorm_quantize, from the residual stream)
    and the SwiGLU between gate/up and down (swiglu_quantize, from the gate/up GEMM's bf16
    output); the attention output keeps quantize_per_token. Both chains are reported, with
    the time of their four quantization-side kernels."""
    from synth_inputs import qwen3_8b_block_inputs, QWEN3_8B_BLOCK

    M = 2048
    inputs, weights = qwen3_8b_block_inputs(M=M, seed=0)
    groups = (("attn_in", ("q", "k", "v")), ("o_in", ("o",)), ("mlp_in", ("gate", "up")), ("down_in", ("down",)))
    ops = sum(2.0 * M * N * K for _, K, N in QWEN3_8B_BLOCK)
    stages = []
    for in_name, projs in groups:
        x = torch.from_numpy(inputs[in_name]).cuda()
        W_host = np.concatenate([weights[n] for n in projs])
        wq, sw = w8a8.quantize_weight(torch.from_numpy(W_host).cuda(), 8, 0)  # offline: not timed
        K, N = x.shape[1], wq.shape[0]
        stages.append({"name": "+".join(projs), "x": x, "wq": wq, "sw": sw, "N": N, "K": K,
                       "x_host": inputs[in_name], "W_host": W_host,
                       "xq": torch.empty((M, K), dtype=torch.int8, device="cuda"),
                       "sx": torch.empty((M,), dtype=torch.float32, device="cuda"),
                       "y": torch.empty((M, N), dtype=torch.bfloat16, device="cuda")})
    del inputs, weights
    qkv, o, gu, down = stages
    I = down["K"]
    # norm weights of the two RMSNorms (near one, as trained ones are)
    rng = np.random.default_rng(1)
    g_attn = torch.from_numpy((1 + 0.1 * rng.standard_normal(qkv["K"])).astype(np.float16)).cuda()
    g_mlp = torch.from_numpy((1 + 0.1 * rng.standard_normal(gu["K"])).astype(np.float16)).cuda()
    eps = 1e-6

    def gemm(st, stream):
        w8a8.w8a8_gemm_pc(st["xq"], st["sx"], st["wq"], st["sw"], y=st["y"], stream=stream)

    quant = {  # the quantization-side kernel of each stage, per chain
        "standalone": [lambda st_, cur: w8a8.quantize_per_token(st_["x"], st_["xq"], st_["sx"], stream=cur)] * 4,
        "producers": [
            lambda st_, cur: w8a8.rmsnorm_quantize(st_["x"], g_attn, eps, st_["xq"], st_["sx"], stream=cur),
            lambda st_, cur: w8a8.quantize_per_token(st_["x"], st_["xq"], st_["sx"], stream=cur),
            lambda st_, cur: w8a8.rmsnorm_quantize(st_["x"], g_mlp, eps, st_["xq"], st_["sx"], stream=cur),
            lambda st_, cur: w8a8.swiglu_quantize(gu["y"][:, :I], gu["y"][:, I:], st_["xq"], st_["sx"], stream=cur),
        ],
    }

    def make_step(chain):
        def step(i):
            cur = torch.cuda.current_stream()
            for st, q in zip(stages, quant[chain]):
                q(st, cur)
                gemm(st, cur)
        return step

    stream = torch.cuda.current_stream()

    def launch_ms(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(args.steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    ms_per_step, event_ms = timed_steps(args, torch, make_step("standalone"), w8a8)
    sclk = dict(CLOCK) or None
    value = ops / (ms_per_step * 1e-3) / 1e12
    prod_ms, prod_event_ms = timed_steps(args, torch, make_step("producers"), w8a8)
    chains = {}
    for chain in ("standalone", "producers"):
        kernels = [launch_ms(lambda st=st, q=q: q(st, stream)) for st, q in zip(stages, quant[chain])]
        chains[chain] = {"quantize_side_us": [k * 1e3 for k in kernels], "quantize_side_total_us": sum(kernels) * 1e3}
    chains["standalone"].update({"ms_per_step": ms_per_step, "tops": value,
                                 "kernels": "quantize_per_token x4"})
    chains["producers"].update({"ms_per_step": prod_ms, "tops": ops / (prod_ms * 1e-3) / 1e12,
                                "kernels": "rmsnorm_quantize (q|k|v), quantize_per_token (o), rmsnorm_quantize "
                                           "(gate|up), swiglu_quantize (down, from the gate|up output)"})
    # dominant kernel: the gate+up GEMM (N = 24576, 52 % of the block's operations)
    gemm_ms = launch_ms(lambda: gemm(gu, stream))
    big_ops = 2.0 * M * gu["N"] * gu["K"]
    achieved = big_ops / (gemm_ms * 1e-3) / 1e12
    result = {
        "metric": "INT8 TOPS of one Qwen3-8B block's seven W8A8 linears (quantize + GEMM + dequant), M=2048",
        "value": value, "unit": "TOPS", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "i8", "data": "synthetic",
        "config": {"workload": "Qwen3-8B block linears at prefill: q,k,v | o | gate,up | down, per-channel, "
                               "each input quantized per token in the step",
                   "M": M, "shapes_NK": [[st["N"], st["K"]] for st in stages], "out": "bf16",
                   "parallelism": "single GPU"},
        "frac_of_peak_step": value / PEAK_INT8_TOPS,
        "step_event_ms": event_ms, "sclk": sclk,
        "chains": chains,
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_INT8_TOPS, "unit": "TOPS",
                     "frac": achieved / PEAK_INT8_TOPS, "traffic": None,
                     "kernel": f"gemm ({gu['name']}: M={M} N={gu['N']} K={gu['K']})", "launch_ms": gemm_ms},
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = qwen3_cpu_baseline(stages, args.cpu_seconds)
    return result


def qwen3_cpu_baseline(stages, budget_s):
    """The CPU oracle on a bounded sample of token rows of every projection of the block."""
    import oracle

    oracle.build(force=False)
    host = [(st["x_host"], *oracle.quantize_weight(st["W_host"], 8, 0)) for st in stages]
    rows_done, chunk = 0, 8
    t0 = time.perf_counter()
    while rows_done < 2048:
        for x, wq, sw in host:
            oracle.linear_pc(x[rows_done:rows_done + chunk], wq, sw)
        rows_done += chunk
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    ops = sum(2.0 * rows_done * wq.shape[0] * wq.shape[1] for _, wq, _ in host)
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": ops / dt / 1e12, "unit": "TOPS", "cores": cores, "kind": "oracle",
            "sample": f"first {rows_done} of 2048 token rows of each of the block's projections; "
                      f"per-token quantize + int GEMM + fp64 dequant; {dt:.2f} s"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path is single-GPU; see the sharding notes in the design document)",
              file=sys.stderr)
        return 2

    import torch
    import w8a8_activation_quantized_amd as w8a8
    from synth_inputs import linear_inputs

    if not torch.cuda.is_available() or not w8a8.w8a8_is_available(0):
        print("no gfx950 GPU available: " + w8a8.w8a8_last_error(), file=sys.stderr)
        return 1

    if args.copy_ref_mb:
        src = torch.empty(args.copy_ref_mb << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if args.workload == "qwen3":
        print(json.dumps(qwen3_block(args, torch, w8a8)), flush=True)
        return 0
    if args.workload == "sdpa":
        print(json.dumps(sdpa_bench(args, torch, w8a8)), flush=True)
        return 0
    if args.workload == "rmsnorm":
        print(json.dumps(rmsnorm_bench(args, torch, w8a8)), flush=True)
        return 0
    if args.workload in ("mv", "mvg128"):
        print(json.dumps(mv_decode(args, torch, w8a8, 0 if args.workload == "mv" else 128)), flush=True)
        return 0

    result = linear_bench(args, torch, w8a8, args.workload)
    if args.workload == "pc" and not args.no_m1:
        # the second bar of the target: the fused M = 1 layer (one kernel per step), weights
        # streamed from HBM, int8 and int4 (gs = 128) weights
        result["m1"] = {}
        for name in ("m1", "m1w4"):
            r = linear_bench(args, torch, w8a8, name)
            ro = r["roofline"]
            result["m1"][name] = {"M": 1, "N": r["config"]["N"], "K": r["config"]["K"],
                                  "weight_bits": r["config"]["weight_bits"], "group_size": r["config"]["group_size"],
                                  "us_per_step": r["ms_per_step"] * 1e3, "kernel_us": ro["launch_ms"] * 1e3,
                                  "gbs": ro["achieved"], "frac_of_hbm": ro["frac"], "alg_bytes": ro["alg_bytes"],
                                  "sclk": r.get("sclk")}
    if not args.no_cpu_baseline:
        M, N, K, bits, gs = WORKLOADS[args.workload]
        x_np, W_np = linear_inputs(M, N, K, seed=0)
        result["cpu_baseline"] = cpu_baseline(x_np, W_np, bits, gs, args.cpu_seconds)
        if args.workload == "pc":
            result["cpu_baseline"]["single_thread"] = cpu_single_thread()
    print(json.dumps(result), flush=True)
    return 0


def linear_bench(args, torch, w8a8, workload):
    """One w8a8 linear workload (quantize + GEMM, or the one-kernel layer for M <= 16):
    the timed steps, the per-kernel launch times and the roofline of the dominant kernel."""
    from synth_inputs import linear_inputs

    M, N, K, bits, gs = WORKLOADS[workload]
    x_np, W_np = linear_inputs(M, N, K, seed=0)
    x = torch.from_numpy(x_np).cuda()
    Wd = torch.from_numpy(W_np).cuda()
    wq, sw = w8a8.quantize_weight(Wd, bits, gs)  # offline: not timed
    del Wd
    # small M is bound by streaming the weights: rotate over copies larger than the MALL
    wbytes = wq.numel() * wq.element_size()
    copies = [wq] + ([wq.clone() for _ in range((512 << 20) // wbytes)] if M <= 128 else [])
    xq = torch.empty((M, K), dtype=torch.int8, device="cuda")
    sx = torch.empty((M,), dtype=torch.float32, device="cuda")
    y = torch.empty((M, N), dtype=torch.float16, device="cuda")
    stream = torch.cuda.current_stream()
    fused = M <= 16

    if bits == 4 and gs == 0:
        def gemm(w, st):
            w8a8.w4a8_gemm_pc(xq, sx, w, sw, y=y, stream=st)
    elif bits == 4:
        def gemm(w, st):
            w8a8.w4a8_gemm_pg(xq, sx, w, sw, gs, y=y, stream=st)
    elif gs:
        def gemm(w, st):
            w8a8.w8a8_gemm_pg(xq, sx, w, sw, gs, y=y, stream=st)
    else:
        def gemm(w, st):
            w8a8.w8a8_gemm_pc(xq, sx, w, sw, y=y, stream=st)

    def step(i):
        w = copies[i % len(copies)]
        cur = torch.cuda.current_stream()
        if fused:
            w8a8.w8a8_linear(x, w, sw, bits, gs, y=y, x_q=xq, s_x=sx, stream=cur)
            return
        w8a8.quantize_per_token(x, xq, sx, stream=cur)
        gemm(w, cur)

    def launch_ms(launch, stream):
        """Average duration of one launch: args.steps launches issued back to back on the
        stream the kernel runs on, between two events on that stream. Events between the
        launches themselves would add their own time to every kernel they bracket."""
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(args.steps):
            launch(args.warmup + i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    # setup, not a step: touch every weight copy once (page tables warm, as in a serving
    # loop); then the warmup and timed steps
    for i in range(len(copies) if len(copies) > 1 else 0):
        step(i)
    ms_per_step, step_event_ms = timed_steps(args, torch, step, w8a8)
    sclk = dict(CLOCK) or None
    dist = None if fused else step_distribution(torch, step, min(args.steps, 200), args.warmup)
    if fused:
        quant_ms = gemm_ms = step_event_ms if step_event_ms is not None else launch_ms(step, stream)
    else:
        # per-kernel durations on the same stream, right after the timed steps; the
        # quantization rotates over copies of x larger than the Infinity Cache, since in a
        # step the GEMM's traffic evicts x between two quantizations
        xs = [x] + [x.clone() for _ in range((512 << 20) // (x.numel() * x.element_size()))]
        quant_ms = launch_ms(lambda i: w8a8.quantize_per_token(xs[i % len(xs)], xq, sx, stream=stream), stream)
        gemm_ms = launch_ms(lambda i: gemm(copies[i % len(copies)], stream), stream)
        del xs

    ops = 2.0 * M * N * K
    value = ops / (ms_per_step * 1e-3) / 1e12

    if fused:
        # one kernel per step: quantization + GEMV + dequant; HBM-bound on the weight stream
        kernel_ms = quant_ms
        alg_bytes = wbytes + sw.numel() * 4 + M * K * 2 + M * N * 2  # weights + scales, x in, y out
        achieved = alg_bytes / (kernel_ms * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": achieved / PEAK_HBM_GBS, "traffic": measured_traffic(workload),
                    "kernel": "fused quantize + GEMV + dequant (w8a8_linear, M <= 16)",
                    "launch_ms": kernel_ms, "alg_bytes": alg_bytes}
    else:
        achieved = ops / (gemm_ms * 1e-3) / 1e12
        roofline = {"bound": "mfma", "achieved": achieved, "peak": PEAK_INT8_TOPS, "unit": "TOPS",
                    "frac": achieved / PEAK_INT8_TOPS, "traffic": measured_traffic(workload),
                    "kernel": "gemm (int8 MFMA" + (", int4 weights unpacked in the operand load" if bits == 4 else "")
                              + (f", fused per-group dequant, gs={gs})" if gs else ", fused per-channel dequant)"),
                    "launch_ms": gemm_ms}

    result = {
        "metric": f"INT8 TOPS & % MFMA peak of fused quant-GEMM-dequant, M={M} N={N} K={K}",
        "value": value,
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic",
        "config": {"workload": f"w8a8 linear ({workload}): per-token quantize + int8 GEMM + fused dequant"
                               + (" in one kernel" if fused else ""),
                   "M": M, "N": N, "K": K, "weight_bits": bits, "group_size": gs, "out": "fp16",
                   "parallelism": "single GPU"},
        "frac_of_peak_step": value / PEAK_INT8_TOPS,
        "step_event_ms": step_event_ms,
        "gemm_ms": None if fused else gemm_ms,
        "quantize_ms": None if fused else quant_ms,
        "fused_ms": quant_ms if fused else None,
        "quantize_gbs": None if fused else (3.0 * M * K + 4 * M) / (quant_ms * 1e-3) / 1e9,
        "weight_copies": len(copies),
        "sclk": sclk,
        "step_times": dist,
        "roofline": roofline,
    }
    return result




if __name__ == "__main__":
    sys.exit(main())
