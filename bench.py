#!/usr/bin/env python3
"""Benchmark of the routed FP4 expert FFN hot path on one MI355X.

A step is one pass of the whole hot path over one batch: for the batch-1 decode workload
(one 384-expert MoE layer, hidden 4096, intermediate 2880, top-6, FP4 E2M1 weights with
ue8m0 block-32 scales) that is moe_fp4_route (router GEMV in fp64 + top-6 softmax) then
moe_fp4_expert_ffn (gate/up/SiLU, down and the weighted combine) for one fresh token.
Every step reads a different token's activations, already resident in HBM, so routing
(and the experts read) changes from step to step.

Prints one JSON line (the last line of stdout).
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
MFMA_FP4_PEAK_TFLOPS = 10100.0  # MI355X dense MXFP4 matrix cores, published
MFMA_FP8_PEAK_TFLOPS = 5000.0  # MI355X dense FP8 (the f8f6f4 MFMA's rate with an FP8 operand)


def log(msg: str) -> None:
    sys.stderr.write(f"[bench {time.strftime('%H:%M:%S')}] {msg}\n")
    sys.stderr.flush()


def expert_bytes(hidden: int, inter: int) -> int:
    n = 3 * hidden * inter
    return n // 2 + n // 32


def gate_up_bytes(hidden: int, inter: int) -> int:
    n = 2 * hidden * inter
    return n // 2 + n // 32


def grouped_gate_up_bytes(d_avg: float, T: int, k: int, hidden: int, inter: int, fp8: bool) -> float:
    """Algorithmic bytes of one grouped gate/up launch: each distinct expert's gate and up
    once, x read and h written as MX activations (per element and term: E4M3 one term,
    E2M3 two; plus the ue8m0 scale byte per 32 elements of each term), over H and I rounded
    up to 128."""
    Hp, Ip = (hidden + 127) // 128 * 128, (inter + 127) // 128 * 128
    nterm, elem = (1, 1.0) if fp8 else (2, 0.75)
    return (d_avg * gate_up_bytes(hidden, inter) + T * Hp * nterm * (elem + 1 / 32)
            + T * k * Ip * nterm * (elem + 1 / 32))


TRAFFIC_SUMMARIES = [os.path.join(ROOT, "profiles", "decode_layer_hbm_traffic.md"),
                     os.path.join(ROOT, "profiles", "grouped_hbm_traffic.md"),
                     os.path.join(ROOT, "profiles", "small_m_kernel_trace_and_traffic.md")]
KERNEL_SOURCES = {"gate_up_kernel": "kernels_ffn.hip", "down_combine_kernel": "kernels_ffn.hip",
                  "route_decode_kernel": "kernels_route.hip",
                  "gemm_gate_up_kernel": "kernels_batched.hip", "gemm_down_kernel": "kernels_batched.hip",
                  "gate_up_multi_kernel": "kernels_small_m.hip"}


def measured_traffic(kernel: str, workload: str = ""):
    """HBM bytes per launch of `kernel` (on `workload`, for the grouped kernels) from the
    committed rocprofv3 counter summaries (FETCH_SIZE + WRITE_SIZE, calibrated on a plain
    copy), or None when there is no entry or the kernel's source has changed since the
    counters were taken."""
    import hashlib

    key = f"{kernel}@{workload}" if workload else kernel
    try:
        src = os.path.join(ROOT, "fp4_expert_ffn_amd", "csrc", KERNEL_SOURCES[kernel])
        digest = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
    except (OSError, KeyError):
        return None
    for path in TRAFFIC_SUMMARIES:
        try:
            lines = open(path).read().splitlines()
        except OSError:
            continue
        for line in lines:
            f = line.split()
            if len(f) == 5 and f[0] == "traffic_bytes_per_launch" and f[1] == key and f[3] == "source":
                return int(f[2]) if f[4] == digest else None
    return None


TRACE_SUMMARIES = {"gate_up_kernel": os.path.join(ROOT, "profiles", "decode_layer_kernel_trace.md")}


def traced_avg_us(kernel: str):
    """Average duration (us) of `kernel` in the committed rocprofv3 kernel-trace summary of
    the default bench command, or None when the summary is missing or was taken on another
    version of the kernel's source (its recorded sha256/16 differs)."""
    import hashlib
    import re

    try:
        text = open(TRACE_SUMMARIES[kernel]).read()
        src_name = KERNEL_SOURCES[kernel]
        digest = hashlib.sha256(open(os.path.join(ROOT, "fp4_expert_ffn_amd", "csrc", src_name),
                                     "rb").read()).hexdigest()[:16]
    except (OSError, KeyError):
        return None
    if f"{src_name} sha256/16 {digest}" not in text:
        return None
    m = re.search(r"\|\s*`" + re.escape(kernel) + r"<[^`]*>`\s*\|\s*\d+\s*\|\s*(\d+)\s*\|", text)
    return int(m.group(1)) / 1e3 if m else None


def host_cpu_info() -> dict:
    """The host cores this process may run on and the BLAS thread pools NumPy would use."""
    from threadpoolctl import threadpool_info

    blas = [{"api": d.get("internal_api"), "threads": d.get("num_threads")}
            for d in threadpool_info() if d.get("user_api") == "blas"]
    return {"host_cores_available": len(os.sched_getaffinity(0)), "blas_default_threads": blas}


def cpu_baseline(wl, n_tokens: int, first_step: int):
    """Time the fp64 oracle (route + expert FFN) on the host for a bounded sample of the
    same workload: n_tokens tokens, one BLAS thread."""
    from threadpoolctl import threadpool_limits

    from oracle import moe_oracle as O
    from synth import moe_inputs as S

    wr = S.router_weights(wl, 0)
    xs = [S.activations(wl, 0, first_step + i) for i in range(n_tokens)]
    # expert blobs generated up front (input preparation, not timed)
    ids_all = [O.route(x, wr, wl.k)[0] for x in xs]
    need = sorted(set(int(e) for ids in ids_all for e in ids.ravel()))
    blobs = {e: S.expert_blob(wl, 0, e) for e in need}
    src = lambda e: blobs[e]  # noqa: E731
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        for x in xs:
            ids, w, _ = O.route(x, wr, wl.k)
            O.expert_ffn(x, ids, w, src, wl.n_experts, wl.hidden, wl.inter)
        dt = time.perf_counter() - t0
    out = {"value": n_tokens / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
           "sample": f"{n_tokens} tokens of the same one-layer batch-1 decode workload "
                     f"(route + expert FFN, fp64 NumPy, BLAS limited to 1 thread), {dt:.1f} s"}
    out.update(host_cpu_info())
    return out


def measure_peaks(torch, C, dev) -> dict:
    """What this chip sustains, measured with the library's two probe kernels: a streaming
    read of 4 GiB with the expert kernels' 16-byte non-temporal loads, and a loop of the
    block-scaled 16x16x128 matrix-core operation with FP4 x FP4 and FP8 x FP4 operands."""
    out = {}
    nbytes = 4 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    for _ in range(2):
        C.moe_fp4_debug_stream_read(buf, nbytes, sink)
    torch.cuda.synchronize()
    C.moe_fp4_timing_reset()
    C.moe_fp4_timing_enable(True)
    for _ in range(10):
        C.moe_fp4_debug_stream_read(buf, nbytes, sink)
    torch.cuda.synchronize()
    C.moe_fp4_timing_enable(False)
    n, ms = C.moe_fp4_timing_read(C.KERNEL_NAMES.index("probe_stream"))
    out["hbm_stream_read_gbs"] = round(nbytes * n / (ms * 1e-3) / 1e9, 1)
    del buf
    n_wg, iters = 1024, 2000  # 4 wavefronts per SIMD on 256 CUs
    flops = n_wg * 4 * iters * C.PROBE_MFMA_CHAINS * 2.0 * 16 * 16 * 128
    for fmt, key in ((4, "mfma_fp4xfp4_tflops"), (0, "mfma_fp8xfp4_tflops")):
        C.moe_fp4_debug_mfma_loop(fmt, n_wg, iters, sink)
        torch.cuda.synchronize()
        C.moe_fp4_timing_reset()
        C.moe_fp4_timing_enable(True)
        for _ in range(5):
            C.moe_fp4_debug_mfma_loop(fmt, n_wg, iters, sink)
        torch.cuda.synchronize()
        C.moe_fp4_timing_enable(False)
        n, ms = C.moe_fp4_timing_read(C.KERNEL_NAMES.index("probe_mfma"))
        out[key] = round(flops * n / (ms * 1e-3) / 1e12, 1)
    C.moe_fp4_timing_reset()
    log("measured peaks: " + json.dumps(out))
    return out


def step_percentiles(torch, step, indices) -> dict:
    """Per-step GPU time (us) of stream-launched steps, each bracketed by its own events."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in indices]
    torch.cuda.synchronize()
    for (a, b), i in zip(evs, indices):
        a.record()
        step(i)
        b.record()
    torch.cuda.synchronize()
    us = np.array([a.elapsed_time(b) * 1e3 for a, b in evs])
    return {"p10": round(float(np.percentile(us, 10)), 2), "p50": round(float(np.median(us)), 2),
            "p90": round(float(np.percentile(us, 90)), 2), "n": len(us),
            "how": "stream launches, one event pair per step"}


def with_measured_peak(roofline, peaks):
    if roofline is None or not peaks:
        return roofline
    key = {"GB/s": "hbm_stream_read_gbs", "TFLOP/s": "mfma_fp8xfp4_tflops"}[roofline["unit"]]
    mp = peaks.get(key)
    if mp:
        roofline["measured_peak"] = mp
        roofline["frac_of_measured_peak"] = round(roofline["achieved"] / mp, 4)
    return roofline


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--workload", default="layer_decode_h4096_i2880_e384",
                    choices=["layer_decode_h4096_i2880_e384", "batched64_zipf", "prefill8192_uniform",
                             "prefill32768_uniform", "stack16_decode", "expert_h256_i128",
                             "mtp4_correlated", "streams8_uniform", "shared_expert_fp8_h4096_i2880"],
                    help="the batch-1 decode layer (default, the headline line), or one of the "
                         "multi-token shapes (small-M path below 24 tokens, grouped GEMM path "
                         "from 24 on)")
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--mode", choices=["graph", "stream"], default="graph")
    ap.add_argument("--api", choices=["fused", "split"], default="fused",
                    help="fused: one moe_fp4_moe_forward call; split: moe_fp4_route then "
                         "moe_fp4_expert_ffn (three kernel launches either way)")
    ap.add_argument("--stack-route", choices=["fused", "separate"], default="fused",
                    help="stack16_decode: route each later layer straight from the residual "
                         "stream (fused) or run residual + RMSNorm as its own launch (separate)")
    ap.add_argument("--act-terms", type=int, choices=[1, 2], default=2,
                    help="grouped-path workloads: activations as two MXFP6 terms (default, meets "
                         "the output tolerance) or one (the opt-in FP8-activation path)")
    ap.add_argument("--cpu-tokens", type=int, default=30)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-roofline-pass", action="store_true")
    ap.add_argument("--prefetch", choices=["none", "oracle", "router"], default="none",
                    help="stack16_decode: prefetch the next layer's experts into the memory-side "
                         "cache on a side stream (oracle: true ids from a prior pass; router: the "
                         "next layer's router on this layer's input)")
    ap.add_argument("--prefetch-top", type=int, default=2,
                    help="experts prefetched per layer (the top of the prediction)")
    ap.add_argument("--prefetch-mats", type=int, default=3,
                    help="matrices prefetched: bit 0 gate, 1 up, 2 down")
    ap.add_argument("--no-batched", action="store_true",
                    help="skip the batched (grouped GEMM) half of the metric in the decode run")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the measured-peak probes (streaming read, matrix-core loop)")
    ap.add_argument("--pmc-calibration", action="store_true",
                    help="before the steps, run a plain elementwise copy of 256 MiB three times "
                         "(a known-size kernel that scales the FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(this build runs on a single MI355X).", file=sys.stderr)
        return 2

    if args.workload == "stack16_decode":
        return run_stack(args)
    if args.workload == "expert_h256_i128":
        return run_single_expert(args)
    if args.workload == "shared_expert_fp8_h4096_i2880":
        return run_shared_expert(args)
    if args.workload != "layer_decode_h4096_i2880_e384":
        return run_batched(args)

    import torch

    from fp4_expert_ffn_amd import device as D
    from fp4_expert_ffn_amd import moe_fp4 as C
    from synth import moe_inputs as S

    C.lib()
    dev = torch.device("cuda:0")
    wl = S.WORKLOADS["layer_decode_h4096_i2880_e384"]
    H, I, E, k = wl.hidden, wl.inter, wl.n_experts, wl.k
    K, W = args.steps, args.warmup

    log(f"uploading {E} experts ({E * expert_bytes(H, I) / 1e9:.2f} GB)")
    t0 = time.time()
    packed = D.upload_experts(S.expert_source(wl, 0), E, H, I, dev, chunk=32)
    wr = D.upload_bf16(S.router_weights(wl, 0), dev)
    layer = D.MoeFp4Layer(packed, E, H, I, k, wr)
    n_x = W + 2 * K
    xs_bits = np.concatenate([S.activations(wl, 0, s) for s in range(n_x)])
    xs = D.upload_bf16(xs_bits, dev)
    log(f"setup done in {time.time() - t0:.1f} s")

    if args.pmc_calibration:
        # 64 Mi fp32 elements: 268,435,456 B read and 268,435,456 B written per launch
        src = torch.empty(64 << 20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst

    ids = torch.empty((1, k), dtype=torch.int32, device=dev)
    w = torch.empty((1, k), dtype=torch.float32, device=dev)
    y = torch.empty((1, H), dtype=torch.bfloat16, device=dev)
    layer._workspace(1)
    layer._route_workspace(1)
    layer._forward_workspace(1)

    def step(i: int) -> None:
        x = xs[i:i + 1]
        if args.api == "fused":
            layer.forward_fused(x, ids, w, y)
        else:
            layer.route(x, ids, w)
            layer.ffn(x, ids, w, y)

    for i in range(W):
        step(i)
    torch.cuda.synchronize()

    graph = None
    if args.mode == "graph":
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=side):
            for i in range(W, W + K):
                step(i)
        torch.cuda.synchronize()
        graph.replay()  # one untimed replay
        torch.cuda.synchronize()

    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ev0.record()
    if graph is not None:
        graph.replay()
    else:
        for i in range(W, W + K):
            step(i)
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    gpu_ms = ev0.elapsed_time(ev1)
    elapsed_s = max(gpu_ms / 1e3, 1e-9)
    value = K / elapsed_s
    ms_per_step = gpu_ms / K
    step_bytes = k * expert_bytes(H, I) + E * H * 2 + 2 * H * 2
    log(f"timed {K} steps ({args.mode}): {gpu_ms:.3f} ms GPU, {wall * 1e3:.3f} ms wall -> "
        f"{value:.0f} layer-tokens/s, {step_bytes * K / elapsed_s / 1e9:.0f} GB/s algorithmic")

    # Per-kernel durations: the library's own HIP events bracket each launch on the launch
    # stream. A second pass over fresh tokens, stream-launched, with timing enabled.
    roofline = None
    kernels = {}
    if not args.no_roofline_pass:
        C.moe_fp4_timing_reset()
        C.moe_fp4_timing_enable(True)
        for i in range(W + K, W + 2 * K):
            step(i)
        torch.cuda.synchronize()
        C.moe_fp4_timing_enable(False)
        for kind, name in enumerate(C.KERNEL_NAMES):
            n, ms = C.moe_fp4_timing_read(kind)
            if n:
                kernels[name] = {"launches": n, "avg_us": ms * 1e3 / n}
        C.moe_fp4_timing_reset()
        gu = kernels.get("gate_up")
        if gu:
            # algorithmic bytes of one gate_up launch at batch 1: the k selected experts'
            # gate and up codes + scales, the token's x, and h (bf16) written
            alg = k * gate_up_bytes(H, I) + H * 2 + k * I * 2
            achieved = alg / (gu["avg_us"] * 1e-6) / 1e9
            roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                        "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                        "traffic": measured_traffic("gate_up_kernel"), "kernel": "gate_up",
                        "bytes_per_launch": alg,
                        "avg_launch_us": round(gu["avg_us"], 3),
                        "avg_launch_us_source": "library HIP events on the launch stream, "
                                                "stamped with the dispatch's start and end"}
            tr = traced_avg_us("gate_up_kernel")
            if tr:
                roofline["trace_avg_launch_us"] = tr
                roofline["trace_frac"] = round(alg / (tr * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
                roofline["trace_source"] = "profiles/decode_layer_kernel_trace.md (rocprofv3 --kernel-trace --stats)"
        log("kernels: " + json.dumps(kernels))

    pct = step_percentiles(torch, step, range(W + K, W + 2 * K))
    log(f"per-step us (stream): {json.dumps(pct)}")
    peaks = None if args.no_peaks else measure_peaks(torch, C, dev)
    roofline = with_measured_peak(roofline, peaks)

    batched = None
    if not args.no_batched:
        # the other half of the metric: batched FP4 TFLOP/s of the grouped path on the same
        # 384 experts (8192 tokens, and the matrix-core-bound 32768)
        batched = {"metric": "batched FP4 TFLOP/s (algorithmic: 6 H I flops per (token, slot) "
                             "pair, no hi/lo duplication)",
                   "experts": "the decode layer's 384 experts"}
        for name in ("prefill8192_uniform", "prefill32768_uniform"):
            batched[name] = grouped_measure(torch, C, D, S, layer, S.WORKLOADS[name], dev,
                                            K=10, W=2, terms=2)
            log(f"batched {name}: " + json.dumps(batched[name]))

    cpu = None
    if not args.no_cpu_baseline:
        log(f"cpu baseline: oracle on {args.cpu_tokens} tokens")
        cpu = cpu_baseline(wl, args.cpu_tokens, first_step=0)
        log(f"cpu baseline: {cpu['value']:.3f} tokens/s")

    out = {
        "metric": "MoE-layer tokens/s at batch 1 (+ achieved HBM GB/s)",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "hidden": H, "intermediate": I, "experts": E, "top_k": k,
                   "weights": "fp4-e2m1 + ue8m0/32", "batch_tokens": 1, "launch": args.mode, "api": args.api,
                   "parallelism": "none (1 GPU)"},
        "algorithmic_gbps": round(step_bytes * K / elapsed_s / 1e9, 1),
        "hbm_frac_step": round(step_bytes * K / elapsed_s / 1e9 / HBM_PEAK_GBS, 4),
        "bytes_per_step": step_bytes,
        "step_us": pct,
        "kernels": kernels,
        "measured_peaks": peaks,
        "roofline": roofline,
        "batched": batched,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    return 0


def grouped_measure(torch, C, D, S, layer, wl, dev, K: int, W: int, terms: int) -> dict:
    """One grouped-path workload on a resident layer: K graph-replayed steps of top-k on the
    workload's fresh router logits + moe_fp4_expert_ffn (the grouped GEMM path), then a
    stream-launched pass with the library's kernel timing. Algorithmic flops are 6 H I per
    (token, slot) pair (2 H I for each of gate, up and down; the two MXFP6 activation terms
    are not counted twice); algorithmic bytes are each distinct expert once plus the
    activations, logits and routing."""
    H, I, E, k, T = wl.hidden, wl.inter, layer.n_experts, wl.k, wl.tokens
    lgs = torch.stack([torch.from_numpy(S.router_logits(wl, 0, i)) for i in range(W + 2 * K)]).to(dev)
    x = D.upload_bf16(S.activations(wl, 0, 0), dev)
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    y = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    layer._workspace(T, k)
    path = C.PATH_GROUPED if terms == 2 else C.PATH_GROUPED_FP8

    def step(i: int) -> None:
        C.moe_fp4_route_logits(lgs[i], T, E, k, ids, w)
        layer.ffn(x, ids, w, y, path=path)

    for i in range(W):
        step(i)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        for i in range(W, W + K):
            step(i)
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    graph.replay()
    ev1.record()
    torch.cuda.synchronize()
    step_s = ev0.elapsed_time(ev1) / 1e3 / K
    del graph
    distinct = []
    for i in range(W, W + K):
        C.moe_fp4_route_logits(lgs[i], T, E, k, ids, w)
        distinct.append(int(torch.unique(ids).numel()))
    d_avg = float(np.mean(distinct))
    pairs = T * k
    flops = pairs * 6.0 * H * I
    step_bytes = d_avg * expert_bytes(H, I) + 2 * T * H * 2 + T * E * 4 + pairs * 8
    C.moe_fp4_timing_reset()
    C.moe_fp4_timing_enable(True)
    for i in range(W + K, W + 2 * K):
        step(i)
    torch.cuda.synchronize()
    C.moe_fp4_timing_enable(False)
    kern = {}  # GPU time per step of each kernel kind (the split sort is three launches)
    for kind, name in enumerate(C.KERNEL_NAMES):
        n, ms = C.moe_fp4_timing_read(kind)
        if n:
            kern[name] = round(ms * 1e3 / K, 2)
    C.moe_fp4_timing_reset()
    out = {"tokens": T, "steps": K, "ms_per_step": round(step_s * 1e3, 4),
           "tflops": round(flops / step_s / 1e12, 1),
           "frac_fp4_peak": round(flops / step_s / 1e12 / MFMA_FP4_PEAK_TFLOPS, 4),
           "algorithmic_gbps": round(step_bytes / step_s / 1e9, 1),
           "frac_hbm": round(step_bytes / step_s / 1e9 / HBM_PEAK_GBS, 4),
           "distinct_experts": round(d_avg, 1), "kernel_us_per_step": kern}
    gu = kern.get("grouped_gate_up")
    if gu:
        gflops = pairs * 4.0 * H * I  # gate and up
        out["gate_up_tflops"] = round(gflops / (gu * 1e-6) / 1e12, 1)
        out["gate_up_frac_fp4_peak"] = round(gflops / (gu * 1e-6) / 1e12 / MFMA_FP4_PEAK_TFLOPS, 4)
        # HBM bytes per gate/up launch from the committed counter summary (null when it has
        # none for this workload or the kernel source changed since), against the algorithmic
        tr = measured_traffic("gemm_gate_up_kernel", wl.name) if terms == 2 else None
        out["gate_up_traffic_bytes"] = tr
        out["gate_up_traffic_ratio"] = (round(tr / grouped_gate_up_bytes(d_avg, T, k, H, I, False), 3)
                                        if tr else None)
    del lgs, x, ids, w, y
    return out


def run_stack(args) -> int:
    """16 chained MoE layers at batch 1 (about 116 GB of FP4 experts resident): per token,
    the residual starts as the token's x; every layer routes x (one-launch routing), runs
    the expert FFN, then residual += y and x = RMSNorm(residual) feed the next layer."""
    import torch

    from fp4_expert_ffn_amd import device as D
    from fp4_expert_ffn_amd import moe_fp4 as C
    from synth import moe_inputs as S

    C.lib()
    dev = torch.device("cuda:0")
    wl = S.WORKLOADS["stack16_decode"]
    H, I, E, k, L = wl.hidden, wl.inter, wl.n_experts, wl.k, wl.layers
    K, W = min(args.steps, 200), min(args.warmup, 10)
    stride = C.moe_fp4_packed_expert_stride(H, I)
    log(f"{wl.name}: generating and packing {L} x {E} experts on the device "
        f"({L * E * expert_bytes(H, I) / 1e9:.1f} GB)")
    t0 = time.time()
    layers = []
    for l in range(L):
        packed = torch.empty(stride * E, dtype=torch.uint8, device=dev)
        for e0 in range(0, E, S.STACK_CHUNK):
            e1 = min(E, e0 + S.STACK_CHUNK)
            codes, scales = S.device_expert_blobs(wl, l, e0, e1, dev)
            C.moe_fp4_pack(codes, scales, e1 - e0, H, I, packed.data_ptr() + e0 * stride,
                           (e1 - e0) * stride)
            del codes, scales
        wr = D.upload_bf16(S.router_weights(wl, l), dev)
        layers.append(D.MoeFp4Layer(packed, E, H, I, k, wr))
    torch.cuda.synchronize()
    xs = D.upload_bf16(np.concatenate([S.activations(wl, 0, t) for t in range(W + 2 * K)]), dev)
    log(f"setup done in {time.time() - t0:.1f} s")
    ws = layers[0]._forward_workspace(1)
    for lay in layers:
        lay._fws = ws  # one workspace for the whole stack (stream-ordered)
    r = torch.empty((1, H), dtype=torch.float32, device=dev)
    r2 = torch.empty_like(r)
    xa = torch.empty((1, H), dtype=torch.bfloat16, device=dev)
    xb = torch.empty_like(xa)
    ids = torch.empty((1, k), dtype=torch.int32, device=dev)
    w = torch.empty((1, k), dtype=torch.float32, device=dev)
    y = torch.empty((1, H), dtype=torch.bfloat16, device=dev)

    # Speculative prefetch of layer l + 1's experts into the memory-side cache
    # (moe_fp4_prefetch_experts on a side stream, forked once layer l's FFN is enqueued, so it
    # runs while layer l + 1 routes): "oracle" prefetches the true top experts of the next
    # layer (recorded in an untimed pass over the same tokens), "router" the top experts of
    # the next layer's router applied to this layer's input, computed on the side stream.
    pf = args.prefetch
    top = max(1, min(k, args.prefetch_top))
    side = torch.cuda.Stream() if pf != "none" else None
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    true_ids = None
    pred_ids = torch.empty((L, k), dtype=torch.int32, device=dev)
    pred_w = torch.empty((L, k), dtype=torch.float32, device=dev)
    pred_ws = torch.empty(C.moe_fp4_route_workspace_bytes(1, E), dtype=torch.uint8, device=dev)

    def prefetch_next(l: int, t: int, x_l) -> None:
        """Enqueue the prefetch of layer l + 1's experts (and, for the router predictor, the
        prediction on x_l) on the side stream; returns the event main must wait on before
        overwriting x_l."""
        if pf == "none" or l + 1 >= L:
            return None
        main = torch.cuda.current_stream()
        ev_x = main.record_event()
        ev_pred = None
        if pf == "router":
            side.wait_event(ev_x)
            with torch.cuda.stream(side):  # its own route workspace: it runs beside the stack's
                C.moe_fp4_route(x_l, layers[l + 1].w_router, 1, H, E, k, pred_ids[l + 1:l + 2],
                                pred_w[l + 1:l + 2], pred_ws)
            ev_pred = side.record_event()
        return ev_pred

    def prefetch_issue(l: int, t: int) -> None:
        if pf == "none" or l + 1 >= L:
            return
        side.wait_stream(torch.cuda.current_stream())  # after layer l's FFN
        ids_src = true_ids[t, l + 1] if pf == "oracle" else pred_ids[l + 1]
        with torch.cuda.stream(side):
            C.moe_fp4_prefetch_experts(ids_src, top, layers[l + 1].packed, E, H, I,
                                       args.prefetch_mats, sink)

    def step(t: int) -> None:
        x = xs[t:t + 1]
        C.moe_fp4_residual_init(x, r, 1, H)
        if pf != "none":
            rc, rn = r, r2
            pending = {}
            for l, lay in enumerate(layers):
                if l == 0:
                    x_l = x
                    lay.forward_fused(x, ids, w, y)
                else:
                    xn = xa if l % 2 == 0 else xb
                    if l - 2 in pending and pending[l - 2] is not None:
                        torch.cuda.current_stream().wait_event(pending[l - 2])
                    lay.route_residual(rc, y, rn, xn, 1e-6, ids, w)
                    x_l = xn
                pending[l] = prefetch_next(l, t, x_l)
                if l > 0:
                    lay.ffn(x_l, ids, w, y)
                    rc, rn = rn, rc
                prefetch_issue(l, t)
            C.moe_fp4_residual_rmsnorm(rc, y, xa, 1, H, 1e-6)
            torch.cuda.current_stream().wait_stream(side)
            return
        if args.stack_route == "separate":
            for l, lay in enumerate(layers):
                lay.forward_fused(x, ids, w, y)
                xn = xa if l % 2 == 0 else xb
                C.moe_fp4_residual_rmsnorm(r, y, xn, 1, H, 1e-6)
                x = xn
            return
        # layers after the first route straight from the residual stream: the router kernel
        # adds the previous layer's y, normalises and routes in one launch
        rc, rn = r, r2
        for l, lay in enumerate(layers):
            if l == 0:
                lay.forward_fused(x, ids, w, y)
                continue
            xn = xa if l % 2 == 0 else xb
            lay.route_residual(rc, y, rn, xn, 1e-6, ids, w)
            lay.ffn(xn, ids, w, y)
            rc, rn = rn, rc
        C.moe_fp4_residual_rmsnorm(rc, y, xa, 1, H, 1e-6)  # the last layer's residual + norm

    if pf == "oracle":
        # the true ids of every (token, layer) of the timed tokens, from one untimed pass of
        # the same stack without prefetch
        true_ids = torch.empty((W + 2 * K, L, k), dtype=torch.int32, device=dev)
        pf_saved, pf = pf, "none"
        for t in range(W + 2 * K):
            x = xs[t:t + 1]
            C.moe_fp4_residual_init(x, r, 1, H)
            rc, rn = r, r2
            for l, lay in enumerate(layers):
                if l == 0:
                    lay.forward_fused(x, ids, w, y)
                else:
                    xn = xa if l % 2 == 0 else xb
                    lay.route_residual(rc, y, rn, xn, 1e-6, ids, w)
                    lay.ffn(xn, ids, w, y)
                    rc, rn = rn, rc
                true_ids[t, l].copy_(ids[0])
        torch.cuda.synchronize()
        pf = pf_saved
        log("oracle predictor: true ids recorded")

    for t in range(W):
        step(t)
    torch.cuda.synchronize()
    graph = None
    if args.mode == "graph":
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=cap):
            for t in range(W, W + K):
                step(t)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record()
    if graph is not None:
        graph.replay()
    else:
        for t in range(W, W + K):
            step(t)
    ev1.record()
    torch.cuda.synchronize()
    gpu_ms = ev0.elapsed_time(ev1)
    elapsed_s = max(gpu_ms / 1e3, 1e-9)
    token_bytes = L * (k * expert_bytes(H, I) + E * H * 2 + 2 * H * 2)
    log(f"timed {K} tokens x {L} layers ({args.mode}): {gpu_ms:.3f} ms -> {K / elapsed_s:.1f} tokens/s, "
        f"{token_bytes * K / elapsed_s / 1e9:.0f} GB/s")
    kernels = {}
    if not args.no_roofline_pass:
        C.moe_fp4_timing_reset()
        C.moe_fp4_timing_enable(True)
        for t in range(W + K, W + 2 * K):
            step(t)
        torch.cuda.synchronize()
        C.moe_fp4_timing_enable(False)
        for kind, name in enumerate(C.KERNEL_NAMES):
            n, ms = C.moe_fp4_timing_read(kind)
            if n:
                kernels[name] = {"launches": n, "avg_us": ms * 1e3 / n}
        C.moe_fp4_timing_reset()
        log("kernels: " + json.dumps(kernels))
    out = {
        "metric": "16-layer MoE decode tokens/s at batch 1 (+ achieved HBM GB/s)",
        "value": round(K / elapsed_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(gpu_ms / K, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "layers": L, "stack_route": args.stack_route, "hidden": H,
                   "intermediate": I, "experts": E,
                   "top_k": k, "batch_tokens": 1, "launch": args.mode, "parallelism": "none (1 GPU)",
                   "prefetch": pf, "prefetch_top": top if pf != "none" else 0,
                   "prefetch_matrices": args.prefetch_mats if pf != "none" else 0},
        "algorithmic_gbps": round(token_bytes * K / elapsed_s / 1e9, 1),
        "hbm_frac_step": round(token_bytes * K / elapsed_s / 1e9 / HBM_PEAK_GBS, 4),
        "bytes_per_step": token_bytes,
        "kernels": kernels,
    }
    if pf == "router":
        # how often the next layer's router on this layer's input names one of the next
        # layer's true experts (untimed, 20 tokens, everything on one stream)
        hits = total = 0
        for t in range(20):
            x = xs[t:t + 1]
            C.moe_fp4_residual_init(x, r, 1, H)
            rc, rn = r, r2
            x_l = x
            for l, lay in enumerate(layers):
                if l > 0:
                    xn = xa if l % 2 == 0 else xb
                    lay.route_residual(rc, y, rn, xn, 1e-6, ids, w)
                    x_l = xn
                else:
                    lay.route(x, ids, w)
                if l > 0:
                    truth = set(ids[0].tolist())
                    hits += len(truth & set(pred_ids[l, :top].tolist()))
                    total += top
                lay.ffn(x_l, ids, w, y)
                if l > 0:
                    rc, rn = rn, rc
                if l + 1 < L:
                    C.moe_fp4_route(x_l, layers[l + 1].w_router, 1, H, E, k, pred_ids[l + 1:l + 2],
                                    pred_w[l + 1:l + 2], pred_ws)
        out["prefetch_hit_rate"] = round(hits / max(total, 1), 4)
        log(f"router predictor: {hits} of {total} predicted experts were among the next layer's top-{k}")
    print(json.dumps(out), flush=True)
    return 0


def run_single_expert(args) -> int:
    """One SwiGLU expert at batch 1 (hidden 256, intermediate 128): microseconds per
    moe_fp4_expert_ffn call, stream-launched (launch latency bound, weights in L2)."""
    import torch

    from fp4_expert_ffn_amd import device as D
    from fp4_expert_ffn_amd import moe_fp4 as C
    from synth import moe_inputs as S

    C.lib()
    dev = torch.device("cuda:0")
    wl = S.WORKLOADS["expert_h256_i128"]
    H, I = wl.hidden, wl.inter
    K, W = min(args.steps, 2000), min(args.warmup, 100)
    packed = D.upload_experts(S.expert_source(wl, 0), 1, H, I, dev)
    layer = D.MoeFp4Layer(packed, 1, H, I, 1)
    x = D.upload_bf16(S.activations(wl, 0, 0), dev)
    ids = torch.zeros((1, 1), dtype=torch.int32, device=dev)
    w = torch.ones((1, 1), dtype=torch.float32, device=dev)
    y = torch.empty((1, H), dtype=torch.bfloat16, device=dev)
    layer._workspace(1, 1)
    for _ in range(W):
        layer.ffn(x, ids, w, y)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record()
    for _ in range(K):
        layer.ffn(x, ids, w, y)
    ev1.record()
    torch.cuda.synchronize()
    us = ev0.elapsed_time(ev1) * 1e3 / K
    log(f"single expert H{H} I{I}: {us:.2f} us per call (two kernel launches)")
    out = {"metric": "single-expert FFN call latency", "value": round(us, 3), "unit": "us/call",
           "n_gpus": 1, "steps": K, "warmup": W, "ms_per_step": round(us / 1e3, 6),
           "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic", "config": {"workload": wl.name, "hidden": H, "intermediate": I,
                                            "launch": "stream"}}
    print(json.dumps(out), flush=True)
    return 0


def run_shared_expert(args) -> int:
    """The FP8 SwiGLU shared expert (hidden 4096, intermediate 2880, E4M3 weights with one
    fp32 multiplier per 128 x 128 block) at batch 1: one fresh token per step, two kernel
    launches (gate/up + SwiGLU, then down). HBM-bound: 1 byte per weight."""
    import torch

    from fp4_expert_ffn_amd import moe_fp4 as C
    from synth import moe_inputs as S

    C.lib()
    dev = torch.device("cuda:0")
    H, I = 4096, 2880
    K, W = min(args.steps, 2000), min(args.warmup, 100)
    mats = [S.fp8_matrix(I, H, seed=1), S.fp8_matrix(I, H, seed=2), S.fp8_matrix(H, I, seed=3)]
    packed = []
    for codes, scales in mats:
        nb = C.moe_fp4_fp8_packed_bytes(codes.shape[0], codes.shape[1])
        p = torch.empty(nb, dtype=torch.uint8, device=dev)
        C.moe_fp4_fp8_pack(torch.from_numpy(codes).to(dev), torch.from_numpy(scales).to(dev),
                           codes.shape[0], codes.shape[1], p, nb)
        packed.append(p)
    n_x = W + 2 * K
    xs = (torch.randn((n_x, H), device=dev) * 0.5).to(torch.bfloat16)
    y = torch.empty((1, H), dtype=torch.bfloat16, device=dev)
    wsb = C.moe_fp4_shared_expert_workspace_bytes(1, I)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)

    def step(i: int) -> None:
        C.moe_fp4_shared_expert(xs[i:i + 1], 1, packed[0], packed[1], packed[2], H, I, y, ws, wsb)

    for i in range(W):
        step(i)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        for i in range(W, W + K):
            step(i)
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record()
    graph.replay()
    ev1.record()
    torch.cuda.synchronize()
    us = ev0.elapsed_time(ev1) * 1e3 / K
    weight_bytes = sum(C.moe_fp4_fp8_packed_bytes(c.shape[0], c.shape[1]) for c, _ in mats)
    alg = 3 * H * I + sum(s.size * 4 for _, s in mats) + 2 * H * 2 + 2 * I * 2
    kernels = {}
    C.moe_fp4_timing_reset()
    C.moe_fp4_timing_enable(True)
    for i in range(W + K, W + 2 * K):
        step(i)
    torch.cuda.synchronize()
    C.moe_fp4_timing_enable(False)
    n, ms = C.moe_fp4_timing_read(C.KERNEL_NAMES.index("fp8_gemv"))
    C.moe_fp4_timing_reset()
    if n:
        kernels["fp8_gemv"] = {"launches": n, "avg_us": ms * 1e3 / n}
    # the roofline kernel time: both launches of a step (gate/up and down share one kernel
    # kind), from the library's HIP events on the launch stream
    kern_us = 2 * kernels["fp8_gemv"]["avg_us"] if kernels else us
    log(f"FP8 shared expert H{H} I{I}: {us:.2f} us per token (graph replay), kernels "
        f"{kern_us:.2f} us, {alg / (kern_us * 1e-6) / 1e9:.0f} GB/s algorithmic")
    peaks = None if args.no_peaks else measure_peaks(torch, C, dev)
    achieved = alg / (kern_us * 1e-6) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                "kernel": "fp8_gemv (gate/up and down launches of a step)", "bytes_per_step": alg,
                "kernel_us_per_step": round(kern_us, 3), "packed_weight_bytes": weight_bytes}
    roofline = with_measured_peak(roofline, peaks)
    cpu = None
    if not args.no_cpu_baseline:
        from threadpoolctl import threadpool_limits

        from oracle import moe_oracle as O
        x_bits = xs[:2].view(torch.int16).cpu().numpy().view(np.uint16)
        with threadpool_limits(limits=1):
            t0 = time.perf_counter()
            O.shared_expert_fp8(x_bits, *mats)
            dt = time.perf_counter() - t0
        cpu = {"value": 2 / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
               "sample": f"2 tokens through the FP8 shared expert (fp64 NumPy, 1 thread), {dt:.1f} s"}
    out = {"metric": "FP8 shared-expert tokens/s at batch 1", "value": round(1e6 / us, 1),
           "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": W, "ms_per_step": round(us / 1e3, 6),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16 x fp8",
           "data": "synthetic", "config": {"workload": "shared_expert_fp8_h4096_i2880", "hidden": H,
                                            "intermediate": I, "launch": "graph"},
           "kernels": kernels, "measured_peaks": peaks, "roofline": roofline, "cpu_baseline": cpu}
    print(json.dumps(out), flush=True)
    return 0




def run_batched(args) -> int:
    """A multi-token step: top-k of the step's router logits (drawn directly, as the workload
    defines them) then moe_fp4_expert_ffn, which takes the small-M path below 24 tokens and
    the grouped GEMM path from 24 on. Fresh logits every step, so the experts read and their
    token counts change from step to step."""
    import torch

    from fp4_expert_ffn_amd import device as D
    from fp4_expert_ffn_amd import moe_fp4 as C
    from synth import moe_inputs as S

    C.lib()
    dev = torch.device("cuda:0")
    wl = S.WORKLOADS[args.workload]
    H, I, E, k, T = wl.hidden, wl.inter, wl.n_experts, wl.k, wl.tokens
    # bounded so one run stays within about a minute of GPU time
    K = min(args.steps, 100 if T <= 64 else 10)
    W = min(args.warmup, 10 if T <= 64 else 2)
    log(f"{wl.name}: uploading {E} experts")
    packed = D.upload_experts(S.expert_source(wl, 0), E, H, I, dev, chunk=32)
    layer = D.MoeFp4Layer(packed, E, H, I, k)
    n_lg = W + 2 * K
    lgs = torch.stack([torch.from_numpy(S.router_logits(wl, 0, i)) for i in range(n_lg)]).to(dev)
    xs = [D.upload_bf16(S.activations(wl, 0, i), dev) for i in range(2)]
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    y = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    layer._workspace(T, k)
    fp8 = args.act_terms == 1 and T >= 24
    path = C.PATH_GROUPED_FP8 if fp8 else None  # None: the automatic choice

    def step(i: int) -> None:
        C.moe_fp4_route_logits(lgs[i], T, E, k, ids, w)
        layer.ffn(xs[i % 2], ids, w, y, path=path)

    for i in range(W):
        step(i)
    torch.cuda.synchronize()
    graph = None
    if args.mode == "graph":
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=side):
            for i in range(W, W + K):
                step(i)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record()
    if graph is not None:
        graph.replay()
    else:
        for i in range(W, W + K):
            step(i)
    ev1.record()
    torch.cuda.synchronize()
    gpu_ms = ev0.elapsed_time(ev1)
    elapsed_s = max(gpu_ms / 1e3, 1e-9)

    # distinct experts per step (outside the timed region)
    distinct = []
    for i in range(W, W + K):
        C.moe_fp4_route_logits(lgs[i], T, E, k, ids, w)
        distinct.append(int(torch.unique(ids).numel()))
    d_avg = float(np.mean(distinct))
    pairs = T * k
    flops = pairs * 6.0 * H * I
    step_bytes = d_avg * expert_bytes(H, I) + 2 * T * H * 2 + T * E * 4 + pairs * 8
    tflops = flops * K / elapsed_s / 1e12
    log(f"timed {K} steps ({args.mode}): {gpu_ms:.3f} ms -> {gpu_ms / K:.3f} ms/step, "
        f"{tflops:.1f} TFLOP/s, {step_bytes * K / elapsed_s / 1e9:.0f} GB/s, {d_avg:.1f} experts/step")

    kernels = {}
    roofline = None
    if not args.no_roofline_pass:
        C.moe_fp4_timing_reset()
        C.moe_fp4_timing_enable(True)
        for i in range(W + K, W + 2 * K):
            step(i)
        torch.cuda.synchronize()
        C.moe_fp4_timing_enable(False)
        for kind, name in enumerate(C.KERNEL_NAMES):
            n, ms = C.moe_fp4_timing_read(kind)
            if n:
                kernels[name] = {"launches": n, "avg_us": ms * 1e3 / n}
        C.moe_fp4_timing_reset()
        gu = kernels.get("grouped_gate_up")
        sg = kernels.get("small_m_gate_up")
        if sg:
            # algorithmic bytes: each distinct expert's gate and up once, x read, h written
            t_s = sg["avg_us"] * 1e-6
            alg = d_avg * gate_up_bytes(H, I) + T * H * 2 + pairs * I * 2
            achieved = alg / t_s / 1e9
            roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                        "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                        "traffic": measured_traffic("gate_up_multi_kernel", wl.name),
                        "kernel": "small_m_gate_up", "bytes_per_launch": round(alg),
                        "avg_launch_us": round(sg["avg_us"], 3)}
        if gu:
            t_s = gu["avg_us"] * 1e-6
            if wl.tokens >= 32768:  # enough tokens per expert for a matrix-core bound
                achieved = pairs * 4.0 * H * I / t_s / 1e12
                roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_FP4_PEAK_TFLOPS,
                            "unit": "TFLOP/s", "frac": round(achieved / MFMA_FP4_PEAK_TFLOPS, 4),
                            # matrix-core time the operands imply: two E2M3 products per
                            # pair at the FP4 rate, or one E4M3 product at the FP8 rate
                            "mfma_busy_frac": round(achieved / MFMA_FP8_PEAK_TFLOPS if fp8
                                                    else 2 * achieved / MFMA_FP4_PEAK_TFLOPS, 4),
                            "traffic": None, "kernel": "grouped_gate_up",
                            "flops_per_launch": pairs * 4.0 * H * I, "avg_launch_us": round(gu["avg_us"], 3)}
            else:
                alg = grouped_gate_up_bytes(d_avg, T, k, H, I, fp8)
                achieved = alg / t_s / 1e9
                roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                            "traffic": None if fp8 else measured_traffic("gemm_gate_up_kernel", wl.name),
                            "kernel": "grouped_gate_up", "bytes_per_launch": round(alg),
                            "avg_launch_us": round(gu["avg_us"], 3)}
        log("kernels: " + json.dumps(kernels))

    pct = step_percentiles(torch, step, range(W + K, W + 2 * K))
    log(f"per-step us (stream): {json.dumps(pct)}")
    decode_pct = None
    if T < 24:  # the one-pair-at-a-time decode kernels on the same steps, for comparison
        def step_decode(i: int) -> None:
            C.moe_fp4_route_logits(lgs[i], T, E, k, ids, w)
            layer.ffn(xs[i % 2], ids, w, y, path=1)
        decode_pct = step_percentiles(torch, step_decode, range(W + K, W + 2 * K))
        log(f"per-step us with the decode path (stream): {json.dumps(decode_pct)}")
    peaks = None if args.no_peaks else measure_peaks(torch, C, dev)
    roofline = with_measured_peak(roofline, peaks)

    cpu = None
    if not args.no_cpu_baseline:
        from threadpoolctl import threadpool_limits

        from oracle import moe_oracle as O

        n_tok = min(args.cpu_tokens, 8, T)
        lg = S.router_logits(wl, 0, W).astype(np.float64)[:n_tok]
        x_bits = S.activations(wl, 0, W % 2)[:n_tok]
        with threadpool_limits(limits=1):
            t0 = time.perf_counter()
            ids_o, w_o = O.topk_softmax(lg, k)
            O.expert_ffn(x_bits, ids_o, w_o, S.expert_source(wl, 0), E, H, I)
            dt = time.perf_counter() - t0
        cpu = {"value": n_tok / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
               "sample": f"{n_tok} tokens of one step (top-k + expert FFN, fp64 NumPy, 1 thread), {dt:.1f} s"}

    small = T < 24
    out = {
        "metric": "multi-token decode tokens/s" if small else "batched FP4 TFLOP/s",
        "value": round(T * K / elapsed_s, 1) if small else round(tflops, 2),
        "unit": "tokens/s" if small else "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(gpu_ms / K, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 x fp4" if small else ("fp8 x fp4" if fp8 else "fp8(hi+lo) x fp4"),
        "data": "synthetic",
        "config": {"workload": wl.name, "hidden": H, "intermediate": I, "experts": E, "top_k": k,
                   "tokens": T, "routing": wl.routing, "launch": args.mode, "parallelism": "none (1 GPU)",
                   "activations": "bf16" if small else ("MXFP8 one term" if fp8 else "MXFP6 hi + lo")},
        "tokens_per_s": round(T * K / elapsed_s, 1),
        "tflops": round(tflops, 2),
        "decode_path_step_us": decode_pct,
        "algorithmic_gbps": round(step_bytes * K / elapsed_s / 1e9, 1),
        "distinct_experts_per_step": d_avg,
        "step_us": pct,
        "kernels": kernels,
        "measured_peaks": peaks,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
