#!/usr/bin/env python3
"""Throughput of the batch-1 fused dequantise + GEMV on one MI355X.

One step = one Q4_K GEMV y = x . dequant(W)^T at N = 4096 rows, K = 14336 (the
Llama-8B down-projection shape) on synthetic seeded weights, i.e. every row of
the hot path: weight stream, activation staging, block decode, factored dot,
reductions, store.  Inputs are resident in HBM before the timed region.  Each
step reads a different one of R copies of the weights (R * 33 MB well above
the 256 MB Infinity Cache), so every launch streams its weights from HBM.

Printed: ONE JSON line with the metric (achieved HBM GB/s of the kernel over
the algorithmic bytes weights + x + y), the roofline object of the dominant
kernel, the CPU baseline (the fp64 oracle on the host cores) and extra context
(pure-read ceiling over the same bytes, the other formats' shapes, the dense
bf16 GEMV of the same shape, the general output stage, row materialisation,
prefill on the matrix cores and a Llama-8B per-token sweep).
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

METRIC = "achieved HBM GB/s (% of ~8 TB/s peak), M=1 Q4_K GEMV N=4096 K=14336"
HBM_PEAK_GBPS = 8000.0

# (format, rows, K, description) of the measured shapes
MAIN = ("q4k", 4096, 14336, "Q4_K GEMV M=1, N=4096 x K=14336 (Llama-8B MLP down projection)")
EXTRA = [
    ("q4k", 14336, 4096, "Q4_K GEMV M=1, N=14336 x K=4096 (gate/up)"),
    ("q4k", 4096, 4096, "Q4_K GEMV M=1, N=4096 x K=4096"),
    ("nvfp4", 4096, 14336, "NVFP4 W4A16 GEMV M=1, N=4096 x K=14336"),
    ("tq1", 14336, 4096, "TQ1_0 GEMV M=1, N=14336 x K=4096"),
    ("bf16", 4096, 14336, "dense bf16 GEMV M=1, N=4096 x K=14336 (the Mojo fp4_gemv page's comparison)"),
]
CASE_SEED = {("q4k", 4096, 4096): 0, ("q4k", 14336, 4096): 1, ("q4k", 4096, 14336): 1,
             ("nvfp4", 4096, 14336): 2, ("tq1", 14336, 4096): 3, ("bf16", 4096, 14336): 4}
# The Mojo fp4_gemv page reports its NVFP4 GEMV 1.53x faster than a bf16 GEMV
# at N = 4096, K = 14336 on an Apple M5 Max (context, not a target).
PAGE_FP4_VS_BF16 = 1.53


def algorithmic_bytes(fmt: str, n: int, k: int) -> int:
    """Bytes the method must move once: packed weights + x (2 B/elem) + y (fp32)."""
    from dequant_gemv_amd import synth

    return synth.weight_bytes(fmt, n, k) + 2 * k + 4 * n


TRAFFIC_SUMMARY = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                               "q4k_gemv_4096x14336_hbm_bytes.md")


def measured_traffic(build_id: str):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE + WRITE_SIZE
    summary, only if it was taken with this very build of the library."""
    try:
        fields = dict(line.split(":", 1) for line in open(TRAFFIC_SUMMARY) if ":" in line)
    except OSError:
        return None
    if fields.get("traffic_build_id", "").strip() != build_id:
        return None
    try:
        return int(fields["traffic_bytes_per_launch"].strip())
    except (KeyError, ValueError):
        return None


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def measure_gpu(fmt, n, k, steps, warmup, rotate, launch, with_ceiling=True):
    import numpy as np
    import torch

    from dequant_gemv_amd import qgemv, synth

    dev = torch.device("cuda:0")
    seed = CASE_SEED.get((fmt, n, k), 9)
    w_host = synth.weights(fmt, n, k, synth.W_SEED + seed)
    x_host = synth.activations(fmt, k, synth.X_SEED + seed)
    w0 = torch.from_numpy(w_host).to(dev)
    ws = [w0] + [w0.clone() for _ in range(rotate - 1)]
    x = torch.from_numpy(x_host.view(np.int16).copy()).to(dev)
    y = torch.empty(n, dtype=torch.float32, device=dev)
    fn = qgemv.GEMV[fmt]
    stream = torch.cuda.Stream()
    s_handle = stream.cuda_stream
    nbytes = algorithmic_bytes(fmt, n, k)

    def one(i):
        fn(ws[i % rotate], x, y, n, k, s_handle)

    with torch.cuda.stream(stream):
        for i in range(rotate):  # first touch of every copy
            one(i)
    torch.cuda.synchronize()

    graph = None
    if launch == "graph":
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            for i in range(rotate):
                one(i)
        torch.cuda.synchronize()
        # the untimed warm-up steps, as replays of the same graph right before
        # the timed region (the GPU leaves its idle state before timing starts)
        with torch.cuda.stream(stream):
            for _ in range(max(1, warmup // rotate)):
                graph.replay()
        torch.cuda.synchronize()
    else:
        with torch.cuda.stream(stream):
            for i in range(warmup):
                one(i)
        torch.cuda.synchronize()

    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    with torch.cuda.stream(stream):
        if graph is not None:
            for _ in range(steps // rotate):
                graph.replay()
            for i in range(steps % rotate):
                one(i)
        else:
            for i in range(steps):
                one(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev_ms = ev0.elapsed_time(ev1)
    res = {
        "wall_s": wall,
        "event_ms": ev_ms,
        "us_per_launch_event": 1e3 * ev_ms / steps,
        "us_per_step_wall": 1e6 * wall / steps,
        "bytes": nbytes,
    }
    res["gbps_event"] = nbytes / (res["us_per_launch_event"] * 1e-6) / 1e9
    res["gbps_wall"] = nbytes / (res["us_per_step_wall"] * 1e-6) / 1e9

    if with_ceiling:
        wb = synth.weight_bytes(fmt, n, k)
        sink = torch.empty(qgemv.qgemv_read_sink_len(wb), dtype=torch.float32, device=dev)
        cg = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            for i in range(rotate):
                qgemv.qgemv_read_ceiling(ws[i], wb, sink, s_handle)
        torch.cuda.synchronize()
        with torch.cuda.graph(cg, stream=stream):
            for i in range(rotate):
                qgemv.qgemv_read_ceiling(ws[i], wb, sink, s_handle)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            for _ in range(max(1, warmup // rotate)):
                cg.replay()
        reps = max(1, steps // rotate)
        torch.cuda.synchronize()
        ev0.record(stream)
        with torch.cuda.stream(stream):
            for _ in range(reps):
                cg.replay()
        ev1.record(stream)
        torch.cuda.synchronize()
        us = 1e3 * ev0.elapsed_time(ev1) / (reps * rotate)
        res["ceiling_us"] = us
        res["ceiling_gbps"] = wb / (us * 1e-6) / 1e9
    del ws
    torch.cuda.empty_cache()
    return res


# Llama-8B per-token decode: per layer Q, K, V, O (attention), gate, up, down
# (MLP), 32 layers, then lm_head: 225 batch-1 GEMVs (rows, K).
LLAMA8B_LAYER = [("q", 4096, 4096), ("k", 1024, 4096), ("v", 1024, 4096), ("o", 4096, 4096),
                 ("gate", 14336, 4096), ("up", 14336, 4096), ("down", 4096, 14336)]
LLAMA8B_HEAD = ("lm_head", 128256, 4096)
# The same layer with the GEMVs that share an activation row stored as one
# matrix (Q, K, V rows concatenated; gate and up rows concatenated): 4 launches
# per layer instead of 7, the same weight bytes.
LLAMA8B_LAYER_FUSED = [("qkv", 6144, 4096), ("o", 4096, 4096), ("gate_up", 28672, 4096), ("down", 4096, 14336)]
FUSED_ROLE_OF = {"qkv": "q", "gate_up": "gate"}
SWEEP_MIXES = {
    # attention and lm_head Q4_K, gate/up TQ1_0, down NVFP4
    "mixed": {"q": "q4k", "k": "q4k", "v": "q4k", "o": "q4k", "gate": "tq1", "up": "tq1",
              "down": "nvfp4", "lm_head": "q4k"},
    "q4k": None, "nvfp4": None, "tq1": None,  # every matrix in one format
}


def measure_sweep(mix: str, tokens: int, layers: int = 32):
    """One token = the 225 GEMVs of a Llama-8B decode step, each layer with its
    own weight buffers (cloned on the device from one generated matrix per
    shape, so every launch reads cold bytes: ~2.9 GB for the mixed sweep),
    captured in one HIP graph and replayed per token.  A mix named "<mix>-fused"
    stores Q/K/V and gate/up as concatenated matrices (129 launches)."""
    import numpy as np
    import torch

    from dequant_gemv_amd import qgemv, synth

    dev = torch.device("cuda:0")
    fused = mix.endswith("-fused")
    mix = mix[: -len("-fused")] if fused else mix
    layer_shapes = LLAMA8B_LAYER_FUSED if fused else LLAMA8B_LAYER
    fmt_of = dict(SWEEP_MIXES[mix] or {r: mix for r, _, _ in LLAMA8B_LAYER + [LLAMA8B_HEAD]})
    for role, base in FUSED_ROLE_OF.items():
        fmt_of[role] = fmt_of[base]
    proto, xs = {}, {}
    for role, n, k in layer_shapes + [LLAMA8B_HEAD]:
        fmt = fmt_of[role]
        key = (fmt, n, k)
        if key not in proto:
            seed = 3000 + len(proto)
            proto[key] = torch.from_numpy(synth.weights(fmt, n, k, seed)).to(dev)
            xs[key] = torch.from_numpy(synth.activations(fmt, k, seed + 1).view(np.int16).copy()).to(dev)
    calls, total_bytes = [], 0
    for layer in range(layers):
        for role, n, k in layer_shapes:
            fmt = fmt_of[role]
            w = proto[(fmt, n, k)].clone()
            calls.append((fmt, w, xs[(fmt, n, k)], torch.empty(n, dtype=torch.float32, device=dev), n, k))
            total_bytes += algorithmic_bytes(fmt, n, k)
    role, n, k = LLAMA8B_HEAD
    fmt = fmt_of[role]
    calls.append((fmt, proto[(fmt, n, k)], xs[(fmt, n, k)], torch.empty(n, dtype=torch.float32, device=dev), n, k))
    total_bytes += algorithmic_bytes(fmt, n, k)
    stream = torch.cuda.Stream()
    h = stream.cuda_stream

    def token():
        for fmt, w, x, y, n, k in calls:
            qgemv.GEMV[fmt](w, x, y, n, k, h)

    with torch.cuda.stream(stream):
        token()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        token()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for _ in range(3):
            g.replay()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    with torch.cuda.stream(stream):
        for _ in range(tokens):
            g.replay()
    ev1.record(stream)
    torch.cuda.synchronize()
    us = 1e3 * ev0.elapsed_time(ev1) / tokens
    res = {
        "workload": f"Llama-8B decode step, {len(calls)} GEMVs ({layers} layers + lm_head), formats: {mix}"
                    + (", Q/K/V and gate/up as concatenated matrices" if fused else ""),
        "gemvs_per_token": len(calls),
        "algorithmic_bytes_per_token": total_bytes,
        "us_per_token": round(us, 2),
        "gbps": round(total_bytes / (us * 1e-6) / 1e9, 1),
        "pct_of_hbm_peak": round(100 * total_bytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 1),
        "tokens_timed": tokens,
    }
    del calls, proto, xs, g
    torch.cuda.empty_cache()
    return res


def time_graph(launch, count, steps, warmup, stream, min_warm_ms=0.0, min_timed_ms=0.0):
    """Average microseconds of one of `count` distinct launches (launch(i, h)
    enqueues number i on stream handle h), captured together in one HIP graph
    and replayed; every copy first touched once, eagerly, and the timed
    replays queued right behind the warm-up replays.  With min_warm_ms /
    min_timed_ms the warm-up and the timed region also last at least that
    long (long kernels: the clocks take several ms of load to settle)."""
    import math

    import torch

    h = stream.cuda_stream
    with torch.cuda.stream(stream):
        for i in range(count):
            launch(i, h)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for i in range(count):
            launch(i, h)
    torch.cuda.synchronize()
    warm_reps, reps = max(1, warmup // count), max(1, steps // count)
    if min_warm_ms > 0 or min_timed_ms > 0:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        with torch.cuda.stream(stream):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        per = max(e0.elapsed_time(e1), 1e-3)  # ms per replay
        warm_reps = max(warm_reps, math.ceil(min_warm_ms / per))
        reps = max(reps, math.ceil(min_timed_ms / per))
    with torch.cuda.stream(stream):
        for _ in range(warm_reps):
            g.replay()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # no synchronize between the warm-up replays and the timed ones: after an
    # idle gap the part's clocks ramp up again over the first ~0.75 ms of work
    ev0.record(stream)
    with torch.cuda.stream(stream):
        for _ in range(reps):
            g.replay()
    ev1.record(stream)
    torch.cuda.synchronize()
    us = 1e3 * ev0.elapsed_time(ev1) / (reps * count)
    del g
    return us


def measure_epilogue(steps, warmup, rotate):
    """The main Q4_K shape through the general output stage: fp16 y updated in
    place, y = v + 0.5 y (a residual-style accumulate), against the plain call."""
    import numpy as np
    import torch

    from dequant_gemv_amd import qgemv, synth

    fmt, n, k, _ = MAIN
    dev = torch.device("cuda:0")
    seed = CASE_SEED[(fmt, n, k)]
    w0 = torch.from_numpy(synth.weights(fmt, n, k, synth.W_SEED + seed)).to(dev)
    ws = [w0] + [w0.clone() for _ in range(rotate - 1)]
    x = torch.from_numpy(synth.activations(fmt, k, synth.X_SEED + seed).view(np.int16).copy()).to(dev)
    y16 = torch.zeros(n, dtype=torch.float16, device=dev)
    y32 = torch.empty(n, dtype=torch.float32, device=dev)
    stream = torch.cuda.Stream()
    us_ex = time_graph(lambda i, h: qgemv.qgemv_q4k_ex(ws[i], x, y16, n, k, 1.0, 0.5, y16, h),
                       rotate, steps, warmup, stream)
    us_plain = time_graph(lambda i, h: qgemv.qgemv_q4k(ws[i], x, y32, n, k, h), rotate, steps, warmup, stream)
    del ws
    torch.cuda.empty_cache()
    return {
        "workload": f"Q4_K GEMV M=1, N={n} x K={k}, y (fp16) = x.W^T + 0.5 y in place",
        "us_per_gemv": round(us_ex, 3),
        "us_per_gemv_plain_fp32": round(us_plain, 3),
        "overhead_us": round(us_ex - us_plain, 3),
    }


ROWS_CASES = [
    # (format, rows of W, K, gathered rows or None for all, output type, description)
    ("q4k", 4096, 14336, None, "f16", "Q4_K 4096 x 14336 materialised to fp16"),
    ("nvfp4", 4096, 14336, None, "bf16", "NVFP4 4096 x 14336 materialised to bf16"),
    ("tq1", 14336, 4096, None, "f16", "TQ1_0 14336 x 4096 materialised to fp16"),
    ("q4k", 128256, 4096, 512, "f16", "Q4_K 128256 x 4096 table, 512 random rows to fp16 (prefill embedding lookup)"),
]


def measure_rows(steps, warmup, rotate):
    """Row materialisation throughput: HBM bytes = packed bytes read + outputs
    written (+ the int32 indices) per call."""
    import numpy as np
    import torch

    from dequant_gemv_amd import qgemv, synth

    dev = torch.device("cuda:0")
    out = {}
    for fmt, n, k, nsel, dtype, desc in ROWS_CASES:
        w0 = torch.from_numpy(synth.weights(fmt, n, k, 4100)).to(dev)
        copies = max(1, min(rotate, (1 << 30) // w0.numel())) if nsel is None else 1
        ws = [w0] + [w0.clone() for _ in range(copies - 1)]
        rows = None
        nrows = n
        if nsel is not None:
            rows = torch.from_numpy(np.random.default_rng(4101).integers(0, n, nsel).astype(np.int32)).to(dev)
            nrows = nsel
        tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype]
        o = torch.empty((nrows, k), dtype=tdt, device=dev)
        # outputs rotate too (all-rows cases), so no call rewrites lines another left in the cache
        ocount = max(1, min(copies, (1 << 30) // (o.numel() * o.element_size())))
        os_ = [o] + [torch.empty_like(o) for _ in range(ocount - 1)]
        fn = qgemv.GET_ROWS[fmt]
        stream = torch.cuda.Stream()
        us = time_graph(lambda i, h: fn(ws[i % copies], n, k, rows, nrows, os_[i % ocount], h), max(copies, 8),
                        max(64, steps // 8), max(64, warmup // 8), stream)
        per_row = synth.weight_bytes(fmt, 1, k)
        nbytes = nrows * per_row + nrows * k * o.element_size() + (4 * nrows if rows is not None else 0)
        out[f"{fmt}_{n}x{k}_{nsel or 'all'}_{dtype}"] = {
            "workload": desc,
            "us_per_call": round(us, 3),
            "bytes_per_call": nbytes,
            "gbps": round(nbytes / (us * 1e-6) / 1e9, 1),
            "pct_of_hbm_peak": round(100 * nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 1),
        }
        log(f"[bench] rows {desc}: {us:.3f} us, {out[list(out)[-1]]['gbps']} GB/s")
        del ws, o, os_
        torch.cuda.empty_cache()
    return out


MFMA_PEAK_TFLOPS = 2500.0  # dense fp16 / bf16 matrix-core peak of the part

PREFILL_CASES = [
    # (format, tokens, weight rows, K)
    ("q4k", 512, 4096, 14336), ("q4k", 512, 14336, 4096), ("q4k", 4096, 14336, 4096),
    ("q4k", 4096, 4096, 14336), ("q4k", 1024, 14336, 4096),
    ("nvfp4", 512, 4096, 14336), ("nvfp4", 512, 14336, 4096),
    ("tq1", 512, 4096, 14336), ("tq1", 512, 14336, 4096),
]


# prefill launches run 0.1-0.6 ms: warm up and time each case for at least
# this long, so that every case is timed at settled clocks
PREFILL_WARM_MS = 25.0
PREFILL_TIMED_MS = 15.0


def measure_prefill(steps, warmup, cases=None, unfused=True):
    """Prefill (many tokens): y = X . dequant(W)^T on the matrix cores, in
    TFLOP/s of 2 T N K flops; for Q4_K also the unfused path (materialise W
    as fp16 with the row kernel, then the library fp16 GEMM) for comparison."""
    import math

    import numpy as np
    import torch

    from dequant_gemv_amd import qgemv, synth

    dev = torch.device("cuda:0")
    out = {}
    stream = torch.cuda.Stream()
    for fmt, t, n, k in cases or PREFILL_CASES:
        w0 = torch.from_numpy(synth.weights(fmt, n, k, 4200)).to(dev)
        ws = [w0] + [w0.clone() for _ in range(3)]
        xs = np.stack([synth.activations(fmt, k, 4300 + i) for i in range(t)])
        x = torch.from_numpy(xs.view(np.int16)).to(dev)
        y = torch.empty((t, n), dtype=torch.float32, device=dev)
        fn = qgemv.GEMM[fmt]
        us = time_graph(lambda i, h: fn(ws[i], x, y, t, n, k, h), 4, max(16, steps // 80), max(8, warmup // 80), stream,
                        PREFILL_WARM_MS, PREFILL_TIMED_MS)
        flops = 2.0 * t * n * k
        rec = {
            "workload": f"{fmt} prefill, {t} tokens x {n} rows x K {k}",
            "us": round(us, 2),
            "tflops": round(flops / us / 1e6, 1),
            "pct_of_mfma_peak": round(100 * flops / us / 1e6 / MFMA_PEAK_TFLOPS, 1),
        }
        if fmt == "q4k" and unfused:
            wf = torch.empty((n, k), dtype=torch.float16, device=dev)
            us_rows = time_graph(lambda i, h: qgemv.qget_rows_q4k(ws[i], n, k, None, n, wf, h), 4,
                                 max(16, steps // 80), max(8, warmup // 80), stream, PREFILL_WARM_MS,
                                 PREFILL_TIMED_MS)
            xf = x.view(torch.float16)
            with torch.cuda.stream(stream):  # first calls (library set-up) before the estimate
                for _ in range(3):
                    torch.matmul(xf, wf.t())
            torch.cuda.synchronize()
            ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            ev0.record(stream)
            with torch.cuda.stream(stream):
                torch.matmul(xf, wf.t())
            ev1.record(stream)
            torch.cuda.synchronize()
            per = max(ev0.elapsed_time(ev1), 1e-3)  # ms, a first estimate
            n_mm = max(10, math.ceil(PREFILL_TIMED_MS / per))
            with torch.cuda.stream(stream):
                for _ in range(max(3, math.ceil(PREFILL_WARM_MS / per))):
                    torch.matmul(xf, wf.t())
            ev0.record(stream)  # right behind the warm-up products, as in time_graph
            with torch.cuda.stream(stream):
                for _ in range(n_mm):
                    torch.matmul(xf, wf.t())
            ev1.record(stream)
            torch.cuda.synchronize()
            us_mm = 1e3 * ev0.elapsed_time(ev1) / n_mm
            rec["unfused_us"] = round(us_rows + us_mm, 2)
            rec["unfused_note"] = (f"fp16 materialisation {us_rows:.1f} us + library fp16 GEMM {us_mm:.1f} us "
                                   f"({flops / us_mm / 1e6:.0f} TFLOP/s)")
            del wf
        out[f"{fmt}_{t}x{n}x{k}"] = rec
        log(f"[bench] prefill {fmt} T={t} {n}x{k}: {us:.1f} us, {rec['tflops']} TFLOP/s"
            + (f" (unfused {rec['unfused_us']} us)" if "unfused_us" in rec else ""))
        del ws, x, y
        torch.cuda.empty_cache()
    return out


def measure_ceiling_sweep():
    """Per-launch time of the pure-read kernel against the bytes it reads (a
    graph of 32 launches over 32 buffers, as for the metric), and the least-
    squares fit t = fixed + bytes / bandwidth over the launches of >= 4 MB:
    the fixed part is what one launch costs beyond streaming its bytes."""
    import numpy as np
    import torch

    from dequant_gemv_amd import qgemv

    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream()
    points = []
    for mb in (0.0625, 0.25, 1, 4, 8, 16, 33.0752, 64, 128):
        nbytes = int(mb * 1e6) // 16 * 16
        bufs = [torch.ones(nbytes, dtype=torch.uint8, device=dev) for _ in range(32)]
        sink = torch.zeros(qgemv.qgemv_read_sink_len(nbytes), dtype=torch.float32, device=dev)
        us = time_graph(lambda i, h: qgemv.qgemv_read_ceiling(bufs[i], nbytes, sink, h), 32, 3200, 1280, stream)
        points.append({"bytes": nbytes, "us": round(us, 3), "gbps": round(nbytes / us / 1e3, 1)})
        log(f"[bench] read {nbytes / 1e6:.3f} MB: {us:.3f} us/launch, {nbytes / us / 1e3:.1f} GB/s")
        del bufs, sink
        torch.cuda.empty_cache()
    b = np.array([p["bytes"] for p in points if p["bytes"] >= 4e6], dtype=np.float64)
    t = np.array([p["us"] for p in points if p["bytes"] >= 4e6], dtype=np.float64)
    (fixed, per_byte), *_ = np.linalg.lstsq(np.vstack([np.ones_like(b), b]).T, t, rcond=None)
    return {"points": points, "fit_fixed_us": round(float(fixed), 3), "fit_gbps": round(1e-3 / float(per_byte), 1)}


def cpu_baseline(fmt, n, k, budget_s=10.0):
    """The fp64 oracle as it stands, all host cores, on the same workload."""
    import numpy as np

    import oracle
    from dequant_gemv_amd import synth

    seed = CASE_SEED.get((fmt, n, k), 9)
    w = synth.weights(fmt, n, k, synth.W_SEED + seed)
    x = synth.activations(fmt, k, synth.X_SEED + seed)
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    cores = min(cores, int(os.environ.get("OMP_NUM_THREADS", cores)))
    oracle.set_threads(cores)
    oracle.gemv(fmt, w, x, n, k)  # warm-up
    times = []
    t_start = time.perf_counter()
    while len(times) < 3 or (time.perf_counter() - t_start) * cores < budget_s and len(times) < 50:
        t0 = time.perf_counter()
        oracle.gemv(fmt, w, x, n, k)
        times.append(time.perf_counter() - t0)
    t = statistics.median(times)
    return {
        "value": algorithmic_bytes(fmt, n, k) / t / 1e9,
        "unit": "GB/s",
        "cores": oracle.threads(),
        "kind": "oracle",
        "sample": f"full {n}x{k} {fmt} matrix, median of {len(times)} runs "
                  f"({t * 1e3:.1f} ms each, fp64 scalar dequantise-then-dot, OpenMP over rows)",
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3200)
    ap.add_argument("--warmup", type=int, default=1280)
    ap.add_argument("--rotate", type=int, default=32, help="distinct weight copies cycled through")
    ap.add_argument("--launch", choices=["graph", "eager"], default="graph")
    ap.add_argument("--no-extra", action="store_true", help="skip the other formats' shapes")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--sweep", default="mixed,mixed-fused",
                    help="Llama-8B per-token sweep(s) to time among mixed,q4k,nvfp4,tq1, each also as "
                         "<mix>-fused (comma list; 'none' to skip)")
    ap.add_argument("--sweep-tokens", type=int, default=20)
    ap.add_argument("--fmt", default=None, help="measure only this format (q4k, nvfp4, tq1, f16, bf16) at N,K")
    ap.add_argument("--n", type=int, default=None)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 64 MiB device copy (a known-size reference for the HBM byte counters)")
    ap.add_argument("--k", type=int, default=None)
    ap.add_argument("--prefill-only", default=None, metavar="FMT,T,N,K",
                    help="time only this prefill case (e.g. q4k,4096,14336,4096) and print its record")
    ap.add_argument("--ceiling-sweep", action="store_true",
                    help="time only the pure-read kernel over 0.06-128 MB per launch and fit t = fixed + bytes / BW")
    ap.add_argument("--rows-only", action="store_true",
                    help="time only the row-materialisation cases (after --calibrate-copy if given) and print them")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
              "(the path shards by rows with no exchange; see the design notes)", file=sys.stderr)
        sys.exit(2)

    import torch

    from dequant_gemv_amd import build, qgemv

    # Provenance: the library must be built from the sources in this tree.
    want, have = build.build_id(), qgemv.qgemv_build_id()
    if want != have:
        print(f"libqgemv.so build id {have} does not match the sources ({want}); rebuild", file=sys.stderr)
        sys.exit(3)

    if args.ceiling_sweep:
        print(json.dumps({"ceiling_sweep": measure_ceiling_sweep(), "build_id": have}), flush=True)
        return

    if args.prefill_only:
        f, t, n, k = args.prefill_only.split(",")
        res = measure_prefill(args.steps, args.warmup, [(f, int(t), int(n), int(k))], unfused=False)
        print(json.dumps({"prefill": res, "build_id": have}), flush=True)
        return

    if args.calibrate_copy:
        src = torch.empty(64 << 20, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(8):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log("[bench] calibration: 8 copies of 64 MiB (read 65536 KiB + write 65536 KiB each)")

    if args.rows_only:
        print(json.dumps({"get_rows": measure_rows(args.steps, args.warmup, args.rotate), "build_id": have}),
              flush=True)
        return

    fmt, n, k, desc = MAIN
    if args.fmt:
        fmt, n, k, desc = args.fmt, args.n or n, args.k or k, f"{args.fmt} GEMV M=1, N={args.n or n} x K={args.k or k}"
    log(f"[bench] build {have} on {torch.cuda.get_device_name(0)}; main {fmt} {n}x{k}")
    main_res = measure_gpu(fmt, n, k, args.steps, args.warmup, args.rotate, args.launch)
    log(f"[bench] main: {main_res['us_per_launch_event']:.3f} us/launch, {main_res['gbps_event']:.1f} GB/s "
        f"(ceiling {main_res['ceiling_gbps']:.1f} GB/s)")

    extra = {}
    if not args.no_extra and not args.fmt:
        for efmt, en, ek, edesc in EXTRA:
            r = measure_gpu(efmt, en, ek, max(args.rotate, args.steps // 4), args.warmup, args.rotate, args.launch)
            extra[f"{efmt}_{en}x{ek}"] = {
                "workload": edesc,
                "us_per_gemv": round(r["us_per_launch_event"], 3),
                "gbps": round(r["gbps_event"], 1),
                "pct_of_hbm_peak": round(100 * r["gbps_event"] / HBM_PEAK_GBPS, 1),
                "read_ceiling_gbps": round(r["ceiling_gbps"], 1),
            }
            log(f"[bench] {efmt} {en}x{ek}: {r['us_per_launch_event']:.3f} us, {r['gbps_event']:.1f} GB/s")

    fp4_vs_bf16 = None
    if "nvfp4_4096x14336" in extra and "bf16_4096x14336" in extra:
        fp4_vs_bf16 = {
            "speedup": round(extra["bf16_4096x14336"]["us_per_gemv"] / extra["nvfp4_4096x14336"]["us_per_gemv"], 3),
            "bytes_ratio": round(algorithmic_bytes("bf16", 4096, 14336) / algorithmic_bytes("nvfp4", 4096, 14336), 3),
            "page_speedup_apple_m5_max": PAGE_FP4_VS_BF16,
        }
        log(f"[bench] NVFP4 vs bf16 at 4096x14336: {fp4_vs_bf16['speedup']}x")

    epilogue = rows_res = prefill_res = None
    if not args.no_extra and not args.fmt:
        epilogue = measure_epilogue(max(args.rotate, args.steps // 4), args.warmup, args.rotate)
        log(f"[bench] epilogue: {epilogue['us_per_gemv']} us (plain {epilogue['us_per_gemv_plain_fp32']} us)")
        rows_res = measure_rows(args.steps, args.warmup, args.rotate)
        prefill_res = measure_prefill(args.steps, args.warmup)

    sweeps = {}
    if not args.no_extra and not args.fmt and args.sweep != "none":
        for mix in args.sweep.split(","):
            r = measure_sweep(mix, args.sweep_tokens)
            sweeps[mix] = r
            log(f"[bench] sweep {mix}: {r['us_per_token']} us/token, {r['gbps']} GB/s over {r['gemvs_per_token']} GEMVs")

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(fmt, n, k)
        log(f"[bench] cpu oracle: {cpu['value']:.2f} GB/s on {cpu['cores']} threads")

    value = main_res["gbps_wall"]
    achieved = main_res["gbps_event"]
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(main_res["us_per_step_wall"] / 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": desc,
            "format": fmt, "n": n, "k": k,
            "algorithmic_bytes_per_gemv": main_res["bytes"],
            "rotated_weight_copies": args.rotate,
            "launch": "hipGraph of %d launches" % args.rotate if args.launch == "graph" else "eager",
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": measured_traffic(have) if (fmt, n, k) == MAIN[:3] else None,
        },
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "us_per_gemv": round(main_res["us_per_launch_event"], 3),
        "read_ceiling": {"gbps": round(main_res["ceiling_gbps"], 1), "us": round(main_res["ceiling_us"], 3),
                         "note": "pure dwordx4 read of the same weight bytes, same rotation"},
        "cpu_baseline": cpu,
        "other_shapes": extra,
        "fp4_vs_bf16": fp4_vs_bf16,
        "epilogue": epilogue,
        "get_rows": rows_res,
        "prefill": prefill_res,
        "decode_sweep": sweeps,
        "build_id": have,
        "gpu": torch.cuda.get_device_name(0),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
