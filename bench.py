#!/usr/bin/env python3
"""Throughput of the batch-1 fused dequantise + GEMV on one MI355X.

One step = one Q4_K GEMV y = x . dequant(W)^T at N = 4096 rows, K = 14336 (the
Llama-8B down-projection shape) on synthetic seeded weights, i.e. every row of
the hot path: weight stream, activation staging, block decode, factored dot,
reductions, store.  Inputs are resident in HBM before the timed region.

The timed region is ONE replay of a captured HIP graph of exactly --steps
dependent launches; launch i reads weight copy i mod C with C = max(16,
min(steps, 32)) distinct copies (>= 529 MB, above the 256 MB Infinity Cache),
so every launch streams its weights from HBM.  It is bracketed by HIP events
on the launch stream and queued right behind a clock pre-roll (replays of the
same graph for --preroll-ms) and --warmup replays of the same graph, all
between two device synchronisations.  value, ms_per_step and the roofline
come from that event time.

Printed: ONE JSON line with the metric (achieved HBM GB/s of the kernel over
the algorithmic bytes weights + x + y), the roofline object of the dominant
kernel, the CPU baseline (the fp64 oracle on the host cores, and on one) and
extra context (pure-read ceiling over the same bytes, the other formats'
shapes, the dense bf16 GEMV of the same shape, the general output stage, row
materialisation, prefill on the matrix cores and a Llama-8B per-token sweep
with its per-role breakdown).
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


VALU_SUMMARY = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", "gemv_valu_counters.md")
CLOCK_GHZ = 2.4  # nominal peak engine clock of the part


def valu_estimates(build_id: str) -> dict:
    """Per-shape VALU figures from the committed rocprofv3 counter summary
    (lines `valu <fmt>_<n>x<k>: insts_per_wave=A busy_cycles_per_simd=B`),
    only if it was taken with this very build of the library."""
    out = {}
    try:
        lines = open(VALU_SUMMARY).read().splitlines()
    except OSError:
        return out
    bid = [ln.split(":", 1)[1].strip() for ln in lines if ln.startswith("valu_build_id:")]
    if not bid or bid[0] != build_id:
        return out
    for ln in lines:
        if not ln.startswith("valu ") or ":" not in ln:
            continue
        key, rest = ln[len("valu "):].split(":", 1)
        try:
            vals = dict(kv.split("=") for kv in rest.split())
            out[key.strip()] = {k: float(v) for k, v in vals.items()}
        except ValueError:
            continue
    return out


def valu_fields(valu: dict, fmt: str, n: int, k: int, us: float) -> dict:
    """Estimated VALU issue share of one launch: the SIMD-cycles the counters
    saw spent issuing VALU instructions, per SIMD, over the launch's cycles at
    the nominal clock (empty when no counter summary of the loaded library's build id covers the shape)."""
    v = valu.get(f"{fmt}_{n}x{k}")
    if not v or "busy_cycles_per_simd" not in v:
        return {}
    return {"valu_insts_per_wave": round(v.get("insts_per_wave", float("nan")), 1),
            "est_valu_issue_pct": round(100 * v["busy_cycles_per_simd"] / (us * 1e-6 * CLOCK_GHZ * 1e9), 1)}


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


# Timed region: ONE captured HIP graph of exactly `steps` dependent launches
# (launch i reads weight copy i mod `copies`), replayed once between two HIP
# events on the launch stream.  Before it, on the same stream and with no
# synchronisation in between: a clock pre-roll (replays of the same graph for
# at least `preroll_ms`; the part's clocks ramp up over the first ~0.75 ms of
# work after an idle gap) and `warmup` replays of the graph.  A device
# synchronisation brackets the whole sequence.
PREROLL_MS = 20.0


def copies_for(steps: int, max_copies: int = 32) -> int:
    """Distinct weight copies a timed graph cycles through: every launch of a
    run of up to 16 consecutive ones reads its own copy (>= 16 x the bytes of
    one launch, well above the 256 MB Infinity Cache for the 33 MB shapes)."""
    return max(16, min(steps, max_copies))


def time_graph(launch, steps, copies, warmup, stream, preroll_ms=PREROLL_MS, min_timed_ms=0.0, min_warm_ms=0.0,
               reps=1):
    """Per-launch device time of a graph of `steps` launches (launch(i, h)
    enqueues launch i on stream handle h, i < copies).  Returns a dict: `us`
    (event time of the timed replays / launches), `preroll_ms`, `replays`
    (timed replays of the graph; 1 unless min_timed_ms asks for more),
    `warmup_replays` and `wall_ms` (host time between the two
    synchronisations, pre-roll and warm-up included).  `reps` timed replays
    (default one) are queued back to back."""
    import math

    import torch

    h = stream.cuda_stream
    with torch.cuda.stream(stream):
        for i in range(copies):  # first touch of every copy, outside the graph
            launch(i, h)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for i in range(steps):
            launch(i % copies, h)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    with torch.cuda.stream(stream):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    per = max(e0.elapsed_time(e1), 1e-3)  # ms per replay, a first estimate
    n_pre = math.ceil(preroll_ms / per) if preroll_ms > 0 else 0
    warm = max(warmup, math.ceil(min_warm_ms / per)) if min_warm_ms > 0 else warmup
    reps = max(reps, math.ceil(min_timed_ms / per)) if min_timed_ms > 0 else max(1, reps)
    p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    p0.record(stream)
    with torch.cuda.stream(stream):
        for _ in range(n_pre):
            g.replay()
    p1.record(stream)
    with torch.cuda.stream(stream):
        for _ in range(warm):
            g.replay()
    ev0.record(stream)  # right behind the warm-up: no idle gap before the timed launches
    with torch.cuda.stream(stream):
        for _ in range(reps):
            g.replay()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    res = {"us": 1e3 * ev0.elapsed_time(ev1) / (reps * steps), "preroll_ms": p0.elapsed_time(p1),
           "replays": reps, "warmup_replays": warm, "wall_ms": 1e3 * wall}
    del g
    return res


def measure_gpu(fmt, n, k, steps, warmup, preroll_ms=PREROLL_MS, with_ceiling=True):
    """One GEMV shape: a graph of `steps` launches over copies_for(steps)
    weight copies (and the pure-read kernel over the same bytes and copies)."""
    import numpy as np
    import torch

    from dequant_gemv_amd import qgemv, synth

    dev = torch.device("cuda:0")
    seed = CASE_SEED.get((fmt, n, k), 9)
    w_host = synth.weights(fmt, n, k, synth.W_SEED + seed)
    x_host = synth.activations(fmt, k, synth.X_SEED + seed)
    copies = copies_for(steps)
    w0 = torch.from_numpy(w_host).to(dev)
    ws = [w0] + [w0.clone() for _ in range(copies - 1)]
    x = torch.from_numpy(x_host.view(np.int16).copy()).to(dev)
    y = torch.empty(n, dtype=torch.float32, device=dev)
    fn = qgemv.GEMV[fmt]
    stream = torch.cuda.Stream()
    nbytes = algorithmic_bytes(fmt, n, k)

    t = time_graph(lambda i, h: fn(ws[i], x, y, n, k, h), steps, copies, warmup, stream, preroll_ms)
    res = {"us": t["us"], "bytes": nbytes, "copies": copies, "preroll_ms": t["preroll_ms"],
           "wall_ms": t["wall_ms"], "gbps": nbytes / (t["us"] * 1e-6) / 1e9}
    if with_ceiling:
        wb = synth.weight_bytes(fmt, n, k)
        sink = torch.empty(qgemv.qgemv_read_sink_len(wb), dtype=torch.float32, device=dev)
        c = time_graph(lambda i, h: qgemv.qgemv_read_ceiling(ws[i], wb, sink, h), steps, copies, warmup, stream,
                       preroll_ms)
        res["ceiling_us"] = c["us"]
        res["ceiling_gbps"] = wb / (c["us"] * 1e-6) / 1e9
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


def measure_sweep(mix: str, tokens: int, warmup: int, layers: int = 32, preroll_ms=PREROLL_MS):
    """One token = the 225 GEMVs of a Llama-8B decode step, each layer with its
    own weight buffers (cloned on the device from one generated matrix per
    shape, so every launch reads cold bytes: ~2.9 GB for the mixed sweep),
    captured in one HIP graph and replayed per token.  A mix named "<mix>-fused"
    stores Q/K/V and gate/up as concatenated matrices (129 launches).  The
    breakdown times each role's launches alone (one graph of its 32 launches,
    or of 16 launches of lm_head) and sums them per token."""
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
            calls.append((role, fmt, w, xs[(fmt, n, k)], torch.empty(n, dtype=torch.float32, device=dev), n, k))
            total_bytes += algorithmic_bytes(fmt, n, k)
    role, n, k = LLAMA8B_HEAD
    fmt = fmt_of[role]
    calls.append((role, fmt, proto[(fmt, n, k)], xs[(fmt, n, k)], torch.empty(n, dtype=torch.float32, device=dev), n, k))
    total_bytes += algorithmic_bytes(fmt, n, k)
    stream = torch.cuda.Stream()

    def call(c, h):
        _, fmt, w, x, y, n, k = c
        qgemv.GEMV[fmt](w, x, y, n, k, h)

    t = time_graph(lambda i, h: call(calls[i], h), len(calls), len(calls), warmup, stream, preroll_ms, reps=tokens)
    us = t["us"] * len(calls)
    breakdown, summed = {}, 0.0
    for role, n, k in layer_shapes + [LLAMA8B_HEAD]:
        mine = [c for c in calls if c[0] == role]
        per_token = len(mine)
        if len(mine) == 1:  # lm_head: one 296 MB matrix, larger than the Infinity Cache
            mine = mine * 16
        r = time_graph(lambda i, h: call(mine[i], h), len(mine), len(mine), warmup, stream, preroll_ms)
        fmt = fmt_of[role]
        b = algorithmic_bytes(fmt, n, k)
        breakdown[role] = {"format": fmt, "rows": n, "k": k, "launches_per_token": per_token,
                           "us_per_launch": round(r["us"], 3), "us_per_token": round(r["us"] * per_token, 2),
                           "gbps": round(b / (r["us"] * 1e-6) / 1e9, 1)}
        summed += r["us"] * per_token
    res = {
        "workload": f"Llama-8B decode step, {len(calls)} GEMVs ({layers} layers + lm_head), formats: {mix}"
                    + (", Q/K/V and gate/up as concatenated matrices" if fused else ""),
        "gemvs_per_token": len(calls),
        "algorithmic_bytes_per_token": total_bytes,
        "us_per_token": round(us, 2),
        "gbps": round(total_bytes / (us * 1e-6) / 1e9, 1),
        "pct_of_hbm_peak": round(100 * total_bytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 1),
        "tokens_timed": t["replays"],
        "breakdown": breakdown,
        "breakdown_sum_us": round(summed, 2),
    }
    del calls, proto, xs
    torch.cuda.empty_cache()
    return res


def measure_epilogue(steps, warmup, preroll_ms=PREROLL_MS):
    """The main Q4_K shape through the general output stage: fp16 y updated in
    place, y = v + 0.5 y (a residual-style accumulate), against the plain call."""
    import numpy as np
    import torch

    from dequant_gemv_amd import qgemv, synth

    fmt, n, k, _ = MAIN
    dev = torch.device("cuda:0")
    seed = CASE_SEED[(fmt, n, k)]
    copies = copies_for(steps)
    w0 = torch.from_numpy(synth.weights(fmt, n, k, synth.W_SEED + seed)).to(dev)
    ws = [w0] + [w0.clone() for _ in range(copies - 1)]
    x = torch.from_numpy(synth.activations(fmt, k, synth.X_SEED + seed).view(np.int16).copy()).to(dev)
    y16 = torch.zeros(n, dtype=torch.float16, device=dev)
    y32 = torch.empty(n, dtype=torch.float32, device=dev)
    stream = torch.cuda.Stream()
    us_ex = time_graph(lambda i, h: qgemv.qgemv_q4k_ex(ws[i], x, y16, n, k, 1.0, 0.5, y16, h),
                       steps, copies, warmup, stream, preroll_ms)["us"]
    us_plain = time_graph(lambda i, h: qgemv.qgemv_q4k(ws[i], x, y32, n, k, h), steps, copies, warmup, stream,
                          preroll_ms)["us"]
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


def measure_rows(steps, warmup, preroll_ms=PREROLL_MS):
    """Row materialisation throughput: HBM bytes = packed bytes read + outputs
    written (+ the int32 indices) per call.  A graph of `steps` launches cycles
    through up to 1 GiB of weight copies and of output buffers."""
    import numpy as np
    import torch

    from dequant_gemv_amd import qgemv, synth

    dev = torch.device("cuda:0")
    out = {}
    for fmt, n, k, nsel, dtype, desc in ROWS_CASES:
        w0 = torch.from_numpy(synth.weights(fmt, n, k, 4100)).to(dev)
        copies = max(1, min(copies_for(steps), (1 << 30) // w0.numel())) if nsel is None else 1
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
        us = time_graph(lambda i, h: fn(ws[i % copies], n, k, rows, nrows, os_[i % ocount], h), steps,
                        max(copies, ocount), warmup, stream, preroll_ms)["us"]
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
        us = time_graph(lambda i, h: fn(ws[i], x, y, t, n, k, h), 4, 4, 0, stream, 0.0, PREFILL_TIMED_MS,
                        PREFILL_WARM_MS)["us"]
        flops = 2.0 * t * n * k
        rec = {
            "workload": f"{fmt} prefill, {t} tokens x {n} rows x K {k}",
            "us": round(us, 2),
            "tflops": round(flops / us / 1e6, 1),
            "pct_of_mfma_peak": round(100 * flops / us / 1e6 / MFMA_PEAK_TFLOPS, 1),
        }
        nws = qgemv.qgemm_workspace_bytes(t, n, k)
        if nws:  # K split: the same call through a workspace (fixed addition order)
            wsb = torch.empty(nws // 4, dtype=torch.float32, device=dev)
            rec["workspace_us"] = round(time_graph(lambda i, h: qgemv.GEMM_WS[fmt](ws[i], x, y, t, n, k, wsb, h), 4, 4,
                                                   0, stream, 0.0, PREFILL_TIMED_MS, PREFILL_WARM_MS)["us"], 2)
            rec["workspace_mb"] = round(nws / 1e6, 1)
            del wsb
        if fmt == "q4k" and unfused:
            wf = torch.empty((n, k), dtype=torch.float16, device=dev)
            us_rows = time_graph(lambda i, h: qgemv.qget_rows_q4k(ws[i], n, k, None, n, wf, h), 4, 4, 0, stream,
                                 0.0, PREFILL_TIMED_MS, PREFILL_WARM_MS)["us"]
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
    graph of 320 launches over 32 buffers, as for the metric), and the least-
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
        us = time_graph(lambda i, h: qgemv.qgemv_read_ceiling(bufs[i], nbytes, sink, h), 320, 32, 10, stream)["us"]
        points.append({"bytes": nbytes, "us": round(us, 3), "gbps": round(nbytes / us / 1e3, 1)})
        log(f"[bench] read {nbytes / 1e6:.3f} MB: {us:.3f} us/launch, {nbytes / us / 1e3:.1f} GB/s")
        del bufs, sink
        torch.cuda.empty_cache()
    b = np.array([p["bytes"] for p in points if p["bytes"] >= 4e6], dtype=np.float64)
    t = np.array([p["us"] for p in points if p["bytes"] >= 4e6], dtype=np.float64)
    (fixed, per_byte), *_ = np.linalg.lstsq(np.vstack([np.ones_like(b), b]).T, t, rcond=None)
    return {"points": points, "fit_fixed_us": round(float(fixed), 3), "fit_gbps": round(1e-3 / float(per_byte), 1)}


SIMDS = 1024  # 256 compute units x 4 SIMDs


def counter_summary(dirs, shapes, build_id):
    """Text summary of `rocprofv3 --pmc ... -- python3 bench.py ...` runs (the
    counter_collection.csv files under `dirs`): per GEMV kernel, in the order
    the run first dispatched them (one per entry of `shapes`), the median per
    dispatch of every counter collected (cycle counters such as GRBM_GUI_ACTIVE
    include the profiler's per-dispatch serialisation and are listed only).  FETCH_SIZE / WRITE_SIZE (KiB) are
    scaled by what the same counter read for the run's first 8 copy dispatches
    (--calibrate-copy: 64 MiB read + 64 MiB written each); the VALU counters
    give instructions per wave and SIMD-cycles spent issuing VALU per SIMD
    (SQ_ACTIVE_INST_VALU x 4 / SIMDs, the convention of rocprof's VALUBusy).
    Returns the summary lines (those bench.py reads back included)."""
    import csv
    import glob

    per = {}  # kernel name -> counter -> [values]
    first = {}  # kernel name -> first dispatch id
    copies = {}  # counter -> [values of copy dispatches, in dispatch order]
    for d in dirs:
        for f in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
            for r in csv.DictReader(open(f)):
                name, did = r["Kernel_Name"], int(r["Dispatch_Id"])
                val = float(r["Counter_Value"])
                if "copyBuffer" in name:
                    copies.setdefault(r["Counter_Name"], []).append((did, val))
                if "_gemv_" not in name:
                    continue
                per.setdefault(name, {}).setdefault(r["Counter_Name"], []).append(val)
                first[name] = min(first.get(name, did), did)
    names = sorted(per, key=first.get)
    if len(names) != len(shapes):
        raise SystemExit(f"{len(names)} GEMV kernels in the counter files, {len(shapes)} shapes expected")
    scale = {}
    for c, want_kib in (("FETCH_SIZE", 65536.0), ("WRITE_SIZE", 65536.0)):
        vals = [v for _, v in sorted(copies.get(c, []))[:8]]
        if len(vals) == 8 and statistics.median(vals) > 0:
            scale[c] = want_kib / statistics.median(vals)
    out = [f"valu_build_id: {build_id}" if any("SQ_INSTS_VALU" in per[n] for n in names) else
           f"counters_build_id: {build_id}"]
    for c, s in scale.items():
        out.append(f"calibration {c}: copy of 64 MiB counts {65536.0 / s:.1f} KiB per dispatch, scale {s:.4f}")
    for (fmt, n, k, _), name in zip(shapes, names):
        cs = per[name]
        med = {c: statistics.median(v) for c, v in cs.items()}
        key = f"{fmt}_{n}x{k}"
        out.append(f"kernel {key}: {name.split('(')[0]} ({len(next(iter(cs.values())))} dispatches)")
        for c in sorted(med):
            out.append(f"  {c}: {med[c]:.6g}")
        if "FETCH_SIZE" in med and "WRITE_SIZE" in med and len(scale) == 2:
            tb = int(round(1024 * (med["FETCH_SIZE"] * scale["FETCH_SIZE"] + med["WRITE_SIZE"] * scale["WRITE_SIZE"])))
            ab = algorithmic_bytes(fmt, n, k)
            out.append(f"traffic {key}: bytes_per_launch={tb} algorithmic={ab} ratio={tb / ab:.4f}")
        if "SQ_INSTS_VALU" in med and "SQ_WAVES" in med:
            line = f"valu {key}: insts_per_wave={med['SQ_INSTS_VALU'] / med['SQ_WAVES']:.1f}"
            if "SQ_ACTIVE_INST_VALU" in med:
                line += f" busy_cycles_per_simd={4 * med['SQ_ACTIVE_INST_VALU'] / SIMDS:.0f}"
            out.append(line)
    return out


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform

    return platform.processor() or "unknown"


def cpu_baseline(fmt, n, k, budget_s=10.0, one_thread_rows=256):
    """The fp64 oracle as it stands, on the same workload: all host cores on
    the full matrix (median of repeated runs within about `budget_s` of CPU
    time), and one thread on the first `one_thread_rows` rows."""
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
    threads = oracle.threads()
    # one thread on a row prefix: the same per-row work, scaled by its bytes
    n1 = min(n, one_thread_rows)
    if fmt == "nvfp4":  # nibbles [n][k/2], then scales [n][k/16]
        nib, sc = w[: n * k // 2].reshape(n, -1), w[n * k // 2:].reshape(n, -1)
        w1 = np.concatenate([nib[:n1].reshape(-1), sc[:n1].reshape(-1)])
    else:
        w1 = np.ascontiguousarray(w.reshape(n, -1)[:n1]).reshape(-1)
    oracle.set_threads(1)
    oracle.gemv(fmt, w1, x, n1, k)
    t1s = []
    for _ in range(3):
        t0 = time.perf_counter()
        oracle.gemv(fmt, w1, x, n1, k)
        t1s.append(time.perf_counter() - t0)
    t1 = statistics.median(t1s)
    oracle.set_threads(cores)
    return {
        "value": algorithmic_bytes(fmt, n, k) / t / 1e9,
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "cpu_model": cpu_model(),
        "sample": f"full {n}x{k} {fmt} matrix, median of {len(times)} runs "
                  f"({t * 1e3:.1f} ms each, fp64 scalar dequantise-then-dot, OpenMP over rows)",
        "one_thread": {"value": algorithmic_bytes(fmt, n1, k) / t1 / 1e9, "unit": "GB/s",
                       "sample": f"first {n1} rows of the same shape ({synth.weight_bytes(fmt, n1, k)} packed bytes), "
                                 f"median of 3 runs ({t1 * 1e3:.1f} ms each)"},
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=320,
                    help="launches in the timed graph (one replay of it is the timed region)")
    ap.add_argument("--warmup", type=int, default=10, help="untimed replays of that graph right before it")
    ap.add_argument("--preroll-ms", type=float, default=PREROLL_MS,
                    help="clock pre-roll: replays of the same graph for at least this long before the warm-up")
    ap.add_argument("--no-extra", action="store_true", help="skip the other formats' shapes")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--sweep", default="mixed,mixed-fused",
                    help="Llama-8B per-token sweep(s) to time among mixed,q4k,nvfp4,tq1, each also as "
                         "<mix>-fused (comma list; 'none' to skip)")
    ap.add_argument("--sweep-tokens", type=int, default=20)
    ap.add_argument("--fmt", default=None, help="measure only this format (q4k, nvfp4, tq1, f16, bf16) at N,K")
    ap.add_argument("--n", type=int, default=None)
    ap.add_argument("--k", type=int, default=None)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 64 MiB device copy (a known-size reference for the HBM byte counters)")
    ap.add_argument("--prefill-only", default=None, metavar="FMT,T,N,K",
                    help="time only this prefill case (e.g. q4k,4096,14336,4096) and print its record")
    ap.add_argument("--ceiling-sweep", action="store_true",
                    help="time only the pure-read kernel over 0.06-128 MB per launch and fit t = fixed + bytes / BW")
    ap.add_argument("--rows-only", action="store_true",
                    help="time only the row-materialisation cases (after --calibrate-copy if given) and print them")
    ap.add_argument("--shapes-only", action="store_true",
                    help="time only the GEMV shapes (main and other formats) with their read ceilings")
    ap.add_argument("--sweep-only", action="store_true",
                    help="time only the Llama-8B decode sweeps (--sweep) and print them")
    ap.add_argument("--counter-summary", nargs="+", metavar="DIR", default=None,
                    help="print a summary of rocprofv3 --pmc output directories of a run of this script with the "
                         "same shape flags (--fmt/--n/--k, else the main and other shapes) and exit (no GPU used)")
    args = ap.parse_args()

    if args.counter_summary:
        from dequant_gemv_amd import build

        shapes = [MAIN] if args.no_extra else [MAIN] + EXTRA
        if args.fmt:
            shapes = [(args.fmt, args.n or MAIN[1], args.k or MAIN[2], "")]
        print("\n".join(counter_summary(args.counter_summary, shapes, build.build_id())))
        return

    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
              "(the path shards by rows with no exchange; see the design notes)", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0:
        print("--steps must be >= 1 and --warmup >= 0", file=sys.stderr)
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
        print(json.dumps({"get_rows": measure_rows(args.steps, args.warmup, args.preroll_ms), "build_id": have}),
              flush=True)
        return

    if args.sweep_only:
        sweeps = {}
        for mix in args.sweep.split(","):
            sweeps[mix] = measure_sweep(mix, args.sweep_tokens, args.warmup, preroll_ms=args.preroll_ms)
            log(f"[bench] sweep {mix}: {sweeps[mix]['us_per_token']} us/token")
        print(json.dumps({"decode_sweep": sweeps, "build_id": have}), flush=True)
        return

    fmt, n, k, desc = MAIN
    if args.fmt:
        fmt, n, k, desc = args.fmt, args.n or n, args.k or k, f"{args.fmt} GEMV M=1, N={args.n or n} x K={args.k or k}"
    log(f"[bench] build {have} on {torch.cuda.get_device_name(0)}; main {fmt} {n}x{k}")
    main_res = measure_gpu(fmt, n, k, args.steps, args.warmup, args.preroll_ms)
    log(f"[bench] main: {main_res['us']:.3f} us/launch, {main_res['gbps']:.1f} GB/s "
        f"(ceiling {main_res['ceiling_us']:.3f} us, {main_res['ceiling_gbps']:.1f} GB/s)")

    valu = valu_estimates(have)
    extra = {}
    if not args.no_extra and not args.fmt:
        for efmt, en, ek, edesc in EXTRA:
            r = measure_gpu(efmt, en, ek, args.steps, args.warmup, args.preroll_ms)
            rec = {
                "workload": edesc,
                "us_per_gemv": round(r["us"], 3),
                "gbps": round(r["gbps"], 1),
                "pct_of_hbm_peak": round(100 * r["gbps"] / HBM_PEAK_GBPS, 1),
                "read_ceiling_us": round(r["ceiling_us"], 3),
                "read_ceiling_gbps": round(r["ceiling_gbps"], 1),
                "pct_of_read_ceiling": round(100 * r["ceiling_us"] / r["us"], 1),
            }
            rec.update(valu_fields(valu, efmt, en, ek, r["us"]))
            extra[f"{efmt}_{en}x{ek}"] = rec
            log(f"[bench] {efmt} {en}x{ek}: {r['us']:.3f} us, {r['gbps']:.1f} GB/s")

    fp4_vs_bf16 = None
    if "nvfp4_4096x14336" in extra and "bf16_4096x14336" in extra:
        fp4_vs_bf16 = {
            "speedup": round(extra["bf16_4096x14336"]["us_per_gemv"] / extra["nvfp4_4096x14336"]["us_per_gemv"], 3),
            "bytes_ratio": round(algorithmic_bytes("bf16", 4096, 14336) / algorithmic_bytes("nvfp4", 4096, 14336), 3),
            "page_speedup_apple_m5_max": PAGE_FP4_VS_BF16,
        }
        log(f"[bench] NVFP4 vs bf16 at 4096x14336: {fp4_vs_bf16['speedup']}x")

    epilogue = rows_res = prefill_res = None
    sweeps = {}
    if not args.no_extra and not args.fmt and not args.shapes_only:
        epilogue = measure_epilogue(args.steps, args.warmup, args.preroll_ms)
        log(f"[bench] epilogue: {epilogue['us_per_gemv']} us (plain {epilogue['us_per_gemv_plain_fp32']} us)")
        rows_res = measure_rows(args.steps, args.warmup, args.preroll_ms)
        prefill_res = measure_prefill(args.steps, args.warmup)
        if args.sweep != "none":
            for mix in args.sweep.split(","):
                r = measure_sweep(mix, args.sweep_tokens, args.warmup, preroll_ms=args.preroll_ms)
                sweeps[mix] = r
                log(f"[bench] sweep {mix}: {r['us_per_token']} us/token, {r['gbps']} GB/s over "
                    f"{r['gemvs_per_token']} GEMVs (roles summed: {r['breakdown_sum_us']} us)")

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(fmt, n, k)
        log(f"[bench] cpu oracle: {cpu['value']:.2f} GB/s on {cpu['cores']} threads, "
            f"{cpu['one_thread']['value']:.3f} GB/s on one")

    us = main_res["us"]
    achieved = main_res["gbps"]
    out = {
        "metric": METRIC,
        "value": round(achieved, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us / 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": desc,
            "format": fmt, "n": n, "k": k,
            "algorithmic_bytes_per_gemv": main_res["bytes"],
            "weight_copies": main_res["copies"],
            "launch": (f"one HIP graph of {args.steps} dependent launches (launch i reads weight copy i mod "
                       f"{main_res['copies']}), replayed once between two HIP events on its stream, right behind "
                       f"{args.warmup} warm-up replays of the same graph"),
            "clock_preroll_ms": round(main_res["preroll_ms"], 3),
            "wall_ms_sync_to_sync": round(main_res["wall_ms"], 3),
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": measured_traffic(have) if (fmt, n, k) == MAIN[:3] else None,
        },
        "pct_of_hbm_peak": round(100 * achieved / HBM_PEAK_GBPS, 2),
        "us_per_gemv": round(us, 3),
        "read_ceiling": {"gbps": round(main_res["ceiling_gbps"], 1), "us": round(main_res["ceiling_us"], 3),
                         "pct_of_read_ceiling": round(100 * main_res["ceiling_us"] / us, 1),
                         "note": "pure dwordx4 read of the same weight bytes, same graph and copies"},
        "valu": valu_fields(valu, fmt, n, k, us),
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
