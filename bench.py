#!/usr/bin/env python3
"""Benchmark of the NVFP4 hot path on one MI355X.

A step is one pass of the path over one batch: per-token NVFP4 quantization
of the activations (nvfp4_act_quant) followed by the block-scaled NVFP4 GEMM
against weights prepared offline (quantized per tensor and pre-tiled by
nvfp4_pretile_weight; nvfp4_gemm_pretiled).  The headline workload is the
prefill GEMM B=4096, K=8192, N=8192 (bf16 activations ~N(0,1), weights
~N(0,0.02), FP16 output); `value` is whole-step TFLOP/s (2*B*N*K per step).
The same GEMM on the plain [N, K/2] weight layout (nvfp4_gemm) is timed after
the steps and reported under "workloads".  The other workloads (decode GEMM, fused SwiGLU quantize,
quantize + GEMM small case, the MXFP4 variant's prefill step and decode GEMM
on the FP4 MFMA, MoE) are measured after it and reported under "workloads".

Timing: inputs are resident in HBM before the timed region; untimed settle
steps (SETTLE_MS of back-to-back steps, so the GPU clocks have risen from
idle; reported as clock_settle), then W warmup steps,
then exactly K steps between synchronizations, timed with HIP events on the
stream the kernels run on; per-call events give the average duration of the
GEMM call and of the quantize call.  The micro-second workloads (decode,
small, MoE, SwiGLU) are timed by replaying a HIP graph of many calls, so the
host's per-call launch cost is not counted as GPU time.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--quick]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
FP16_MFMA_PEAK_TFLOPS = 2500.0  # dense fp16 MFMA
FP4_MFMA_PEAK_TFLOPS = 10100.0  # dense fp4 MFMA (context: the path runs fp16 MFMA)
ALGO_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
# Untimed steps run back to back before the W warmup steps of a prefill
# workload, until this much wall time has passed: after the host-side input
# generation the GPU has been idle for about a second, and its clocks rise
# over the first tens of milliseconds of sustained load (measured: the
# pre-tiled GEMM call takes 565 us on the first step after 10 settle steps,
# falling to 470 us by step 25 and 452-465 us from then on).  The timed region
# is still exactly K full steps; the settle phase is reported in the line.
SETTLE_MS = 100.0


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--quick", action="store_true", help="skip the secondary workloads and the CPU baseline")
    p.add_argument("--no-cpu", action="store_true")
    p.add_argument("--only", choices=["prefill", "decode", "swiglu", "quant", "small", "moe", "copy",
                                      "mx_prefill", "mx_decode"],
                   help="run one workload and print its measurement (for profiler runs)")
    return p.parse_args()


class EventTimer:
    """Average duration of a repeated call, measured with HIP events on `stream`."""

    def __init__(self, torch, stream):
        self.torch, self.stream, self.pairs = torch, stream, []

    def __call__(self, fn):
        t = self.torch
        a, b = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        a.record(self.stream)
        r = fn()
        b.record(self.stream)
        self.pairs.append((a, b))
        return r

    def mean_ms(self):
        return sum(a.elapsed_time(b) for a, b in self.pairs) / max(len(self.pairs), 1)


def quant_bytes(rows, k_in, k_out, scale=True):
    """Algorithmic HBM bytes of one quantize call: read input, write codes,
    E4M3 bytes, the FP32 global per row and (optionally) the combined scales."""
    return rows * k_in * 2 + rows * k_out // 2 + rows * k_out // 16 + rows * 4 + (rows * k_out // 16 * 4 if scale else 0)


def gemm_bytes(B, N, K):
    """Algorithmic bytes of one GEMM call: each operand read once, output written once."""
    return B * K // 2 + B * (K // 16) * 4 + N * K // 2 + N * (K // 16) + 4 + B * N * 2


def settle(torch, step, ms=SETTLE_MS, max_steps=2000):
    """Runs `step` untimed, in groups of 10, until `ms` of wall time have
    passed (or max_steps); returns (steps, ms)."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n = 0
    while n < max_steps:
        for _ in range(10):
            step()
        n += 10
        torch.cuda.synchronize()
        if (time.perf_counter() - t0) * 1e3 >= ms:
            break
    return n, (time.perf_counter() - t0) * 1e3


def run_prefill(torch, nv, si, steps, warmup):
    c = si.CONFIGS["C3"]
    B, K, N = c["B"], c["K"], c["N"]
    dev = torch.device("cuda:0")
    a, w = si.gemm_inputs("C3")
    x = a.to(dev)
    # offline weight preparation (not timed): NVFP4 quantization per tensor,
    # then the pre-tiled layout the GEMM's lanes read (nvfp4_pretile_weight)
    wq = nv.quantize(w.to(dev), group_rows=N, want_scale=False)
    wt = nv.pretile_weight(wq["codes"], wq["sf"])
    del w
    stream = torch.cuda.current_stream()
    qa = {"codes": torch.empty((B, K // 2), dtype=torch.uint8, device=dev),
          "sf": torch.empty((B, K // 16), dtype=torch.uint8, device=dev),
          "g_dec": torch.empty((B,), dtype=torch.float32, device=dev),
          "scale": torch.empty((B, K // 16), dtype=torch.float32, device=dev)}
    y = torch.empty((B, N), dtype=torch.float16, device=dev)
    ws = torch.empty(max(nv.gemm_workspace_size(B, N, K), 1), dtype=torch.uint8, device=dev)

    def step(tq=None, tg=None):
        fq = lambda: nv.act_quant(x, "none", out=qa)
        fg = lambda: nv.gemm_pretiled(qa["codes"], qa["scale"], wt, wq["g_dec"], out=y, workspace=ws)
        tq(fq) if tq else fq()
        tg(fg) if tg else fg()

    n_settle, ms_settle = settle(torch, step)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    tq, tg = EventTimer(torch, stream), EventTimer(torch, stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        step(tq, tg)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = e0.elapsed_time(e1) / steps
    # the same GEMM on the weights in the plain [N, K/2] layout (nvfp4_gemm)
    tu = EventTimer(torch, stream)
    for i in range(warmup + steps):
        f = lambda: nv.gemm(qa["codes"], qa["scale"], wq["codes"], wq["sf"], wq["g_dec"], out=y, workspace=ws)
        tu(f) if i >= warmup else f()
    torch.cuda.synchronize()
    return dict(B=B, K=K, N=N, ms_step=ms_step, wall_s=wall, ms_gemm=tg.mean_ms(), ms_quant=tq.mean_ms(),
                ms_gemm_untiled=tu.mean_ms(), settle_steps=n_settle, settle_ms=ms_settle,
                flops=2.0 * B * N * K, qbytes=quant_bytes(B, K, K), gbytes=gemm_bytes(B, N, K))


def graph_time_ms(torch, fns, reps=5):
    """Average GPU time per call of `fns` (a list of launch callables), timed by
    replaying a HIP graph that holds one call of each: the host-side cost of
    issuing micro-second kernels one by one does not enter the figure.  The
    graph is replayed untimed for SETTLE_MS first (the GPU clocks rise from
    idle under sustained load), then `reps` replays are timed."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for f in fns:
            f()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for f in fns:
            f()
    g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < SETTLE_MS:
        g.replay()
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (reps * len(fns))


def run_decode(torch, nv, si, B, iters=None):
    """Decode GEMM (one rank's K-share) with the weights rotated through 32
    copies (> 512 MB) so the 256 MB Infinity Cache cannot hold them."""
    c = si.CONFIGS["C2"]
    K, N = c["K"], c["N"]
    dev = torch.device("cuda:0")
    a, w = si.gemm_inputs("C2", B=B)
    wq = nv.quantize(w.to(dev), group_rows=N, want_scale=False)
    copies = 32
    Ws = [(wq["codes"].clone(), wq["sf"].clone(), wq["g_dec"].clone()) for _ in range(copies)]
    x = a.to(dev)
    qa = nv.act_quant(x, "none")
    y = torch.empty((B, N), dtype=torch.float16, device=dev)
    ms_gemm = graph_time_ms(torch, [(lambda Wi=Wi: nv.gemm(qa["codes"], qa["scale"], *Wi, out=y)) for Wi in Ws])
    ms_quant = graph_time_ms(torch, [lambda: nv.act_quant(x, "none", out=qa)] * 8)
    # the same weights pre-tiled offline (nvfp4_pretile_weight)
    Wt = [(nv.pretile_weight(Wi[0], Wi[1]), Wi[2]) for Wi in Ws]
    del Ws
    ms_tiled = graph_time_ms(torch, [(lambda Wi=Wi: nv.gemm_pretiled(qa["codes"], qa["scale"], Wi[0], Wi[1], out=y))
                                     for Wi in Wt])
    gb = gemm_bytes(B, N, K)
    return dict(B=B, us_gemm=ms_gemm * 1e3, us_quant=ms_quant * 1e3, gemm_bytes=gb,
                gemm_GBps=gb / (ms_gemm * 1e-3) / 1e9, hbm_frac=gb / (ms_gemm * 1e-3) / 1e9 / HBM_PEAK_GBS,
                us_gemm_pretiled=ms_tiled * 1e3, hbm_frac_pretiled=gb / (ms_tiled * 1e-3) / 1e9 / HBM_PEAK_GBS)


def run_quant_rotating(torch, nv, si, copies=5, reps=4):
    """Per-token quantize of the prefill activations ([4096, 8192] bf16, codes +
    E4M3 bytes + globals + combined scales) with the input rotated through
    `copies` buffers (5 x 64 MB > the 256 MB Infinity Cache), so every call
    reads its input from HBM."""
    c = si.CONFIGS["C3"]
    B, K = c["B"], c["K"]
    dev = torch.device("cuda:0")
    a, _ = si.gemm_inputs("C3", N=16)
    xs = [a.to(dev) for _ in range(copies)]
    outs = [nv.act_quant(x, "none") for x in xs]
    ms = graph_time_ms(torch, [(lambda x=x, o=o: nv.act_quant(x, "none", out=o)) for x, o in zip(xs, outs)],
                       reps=reps)
    by = quant_bytes(B, K, K)
    return dict(rows=B, K=K, us=ms * 1e3, bytes=by, GBps=by / (ms * 1e-3) / 1e9,
                hbm_frac=by / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS)


def run_swiglu(torch, nv, si, iters=10):
    c = si.CONFIGS["C4"]
    rows, H = c["rows"], c["H"]
    dev = torch.device("cuda:0")
    x = si.swiglu_input().to(dev)
    out = nv.act_quant(x, "swiglu", want_scale=False)
    ms = graph_time_ms(torch, [lambda: nv.act_quant(x, "swiglu", out=out)] * iters, reps=2)
    by = quant_bytes(rows, 2 * H, H, scale=False)
    return dict(rows=rows, H=H, us=ms * 1e3, bytes=by, GBps=by / (ms * 1e-3) / 1e9,
                hbm_frac=by / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS)


def run_small(torch, nv, si, iters=20):
    c = si.CONFIGS["C1"]
    B, K, N = c["B"], c["K"], c["N"]
    dev = torch.device("cuda:0")
    a, w = si.gemm_inputs("C1")
    x = a.to(dev)
    wq = nv.quantize(w.to(dev), group_rows=N, want_scale=False)
    qa = nv.act_quant(x, "none")
    y = nv.gemm(qa["codes"], qa["scale"], wq["codes"], wq["sf"], wq["g_dec"])

    def step():
        nv.act_quant(x, "none", out=qa)
        nv.gemm(qa["codes"], qa["scale"], wq["codes"], wq["sf"], wq["g_dec"], out=y)
    ms = graph_time_ms(torch, [step] * iters)
    return dict(B=B, K=K, N=N, us_step=ms * 1e3)


def run_moe(torch, nv, si, iters=None):
    c = si.CONFIGS["C5"]
    dev = torch.device("cuda:0")
    d = si.moe_inputs()
    T, E, Hd, I = d["T"], d["E"], d["hidden"], d["inter"]
    w1 = nv.quantize(d["w1"].to(dev), group_rows=I, want_scale=False)
    w2 = nv.quantize(d["w2"].to(dev), group_rows=Hd, want_scale=False)
    args = [torch.from_numpy(d["logits"]).to(dev), torch.from_numpy(d["bias"]).to(dev), d["x"].to(dev),
            w1["codes"].view(E, I, Hd // 2), w1["sf"].view(E, I, Hd // 16), w1["g_dec"],
            w2["codes"].view(E, Hd, I // 2), w2["sf"].view(E, Hd, I // 16), w2["g_dec"]]
    copies = 4   # 4 x 151 MB of expert weights rotate past the 256 MB Infinity Cache
    sets = [args] + [[t.clone() if i >= 3 else t for i, t in enumerate(args)] for _ in range(copies - 1)]
    out = torch.empty((T, Hd), dtype=torch.float16, device=dev)
    ws = torch.empty(nv.moe_workspace_size(T, E, c["top_k"], Hd, I), dtype=torch.uint8, device=dev)
    kw = dict(top_k=c["top_k"], n_group=c["n_group"], topk_group=c["topk_group"],
              norm_topk_prob=c["norm_topk_prob"], routed_scaling=c["routed_scaling"], out=out, workspace=ws)
    ms_plain = graph_time_ms(torch, [(lambda st=st: nv.moe_w4a16(*st, **kw)) for st in sets], reps=3)
    # the same expert weights pre-tiled offline (moe_pretile_weights): the timed layer
    tiled = []
    for st in sets:
        w1t, s1t = nv.moe_pretile_weights(st[3], st[4])
        w2t, s2t = nv.moe_pretile_weights(st[6], st[7])
        tiled.append(st[:3] + [w1t, s1t, st[5], w2t, s2t, st[8]])
    del sets
    ms = graph_time_ms(torch, [(lambda st=st: nv.moe_w4a16_pretiled(*st, **kw)) for st in tiled], reps=3)
    wbytes = E * (I * Hd // 2 + I * Hd // 16 + Hd * I // 2 + Hd * I // 16) + 2 * E * 4
    by = wbytes + T * Hd * 2 * 2 + T * E * 4 + E * 4
    return dict(T=T, E=E, us=ms * 1e3, bytes=by, GBps=by / (ms * 1e-3) / 1e9,
                hbm_frac=by / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, flops=2.0 * T * c["top_k"] * (2 * Hd * I),
                weights="pre-tiled", us_plain_weights=ms_plain * 1e3)


def mx_gemm_bytes(B, N, K):
    """Algorithmic bytes of one MX GEMM call: codes, E8M0 bytes and globals of
    both operands read once (padding rows excluded), output written once."""
    return B * K // 2 + B * K // 32 + B * 4 + N * K // 2 + N * K // 32 + 4 + B * N * 2


def mx_quant_bytes(rows, k):
    return rows * k * 2 + rows * k // 2 + rows * k // 32 + rows * 4


def run_mx_prefill(torch, nv, si, steps, warmup):
    """MXFP4 variant of the prefill step: per-token MX quantization of the same
    [4096, 8192] bf16 activations straight into the MX tile layout, then the
    block-scaled FP4 MFMA GEMM against the same weights, MX-quantized per tensor
    into the tile layout before timing."""
    c = si.CONFIGS["C3"]
    B, K, N = c["B"], c["K"], c["N"]
    dev = torch.device("cuda:0")
    a, w = si.gemm_inputs("C3")
    x = a.to(dev)
    wt = nv.mx_quantize(w.to(dev), group_rows=N, tiled=True)
    del w
    stream = torch.cuda.current_stream()
    qa = nv.mx_quantize(x, tiled=True)
    y = torch.empty((B, N), dtype=torch.float16, device=dev)

    def step(tq=None, tg=None):
        fq = lambda: nv.mx_quantize(x, tiled=True, out=qa)
        fg = lambda: nv.mx_gemm(qa, qa["g_dec"], wt, wt["g_dec"], out=y)
        tq(fq) if tq else fq()
        tg(fg) if tg else fg()

    n_settle, _ = settle(torch, step)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    tq, tg = EventTimer(torch, stream), EventTimer(torch, stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        step(tq, tg)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / steps
    flops = 2.0 * B * N * K
    ms_g, ms_q = tg.mean_ms(), tq.mean_ms()
    return dict(B=B, K=K, N=N, ms_step=ms_step, ms_gemm=ms_g, ms_quant=ms_q,
                gemm_TFLOPs=flops / (ms_g * 1e-3) / 1e12,
                gemm_frac_fp4_peak=flops / (ms_g * 1e-3) / 1e12 / FP4_MFMA_PEAK_TFLOPS,
                quant_GBps=mx_quant_bytes(B, K) / (ms_q * 1e-3) / 1e9,
                quant_hbm_frac=mx_quant_bytes(B, K) / (ms_q * 1e-3) / 1e9 / HBM_PEAK_GBS,
                step_TFLOPs=flops / (ms_step * 1e-3) / 1e12, settle_steps=n_settle)


def run_mx_decode(torch, nv, si, B):
    """MX decode GEMM (K=4096, N=8192) with the weight tiles rotated through 32
    copies (> 512 MB) past the Infinity Cache; HIP-graph replay."""
    c = si.CONFIGS["C2"]
    K, N = c["K"], c["N"]
    dev = torch.device("cuda:0")
    a, w = si.gemm_inputs("C2", B=B)
    w0 = nv.mx_quantize(w.to(dev), group_rows=N, tiled=True)
    Ws = [dict(w0, codes=w0["codes"].clone(), sf=w0["sf"].clone()) for _ in range(32)]
    qa = nv.mx_quantize(a.to(dev), tiled=True)
    y = torch.empty((B, N), dtype=torch.float16, device=dev)
    ms = graph_time_ms(torch, [(lambda Wi=Wi: nv.mx_gemm(qa, qa["g_dec"], Wi, Wi["g_dec"], out=y)) for Wi in Ws])
    by = mx_gemm_bytes(B, N, K)
    return dict(B=B, us_gemm=ms * 1e3, gemm_bytes=by, GBps=by / (ms * 1e-3) / 1e9,
                hbm_frac=by / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS)


def run_copy(torch):
    """A plain 256 MiB device copy, three times: the reference for scaling the
    FETCH_SIZE / WRITE_SIZE counters to bytes."""
    x = torch.empty(256 * 1024 * 1024, dtype=torch.uint8, device="cuda")
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    return {"bytes_read_per_copy": x.numel(), "bytes_written_per_copy": y.numel()}


def cpu_baseline(si, pre):
    """The oracle as it stands on the prefill step: per-token quantization of the
    activation rows (C oracle, one thread) and the fp64 GEMM reference of those
    rows against the full weight matrix (numpy BLAS), repeated until about ten
    seconds of CPU work have been timed."""
    import numpy as np
    import oracle
    from threadpoolctl import threadpool_info
    c = si.CONFIGS["C3"]
    K, N = c["K"], c["N"]
    a, w = si.gemm_inputs("C3")
    wq = oracle.quantize(w, group_rows=N, want_scale=False)    # offline weight prep: not timed
    R = a.shape[0]
    reps, dt = 0, 0.0
    while dt < 10.0 and reps < 8:
        t0 = time.perf_counter()
        qa = oracle.quantize(a)
        oracle.gemm_ref(qa["codes"], qa["scale"], wq["codes"], wq["sf"], wq["g_dec"][0])
        dt += time.perf_counter() - t0
        reps += 1
    blas = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
    cores = max(blas) if blas else 1
    return {"value": 2.0 * R * N * K * reps / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": "%d repetitions of the full step (%d activation rows): C-oracle per-token quantize "
                      "(1 thread) + fp64 numpy GEMM reference against the %dx%d weight, %.1f s in total"
                      % (reps, R, N, K, dt),
            "quantizers": oracle_quant_rates(si, a), "host": host_info()}


def host_info():
    """Host CPU model and the cores this process may use."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "nproc": len(os.sched_getaffinity(0)), "cpu_count": os.cpu_count()}


def oracle_quant_rates(si, a):
    """The C oracle's quantizer throughput in the GPU figures' byte accounting,
    on a bounded sample of rows: one thread, then all cores of the job's share
    (a thread pool over chunks of rows; the C call releases the GIL)."""
    import oracle
    from concurrent.futures import ThreadPoolExecutor
    # every core this process may use, within the job's CPU share
    ncores = min(len(os.sched_getaffinity(0)), int(os.environ.get("OMP_NUM_THREADS", "16")))

    def rate(x, act, want_scale, k_in, k_out, rows, threads, chunk):
        parts = [x[i:i + chunk] for i in range(0, rows, chunk)]
        f = lambda p: oracle.quantize(p, act, want_scale=want_scale)
        t0 = time.perf_counter()
        if threads == 1:
            for p in parts:
                f(p)
        else:
            with ThreadPoolExecutor(threads) as ex:
                list(ex.map(f, parts))
        dt = time.perf_counter() - t0
        by = quant_bytes(rows, k_in, k_out, scale=want_scale)
        return {"rows": rows, "threads": threads, "s": round(dt, 3), "GBps": by / dt / 1e9}

    c3 = si.CONFIGS["C3"]
    x4 = si.swiglu_input(rows=2048)
    H = x4.shape[1] // 2
    return {
        "C3_act_quant": [rate(a, oracle.ACT_NONE, True, c3["K"], c3["K"], 2048, 1, 256),
                         rate(a, oracle.ACT_NONE, True, c3["K"], c3["K"], a.shape[0], ncores, 64)],
        "C4_swiglu_quant": [rate(x4, oracle.ACT_SWIGLU, False, 2 * H, H, 512, 1, 128),
                            rate(x4, oracle.ACT_SWIGLU, False, 2 * H, H, x4.shape[0], ncores, 32)],
    }


def load_traffic():
    """HBM bytes per GEMM call from the committed counter run, or None when the
    GEMM source has changed since the counters were taken."""
    import hashlib
    try:
        with open(ALGO_TRAFFIC_FILE) as f:
            t = json.load(f)
        src = os.path.join(ROOT, "nvfp4_block_scaled_quantize_amd", "csrc", "gemm.hip")
        with open(src, "rb") as f:
            h = hashlib.sha256(f.read()).hexdigest()
        return t["gemm_call_bytes"] if t.get("gemm_source_sha256") == h else None
    except (OSError, ValueError, KeyError):
        return None


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the NVFP4 path here is a single-GPU build "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch
    import nvfp4_block_scaled_quantize_amd as nv
    import synth_inputs as si
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.only:
        fn = {"prefill": lambda: run_prefill(torch, nv, si, 3, 1),
              "decode": lambda: {B: run_decode(torch, nv, si, B) for B in (1, 4, 8)},
              "swiglu": lambda: run_swiglu(torch, nv, si, iters=3),
              "quant": lambda: run_quant_rotating(torch, nv, si),
              "small": lambda: run_small(torch, nv, si),
              "moe": lambda: run_moe(torch, nv, si),
              "copy": lambda: run_copy(torch),
              "mx_prefill": lambda: run_mx_prefill(torch, nv, si, 3, 1),
              "mx_decode": lambda: {B: run_mx_decode(torch, nv, si, B) for B in (1, 4, 8)}}[args.only]
        print(json.dumps({"only": args.only, "result": fn()}, default=str), flush=True)
        return
    log("prefill: act_quant [4096,8192] + gemm 4096x8192x8192, untimed settle (%.0f ms), %d warmup + %d steps"
        % (SETTLE_MS, args.warmup, args.steps))
    pre = run_prefill(torch, nv, si, args.steps, args.warmup)
    value = pre["flops"] / (pre["ms_step"] * 1e-3) / 1e12
    gemm_tflops = pre["flops"] / (pre["ms_gemm"] * 1e-3) / 1e12
    quant_gbs = pre["qbytes"] / (pre["ms_quant"] * 1e-3) / 1e9
    log("prefill step %.3f ms (gemm %.3f ms = %.1f TFLOP/s, quant %.3f ms = %.0f GB/s)" % (
        pre["ms_step"], pre["ms_gemm"], gemm_tflops, pre["ms_quant"], quant_gbs))
    workloads = {"prefill_C3": {
        "gemm_ms": round(pre["ms_gemm"], 4), "gemm_TFLOPs": round(gemm_tflops, 1),
        "gemm_frac_fp16_peak": round(gemm_tflops / FP16_MFMA_PEAK_TFLOPS, 4),
        "gemm_frac_fp4_peak": round(gemm_tflops / FP4_MFMA_PEAK_TFLOPS, 4),
        "act_quant_ms": round(pre["ms_quant"], 4), "act_quant_GBps": round(quant_gbs, 1),
        "act_quant_hbm_frac": round(quant_gbs / HBM_PEAK_GBS, 4),
        "gemm_untiled_ms": round(pre["ms_gemm_untiled"], 4),
        "gemm_untiled_TFLOPs": round(pre["flops"] / (pre["ms_gemm_untiled"] * 1e-3) / 1e12, 1)}}
    settle_info = {"steps": pre["settle_steps"], "ms": round(pre["settle_ms"], 1),
                   "note": "untimed steps run back to back before the warmup steps, so the GPU clocks "
                           "have risen from idle"}
    if not args.quick:
        for B in (1, 4, 8):
            log("decode B=%d" % B)
            workloads["decode_C2_B%d" % B] = {k: (round(v, 4) if isinstance(v, float) else v)
                                              for k, v in run_decode(torch, nv, si, B).items()}
        log("activation quantize, rotating inputs")
        workloads["quant_C3_rotating"] = {k: (round(v, 4) if isinstance(v, float) else v)
                                          for k, v in run_quant_rotating(torch, nv, si).items()}
        log("swiglu quantize")
        workloads["swiglu_quant_C4"] = {k: (round(v, 4) if isinstance(v, float) else v)
                                        for k, v in run_swiglu(torch, nv, si).items()}
        log("small quantize + gemm")
        workloads["small_C1"] = {k: (round(v, 4) if isinstance(v, float) else v)
                                 for k, v in run_small(torch, nv, si).items()}
        log("mxfp4 prefill step (E8M0 scales, FP4 MFMA)")
        workloads["mx_prefill_C3"] = {k: (round(v, 4) if isinstance(v, float) else v)
                                      for k, v in run_mx_prefill(torch, nv, si, args.steps, args.warmup).items()}
        for B in (1, 4, 8):
            log("mxfp4 decode B=%d" % B)
            workloads["mx_decode_C2_B%d" % B] = {k: (round(v, 4) if isinstance(v, float) else v)
                                                 for k, v in run_mx_decode(torch, nv, si, B).items()}
        try:
            log("moe")
            workloads["moe_C5"] = {k: (round(v, 4) if isinstance(v, float) else v)
                                   for k, v in run_moe(torch, nv, si).items()}
        except Exception as e:  # reported, not hidden
            workloads["moe_C5"] = {"error": str(e)[:200]}
    cpu = None
    if not args.quick and not args.no_cpu:
        log("cpu baseline (oracle sample)")
        cpu = cpu_baseline(si, pre)
    line = {
        "metric": "NVFP4 GEMM TFLOPS + quantize GB/s at 1 MI355X, % of FP4/HBM roofline",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(pre["ms_step"], 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp16",
        "data": "synthetic (seeded bf16 normals; weights quantized to NVFP4 and pre-tiled on the GPU before timing)",
        "config": {"workload": "prefill: per-token act quantize [4096,8192] + NVFP4 GEMM B=4096 K=8192 N=8192",
                   "B": pre["B"], "K": pre["K"], "N": pre["N"], "parallelism": "single GPU"},
        "roofline": {"kernel": "nvfp4_gemm_pretiled (prefill: a_to_f16_rows + gemm_wide<true>)", "bound": "mfma",
                     "achieved": round(gemm_tflops, 1),
                     "peak": FP16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(gemm_tflops / FP16_MFMA_PEAK_TFLOPS, 4),
                     "traffic": load_traffic(), "traffic_unit": "bytes per call"},
        "clock_settle": settle_info,
        "cpu_baseline": cpu,
        "workloads": workloads,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
