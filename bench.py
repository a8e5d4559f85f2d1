#!/usr/bin/env python3
"""Throughput of the Q4 decode path on one MI355X; prints ONE JSON line.

Headline workload: the 7B-class layer in Q4_0 at one token, the configuration
the decode product's roofline target is stated on -- the products
4096->4096, 4096->11008 (x2, gate and up) and 11008->4096, each with its own
seeded activations, 85.5 MB of quantized weights per step. Every product's
weights, activations and outputs are resident in HBM before the timed
region. The four launches are captured once into a HIP graph per weight
copy; each step is one graph launch. The weights rotate over enough copies
(>= 512 MiB) that every step reads them from HBM, not from the 256 MB
Infinity Cache.

  value     = algorithmic bytes per step (quantized W + x + y of the four
              products) x steps / timed seconds  [GB/s]
  roofline  = the dominant kernel, the one-token Q4_0 product at
              4096->11008 (two of the four launches, the most time):
              algorithmic bytes per launch / its average launch time (HIP
              events on the stream its graph is launched on, over a graph of
              launches on rotating copies), against 8 TB/s HBM; beside it the
              median device time of the same launches from the committed
              rocprofv3 trace, when that trace was taken on the current
              kernel sources.

Also reported in "extras": the GPT-2-124M and SmolLM2-360M decode steps as
layer stacks (tokens/s; plain, stacked and gated SmolLM2 stacks), the whole
SmolLM2-360M decode step as a replayed generation loop, the 7B-class shapes
for every format (Q4_0 at one token; Q4_K at 1, 4 and 8 tokens; Q8_0, Q2_K,
Q1_0), the prefill GEMM over a SmolLM2-360M layer at 512 tokens (separate and
stacked matrices), warm steps, launches from a plain stream, the per-launch
floor, and the streaming-read ceiling (a pure read, and the same read storing
a few bytes per wave).
The GPT-2 step and the whole SmolLM2-360M step also carry "device_busy": the
sum of their kernels' traced durations per step from the committed rocprofv3
summary (when taken on the current kernel sources) and the tokens/s it gives.
"cpu_baseline" is the CPU oracle timed on the host cores on whole repeats of
the headline step (bounded to about 10 s).

--profile-shape K,M runs only that product (Q4_0 at one token unless
--profile-fmt / --profile-tokens say otherwise; a graph of launches on rotating
copies, --steps replays) for rocprofv3 runs, one shape per process so that each
trace holds one shape.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
COLD_BYTES = 512 << 20
METRIC = "Q4 decode GEMV effective HBM GB/s (% of peak) + layer-stack tokens/s at 1 GPU"
KERNEL_SOURCES = ["q4_gemv_kernel.h", "q4_gemv_stream.h", "q4_gemv.hip", "q4_gemv_stream.hip", "q4_gemv_q4_0_a.hip",
                  "q4_gemv_q4_0_b.hip"]
DOMINANT = (4096, 11008)  # (K, M) of the headline's dominant product


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def gemv_bytes(q4, fmt, m, k, n, gated=0):
    """Algorithmic bytes of one decode product: quantized W + fp32 x + fp32 y
    (a gated product reads 2m weight rows and writes m outputs)."""
    return q4.q4_weight_bytes(fmt, (2 if gated else 1) * m, k) + 4 * n * k + 4 * n * m


def gemm_bytes(q4, fmt, m, k, n):
    return q4.q4_weight_bytes(fmt, m, k) + 2 * n * k + 4 * n * m


def copies_for(nbytes):
    return max(2, math.ceil(COLD_BYTES / nbytes) + 1)


def kernel_source_hash():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "q4_weight_gemv_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


class Timer:
    """HIP events on torch's current stream, which every launch here uses."""

    def __init__(self, torch):
        self.torch = torch

    def region(self, fn, steps, warmup):
        torch = self.torch
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record()
        for i in range(steps):
            fn(warmup + i)
        end.record()
        torch.cuda.synchronize()
        return start.elapsed_time(end) / 1e3


class Step:
    """A decode step: one set of weights per copy, shared x/y, one graph per copy.
    cold: enough weight copies (>= 512 MiB) that every step reads HBM; warm:
    one copy, replayed (MALL-resident when the step fits in 256 MB).
    run_rotation() replays one graph holding one step per copy, in turn (the
    graph launch's own cost then spreads over the copies' steps)."""

    def __init__(self, torch, q4, shapes, fmt, n, config_id, cold=True, quantize=None):
        import synth

        # Entries (K, M) or (K, M, gated): a gated product reads 2M weight rows.
        # `quantize(fmt, w)` makes the weight buffers (the library's host
        # quantizer unless a caller passes another with the same output).
        quantize = quantize or q4.q4_quantize_ref
        shapes = [tuple(s) + (0,) * (3 - len(s)) for s in shapes]
        self.shapes, self.fmt, self.n, self.q4 = shapes, fmt, n, q4
        self.bytes = sum(gemv_bytes(q4, fmt, m, k, n, g) for k, m, g in shapes)
        self.host_w = [quantize(fmt, synth.weights(synth.seed_for(config_id, i), (2 if g else 1) * m, k))
                       for i, (k, m, g) in enumerate(shapes)]
        self.host_x = [synth.activations(synth.seed_for(config_id, i, True), n, k) for i, (k, m, g) in enumerate(shapes)]
        self.xs = [torch.from_numpy(x).cuda() for x in self.host_x]
        self.ys = [torch.empty((n, m), dtype=torch.float32, device="cuda") for k, m, g in shapes]
        wbytes = sum(h.size for h in self.host_w)
        ncopies = copies_for(wbytes) if cold else 1
        self.copies = [[torch.from_numpy(h).cuda() for h in self.host_w] for _ in range(ncopies)]
        self.graphs = [q4.Q4Graph(fmt, self._ops(ws), n) for ws in self.copies]
        self.seqs = [q4.Q4Sequence(fmt, self._ops(ws), n) for ws in self.copies]
        self.rotation = q4.Q4Graph(fmt, [op for ws in self.copies for op in self._ops(ws)], n)
        self.partial = {}
        torch.cuda.synchronize()

    def _ops(self, ws):
        return [(w, x, y, m, k, g) for w, x, y, (k, m, g) in zip(ws, self.xs, self.ys, self.shapes)]

    def run_graph(self, i):
        self.graphs[i % len(self.graphs)].launch()

    def run_plain(self, q4, i):
        # Back-to-back launches from the library's C loop (arguments marshalled once).
        self.seqs[i % len(self.seqs)].launch()

    def prepare(self, steps):
        """Capture the graph of the remainder steps % copies (before timing)."""
        r = steps % len(self.copies)
        if r and r not in self.partial:
            self.partial[r] = self.q4.Q4Graph(self.fmt, [op for ws in self.copies[:r] for op in self._ops(ws)], self.n)

    def run_steps(self, steps):
        """Exactly `steps` steps: whole rotations (one graph launch each), then
        one launch of a graph holding the remaining steps on the first copies."""
        self.prepare(steps)
        for _ in range(steps // len(self.copies)):
            self.rotation.launch()
        r = steps % len(self.copies)
        if r:
            self.partial[r].launch()

    def close(self):
        for g in list(self.graphs) + [self.rotation] + list(self.partial.values()):
            g.close()


def _profile_field(path, field):
    """A numeric field of a committed rocprofv3 summary, if the summary was
    taken on the current kernel sources (its kernel_source_sha256 line)."""
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"kernel_source_sha256:\s*(\w+)", text)
    t = re.search(field + r":\s*([0-9.eE+]+)", text)
    if not m or not t or m.group(1) != kernel_source_hash():
        return None
    return float(t.group(1))


def traffic_from_profile(path=None):
    """HBM bytes per launch of the dominant product, from the committed counter
    summary, if it was taken on the current kernel sources (else None)."""
    return _profile_field(path or os.path.join(ROOT, "profiles", "pmc_gemv_q4_0_4096x11008.txt"),
                          "hbm_bytes_per_launch")


def trace_median_from_profile(path=None):
    """Median device time (us) of the dominant product's launches, from the
    committed kernel trace, if it was taken on the current kernel sources."""
    return _profile_field(path or os.path.join(ROOT, "profiles", "trace_gemv_q4_0_4096x11008.md"),
                          "median_us")


def kernel_us_per_step_from_profile(path):
    """Device time per step (its kernels' mean traced durations summed) from a
    committed kernel trace summary, if taken on the current kernel sources."""
    return _profile_field(path, "kernel_us_per_step")


def device_busy(name, path=None):
    """The "device_busy" record of a step from its committed trace
    (profiles/<name>), or None. The profiler stretches short kernels, so the
    figure bounds the step's device-busy time from above (it can exceed the
    unprofiled wall time)."""
    us = kernel_us_per_step_from_profile(path or os.path.join(ROOT, "profiles", name))
    if us is None:
        return None
    return {"kernel_us_per_step": us, "tokens_per_s": round(1e6 / us, 1), "from": f"profiles/{name}",
            "note": "sum of traced kernel durations per step; traced short kernels run long"}


def gemm_mfma_busy_from_profile(path=None):
    """MFMA busy (% of the dense bf16 rate) per prefill matrix of the SmolLM2
    layer, from the committed counter summary, if it was taken on the current
    prefill source (else None)."""
    path = path or os.path.join(ROOT, "profiles", "gemm_smollm2_layer_counters.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"kernel_source_sha256:\s*(\w+)", text)
    with open(os.path.join(ROOT, "q4_weight_gemv_amd", "csrc", "q4_gemm.hip"), "rb") as fh:
        cur = hashlib.sha256(fh.read()).hexdigest()[:16]
    if not m or m.group(1) != cur:
        return None
    out = {}
    for k, mm, pct in re.findall(r"^\| (\d+)->(\d+) [^|]*(?:\\\|[^|]*)*\|.*?\| ([0-9.]+) % \|", text, re.M):
        out[f"{k}to{mm}"] = float(pct)
    return out or None


def host_cpu():
    """(cores this process may run on, CPU model) of the host."""
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return cores, model


# Worker threads for the CPU oracle: the host's cores, up to 16 (the CPU share
# of one GPU on a shared GPU host).
CPU_SHARE = 16


def cpu_baseline(step, what, budget_s=10.0, budget_1core_s=6.0):
    """The oracle (as it stands) on whole repeats of the same step, with its
    rows split over the host cores it may use (up to CPU_SHARE), and again on
    one core."""
    import oracle

    def timed(threads, budget):
        t0 = time.perf_counter()
        reps = 0
        while True:
            for i, (k, m, g) in enumerate(step.shapes):
                if g:
                    oracle.matvec_silu_mul(step.fmt, step.host_w[i], m, k, step.host_x[i], threads=threads)
                else:
                    oracle.matvec(step.fmt, step.host_w[i], m, k, step.host_x[i], threads=threads)
            reps += 1
            if time.perf_counter() - t0 >= budget:
                break
        return reps, time.perf_counter() - t0

    cores, model = host_cpu()
    threads = max(1, min(CPU_SHARE, cores))
    reps, dt = timed(threads, budget_s)
    reps1, dt1 = timed(1, budget_1core_s)
    return {
        "value": round(step.bytes * reps / dt / 1e9, 4),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{reps} whole {what} (rows split over {threads} threads), {dt:.1f} s wall",
        "steps_per_s": round(reps / dt, 3),
        "host_cores": cores,
        "cpu_model": model,
        "one_core": {"GB_s": round(step.bytes * reps1 / dt1 / 1e9, 4), "steps_per_s": round(reps1 / dt1, 3),
                     "sample": f"{reps1} whole step(s), {dt1:.1f} s wall"},
    }


def product_time(torch, q4, timer, fmt, k, m, n=1, reps=20, seed_config=4, gated=False):
    """Average launch time (s) of one decode product, cold: a graph of one
    launch per rotating weight copy, replayed, timed with HIP events on the
    stream the graph is launched on. gated: the gated product of a 2m-row
    matrix (m outputs)."""
    import synth

    rows = 2 * m if gated else m
    wq = q4.q4_quantize_ref(fmt, synth.weights(synth.seed_for(seed_config, k + rows), rows, k))
    copies = [torch.from_numpy(wq).cuda() for _ in range(copies_for(wq.size))]
    x = torch.from_numpy(synth.activations(synth.seed_for(seed_config, k, True), n, k)).cuda()
    y = torch.empty((n, m), device="cuda")
    ep = q4.Q4_EPILOGUE_SILU_MUL if gated else q4.Q4_EPILOGUE_NONE
    g = q4.Q4Graph(fmt, [(c, x, y, m, k, ep) for c in copies], n)
    t = timer.region(lambda i: g.launch(), reps, 3) / (reps * len(copies))
    g.close()
    del copies
    return t


def bench_7b(torch, q4, timer, reps=20):
    """7B-class shapes one product at a time, cold: a graph of one launch per
    rotating weight copy, replayed."""
    import synth

    out = {}
    name = {0: "q4_0", 1: "q4_k", 2: "q8_0", 3: "q2_k", 4: "q1_0"}
    # Q4_0 at one token (the headline's format), Q4_K at 1, 4, 8 tokens, and
    # Q8_0, Q2_K and Q1_0 at one token beside them (the pages compare q8_0,
    # q4_k_m and q2_k, and name q1_0 as a format added through one
    # dequantization routine).
    for fmt, ns in ((0, (1,)), (1, (1, 4, 8)), (2, (1,)), (3, (1,)), (4, (1,))):
        layer_t, layer_b = 0.0, 0
        for k, m in synth.llama7b_layer()[:2] + synth.llama7b_layer()[3:]:
            for n in ns:
                t = product_time(torch, q4, timer, fmt, k, m, n, reps)
                nb = gemv_bytes(q4, fmt, m, k, n)
                key = f"{name[fmt]}_{k}to{m}_n{n}"
                out[key] = {"us": round(t * 1e6, 3), "GB_s": round(nb / t / 1e9, 1),
                            "pct_peak": round(100 * nb / t / 1e9 / HBM_PEAK_GBS, 1)}
                log(f"{key}: {t * 1e6:.2f} us {nb / t / 1e9:.0f} GB/s")
                if n == 1:
                    mult = 2 if (k, m) == (4096, 11008) else 1  # gate and up
                    layer_t += mult * t
                    layer_b += mult * nb
        key = f"{name[fmt]}_7b_layer_as_listed_n1"
        out[key] = {"us": round(layer_t * 1e6, 2), "GB_s": round(layer_b / layer_t / 1e9, 1),
                    "pct_peak": round(100 * layer_b / layer_t / 1e9 / HBM_PEAK_GBS, 1),
                    "note": "sum of the products' separate per-launch times"}
        torch.cuda.empty_cache()
    # The gate and up projections as one gated product (4096 -> 2 x 11008,
    # silu(g) * u): Q4_0 at one token, Q4_K at 1, 4 and 8.
    for fmt, ns in ((0, (1,)), (1, (1, 4, 8))):
        for n in ns:
            t = product_time(torch, q4, timer, fmt, 4096, 11008, n, reps, gated=True)
            nb = gemv_bytes(q4, fmt, 11008, 4096, n, gated=1)
            key = f"{name[fmt]}_gated_4096to2x11008_n{n}"
            out[key] = {"us": round(t * 1e6, 3), "GB_s": round(nb / t / 1e9, 1),
                        "pct_peak": round(100 * nb / t / 1e9 / HBM_PEAK_GBS, 1)}
            log(f"{key}: {t * 1e6:.2f} us {nb / t / 1e9:.0f} GB/s")
        torch.cuda.empty_cache()
    return out


def sweep_one_token(torch, q4, timer, reps=10, out=None):
    """Time every streaming geometry and the library's tiled choice for one
    token, cold (a graph of one launch per rotating weight copy), at the
    workload shapes: Q4_0 at every GPT-2-124M, SmolLM2-360M and 7B-class
    shape; the other formats at the 7B-class and SmolLM2 shapes. One JSON
    line per measurement (the evidence behind the library's defaults)."""
    import synth

    name = {0: "q4_0", 1: "q4_k", 2: "q8_0", 3: "q2_k", 4: "q1_0"}
    small = sorted(set(synth.gpt2_124m_step() + synth.smollm2_360m_step()))
    big = sorted(set(synth.llama7b_layer()))
    s = torch.cuda.Stream()
    for fmt in (0, 1, 2, 3, 4):
        shapes = small + big if fmt == 0 else sorted(set(synth.smollm2_360m_step())) + big
        for k, m in shapes:
            if k % (256 if fmt in (1, 3) else 32):
                continue
            wq = q4.q4_quantize_ref(fmt, synth.weights(synth.seed_for(6, k + m), m, k))
            copies = [torch.from_numpy(wq).cuda() for _ in range(copies_for(wq.size))]
            x = torch.from_numpy(synth.activations(synth.seed_for(6, k, True), 1, k)).cuda()
            y = torch.empty((1, m), device="cuda")
            nb = gemv_bytes(q4, fmt, m, k, 1)
            cfgs = [("tiled", dict(kernel=q4.Q4_GEMV_KERNEL_TILED))] + [
                (f"stream L{g[0]} W{g[1]} D{g[2]}", dict(kernel=q4.Q4_GEMV_KERNEL_STREAM, lanes_per_row=g[0],
                                                        waves_per_group=g[1], groups_per_cu=gpc, depth=g[2]))
                for g in q4.GEMV_STREAM_GEOMETRIES for gpc in ((4, 8) if g[1] == 1 else (1, 2) if g[1] <= 8 else (1,))]
            cfgs = [(f"{label} G{kw.get('groups_per_cu', 0)}" if "stream" in label else label, kw) for label, kw in cfgs]
            for label, kw in cfgs:
                g = torch.cuda.CUDAGraph()
                with torch.cuda.stream(s):
                    q4.q4_gemv_tuned(fmt, copies[0], x, y, m, k, stream=s, **kw)
                    torch.cuda.synchronize()
                    with torch.cuda.graph(g, stream=s):
                        for c in copies:
                            q4.q4_gemv_tuned(fmt, c, x, y, m, k, stream=s, **kw)
                t = timer.region(lambda i: g.replay(), reps, 2) / (reps * len(copies))
                del g
                rec = {"format": name[fmt], "shape": f"{k}->{m}", "kernel": label, "us": round(t * 1e6, 3),
                       "pct_peak": round(100 * nb / t / 1e9 / HBM_PEAK_GBS, 2)}
                print(json.dumps(rec), flush=True)
                if out is not None:
                    out.append(rec)
            del copies
            torch.cuda.empty_cache()


def sweep_tokens(torch, q4, timer, reps=10):
    """Q4_K decode products at 2..8 tokens: the tiled kernel (the library's
    tiled choice) against the matrix-core kernel (one and two workgroups per
    compute unit) and the library's default, cold, at the 7B-class shapes and
    two others (short and long rows). One JSON line per measurement (the
    evidence behind the library's choice of kernel)."""
    import synth

    shapes = sorted(set(synth.llama7b_layer())) + [(2048, 8192), (8192, 2048)]
    s = torch.cuda.Stream()
    for k, m in shapes:
        wq = q4.q4_quantize_ref(1, synth.weights(synth.seed_for(6, k + m), m, k))
        copies = [torch.from_numpy(wq).cuda() for _ in range(copies_for(wq.size))]
        for n in range(2, 9):
            x = torch.from_numpy(synth.activations(synth.seed_for(6, k + n, True), n, k)).cuda()
            y = torch.empty((n, m), device="cuda")
            nb = gemv_bytes(q4, 1, m, k, n)
            for label, kw in (("tiled", dict(kernel=q4.Q4_GEMV_KERNEL_TILED)),
                              ("matrix G1", dict(kernel=q4.Q4_GEMV_KERNEL_MATRIX, groups_per_cu=1)),
                              ("matrix G2", dict(kernel=q4.Q4_GEMV_KERNEL_MATRIX, groups_per_cu=2)),
                              ("library", dict())):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.stream(s):
                    q4.q4_gemv_tuned(1, copies[0], x, y, m, k, stream=s, **kw)
                    torch.cuda.synchronize()
                    with torch.cuda.graph(g, stream=s):
                        for c in copies:
                            q4.q4_gemv_tuned(1, c, x, y, m, k, stream=s, **kw)
                t = timer.region(lambda i: g.replay(), reps, 2) / (reps * len(copies))
                del g
                print(json.dumps({"format": "q4_k", "shape": f"{k}->{m}", "tokens": n, "kernel": label,
                                  "us": round(t * 1e6, 3), "pct_peak": round(100 * nb / t / 1e9 / HBM_PEAK_GBS, 2)}),
                      flush=True)
        del copies
        torch.cuda.empty_cache()


def sweep_gemm(torch, q4, timer, n=512, reps=10):
    """Every instantiated prefill tile against the library's choice at the
    SmolLM2-360M layer shapes x 512 tokens, Q4_0 (graphs of 20 launches per
    tile). One JSON line per measurement."""
    import synth

    s = torch.cuda.Stream()
    for k, m in sorted(set(synth.smollm2_360m_layer())):
        wq = torch.from_numpy(q4.q4_quantize_ref(0, synth.weights(synth.seed_for(7, k + m), m, k))).cuda()
        xb = torch.from_numpy(synth.bf16_bits(synth.activations(synth.seed_for(7, k, True), n, k)).view(np.int16)).cuda()
        y = torch.empty((n, m), device="cuda")
        for label, tile in [("library", None)] + [(f"{t[0]}x{t[1]}x{t[2]}", t) for t in q4.GEMM_TILES]:
            def launch():
                if tile is None:
                    q4.q4_gemm(0, wq, xb, y, m, k, stream=s)
                else:
                    q4.q4_gemm_tuned(0, wq, xb, y, m, k, tile[0], tile[1], tile[2], stream=s)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.stream(s):
                launch()
                torch.cuda.synchronize()
                with torch.cuda.graph(g, stream=s):
                    for _ in range(20):
                        launch()
            t = timer.region(lambda i: g.replay(), reps, 2) / (reps * 20)
            del g
            print(json.dumps({"format": "q4_0", "shape": f"{k}->{m}", "tokens": n, "tile": label,
                              "us": round(t * 1e6, 3), "TFLOP_s": round(2 * n * m * k / t / 1e12, 1)}), flush=True)


def bench_gemm(torch, q4, timer, n=512, reps=20, shapes=None, per_matrix=True):
    """Prefill GEMM over the SmolLM2-360M layer's matrices at 512 tokens:
    one graph of the launches, replayed (weights 5.5 MB, L2/MALL-resident);
    and each matrix alone, as a graph of 20 launches."""
    import synth

    fns, flops, per = [], 0, {}
    for i, (k, m) in enumerate(shapes or synth.smollm2_360m_layer()):
        wq = torch.from_numpy(q4.q4_quantize_ref(0, synth.weights(synth.seed_for(3, i), m, k))).cuda()
        xb = torch.from_numpy(synth.bf16_bits(synth.activations(synth.seed_for(3, i, True), n, k)).view(np.int16)).cuda()
        y = torch.empty((n, m), device="cuda")
        fns.append((wq, xb, y, m, k))
        flops += 2 * n * m * k
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        for (w, xb, y, m, k) in fns:
            q4.q4_gemm(0, w, xb, y, m, k)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            for (w, xb, y, m, k) in fns:
                q4.q4_gemm(0, w, xb, y, m, k)
    t = timer.region(lambda i: g.replay(), reps, 3) / reps
    tf = flops / t / 1e12
    log(f"gemm smollm2 layer x{n}: {t * 1e6:.1f} us {tf:.1f} TFLOP/s")
    out = {"layer_us": round(t * 1e6, 2), "TFLOP_s": round(tf, 1), "pct_bf16_peak": round(100 * tf / BF16_PEAK_TFLOPS, 2),
           "GFLOP": round(flops / 1e9, 3), "tokens": n, "launches": len(fns)}
    if per_matrix:
        seen = set()
        for (w, xb, y, m, k) in fns:
            if (k, m) in seen:
                continue
            seen.add((k, m))
            gm = torch.cuda.CUDAGraph()
            with torch.cuda.stream(s):
                with torch.cuda.graph(gm, stream=s):
                    for _ in range(20):
                        q4.q4_gemm(0, w, xb, y, m, k)
            tm = timer.region(lambda i: gm.replay(), reps, 3) / (reps * 20)
            # Context only, not the product path: the vendor library's dense
            # bf16 GEMM (torch.mm -> hipBLASLt) on the same shape with weights
            # already in bf16 (4x the weight bytes, no dequantization), bf16 out.
            wt = (torch.randn(k, m, device="cuda") * 0.02).to(torch.bfloat16).contiguous()
            xd = xb.view(torch.bfloat16)
            yd = torch.empty((n, m), device="cuda", dtype=torch.bfloat16)
            gl = torch.cuda.CUDAGraph()
            with torch.cuda.stream(s):
                torch.mm(xd, wt, out=yd)
                torch.cuda.synchronize()
                with torch.cuda.graph(gl, stream=s):
                    for _ in range(20):
                        torch.mm(xd, wt, out=yd)
            tl = timer.region(lambda i: gl.replay(), reps, 3) / (reps * 20)
            per[f"{k}to{m}"] = {"us": round(tm * 1e6, 2), "TFLOP_s": round(2 * n * m * k / tm / 1e12, 1),
                                "library_dense_bf16_us": round(tl * 1e6, 2)}
        out["per_matrix"] = per
    return out


def bench_full_step(torch, q4, timer, fmt=0, steps=256, warmup=8):
    """The whole SmolLM2-360M decode step (embedding, 32 layers of products with
    the residual add + RMSNorm fused in, attention with its KV cache, the gated
    MLP, LM head, greedy token) as one
    captured graph, replayed as a generation loop: tokens chain on the device.
    One copy of the weights (a generation loop rereads the same model each step;
    203 MB of Q4_0 weights fit the 256 MB memory-side cache)."""
    import synth

    cfg = dict(synth.SMOLLM2_360M)
    fw = synth.llama_float_weights(cfg)
    dev = {}
    wbytes = 0
    for k, v in fw.items():
        if k.startswith("norm"):
            dev[k] = torch.from_numpy(v).cuda()
        else:
            buf = q4.q4_quantize_ref(fmt, v)
            wbytes += buf.size
            dev[k] = torch.from_numpy(buf).cuda()
    del fw
    st = q4.LlamaStep(fmt, cfg, dev)
    st.set(token=1, pos=0)
    st.capture()
    for _ in range(warmup):
        st.replay()
    torch.cuda.synchronize()
    t = timer.region(lambda i: st.replay(), steps, 0) / steps
    pos = int(st.buf["pos"].item())
    st.close()
    launches = 3 + 5 * cfg["layers"]  # embedding; per layer 5; LM head, selection
    log(f"full step smollm2-360m: {t * 1e6:.1f} us/token, {1 / t:.0f} tokens/s")
    return {"us_per_token": round(t * 1e6, 2), "tokens_per_s": round(1 / t, 1), "launches_per_step": launches,
            "weight_bytes": wbytes, "GB_s_weights": round(wbytes / t / 1e9, 1),
            "positions": f"{warmup}..{pos - 1}", "format": {0: "Q4_0", 1: "Q4_K", 2: "Q8_0", 3: "Q2_K", 4: "Q1_0"}[fmt],
            "cache": "one weight copy (a generation loop)"}


def bench_read_ceiling(torch, q4, timer, reps=20):
    """The measured streaming-read ceiling: 1 GiB read once per launch, and the
    7B-class weight sizes read cold (rotating copies, one graph of launches):
    a pure read, and the same read storing one 4-byte fold per wave (as a
    product stores its outputs: the kernel's end then writes dirty lines back)."""
    sink = torch.zeros(4 * 4096, dtype=torch.int32, device="cuda")  # one word per wave
    out = {}
    big = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
    t = timer.region(lambda i: q4.q4_read_probe(big, None, groups=4096), 10, 2) / 10
    out["1GiB"] = {"us": round(t * 1e6, 1), "GB_s": round(big.numel() / t / 1e9, 1)}
    del big
    for nbytes in (9_437_184, 25_362_432):
        copies = [torch.ones(nbytes, dtype=torch.uint8, device="cuda") for _ in range(copies_for(nbytes))]
        for key, sk in ((f"{nbytes}B_cold", None), (f"{nbytes}B_cold_with_fold_stores", sink)):
            g = torch.cuda.CUDAGraph()
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                q4.q4_read_probe(copies[0], sk, groups=2048)
                torch.cuda.synchronize()
                with torch.cuda.graph(g, stream=s):
                    for c in copies:
                        q4.q4_read_probe(c, sk, groups=2048)
            t = timer.region(lambda i: g.replay(), reps, 3) / (reps * len(copies))
            out[key] = {"us": round(t * 1e6, 3), "GB_s": round(nbytes / t / 1e9, 1)}
            del g
        del copies
    torch.cuda.empty_cache()
    log(f"read ceiling: {out}")
    return out


def launch_floor(torch, q4, timer, count=200):
    """Per-launch time of a tiny decode product (64 x 768) in a graph of 200."""
    import synth

    w = torch.from_numpy(q4.q4_quantize_ref(0, synth.weights(9, 64, 768))).cuda()
    x = torch.from_numpy(synth.activations(9, 1, 768)).cuda()
    y = torch.empty((1, 64), device="cuda")
    g = q4.Q4Graph(0, [(w, x, y, 64, 768)] * count, 1)
    t = timer.region(lambda i: g.launch(), 10, 2) / (10 * count)
    g.close()
    return round(t * 1e6, 3)


def arithmetic_label(fmt_name):
    return (f"{fmt_name} weights decoded in registers to exact fp16 codes; activations scaled per 32-element "
            "unit by a power of two and rounded to one fp16 value each (products of 256 rows or more; shorter "
            "ones keep hi+lo fp16 pairs); v_dot2 products, fp32 accumulation")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="only the headline workload")
    ap.add_argument("--extras", default="all",
                    help="comma list of extras to run (default all): gpt2, plain, floor, gate_7b, smollm2, "
                         "smollm2_fused, smollm2_gated, warm, read_ceiling, full_step, gemm")
    ap.add_argument("--profile-shape", default=None,
                    help="K,M: run only this Q4_0 one-token product, cold, --steps graph replays (for rocprofv3)")
    ap.add_argument("--profile-fmt", type=int, default=0,
                    help="with --profile-shape: the format (0 Q4_0, 1 Q4_K, 2 Q8_0, 3 Q2_K, 4 Q1_0)")
    ap.add_argument("--profile-tokens", type=int, default=1, help="with --profile-shape: tokens (1..8)")
    ap.add_argument("--sweep", action="store_true",
                    help="time every one-token geometry at the workload shapes (one JSON line each) and exit")
    ap.add_argument("--sweep-tokens", action="store_true",
                    help="time the tiled and matrix-core kernels for Q4_K at 2..8 tokens (JSON lines), then exit")
    ap.add_argument("--sweep-gemm", action="store_true",
                    help="time every prefill tile at the SmolLM2-360M layer x 512 tokens (JSON lines), then exit")
    ap.add_argument("--calibrate", action="store_true",
                    help="also run a plain 64 MiB device copy (torch) once, as the reference for HBM byte counters")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "bench.py measures one GPU: run with --gpus 1 (nothing here uses a second GPU)"}))
        sys.exit(2)

    import torch

    import q4_weight_gemv_amd as q4
    import synth

    assert torch.cuda.is_available(), "bench needs a GPU"
    torch.cuda.set_device(0)
    timer = Timer(torch)
    K, W = args.steps, args.warmup

    if args.calibrate:
        # A plain copy of known size: its FETCH_SIZE / WRITE_SIZE counters
        # (64 MiB each way) scale the decode kernel's counters to bytes.
        src = torch.ones(64 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        flush.fill_(2)  # 1 GiB of writes evicts src from L2 and the Infinity Cache
        torch.cuda.synchronize()
        del flush
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if args.sweep:
        sweep_one_token(torch, q4, timer)
        return
    if args.sweep_tokens:
        sweep_tokens(torch, q4, timer)
        return
    if args.sweep_gemm:
        sweep_gemm(torch, q4, timer)
        return

    if args.profile_shape:
        pk, pm = (int(v) for v in args.profile_shape.split(","))
        pf, pn = args.profile_fmt, args.profile_tokens
        t = product_time(torch, q4, timer, pf, pk, pm, pn, reps=K)
        nb = gemv_bytes(q4, pf, pm, pk, pn)
        names = {0: "Q4_0", 1: "Q4_K", 2: "Q8_0", 3: "Q2_K", 4: "Q1_0"}
        print(json.dumps({"profile_shape": f"{pk}->{pm}", "format": names.get(pf, str(pf)), "tokens": pn,
                          "us_per_launch": round(t * 1e6, 3), "GB_s": round(nb / t / 1e9, 1),
                          "kernel_source_sha256": kernel_source_hash()}), flush=True)
        return

    shapes = synth.llama7b_layer()
    log(f"setup 7B-class Q4_0 layer: {len(shapes)} products")
    step = Step(torch, q4, shapes, 0, 1, config_id=4)
    # One graph launch runs one step on every weight copy in turn; exactly K
    # steps are timed (whole rotations, then the remainder in one launch).
    nc = len(step.copies)
    step.prepare(K)
    step.run_steps(W)
    torch.cuda.synchronize()
    t = timer.region(lambda i: step.run_steps(K), 1, 0)
    value = step.bytes * K / t / 1e9
    log(f"graph: {t / K * 1e6:.2f} us/step, {value:.1f} GB/s")

    # The dominant kernel: the product at 4096->11008 (gate and up: two of the
    # four launches, the most time), timed alone the same way.
    dk, dm = DOMINANT
    per_launch_bytes = gemv_bytes(q4, 0, dm, dk, 1)
    reps_dom = max(100, K // 10)  # a stable average, whatever K the headline times
    t_dom = product_time(torch, q4, timer, 0, dk, dm, 1, reps=reps_dom)
    achieved = per_launch_bytes / t_dom / 1e9
    per_shape = {}
    for (k, m) in sorted(set(shapes)):
        tp = t_dom if (k, m) == DOMINANT else product_time(torch, q4, timer, 0, k, m, 1, reps=reps_dom)
        nb = gemv_bytes(q4, 0, m, k, 1)
        per_shape[f"{k}to{m}"] = {"us": round(tp * 1e6, 3), "GB_s": round(nb / tp / 1e9, 1),
                                  "pct_peak": round(100 * nb / tp / 1e9 / HBM_PEAK_GBS, 1)}
        # the committed kernel trace of this shape (one process per shape), if current
        med = trace_median_from_profile(os.path.join(ROOT, "profiles", f"trace_gemv_q4_0_{k}x{m}.md"))
        if med is not None:
            per_shape[f"{k}to{m}"]["trace_median_us"] = med
            per_shape[f"{k}to{m}"]["trace_pct_peak"] = round(100 * nb / (med * 1e3) / HBM_PEAK_GBS, 1)
    traffic = traffic_from_profile()
    median_us = trace_median_from_profile()
    log(f"dominant {dk}->{dm}: {t_dom * 1e6:.3f} us/launch, {achieved:.1f} GB/s")

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(t / K * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16 products, fp32 accumulation",
        "arithmetic": arithmetic_label("Q4_0"),
        "data": "synthetic: seeded N(0, 0.02) weights, N(0, 1) activations; no checkpoints",
        "config": {
            "workload": "7B-class layer, Q4_0, one token: 4096->4096, 4096->11008 x2, 11008->4096",
            "format": "Q4_0",
            "tokens": 1,
            "products_per_step": len(shapes),
            "bytes_per_step": step.bytes,
            "launch": f"HIP graph replay: one graph launch runs one step on each of the {nc} weight copies",
            "cache": f"cold: {nc} rotating weight copies (>= 512 MiB)",
        },
        "layer_steps_per_s": round(K / t, 1),
        "pct_of_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": None if traffic is None else round(traffic),
            "kernel": f"one-token Q4_0 decode product at {dk}->{dm}",
            "per_launch_bytes": per_launch_bytes,
            "avg_launch_us": round(t_dom * 1e6, 3),
            "trace_median_us": median_us,
            "frac_trace_median": None if median_us is None else round(per_launch_bytes / (median_us * 1e3) / HBM_PEAK_GBS, 4),
            "kernel_source_sha256": kernel_source_hash(),
        },
        "layer_products": per_shape,
    }

    if not args.no_extras:
        extras = {}
        want = set(args.extras.split(",")) if args.extras != "all" else None
        on = lambda name: want is None or name in want  # noqa: E731
        gpt2 = None
        if on("gpt2") or on("plain"):
            log("setup GPT-2-124M step")
            gpt2 = Step(torch, q4, synth.gpt2_124m_step(), 0, 1, config_id=1)
            ng = max(50, K // 5)
            tg = timer.region(gpt2.run_graph, ng, 5) / ng
            extras["gpt2_step"] = {"us_per_step": round(tg * 1e6, 2), "tokens_per_s": round(1 / tg, 1),
                                   "GB_s": round(gpt2.bytes / tg / 1e9, 1), "products": len(gpt2.shapes),
                                   "avg_launch_us": round(tg / len(gpt2.shapes) * 1e6, 3),
                                   "cache": f"cold: {len(gpt2.copies)} copies", "launch": "HIP graph"}
            busy = device_busy("trace_gemv_gpt2_step.md")
            if busy is not None:
                extras["gpt2_step"]["device_busy"] = busy
            log(f"gpt2 step: {tg * 1e6:.1f} us")
            if on("plain"):
                n_plain = max(20, K // 10)
                tp = timer.region(lambda i: gpt2.run_plain(q4, i), n_plain, 5)
                extras["gpt2_plain_stream"] = {"us_per_step": round(tp / n_plain * 1e6, 2),
                                               "tokens_per_s": round(n_plain / tp, 1)}
            gpt2.close()
            del gpt2
            torch.cuda.empty_cache()
        if on("floor"):
            extras["launch_floor_us"] = launch_floor(torch, q4, timer)
        if on("gate_7b"):
            extras["gate_7b"] = bench_7b(torch, q4, timer, reps=max(2, K // 50))
        for name, key, shapes_fn in (("smollm2", "smollm2_step", synth.smollm2_360m_step),
                                     ("smollm2_fused", "smollm2_step_fused_qkv_gateup", synth.smollm2_360m_step_fused),
                                     ("smollm2_gated", "smollm2_step_qkv_stacked_gated_mlp", synth.smollm2_360m_step_gated)):
            if not on(name):
                continue
            log(f"setup {key}")
            sm = Step(torch, q4, shapes_fn(), 0, 1, config_id=2)
            ns = max(50, K // 10)
            ts = timer.region(sm.run_graph, ns, 5) / ns
            extras[key] = {"us_per_step": round(ts * 1e6, 2), "tokens_per_s": round(1 / ts, 1),
                           "GB_s": round(sm.bytes / ts / 1e9, 1), "products": len(sm.shapes),
                           "cache": f"cold: {len(sm.copies)} copies"}
            log(f"{key}: {ts * 1e6:.1f} us, {1 / ts:.0f} tokens/s")
            sm.close()
            del sm
            torch.cuda.empty_cache()
        if on("warm"):
            for name, shp, cid in (("gpt2_step_warm", synth.gpt2_124m_step(), 1),
                                   ("smollm2_step_warm", synth.smollm2_360m_step(), 2)):
                wst = Step(torch, q4, shp, 0, 1, config_id=cid, cold=False)
                nw = max(50, K // 10)
                tw = timer.region(wst.run_graph, nw, 5) / nw
                extras[name] = {"us_per_step": round(tw * 1e6, 2), "tokens_per_s": round(1 / tw, 1),
                                "GB_s": round(wst.bytes / tw / 1e9, 1), "cache": "warm: one weight copy (MALL-resident)"}
                log(f"{name}: {tw * 1e6:.1f} us")
                wst.close()
                del wst
            torch.cuda.empty_cache()
        if on("read_ceiling"):
            extras["read_ceiling"] = bench_read_ceiling(torch, q4, timer)
        if on("full_step"):
            extras["smollm2_full_decode_step"] = bench_full_step(torch, q4, timer)
            busy = device_busy("step_smollm2_kernel_trace.md")
            if busy is not None:
                extras["smollm2_full_decode_step"]["device_busy"] = busy
        if on("gemm"):
            extras["gemm_smollm2_layer"] = bench_gemm(torch, q4, timer, reps=max(2, K // 50))
            busy = gemm_mfma_busy_from_profile()
            if busy is not None:
                extras["gemm_smollm2_layer"]["mfma_busy_pct_by_counters"] = busy
            extras["gemm_smollm2_layer_fused_qkv_gateup"] = bench_gemm(
                torch, q4, timer, reps=max(2, K // 50), shapes=synth.smollm2_360m_layer_stacked(),
                per_matrix=False)
        result["extras"] = extras

    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline(step, "7B-class Q4_0 layer step(s) (4 products)")
    step.close()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
