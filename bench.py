#!/usr/bin/env python3
"""Throughput of the Q4 decode path on one MI355X.

Default workload: the GPT-2-124M decode step (12 layers x {768->2304,
768->768, 768->3072, 3072->768} + the 768->50257 LM head = 49 Q4_0 decode
products, batch 1), captured once into a HIP graph per weight copy and
replayed, one graph launch per step. Weights rotate over enough copies
(>= 512 MiB in total) that every step reads them from HBM, not from the
256 MB Infinity Cache. Inputs are resident in HBM before timing starts.

value = algorithmic bytes per step (weights + x + y) x steps
        / timed seconds, in GB/s; tokens/s = steps / timed seconds.

Also reported: the 7B-class shapes one at a time (Q4_0 at N=1, and Q4_K at
N=1/4/8), the SmolLM2-360M step, and the prefill GEMM, and the CPU oracle
timed on a bounded sample of the same step.

Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
COLD_BYTES = 512 << 20


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def gemv_bytes(m, k, n, fmt=0):
    """Algorithmic bytes of one decode product: quantized W + x + y."""
    import q4_weight_gemv_amd as q4

    return q4.q4_weight_bytes(fmt, m, k) + 4 * n * k + 4 * n * m


class Step:
    """A decode step: one weight set per copy, shared x/y buffers, one graph per copy."""

    def __init__(self, shapes, fmt, n, config_id, copies, torch, q4):
        import synth

        self.shapes = shapes
        self.fmt = fmt
        self.n = n
        self.bytes = sum(gemv_bytes(m, k, n, fmt) for k, m in shapes)
        host = []
        for i, (k, m) in enumerate(shapes):
            w = synth.weights(synth.seed_for(config_id, i), m, k)
            host.append(q4.q4_quantize_ref(fmt, w))
        self.host_w = host
        self.xs = [torch.from_numpy(synth.activations(synth.seed_for(config_id, i, True), n, k)).cuda()
                   for i, (k, m) in enumerate(shapes)]
        self.ys = [torch.empty((n, m), dtype=torch.float32, device="cuda") for k, m in shapes]
        self.copies = []
        for c in range(copies):
            self.copies.append([torch.from_numpy(h).cuda() for h in host])
        self.graphs = []
        for ws in self.copies:
            ops = [(w, x, y, m, k) for w, x, y, (k, m) in zip(ws, self.xs, self.ys, shapes)]
            self.graphs.append(q4.Q4Graph(fmt, ops, n))
        torch.cuda.synchronize()

    def run_graph(self, i):
        self.graphs[i % len(self.graphs)].launch()

    def run_plain(self, i, q4):
        ws = self.copies[i % len(self.copies)]
        ops = [(w, x, y, m, k) for w, x, y, (k, m) in zip(ws, self.xs, self.ys, self.shapes)]
        q4.q4_gemv_sequence(self.fmt, ops, self.n)

    def close(self):
        for g in self.graphs:
            g.close()


def copies_for(step_bytes):
    return max(2, math.ceil(COLD_BYTES / step_bytes) + 1)


def time_region(torch, fn, steps, warmup):
    """HIP events on torch's current stream (the stream every launch uses)."""
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
    return start.elapsed_time(end) / 1e3  # seconds


def cpu_baseline(step, budget_s=20.0):
    """The oracle on the host cores over a bounded sample of the same step."""
    import oracle

    threads = max(1, min(16, os.cpu_count() or 1))
    host_x = [x.cpu().numpy() for x in step.xs]
    t0 = time.perf_counter()
    done_bytes = 0
    done = 0
    for i, (k, m) in enumerate(step.shapes):
        oracle.matvec(step.fmt, step.host_w[i], m, k, host_x[i], threads=threads)
        done_bytes += gemv_bytes(m, k, step.n, step.fmt)
        done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return {
        "value": round(done_bytes / dt / 1e9, 4),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{done} of {len(step.shapes)} products of one decode step (rows split over {threads} threads), "
                  f"{dt:.1f} s",
        "tokens_per_s": round((done_bytes / step.bytes) / dt, 4),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="only the headline workload")
    ap.add_argument("--workload", default="gpt2", choices=["gpt2", "smollm2", "llama7b"])
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "this build measures one GPU only; --gpus must be 1"}))
        sys.exit(2)

    import torch

    import q4_weight_gemv_amd as q4
    import synth

    assert torch.cuda.is_available(), "bench needs a GPU"
    torch.cuda.set_device(0)
    K, W = args.steps, args.warmup

    shapes = {"gpt2": synth.gpt2_124m_step(), "smollm2": synth.smollm2_360m_step(),
              "llama7b": synth.llama7b_layer()}[args.workload]
    config_id = {"gpt2": 1, "smollm2": 2, "llama7b": 4}[args.workload]
    step_bytes = sum(gemv_bytes(m, k, 1) for k, m in shapes)
    log(f"setup {args.workload}: {len(shapes)} products, {step_bytes / 1e6:.2f} MB/step")
    step = Step(shapes, 0, 1, config_id, copies_for(step_bytes), torch, q4)
    t = time_region(torch, step.run_graph, K, W)
    log(f"graph: {t / K * 1e6:.2f} us/step")
    value = step.bytes * K / t / 1e9
    per_launch_bytes = step.bytes / len(shapes)
    per_launch_s = t / (K * len(shapes))
    result = {
        "metric": "Q4 decode GEMV effective HBM GB/s (% of peak) + layer-stack tokens/s at 1 GPU",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(t / K * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "q4_0 weights, fp16 x products, fp32 accumulate",
        "data": "synthetic (seeded N(0,0.02) weights, N(0,1) activations; no checkpoints)",
        "config": {
            "workload": {"gpt2": "GPT-2-124M decode step", "smollm2": "SmolLM2-360M decode step",
                         "llama7b": "7B-class layer as listed"}[args.workload],
            "format": "Q4_0",
            "tokens": 1,
            "products_per_step": len(shapes),
            "bytes_per_step": step.bytes,
            "launch": "HIP graph replay, one launch per step",
            "cache": f"cold: {len(step.copies)} rotating weight copies",
        },
        "tokens_per_s": round(K / t, 1),
        "pct_of_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "roofline": {
            "bound": "hbm",
            "achieved": round(per_launch_bytes / per_launch_s / 1e9, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(per_launch_bytes / per_launch_s / 1e9 / HBM_PEAK_GBS, 4),
            "traffic": None,
            "kernel": "q4::gemv_kernel (all 49 launches of the step)",
            "per_launch_bytes": round(per_launch_bytes),
            "avg_launch_us": round(per_launch_s * 1e6, 3),
        },
    }

    if not args.no_extras:
        extras = {}
        tp = time_region(torch, lambda i: step.run_plain(i, q4), max(10, K // 4), 3)
        extras["plain_stream_us_per_step"] = round(tp / max(10, K // 4) * 1e6, 2)
        extras["plain_stream_tokens_per_s"] = round(max(10, K // 4) / tp, 1)
        extras.update(bench_shapes(torch, q4, synth))
        result["extras"] = extras

    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline(step)
    step.close()
    print(json.dumps(result))


def bench_shapes(torch, q4, synth, reps=20):
    """Single products at the 7B-class shapes, cold: a graph of one launch per
    rotating weight copy, replayed; HIP events over the replays."""
    out = {}
    for fmt, ns in ((0, (1,)), (1, (1, 4, 8))):
        for k, m in (synth.llama7b_layer()[:2] + synth.llama7b_layer()[3:]):
            wq = q4.q4_quantize_ref(fmt, synth.weights(synth.seed_for(4, k + m), m, k))
            copies = [torch.from_numpy(wq).cuda() for _ in range(copies_for(wq.size))]
            for n in ns:
                x = torch.from_numpy(synth.activations(synth.seed_for(4, k, True), n, k)).cuda()
                y = torch.empty((n, m), device="cuda")
                g = q4.Q4Graph(fmt, [(c, x, y, m, k) for c in copies], n)
                t = time_region(torch, lambda i: g.launch(), reps, 3) / (reps * len(copies))
                g.close()
                gbs = gemv_bytes(m, k, n, fmt) / t / 1e9
                key = f"{'q4_0' if fmt == 0 else 'q4_k'}_{k}x{m}_n{n}"
                out[key] = {"us": round(t * 1e6, 3), "GB_s": round(gbs, 1),
                            "pct_peak": round(100 * gbs / HBM_PEAK_GBS, 1)}
                log(f"{key}: {t * 1e6:.2f} us {gbs:.0f} GB/s")
            del copies
    return out


if __name__ == "__main__":
    main()
