#!/usr/bin/env python3
"""Throughput of the Q4 decode path on one MI355X; prints ONE JSON line.

Headline workload: the GPT-2-124M decode step at batch 1 -- 12 layers of
{768->2304 (QKV), 768->768 (attn-out), 768->3072, 3072->768 (MLP)} plus the
768->50257 LM head = 49 Q4_0 decode products, 69.5 MB of weights. Every
product's weights, activations and outputs are resident in HBM before the
timed region. The 49 launches are captured once into a HIP graph per weight
copy; each step is one graph launch. The weights rotate over enough copies
(>= 512 MiB) that every step reads them from HBM, not from the 256 MB
Infinity Cache.

  value     = algorithmic bytes per step (quantized W + x + y of the 49
              products) x steps / timed seconds  [GB/s]
  tokens/s  = steps / timed seconds
  roofline  = the decode-product kernel: algorithmic bytes per launch /
              average launch time (HIP events on the stream the graphs are
              launched on, timed region / launches), against 8 TB/s HBM.

Also reported in "extras": the 7B-class shapes (Q4_0 at N=1 -- the gate
shapes -- Q4_K at N=1/4/8, the other formats, and the gated gate|up product),
the SmolLM2-360M product stacks (plain, stacked, gated), the whole
SmolLM2-360M decode step as a replayed generation loop, the prefill GEMM over
a SmolLM2-360M layer at 512 tokens (separate and stacked matrices), warm
steps, launches from a plain stream, the per-launch floor, and the streaming-
read ceiling (a pure read, and the same read storing a few bytes per wave).
"cpu_baseline" is the CPU oracle timed on the host cores on whole repeats of
the same step (bounded to about 10 s).
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
KERNEL_SOURCES = ["q4_gemv_kernel.h", "q4_gemv.hip", "q4_gemv_q4_0_a.hip", "q4_gemv_q4_0_b.hip"]


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
    one copy, replayed (MALL-resident when the step fits in 256 MB)."""

    def __init__(self, torch, q4, shapes, fmt, n, config_id, cold=True, quantize=None):
        import synth

        # Entries (K, M) or (K, M, gated): a gated product reads 2M weight rows.
        # `quantize(fmt, w)` makes the weight buffers (the library's host
        # quantizer unless a caller passes another with the same output).
        quantize = quantize or q4.q4_quantize_ref
        shapes = [tuple(s) + (0,) * (3 - len(s)) for s in shapes]
        self.shapes, self.fmt, self.n = shapes, fmt, n
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
        torch.cuda.synchronize()

    def _ops(self, ws):
        return [(w, x, y, m, k, g) for w, x, y, (k, m, g) in zip(ws, self.xs, self.ys, self.shapes)]

    def run_graph(self, i):
        self.graphs[i % len(self.graphs)].launch()

    def run_plain(self, q4, i):
        # Back-to-back launches from the library's C loop (arguments marshalled once).
        self.seqs[i % len(self.seqs)].launch()

    def close(self):
        for g in self.graphs:
            g.close()


def traffic_from_profile(per_launch_bytes, path=None):
    """HBM bytes per launch from the committed counter summary (or the one at
    `path`), if it was taken on the current kernel sources (else None)."""
    path = path or os.path.join(ROOT, "profiles", "pmc_gemv_gpt2_step.txt")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"kernel_source_sha256:\s*(\w+)", text)
    t = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m or not t or m.group(1) != kernel_source_hash():
        return None
    return float(t.group(1))


def cpu_baseline(step, budget_s=10.0, budget_1core_s=6.0):
    """The oracle (as it stands) on whole repeats of the same decode step, with
    its rows split over the host cores, and again on one core."""
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

    threads = max(1, min(16, os.cpu_count() or 1))
    reps, dt = timed(threads, budget_s)
    reps1, dt1 = timed(1, budget_1core_s)
    return {
        "value": round(step.bytes * reps / dt / 1e9, 4),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{reps} whole GPT-2-124M decode step(s) (49 products, rows split over {threads} threads), "
                  f"{dt:.1f} s wall",
        "tokens_per_s": round(reps / dt, 3),
        "one_core": {"GB_s": round(step.bytes * reps1 / dt1 / 1e9, 4), "tokens_per_s": round(reps1 / dt1, 3),
                     "sample": f"{reps1} whole step(s), {dt1:.1f} s wall"},
    }


def bench_7b(torch, q4, timer, reps=20):
    """7B-class shapes one product at a time, cold: a graph of one launch per
    rotating weight copy, replayed."""
    import synth

    out = {}
    name = {0: "q4_0", 1: "q4_k", 2: "q8_0", 3: "q2_k", 4: "q1_0"}
    # Q4_0 at one token (the gate), Q4_K at 1, 4, 8 tokens, and Q8_0, Q2_K and
    # Q1_0 at one token beside them (the pages compare q8_0, q4_k_m and q2_k,
    # and name q1_0 as a format added through one dequantization routine).
    for fmt, ns in ((0, (1,)), (1, (1, 4, 8)), (2, (1,)), (3, (1,)), (4, (1,))):
        layer_t, layer_b = {1: 0.0}, 0
        for k, m in synth.llama7b_layer()[:2] + synth.llama7b_layer()[3:]:
            wq = q4.q4_quantize_ref(fmt, synth.weights(synth.seed_for(4, k + m), m, k))
            copies = [torch.from_numpy(wq).cuda() for _ in range(copies_for(wq.size))]
            for n in ns:
                x = torch.from_numpy(synth.activations(synth.seed_for(4, k, True), n, k)).cuda()
                y = torch.empty((n, m), device="cuda")
                g = q4.Q4Graph(fmt, [(c, x, y, m, k) for c in copies], n)
                t = timer.region(lambda i: g.launch(), reps, 3) / (reps * len(copies))
                g.close()
                nb = gemv_bytes(q4, fmt, m, k, n)
                key = f"{name[fmt]}_{k}to{m}_n{n}"
                out[key] = {"us": round(t * 1e6, 3), "GB_s": round(nb / t / 1e9, 1),
                            "pct_peak": round(100 * nb / t / 1e9 / HBM_PEAK_GBS, 1)}
                log(f"{key}: {t * 1e6:.2f} us {nb / t / 1e9:.0f} GB/s")
                if n == 1:
                    mult = 2 if (k, m) == (4096, 11008) else 1  # gate and up
                    layer_t[1] += mult * t
                    layer_b += mult * nb
            del copies
        key = f"{name[fmt]}_7b_layer_as_listed_n1"
        out[key] = {"us": round(layer_t[1] * 1e6, 2), "GB_s": round(layer_b / layer_t[1] / 1e9, 1),
                    "pct_peak": round(100 * layer_b / layer_t[1] / 1e9 / HBM_PEAK_GBS, 1)}
    return out


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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="only the headline workload")
    ap.add_argument("--extras", default="all",
                    help="comma list of extras to run (default all): plain, floor, gate_7b, smollm2, smollm2_fused, "
                         "smollm2_gated, warm, read_ceiling, full_step, gemm")
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

    shapes = synth.gpt2_124m_step()
    log(f"setup GPT-2-124M step: {len(shapes)} products")
    step = Step(torch, q4, shapes, 0, 1, config_id=1)
    t = timer.region(step.run_graph, K, W)
    value = step.bytes * K / t / 1e9
    launches = K * len(shapes)
    per_launch_bytes = step.bytes / len(shapes)
    achieved = per_launch_bytes / (t / launches) / 1e9
    log(f"graph: {t / K * 1e6:.2f} us/step, {value:.1f} GB/s, {K / t:.0f} tokens/s")
    traffic = traffic_from_profile(per_launch_bytes)

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
        "dtype": "f32",
        "arithmetic": "Q4_0 weights as exact signed fp16 codes; activations as hi+lo fp16 pairs (~2^-23 relative); "
                      "v_dot2 products, fp32 accumulation",
        "data": "synthetic: seeded N(0, 0.02) weights, N(0, 1) activations; no checkpoints",
        "config": {
            "workload": "GPT-2-124M decode step (49 Q4_0 products, batch 1)",
            "format": "Q4_0",
            "tokens": 1,
            "products_per_step": len(shapes),
            "bytes_per_step": step.bytes,
            "launch": "HIP graph replay, one graph launch per step",
            "cache": f"cold: {len(step.copies)} rotating weight copies (>= 512 MiB)",
        },
        "tokens_per_s": round(K / t, 1),
        "pct_of_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": None if traffic is None else round(traffic),
            "kernel": "q4::gemv::gemv_kernel (Q4_0, one token)",
            "per_launch_bytes": round(per_launch_bytes),
            "avg_launch_us": round(t / launches * 1e6, 3),
            "kernel_source_sha256": kernel_source_hash(),
        },
    }

    if not args.no_extras:
        extras = {}
        want = set(args.extras.split(",")) if args.extras != "all" else None
        on = lambda name: want is None or name in want  # noqa: E731
        if on("plain"):
            n_plain = max(20, K // 10)
            tp = timer.region(lambda i: step.run_plain(q4, i), n_plain, 5)
            extras["gpt2_plain_stream"] = {"us_per_step": round(tp / n_plain * 1e6, 2),
                                           "tokens_per_s": round(n_plain / tp, 1)}
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
        if on("gemm"):
            extras["gemm_smollm2_layer"] = bench_gemm(torch, q4, timer, reps=max(2, K // 50))
            extras["gemm_smollm2_layer_fused_qkv_gateup"] = bench_gemm(
                torch, q4, timer, reps=max(2, K // 50), shapes=synth.smollm2_360m_layer_stacked(),
                per_matrix=False)
        result["extras"] = extras

    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline(step)
    step.close()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
