"""The decode steps exactly as bench.py times them, against the oracle.

bench.py's own Step objects are built here: the same shapes, the same
seeded weights and activations, the same weight copies, and one HIP graph
per copy. The only change is that the weight buffers come from the oracle's
quantizer (the CPU tests show that the library's host quantizer writes the
same bytes at every one of these shapes). Each copy's graph is replayed
as the timed loop rotates them, and so is the plain-stream sequence. Every
product's output is compared with the oracle, every row of every product.
Copies and launch paths must also agree bit for bit.
"""
import numpy as np
import pytest

import bench
import synth
from gpu_common import GEMV_TOL, check_tolerance, say, threads

pytestmark = pytest.mark.gpu

CASES = [
    ("gpt2_124m", "gpt2_124m_step", 1),           # the headline step: 49 Q4_0 products
    ("smollm2_360m", "smollm2_360m_step", 2),     # 225 products
    ("smollm2_360m_stacked", "smollm2_360m_step_fused", 2),  # q|k|v and gate|up stacked: 129
    ("smollm2_360m_gated", "smollm2_360m_step_gated", 2),  # q|k|v stacked, gate.up gated: 129
]


@pytest.fixture(scope="module")
def env():
    import torch

    import oracle
    import q4_weight_gemv_amd as q4

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    oracle.lib()
    return torch, q4, oracle


def _check_plain(orc, name, i, buf, x, y, m, k):
    yr, ad = orc.matvec(0, buf, m, k, x, threads=threads(), absdot=True)
    check_tolerance(y, yr, ad, GEMV_TOL, what=f"{name} product {i} ({k}->{m})")


def _check_gated(orc, name, i, buf, x, y, m, k):
    # The gated product's bound, from the plain product's elementwise bound on
    # the gate (g) and up (u) rows and |silu'| <= 1.1:
    #   1.1 |u| tol A_g + |silu(g)| tol A_u + 1.1 tol^2 A_g A_u
    # (A: the rows' sums of |w x|), plus the fp32 epilogue's few ulp.
    yr, g, u = orc.matvec_silu_mul(0, buf, m, k, x, threads=threads(), parts=True)
    _, ad = orc.matvec(0, buf, 2 * m, k, x, threads=threads(), absdot=True)
    ag, au = ad[:, :m], ad[:, m:]
    silu = g / (1.0 + np.exp(-g))
    bound = (1.1 * np.abs(u) * GEMV_TOL * ag + np.abs(silu) * GEMV_TOL * au + 1.1 * GEMV_TOL ** 2 * ag * au
             + 4e-6 * np.abs(yr.astype(np.float64)) + 1e-30)
    err = np.abs(y.astype(np.float64) - yr)
    assert np.all(np.isfinite(y)), f"{name} product {i}: non-finite output"
    bad = np.argwhere(err > bound)
    assert bad.size == 0, (f"{name} product {i} ({k}->{m} gated)", bad[:5])
    assert np.linalg.norm(y[0] - yr[0]) <= GEMV_TOL * np.linalg.norm(yr[0])


@pytest.mark.parametrize("name,shapes_fn,config", CASES)
def test_bench_step_matches_oracle(env, name, shapes_fn, config):
    torch, q4, orc = env
    say(f"bench step {name}: building (oracle-quantized weights)")
    step = bench.Step(torch, q4, getattr(synth, shapes_fn)(), 0, 1, config_id=config, quantize=orc.quantize)
    try:
        assert len(step.graphs) >= 2  # cold: rotating copies, as timed

        def run(launch, what):
            for y in step.ys:
                y.fill_(float("nan"))
            torch.cuda.synchronize()
            say(f"bench step {name}: {what}")
            launch()
            torch.cuda.synchronize()
            return [y.cpu().numpy() for y in step.ys]

        first = run(lambda: step.run_graph(0), "graph of weight copy 0")
        for i, ((k, m, gated), buf, x, y) in enumerate(zip(step.shapes, step.host_w, step.host_x, first)):
            (_check_gated if gated else _check_plain)(orc, name, i, buf, x, y, m, k)
        for c in range(1, len(step.graphs)):
            outs = run(lambda: step.run_graph(c), f"graph of weight copy {c}")
            for i, (a, b) in enumerate(zip(outs, first)):
                assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), (name, c, i)
        outs = run(lambda: step.run_plain(q4, 1), "plain-stream sequence")
        for i, (a, b) in enumerate(zip(outs, first)):
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), (name, "plain", i)
    finally:
        step.close()
        del step
        torch.cuda.empty_cache()
