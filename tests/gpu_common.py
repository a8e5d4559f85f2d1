"""Helpers shared by the GPU tests (device marshalling and tolerance gates)."""
from __future__ import annotations

import os
import sys

import numpy as np

GEMV_TOL = 2e-3   # fp32-accumulate decode product
GEMM_TOL = 1e-2   # bf16 matrix-core prefill product


def threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def say(msg: str) -> None:
    """Name the case before each GPU step, flushed, so a fault points at it."""
    print(msg, flush=True)
    sys.stdout.flush()


def check_tolerance(y_gpu: np.ndarray, y_ref: np.ndarray, absdot: np.ndarray, tol: float, rows=None, what=""):
    """Per token: normwise ||dy|| <= tol ||y|| and elementwise |dy_i| <= tol * sum_k |w_ik x_k|.

    ``rows`` restricts both checks to the listed row indices. For a single
    output the normwise ratio is the per-element |dy| / |y|, which is
    ill-posed where y cancels to nearly zero (any fp32 sum then misses it by
    a large relative amount); there the elementwise forward-error bound is
    the condition.
    """
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    if rows is not None:
        y_gpu, y_ref, absdot = y_gpu[:, rows], y_ref[:, rows], absdot[:, rows]
    assert np.all(np.isfinite(y_gpu)), f"{what}: non-finite output"
    worst_norm = 0.0
    for t in range(y_ref.shape[0]):
        num = np.linalg.norm(y_gpu[t] - y_ref[t])
        den = np.linalg.norm(y_ref[t])
        rel = num / den if den > 0 else num
        worst_norm = max(worst_norm, rel)
        assert rel <= tol or y_ref.shape[1] == 1, f"{what}: token {t} normwise {rel:.3e} > {tol}"
        err = np.abs(y_gpu[t] - y_ref[t])
        bad = np.nonzero(err > tol * absdot[t])[0]
        assert bad.size == 0, (f"{what}: token {t} elementwise at rows {bad[:5]}: "
                               f"{err[bad[:5]]} vs {tol * absdot[t][bad[:5]]}")
    return worst_norm


def sample_rows(m: int, seed: int, edge: int = 192, rand: int = 256):
    """Row ranges for sampled checks: both ends (ragged tail included) and random rows."""
    rng = np.random.default_rng(seed)
    ranges = [(0, min(m, edge))]
    if m > edge:
        ranges.append((max(edge, m - edge), m))
    picks = sorted(set(rng.integers(0, m, size=rand).tolist()))
    ranges += [(r, r + 1) for r in picks]
    idx = sorted({r for a, b in ranges for r in range(a, b)})
    return ranges, idx
