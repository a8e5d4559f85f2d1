"""GPU parity at the size limits the entry points accept.

Every kernel addresses its buffers with 32-bit byte offsets, and offsets from
2^31 up serve as the no-fetch (and no-store) lane offset, so the argument
checks accept weights, activations and outputs of up to 2^31 - 1 bytes each.
These tests run the products with each buffer just under that limit and
check sampled rows (both ends, the last rows holding the highest offsets,
and random rows) against the oracle. Weight buffers are built directly from
random codes with valid fp16 scales (the quantizer is not the subject here).
"""
import numpy as np
import pytest

import synth
from gpu_common import GEMM_TOL, GEMV_TOL, check_tolerance, sample_rows, say, threads

pytestmark = pytest.mark.gpu

LIMIT = 1 << 31


@pytest.fixture(scope="module")
def env():
    import torch

    import oracle
    import q4_weight_gemv_amd as q4

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    oracle.lib()
    return torch, q4, oracle


def _scales(rng, count):
    """Valid fp16 scale bytes (positive, in the range the quantizer writes)."""
    return rng.uniform(0.001, 0.02, size=count).astype(np.float16).view(np.uint8)


def _random_buffer(q4, fmt, m, k, seed):
    """A valid quantized m x k buffer: random codes, finite fp16 scales."""
    rng = np.random.default_rng(seed)
    n = q4.q4_weight_bytes(fmt, m, k)
    buf = rng.integers(0, 256, size=n, dtype=np.uint8)
    if fmt in (0, 2, 4):  # code plane, then one fp16 scale per 32 weights
        nb = m * k // 32
        buf[n - 2 * nb:] = _scales(rng, nb)
    elif fmt == 1:  # 144-byte super-blocks: fp16 d and dmin lead each
        sb = buf.reshape(-1, 144)
        sb[:, 0:4] = _scales(rng, 2 * sb.shape[0]).reshape(-1, 4)
    else:  # Q2_K: codes, scale bytes, then fp16 d and dmin per super-block
        ns = m * k // 256
        buf[n - 4 * ns:] = _scales(rng, 2 * ns)
    return buf


def _rows_check(orc, fmt, buf, m, k, x, y_rows, idx, ranges, tol, what):
    yr, ad = orc.matvec(fmt, buf, m, k, x, threads=threads(), absdot=True, rows=ranges)
    check_tolerance(y_rows, yr[:, idx], ad[:, idx], tol, what=what)


def _largest_rows(q4, fmt, k):
    per_row = q4.q4_weight_bytes(fmt, 1, k)
    return (LIMIT - 1) // per_row


@pytest.mark.parametrize("fmt,n", [(0, 1), (0, 8), (1, 1), (1, 8), (2, 1), (3, 1), (4, 1)])
def test_decode_weights_just_under_2gib(env, fmt, n):
    torch, q4, orc = env
    k = 4096
    m = _largest_rows(q4, fmt, k)
    assert q4.q4_weight_bytes(fmt, m, k) < LIMIT <= q4.q4_weight_bytes(fmt, m + 1, k)
    buf = _random_buffer(q4, fmt, m, k, 7000 + fmt)
    x = synth.activations(7100 + fmt, n, k)
    say(f"limits: weights {buf.size} B fmt={fmt} m={m} k={k} n={n}")
    wd = torch.from_numpy(buf).cuda()
    xd = torch.from_numpy(x).cuda()
    yd = torch.full((n, m), float("nan"), device="cuda")
    q4.q4_gemv(fmt, wd, xd, yd, m, k)
    torch.cuda.synchronize()
    ranges, idx = sample_rows(m, 7200 + fmt, edge=64, rand=128)
    y_rows = yd[:, idx].cpu().numpy()
    del wd, yd
    torch.cuda.empty_cache()
    _rows_check(orc, fmt, buf, m, k, x, y_rows, idx, ranges, GEMV_TOL, f"weights limit fmt={fmt} n={n}")


def test_decode_outputs_just_under_2gib(env):
    # n = 8 tokens of 67,108,863 outputs: y's last element sits 36 bytes
    # below 2^31, the no-store lane offset.
    torch, q4, orc = env
    fmt, k, n = 0, 32, 8
    m = (LIMIT - 1) // (4 * n)
    assert 4 * n * m < LIMIT <= 4 * n * (m + 1)
    buf = _random_buffer(q4, fmt, m, k, 7300)
    x = synth.activations(7301, n, k)
    say(f"limits: outputs {4 * n * m} B m={m} k={k} n={n}")
    wd = torch.from_numpy(buf).cuda()
    xd = torch.from_numpy(x).cuda()
    yd = torch.full((n, m), float("nan"), device="cuda")
    q4.q4_gemv(fmt, wd, xd, yd, m, k)
    torch.cuda.synchronize()
    ranges, idx = sample_rows(m, 7302, edge=64, rand=128)
    y_rows = yd[:, idx].cpu().numpy()
    assert not torch.isnan(yd).any().item()  # every output written
    del wd, yd
    torch.cuda.empty_cache()
    _rows_check(orc, fmt, buf, m, k, x, y_rows, idx, ranges, GEMV_TOL, "outputs limit")


def test_decode_activations_just_under_2gib(env):
    # 8 tokens of 67,108,832 activations (x 36 KB below 2 GiB), 3 ragged
    # rows: the staging runs in LDS-sized chunks up to the last unit. Every
    # activation is random (normal), so every chunk of x up to the buffer's
    # end enters the sums, and the outputs sit deep in cancellation (about
    # 1/sqrt(K) of their term scale): the fp32 sums must carry no same-sign
    # rounding drift to meet the normwise bound there.
    torch, q4, orc = env
    fmt, n, m = 0, 8, 3
    k = (LIMIT - 1) // (4 * n) // 32 * 32
    assert 4 * n * k < LIMIT <= 4 * n * (k + 32)
    buf = _random_buffer(q4, fmt, m, k, 7400)
    rng = np.random.default_rng(7401)
    x = rng.standard_normal((n, k), dtype=np.float32)
    say(f"limits: activations {4 * n * k} B m={m} k={k} n={n}")
    wd = torch.from_numpy(buf).cuda()
    xd = torch.from_numpy(x).cuda()
    yd = torch.full((n, m), float("nan"), device="cuda")
    q4.q4_gemv(fmt, wd, xd, yd, m, k)
    torch.cuda.synchronize()
    y = yd.cpu().numpy()
    del wd, xd, yd
    torch.cuda.empty_cache()
    yr, ad = orc.matvec(fmt, buf, m, k, x, threads=threads(), absdot=True)
    check_tolerance(y, yr, ad, GEMV_TOL, what="activations limit")


def test_prefill_weights_just_under_2gib(env):
    torch, q4, orc = env
    fmt, k, n = 0, 4096, 64
    m = _largest_rows(q4, fmt, k)
    buf = _random_buffer(q4, fmt, m, k, 7500)
    xb = synth.bf16_bits(synth.activations(7501, n, k))
    say(f"limits: prefill weights {buf.size} B m={m} k={k} n={n}")
    wd = torch.from_numpy(buf).cuda()
    xd = torch.from_numpy(np.ascontiguousarray(xb).view(np.int16)).cuda()
    yd = torch.full((n, m), float("nan"), device="cuda")
    q4.q4_gemm(fmt, wd, xd, yd, m, k)
    torch.cuda.synchronize()
    ranges, idx = sample_rows(m, 7502, edge=64, rand=64)
    y = yd[:, idx].cpu().numpy()
    del wd, yd
    torch.cuda.empty_cache()
    yr, ad = orc.matmul(fmt, buf, m, k, xb, threads=threads(), absdot=True, rows=ranges)
    check_tolerance(y, yr[:, idx], ad[:, idx], GEMM_TOL, what="prefill weights limit")
