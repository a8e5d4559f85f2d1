"""GPU parity of the several-token Q4_K decode product on matrix cores.

The kernel (q4_gemv_tuned with Q4_GEMV_KERNEL_MATRIX; the library's choice for
Q4_K at 3-8 tokens on 256 rows or more) forms the products with
v_mfma_f32_16x16x32_f16 from exact fp16 codes and one fp16 per activation.
Checked against the oracle:
* outputs within 2e-3 (normwise and elementwise) for 1..8 tokens, ragged row
  counts, rows split into several LDS chunks, and the 7B-class shapes in full;
* one-hot x returns columns of W_hat bit for bit, and integer weights with
  activations in {-1, 0, 1} give the oracle's sums bit for bit (every step is
  exact there), long rows included;
* the grid size, the library's default dispatch and 4-byte-offset x leave the
  result unchanged bit for bit; a NaN in one token's x poisons only that token.
"""
import numpy as np
import pytest

import synth
from gpu_common import GEMV_TOL, check_tolerance, say, threads
from test_gpu_exact import _integer_buffer

pytestmark = pytest.mark.gpu

Q4_K = 1


@pytest.fixture(scope="module")
def env():
    import torch

    import oracle
    import q4_weight_gemv_amd as q4

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    oracle.lib()
    return torch, q4, oracle


def _matrix(env, buf, x, m, k, groups_per_cu=0, xoff=0):
    torch, q4, _ = env
    wd = torch.from_numpy(buf).cuda()
    n = x.shape[0]
    if xoff:
        # x starting xoff bytes into a float buffer (4-byte aligned only)
        base = torch.zeros(n * k + 4, dtype=torch.float32, device="cuda")
        xd = base[xoff // 4: xoff // 4 + n * k].view(n, k)
        xd.copy_(torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)))
    else:
        xd = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()
    yd = torch.full((n, m), float("nan"), dtype=torch.float32, device="cuda")
    q4.q4_gemv_tuned(Q4_K, wd, xd, yd, m, k, groups_per_cu=groups_per_cu, kernel=q4.Q4_GEMV_KERNEL_MATRIX)
    torch.cuda.synchronize()
    return yd.cpu().numpy()


def _weights(env, m, k, seed):
    _, q4, orc = env
    w = synth.weights(synth.seed_for(seed, m + k), m, k)
    buf = q4.q4_quantize_ref(Q4_K, w)
    assert np.array_equal(buf, orc.quantize(Q4_K, w))
    return buf


# (m, k): one tile and one super-block; ragged tiles; several chunks of the
# LDS at 8 tokens (11008 and 16384 weights per row); the 7B-class shapes.
SHAPES = [(16, 256), (37, 512), (300, 2048), (257, 11008), (1000, 4096), (70, 16384), (4096, 4096)]


@pytest.mark.parametrize("m,k", SHAPES)
@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 6, 7, 8])
def test_matrix_parity(env, m, k, n):
    _, _, orc = env
    buf = _weights(env, m, k, 300 + n)
    x = synth.activations(synth.seed_for(310 + n, k, True), n, k)
    say(f"matrix parity m={m} k={k} n={n}")
    y = _matrix(env, buf, x, m, k)
    yr, ad = orc.matvec(Q4_K, buf, m, k, x, threads=threads(), absdot=True)
    check_tolerance(y, yr, ad, GEMV_TOL, what=f"matrix {m}x{k} n={n}")


@pytest.mark.parametrize("k,m", [(4096, 11008), (11008, 4096)])
@pytest.mark.parametrize("n", [4, 8])
def test_matrix_parity_7b_full(env, k, m, n):
    _, _, orc = env
    buf = _weights(env, m, k, 330 + n)
    x = synth.activations(synth.seed_for(340 + n, k, True), n, k)
    say(f"matrix parity 7B m={m} k={k} n={n}")
    y = _matrix(env, buf, x, m, k)
    yr, ad = orc.matvec(Q4_K, buf, m, k, x, threads=threads(), absdot=True)
    check_tolerance(y, yr, ad, GEMV_TOL, what=f"matrix {m}x{k} n={n}")


@pytest.mark.parametrize("m,k", [(300, 1024), (40, 11008)])
def test_matrix_onehot_columns_exact(env, m, k):
    _, _, orc = env
    buf = _weights(env, m, k, 350)
    what = orc.dequantize(Q4_K, buf, m, k)
    cols = [0, 1, 31, 32, 63, 64, 255, 256, k - 1, k // 2 + 7]
    x = np.zeros((8, k), np.float32)
    for t, c in enumerate(cols[:8]):
        x[t, c] = 1.0
    say(f"matrix onehot m={m} k={k}")
    y = _matrix(env, buf, x, m, k)
    for t, c in enumerate(cols[:8]):
        assert np.array_equal(y[t], what[:, c]), (c, np.nonzero(y[t] != what[:, c])[0][:5])


@pytest.mark.parametrize("m,k,small", [(300, 4096, False), (37, 11008, False), (520, 1 << 16, True)])
@pytest.mark.parametrize("n", [1, 4, 8])
def test_matrix_exact_integer_sums(env, m, k, small, n):
    torch, q4, orc = env
    rng = np.random.default_rng(m + k + n)
    buf = _integer_buffer(q4, Q4_K, m, k, rng, small=small)
    x = rng.integers(-1, 2, size=(n, k)).astype(np.float32)
    say(f"matrix exact sums m={m} k={k} n={n}")
    y = _matrix(env, buf, x, m, k)
    yr = orc.matvec(Q4_K, buf, m, k, x, threads=16)
    assert orc.termscale(Q4_K, buf, m, k, x, threads=16).max() < 2 ** 24, "case exceeds the exact range"
    assert np.array_equal(y, yr), np.argwhere(y != yr)[:5]


def test_matrix_grid_and_default_dispatch(env):
    torch, q4, _ = env
    m, k = 700, 4096
    buf = _weights(env, m, k, 360)
    for n in (4, 5, 8):
        x = synth.activations(synth.seed_for(361, n, True), n, k)
        say(f"matrix grid sizes n={n}")
        y1 = _matrix(env, buf, x, m, k, groups_per_cu=1)
        for g in (2, 3):
            assert np.array_equal(_matrix(env, buf, x, m, k, groups_per_cu=g), y1), g
        # the library's own choice at these sizes is the matrix kernel
        wd = torch.from_numpy(buf).cuda()
        xd = torch.from_numpy(x).cuda()
        yd = torch.full((n, m), float("nan"), dtype=torch.float32, device="cuda")
        q4.q4_gemv(Q4_K, wd, xd, yd, m, k)
        torch.cuda.synchronize()
        assert np.array_equal(yd.cpu().numpy(), y1)


def test_matrix_x_four_byte_aligned(env):
    m, k, n = 300, 2048, 6
    buf = _weights(env, m, k, 370)
    x = synth.activations(synth.seed_for(371, k, True), n, k)
    say("matrix x offsets")
    y0 = _matrix(env, buf, x, m, k)
    for off in (4, 8, 12):
        assert np.array_equal(_matrix(env, buf, x, m, k, xoff=off), y0), off


def test_matrix_nan_token(env):
    _, _, orc = env
    m, k, n = 300, 2048, 4
    buf = _weights(env, m, k, 380)
    x = synth.activations(synth.seed_for(381, k, True), n, k)
    x[2, 777] = np.nan
    say("matrix nan token")
    y = _matrix(env, buf, x, m, k)
    assert np.isnan(y[2]).all()
    keep = [0, 1, 3]
    yr, ad = orc.matvec(Q4_K, buf, m, k, x[keep], threads=threads(), absdot=True)
    check_tolerance(y[keep], yr, ad, GEMV_TOL, what="matrix nan token, other tokens")
