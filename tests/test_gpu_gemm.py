"""GPU parity of the prefill product (LDS dequant -> bf16 MFMA) against the oracle.

* Dequantization bit-exact through the public entry point: X = I_K returns
  bf16(W_hat)^T exactly (one nonzero product per sum, products with 1.0 exact).
* Outputs within 1e-2 of the oracle with exact fp32 weights (normwise and
  elementwise), and within 1e-4 of the oracle with bf16-rounded weights (the
  kernel's own weights: only the fp32 summation order differs).
* SmolLM2-360M layer shapes at 512 tokens (sampled rows), ragged shapes, Q4_K.
"""
import numpy as np
import pytest

import synth
from gpu_common import GEMM_TOL, check_tolerance, say, threads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch

    import oracle
    import q4_weight_gemv_amd as q4

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    oracle.lib()
    return torch, q4, oracle


def _gemm(env, fmt, buf, xb, m, k):
    torch, q4, _ = env
    wd = torch.from_numpy(buf).cuda()
    xd = torch.from_numpy(np.ascontiguousarray(xb).view(np.int16)).cuda()
    yd = torch.full((xb.shape[0], m), float("nan"), dtype=torch.float32, device="cuda")
    q4.q4_gemm(fmt, wd, xd, yd, m, k)
    torch.cuda.synchronize()
    return yd.cpu().numpy()


def _quantize_both(q4, orc, fmt, w):
    buf = q4.q4_quantize_ref(fmt, w)
    assert np.array_equal(buf, orc.quantize(fmt, w)), "host quantizer and oracle disagree"
    return buf


@pytest.mark.parametrize("fmt,m,k", [(0, 37, 96), (0, 130, 960), (0, 64, 2560), (1, 37, 256), (1, 96, 1024),
                                     (2, 37, 96), (2, 130, 960), (3, 37, 256), (3, 96, 1024), (4, 37, 96),
                                     (4, 130, 960)])
def test_identity_gives_bf16_weights_exactly(env, fmt, m, k):
    torch, q4, orc = env
    buf = _quantize_both(q4, orc, fmt, synth.weights(synth.seed_for(30 + fmt, m), m, k))
    eye = synth.bf16_bits(np.eye(k, dtype=np.float32))
    say(f"gemm identity fmt={fmt} m={m} k={k}")
    y = _gemm(env, fmt, buf, eye, m, k)
    what = orc.dequantize(fmt, buf, m, k)
    wb = np.array([[orc.bf16_to_fp32(orc.fp32_to_bf16(float(v))) for v in row] for row in what], np.float32)
    assert np.array_equal(y, wb.T)


def _parity(env, fmt, m, k, n, seed):
    # Every output row and token against the oracle.
    torch, q4, orc = env
    buf = _quantize_both(q4, orc, fmt, synth.weights(synth.seed_for(seed, 2), m, k))
    xb = synth.bf16_bits(synth.activations(synth.seed_for(seed, 2, True), n, k))
    say(f"gemm parity fmt={fmt} m={m} k={k} n={n}")
    y = _gemm(env, fmt, buf, xb, m, k)
    yr, ad = orc.matmul(fmt, buf, m, k, xb, threads=threads(), absdot=True)
    check_tolerance(y, yr, ad, GEMM_TOL, what=f"gemm fmt={fmt} {m}x{k} n={n}")
    yb, adb = orc.matmul(fmt, buf, m, k, xb, round_w_bf16=True, threads=threads(), absdot=True)
    rel = check_tolerance(y, yb, adb, 1e-4, what=f"gemm(bf16 W) fmt={fmt} {m}x{k} n={n}")
    return rel


@pytest.mark.parametrize("fmt,m,k,n", [
    (0, 1, 32, 1), (0, 37, 96, 5), (0, 100, 320, 130), (0, 33, 960, 64), (0, 257, 2560, 200),
    (1, 1, 256, 3), (1, 70, 512, 70), (1, 130, 1024, 257),
    (2, 1, 32, 1), (2, 100, 320, 130), (2, 257, 2560, 200),
    (3, 1, 256, 3), (3, 70, 512, 70), (3, 130, 1024, 257),
    (4, 1, 32, 1), (4, 100, 320, 130), (4, 257, 2560, 200),
])
def test_parity_small(env, fmt, m, k, n):
    _parity(env, fmt, m, k, n, seed=600 + n)


@pytest.mark.parametrize("k,m", sorted(set(synth.smollm2_360m_layer() + synth.smollm2_360m_layer_stacked())))
def test_parity_smollm2_layer_512_tokens(env, k, m):
    # Every matrix the prefill bench times: the layer's seven, and its
    # stacked q|k|v (960 -> 1600) and gate|up (960 -> 5120).
    _parity(env, 0, m, k, 512, seed=700 + k % 13)


@pytest.mark.parametrize("k,m", [(1024, 960), (2560, 960)])
def test_parity_q4_k_512_tokens(env, k, m):
    _parity(env, 1, m, k, 512, seed=800)


@pytest.mark.parametrize("k,m", [(960, 960), (2560, 960)])
def test_parity_q8_0_512_tokens(env, k, m):
    _parity(env, 2, m, k, 512, seed=850)


def _tiles():
    import q4_weight_gemv_amd as q4

    return list(q4.GEMM_TILES)


@pytest.mark.parametrize("tile", _tiles(), ids=lambda t: f"{t[0]}x{t[1]}x{t[2]}")
@pytest.mark.parametrize("fmt", [0, 1, 2, 3, 4])
def test_parity_every_tile(env, fmt, tile):
    """Every instantiated tile through q4_gemm_tuned: 70 rows and 100 tokens
    (ragged in both), K = 1280 (a partial last chunk for every chunk size)."""
    torch, q4, orc = env
    m, k, n = 70, 1280, 100
    buf = _quantize_both(q4, orc, fmt, synth.weights(synth.seed_for(950 + fmt, 2), m, k))
    xb = synth.bf16_bits(synth.activations(synth.seed_for(950 + fmt, 2, True), n, k))
    wd = torch.from_numpy(buf).cuda()
    xd = torch.from_numpy(np.ascontiguousarray(xb).view(np.int16)).cuda()
    yd = torch.full((n, m), float("nan"), dtype=torch.float32, device="cuda")
    say(f"gemm tile {tile} fmt={fmt}")
    q4.q4_gemm_tuned(fmt, wd, xd, yd, m, k, *tile)
    torch.cuda.synchronize()
    y = yd.cpu().numpy()
    yr, ad = orc.matmul(fmt, buf, m, k, xb, threads=threads(), absdot=True)
    check_tolerance(y, yr, ad, GEMM_TOL, what=f"gemm tile {tile} fmt={fmt}")
    yb, adb = orc.matmul(fmt, buf, m, k, xb, round_w_bf16=True, threads=threads(), absdot=True)
    check_tolerance(y, yb, adb, 1e-4, what=f"gemm(bf16 W) tile {tile} fmt={fmt}")


def test_q1_0_hand_built_words(env):
    # Code words all 0, all 1, alternating and random; scales zero,
    # subnormal, negative and the largest finite fp16: the product of the
    # bf16-rounded weights (+-bf16(d)) against the oracle's.
    torch, q4, orc = env
    m, k, n = 70, 512, 40
    rng = np.random.default_rng(5)
    nb = m * k // 32
    words = rng.integers(0, 1 << 32, size=nb, dtype=np.uint64).astype(np.uint32)
    words[0::7] = 0
    words[1::7] = 0xFFFFFFFF
    words[2::7] = 0xAAAAAAAA
    scales = rng.uniform(0.001, 2.0, size=nb).astype(np.float16)
    scales[3::11] = np.float16(0.0)
    scales[4::11] = np.float16(6e-8)
    scales[5::13] = np.float16(65504.0)
    scales[6::17] *= np.float16(-1.0)
    buf = np.concatenate([words.view(np.uint8), scales.view(np.uint8)])
    xb = synth.bf16_bits(synth.activations(960, n, k))
    say("gemm q1_0 hand-built words")
    y = _gemm(env, 4, buf, xb, m, k)
    yb, adb = orc.matmul(4, buf, m, k, xb, round_w_bf16=True, threads=threads(), absdot=True)
    check_tolerance(y, yb, adb, 1e-4, what="gemm q1_0 hand-built (bf16 W)")


@pytest.mark.parametrize("fmt,m,k,n", [(0, 130, 960, 70), (1, 96, 1024, 130), (4, 130, 960, 65)])
def test_nan_activation_makes_its_token_nan(env, fmt, m, k, n):
    # A NaN among one token's bf16 activations makes every output of that
    # token NaN, as in the oracle; the other tokens are unaffected. Outputs
    # start at a finite sentinel, so a NaN below was written by the kernel.
    torch, q4, orc = env
    buf = _quantize_both(q4, orc, fmt, synth.weights(synth.seed_for(1400 + fmt, m), m, k))
    xb = synth.bf16_bits(synth.activations(synth.seed_for(1400 + fmt, m, True), n, k))
    bad = n // 2
    xb[bad, k // 3] = 0x7FC0  # bf16 quiet NaN
    wd = torch.from_numpy(buf).cuda()
    xd = torch.from_numpy(np.ascontiguousarray(xb).view(np.int16)).cuda()
    yd = torch.full((n, m), 12345.0, dtype=torch.float32, device="cuda")
    say(f"gemm nan activation fmt={fmt} m={m} k={k} n={n}")
    q4.q4_gemm(fmt, wd, xd, yd, m, k)
    torch.cuda.synchronize()
    y = yd.cpu().numpy()
    yr, ad = orc.matmul(fmt, buf, m, k, xb, threads=threads(), absdot=True)
    assert np.isnan(yr[bad]).all() and np.isnan(y[bad]).all()
    good = [t for t in range(n) if t != bad]
    check_tolerance(y[good], yr[good], ad[good], GEMM_TOL, what=f"gemm fmt={fmt} tokens without the NaN")


def test_gemm_misaligned_and_noop(env):
    torch, q4, _ = env
    w = torch.zeros(4096, dtype=torch.uint8, device="cuda")
    x = torch.zeros(256, dtype=torch.int16, device="cuda")
    y = torch.full((8,), 5.0, device="cuda")
    lib = q4.raw()
    assert lib.q4_gemm(0, w.data_ptr(), x.data_ptr() + 2, y.data_ptr(), 8, 32, 1, None) == q4.Q4_EALIGN
    assert lib.q4_gemm(0, w.data_ptr(), x.data_ptr(), y.data_ptr(), 0, 32, 1, None) == q4.Q4_OK
    torch.cuda.synchronize()
    assert (y == 5.0).all()


@pytest.mark.parametrize("fmt,m,k,n", [(0, 300, 960, 64), (1, 130, 1024, 33), (0, 2560, 960, 512)])
@pytest.mark.parametrize("shift", [2, 4, 6])
def test_x_four_byte_aligned(env, fmt, m, k, n, shift):
    # bf16 activations 4, 8 or 12 bytes past a 16-byte boundary: the same bits
    # as the same values at an aligned address.
    torch, q4, orc = env
    buf = q4.q4_quantize_ref(fmt, synth.weights(synth.seed_for(60 + fmt, m), m, k))
    xb = synth.bf16_bits(synth.activations(synth.seed_for(60 + fmt, m, True), n, k))
    ref = _gemm(env, fmt, buf, xb, m, k)
    store = torch.zeros(n * k + 16, dtype=torch.int16, device="cuda")
    xd = store[shift:shift + n * k].view(n, k)
    xd.copy_(torch.from_numpy(np.ascontiguousarray(xb).view(np.int16)))
    assert xd.data_ptr() % 16 == 2 * shift
    yd = torch.full((n, m), float("nan"), dtype=torch.float32, device="cuda")
    say(f"gemm x at +{2 * shift} bytes fmt={fmt} m={m} k={k} n={n}")
    q4.q4_gemm(fmt, torch.from_numpy(buf).cuda(), xd, yd, m, k)
    torch.cuda.synchronize()
    assert np.array_equal(yd.cpu().numpy().view(np.uint32), ref.view(np.uint32))
