"""GPU parity of the decode products (Q4_0 and Q4_K GEMV) against the oracle.

* Dequantization bit-exact through the public entry point: a one-hot x = e_j
  returns column j of W_hat exactly (products with one power of two and sums
  of zeros are exact in every step of the kernel).
* Outputs within 2e-3, normwise and elementwise (forward-error form), at
  sizes spanning several tiles with ragged tails, at every workload shape
  (every row), for token counts 1..8.
* Layer-stack sequence and graph replay reproduce the single calls bit for bit.
"""
import numpy as np
import pytest

import synth
from gpu_common import GEMV_TOL, check_tolerance, say, threads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch

    import oracle
    import q4_weight_gemv_amd as q4

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    oracle.lib()
    return torch, q4, oracle


def _quantize_both(q4, orc, fmt, w):
    buf = q4.q4_quantize_ref(fmt, w)
    ref = orc.quantize(fmt, w)
    assert np.array_equal(buf, ref), "host quantizer and oracle disagree"
    return buf


def _gemv(env, fmt, buf, x, m, k):
    torch, q4, _ = env
    wd = torch.from_numpy(buf).cuda()
    xd = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()
    yd = torch.full((x.shape[0], m), float("nan"), dtype=torch.float32, device="cuda")
    q4.q4_gemv(fmt, wd, xd, yd, m, k)
    torch.cuda.synchronize()
    return yd.cpu().numpy()


ONEHOT_CASES = [
    (0, 5, 32), (0, 37, 320), (0, 768, 768), (0, 129, 2560), (0, 300, 4096), (0, 70, 11008),
    (1, 5, 256), (1, 37, 512), (1, 130, 1024), (1, 300, 4096), (1, 70, 11008),
    (2, 5, 32), (2, 37, 320), (2, 768, 768), (2, 300, 4096), (2, 70, 11008),
    (3, 5, 256), (3, 37, 512), (3, 130, 1024), (3, 300, 4096), (3, 70, 11008),
    (4, 5, 32), (4, 37, 320), (4, 768, 768), (4, 300, 4096), (4, 70, 11008),
]


@pytest.mark.parametrize("fmt,m,k", ONEHOT_CASES)
def test_dequant_bit_exact_onehot(env, fmt, m, k):
    torch, q4, orc = env
    w = synth.weights(synth.seed_for(20 + fmt, k % 1000 + m), m, k)
    buf = _quantize_both(q4, orc, fmt, w)
    what = orc.dequantize(fmt, buf, m, k)
    rng = np.random.default_rng(m * 7 + k)
    cols = sorted(set([0, 1, 15, 16, 17, 31, 32, k - 1, k - 17] + rng.integers(0, k, 23).tolist()))
    cols = [c for c in cols if 0 <= c < k]
    for i in range(0, len(cols), 8):
        group = cols[i:i + 8]
        x = np.zeros((len(group), k), np.float32)
        for t, c in enumerate(group):
            x[t, c] = 1.0
        say(f"onehot fmt={fmt} m={m} k={k} cols={group}")
        y = _gemv(env, fmt, buf, x, m, k)
        for t, c in enumerate(group):
            got = y[t]
            exp = what[:, c]
            assert np.array_equal(got, exp), (c, np.nonzero(got != exp)[0][:5])


def _parity(env, fmt, m, k, n, seed, rows=None):
    torch, q4, orc = env
    w = synth.weights(synth.seed_for(seed, 1), m, k)
    x = synth.activations(synth.seed_for(seed, 1, True), n, k)
    buf = _quantize_both(q4, orc, fmt, w)
    say(f"parity fmt={fmt} m={m} k={k} n={n}")
    y = _gemv(env, fmt, buf, x, m, k)
    if rows is None:
        yr, ad = orc.matvec(fmt, buf, m, k, x, threads=threads(), absdot=True)
        idx = None
    else:
        ranges, idx = rows
        yr, ad = orc.matvec(fmt, buf, m, k, x, threads=threads(), absdot=True, rows=ranges)
    check_tolerance(y, yr, ad, GEMV_TOL, rows=idx, what=f"fmt={fmt} {m}x{k} n={n}")
    return y


SMALL_Q4_0 = [(1, 32), (3, 96), (37, 320), (130, 768), (257, 960), (515, 3072), (300, 4096), (77, 11008),
              (1000, 2560), (2049, 768)]


@pytest.mark.parametrize("m,k", SMALL_Q4_0)
@pytest.mark.parametrize("n", [1, 2, 3, 5, 8])
def test_parity_q4_0_small(env, m, k, n):
    _parity(env, 0, m, k, n, seed=100 + n)


def _geometry_ids():
    import q4_weight_gemv_amd as q4

    return [f"L{g[0]}R{g[1]}W{g[2]}" for g in q4.GEMV_GEOMETRIES]


def _geometries():
    import q4_weight_gemv_amd as q4

    return list(q4.GEMV_GEOMETRIES)


@pytest.mark.parametrize("geom", _geometries(), ids=_geometry_ids())
@pytest.mark.parametrize("fmt,n", [(0, 1), (0, 8), (1, 1), (1, 8), (2, 1), (2, 8), (3, 1), (3, 8), (4, 1), (4, 8)])
def test_parity_every_geometry(env, fmt, n, geom):
    """Every instantiated tile geometry through q4_gemv_tuned: 600 ragged rows
    (a grid-stride loop for the short tiles at one group per compute unit) and
    K = 2304, which at n = 8 exceeds one LDS chunk of activations."""
    torch, q4, orc = env
    m, k = 600, 2304
    w = synth.weights(synth.seed_for(900 + fmt, 1), m, k)
    x = synth.activations(synth.seed_for(900 + fmt, 1, True), n, k)
    buf = _quantize_both(q4, orc, fmt, w)
    wd = torch.from_numpy(buf).cuda()
    xd = torch.from_numpy(x).cuda()
    yd = torch.full((n, m), float("nan"), dtype=torch.float32, device="cuda")
    say(f"geometry {geom} fmt={fmt} n={n}")
    q4.q4_gemv_tuned(fmt, wd, xd, yd, m, k, geom[0], geom[1], geom[2], 1)
    torch.cuda.synchronize()
    yr, ad = orc.matvec(fmt, buf, m, k, x, threads=threads(), absdot=True)
    check_tolerance(yd.cpu().numpy(), yr, ad, GEMV_TOL, what=f"geometry {geom} fmt={fmt} n={n}")


def _stream_geometries():
    import q4_weight_gemv_amd as q4

    return list(q4.GEMV_STREAM_GEOMETRIES)


@pytest.mark.parametrize("geom", _stream_geometries(), ids=lambda g: f"L{g[0]}W{g[1]}D{g[2]}")
@pytest.mark.parametrize("fmt", [0, 1, 2, 3, 4])
@pytest.mark.parametrize("m,k", [(600, 2304), (1000, 768), (37, 11008), (300, 4096)])
def test_parity_every_stream_geometry(env, fmt, geom, m, k):
    """Every instantiated geometry of the one-token streaming kernel, every
    format, through q4_gemv_tuned: ragged rows (a partial last row group and a
    partial last slot of units), short rows, a long row, and hi + lo versus
    single fp16 activations (fewer or more than 256 rows)."""
    torch, q4, orc = env
    w = synth.weights(synth.seed_for(910 + fmt, m), m, k)
    x = synth.activations(synth.seed_for(910 + fmt, m, True), 1, k)
    buf = _quantize_both(q4, orc, fmt, w)
    wd = torch.from_numpy(buf).cuda()
    xd = torch.from_numpy(x).cuda()
    yd = torch.full((1, m), float("nan"), dtype=torch.float32, device="cuda")
    say(f"stream geometry {geom} fmt={fmt} m={m} k={k}")
    q4.q4_gemv_tuned(fmt, wd, xd, yd, m, k, lanes_per_row=geom[0], waves_per_group=geom[1], groups_per_cu=1,
                     kernel=q4.Q4_GEMV_KERNEL_STREAM, depth=geom[2])
    torch.cuda.synchronize()
    yr, ad = orc.matvec(fmt, buf, m, k, x, threads=threads(), absdot=True)
    check_tolerance(yd.cpu().numpy(), yr, ad, GEMV_TOL, what=f"stream {geom} fmt={fmt} {m}x{k}")


@pytest.mark.parametrize("m,k", [(1, 32), (3, 64), (7, 768), (9, 960), (255, 4096), (256, 4096), (257, 4096),
                                 (4097, 4096), (2, 14560), (300, 14560), (40, 14592), (5, 1 << 16)])
def test_parity_q4_0_one_token_edges(env, m, k):
    # The library's one-token choice at the edges of the streaming kernel:
    # single rows, fewer rows than a row group, the 256-row switch of the
    # activation precision, the longest row it stages (14560 weights, 65520
    # bytes of LDS) and longer rows (the tiled kernel).
    _parity(env, 0, m, k, 1, seed=330 + m % 11)


@pytest.mark.parametrize("gpc", [1, 2, 3, 4, 8])
def test_stream_groups_per_cu(env, gpc):
    # Workgroups per compute unit change only how the rows are split, never a
    # row's arithmetic: every split gives the same bits.
    torch, q4, orc = env
    m, k = 2311, 2304
    buf = q4.q4_quantize_ref(0, synth.weights(921, m, k))
    x = synth.activations(922, 1, k)
    wd = torch.from_numpy(buf).cuda()
    xd = torch.from_numpy(x).cuda()
    outs = []
    for g in (1, gpc):
        yd = torch.full((1, m), float("nan"), dtype=torch.float32, device="cuda")
        q4.q4_gemv_tuned(0, wd, xd, yd, m, k, lanes_per_row=64, waves_per_group=8, groups_per_cu=g,
                         kernel=q4.Q4_GEMV_KERNEL_STREAM, depth=2)
        torch.cuda.synchronize()
        outs.append(yd.cpu().numpy())
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))
    yr, ad = orc.matvec(0, buf, m, k, x, threads=threads(), absdot=True)
    check_tolerance(outs[1], yr, ad, GEMV_TOL, what=f"stream gpc={gpc}")


SMALL_Q4_K = [(1, 256), (37, 512), (130, 1024), (257, 2560), (300, 4096), (77, 11008), (1025, 768 + 256)]


@pytest.mark.parametrize("m,k", SMALL_Q4_K)
@pytest.mark.parametrize("n", [1, 4, 6, 8])
def test_parity_q4_k_small(env, m, k, n):
    _parity(env, 1, m, k, n, seed=200 + n)


WORKLOAD_SHAPES = sorted(set(synth.gpt2_124m_step() + synth.smollm2_360m_step() + synth.llama7b_layer()))


@pytest.mark.parametrize("k,m", WORKLOAD_SHAPES)
def test_parity_q4_0_workload_shapes(env, k, m):
    # N = 1 (decode) at every matrix shape of the GPT-2, SmolLM2 and 7B workloads.
    _parity(env, 0, m, k, 1, seed=300 + k % 17)


@pytest.mark.parametrize("k,m", synth.llama7b_layer()[:1] + synth.llama7b_layer()[2:])
@pytest.mark.parametrize("n", [1, 4, 8])
def test_parity_q4_k_7b(env, k, m, n):
    _parity(env, 1, m, k, n, seed=400 + n)


@pytest.mark.parametrize("k,m", [(4096, 4096), (11008, 4096)])
@pytest.mark.parametrize("n", [4, 8])
def test_parity_q4_0_7b_batched(env, k, m, n):
    _parity(env, 0, m, k, n, seed=500 + n)


SMALL_Q8_0 = [(1, 32), (37, 320), (130, 768), (257, 960), (300, 4096), (77, 11008), (2049, 768)]


@pytest.mark.parametrize("m,k", SMALL_Q8_0)
@pytest.mark.parametrize("n", [1, 3, 8])
def test_parity_q8_0_small(env, m, k, n):
    _parity(env, 2, m, k, n, seed=150 + n)


@pytest.mark.parametrize("k,m", synth.llama7b_layer()[:2] + synth.llama7b_layer()[3:])
@pytest.mark.parametrize("n", [1, 8])
def test_parity_q8_0_7b(env, k, m, n):
    _parity(env, 2, m, k, n, seed=450 + n)


SMALL_Q2_K = [(1, 256), (37, 512), (130, 1024), (257, 2560), (300, 4096), (77, 11008), (1025, 768 + 256)]


@pytest.mark.parametrize("m,k", SMALL_Q2_K)
@pytest.mark.parametrize("n", [1, 4, 8])
def test_parity_q2_k_small(env, m, k, n):
    _parity(env, 3, m, k, n, seed=250 + n)


@pytest.mark.parametrize("k,m", synth.llama7b_layer()[:2] + synth.llama7b_layer()[3:])
@pytest.mark.parametrize("n", [1, 8])
def test_parity_q2_k_7b(env, k, m, n):
    _parity(env, 3, m, k, n, seed=470 + n)


SMALL_Q1_0 = [(1, 32), (37, 320), (130, 768), (257, 960), (300, 4096), (77, 11008), (2049, 768)]


@pytest.mark.parametrize("m,k", SMALL_Q1_0)
@pytest.mark.parametrize("n", [1, 3, 8])
def test_parity_q1_0_small(env, m, k, n):
    _parity(env, 4, m, k, n, seed=170 + n)


@pytest.mark.parametrize("k,m", synth.llama7b_layer()[:2] + synth.llama7b_layer()[3:])
@pytest.mark.parametrize("n", [1, 8])
def test_parity_q1_0_7b(env, k, m, n):
    _parity(env, 4, m, k, n, seed=490 + n)


@pytest.mark.parametrize("m", [40, 300])
def test_q1_0_hand_built_words(env, m):
    # Code words all 0, all 1, alternating and random, with scales that are
    # zero, subnormal, ordinary and the largest finite fp16, against the
    # oracle's product of the same bytes (below and above the row count where
    # activations lose their lo halves).
    torch, q4, orc = env
    k = 256
    rng = np.random.default_rng(m)
    nb = m * k // 32
    words = rng.integers(0, 1 << 32, size=nb, dtype=np.uint64).astype(np.uint32)
    words[0::7] = 0
    words[1::7] = 0xFFFFFFFF
    words[2::7] = 0x55555555
    scales = rng.uniform(0.001, 2.0, size=nb).astype(np.float16)
    scales[3::11] = np.float16(0.0)
    scales[4::11] = np.float16(6e-8)     # subnormal
    scales[5::13] = np.float16(65504.0)  # largest finite
    scales[6::17] *= np.float16(-1.0)     # negative (the quantizer never writes one)
    buf = np.concatenate([words.view(np.uint8), scales.view(np.uint8)])
    assert buf.size == q4.q4_weight_bytes(4, m, k)
    x = synth.activations(880 + m, 2, k)
    say(f"q1_0 hand-built words m={m}")
    y = _gemv(env, 4, buf, x, m, k)
    yr, ad = orc.matvec(4, buf, m, k, x, threads=threads(), absdot=True)
    check_tolerance(y, yr, ad, GEMV_TOL, what=f"q1_0 hand-built m={m}")


def test_q8_0_extreme_codes(env):
    # Hand-built Q8_0 blocks with every code -128..127 (a code of -128 is legal
    # input though the quantizer never writes it) and mixed scales: one-hot x
    # returns each dequantized weight exactly.
    torch, q4, orc = env
    m, k = 8, 256
    codes = (np.arange(m * k) % 256).astype(np.uint8).reshape(m * k)
    d = np.array([0.5, 0.0078125, 3.0, 1.5e-5] * (m * k // 32 // 4), np.float16)
    buf = np.concatenate([codes, d.view(np.uint8)])
    assert buf.size == q4.q4_weight_bytes(2, m, k)
    what = orc.dequantize(2, buf, m, k)
    for c0 in range(0, k, 8):
        x = np.zeros((8, k), np.float32)
        for t in range(8):
            x[t, c0 + t] = 1.0
        y = _gemv(env, 2, buf, x, m, k)
        assert np.array_equal(y, what[:, c0:c0 + 8].T), c0


def test_zero_rows_and_tokens_are_noops(env):
    torch, q4, _ = env
    y = torch.full((2, 8), 7.0, device="cuda")
    w = torch.zeros(1024, dtype=torch.uint8, device="cuda")
    x = torch.zeros((2, 64), device="cuda")
    q4.q4_gemv(0, w, x, y, 0, 64)
    q4.raw().q4_gemv(0, w.data_ptr(), x.data_ptr(), y.data_ptr(), 8, 64, 0, None)
    torch.cuda.synchronize()
    assert (y == 7.0).all()


@pytest.mark.parametrize("fmt,m,k,n", [(0, 300, 4096, 1), (0, 37, 768, 3), (0, 2049, 768, 1), (1, 300, 4096, 1),
                                         (1, 130, 1024, 8), (2, 300, 960, 1), (3, 130, 1024, 4), (4, 2049, 768, 1)])
@pytest.mark.parametrize("shift", [1, 2, 3])
def test_x_four_byte_aligned(env, fmt, m, k, n, shift):
    # x 4, 8 or 12 bytes past a 16-byte boundary is staged with 4-byte loads:
    # the same bits as the same values at an aligned address, and the
    # oracle's tolerance (one token: the streaming kernel; several: tiled).
    torch, q4, orc = env
    buf = q4.q4_quantize_ref(fmt, synth.weights(synth.seed_for(1500 + fmt, m), m, k))
    x = synth.activations(synth.seed_for(1500 + fmt, m, True), n, k)
    wd = torch.from_numpy(buf).cuda()
    ref = _gemv(env, fmt, buf, x, m, k)
    store = torch.zeros(n * k + 8, dtype=torch.float32, device="cuda")
    xd = store[shift:shift + n * k].view(n, k)
    xd.copy_(torch.from_numpy(x))
    assert xd.data_ptr() % 16 == 4 * shift
    yd = torch.full((n, m), float("nan"), dtype=torch.float32, device="cuda")
    say(f"x at +{4 * shift} bytes fmt={fmt} m={m} k={k} n={n}")
    q4.q4_gemv(fmt, wd, xd, yd, m, k)
    torch.cuda.synchronize()
    y = yd.cpu().numpy()
    assert np.array_equal(y.view(np.uint32), ref.view(np.uint32))
    yr, ad = orc.matvec(fmt, buf, m, k, x, threads=threads(), absdot=True)
    if fmt in (1, 3):
        ad = orc.termscale(fmt, buf, m, k, x, threads=threads())
    check_tolerance(y, yr, ad, GEMV_TOL, what=f"x at +{4 * shift} fmt={fmt}")


def test_misaligned_pointer_rejected(env):
    torch, q4, _ = env
    w = torch.zeros(4096, dtype=torch.uint8, device="cuda")
    x = torch.zeros(128, device="cuda")
    y = torch.full((8,), 3.0, device="cuda")
    st = q4.raw().q4_gemv(0, w.data_ptr() + 8, x.data_ptr(), y.data_ptr(), 8, 64, 1, None)
    assert st == q4.Q4_EALIGN
    torch.cuda.synchronize()
    assert (y == 3.0).all()


def test_deterministic(env):
    torch, q4, orc = env
    m, k = 2304, 768
    w = synth.weights(61, m, k)
    x = synth.activations(62, 3, k)
    buf = q4.q4_quantize_ref(0, w)
    a = _gemv(env, 0, buf, x, m, k)
    b = _gemv(env, 0, buf, x, m, k)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("fmt,m,k,n", [(0, 300, 1024, 1), (0, 100, 960, 4), (1, 300, 1024, 4), (2, 130, 960, 1),
                                         (3, 130, 1024, 4), (4, 130, 960, 4)])
def test_nan_activation_makes_its_token_nan(env, fmt, m, k, n):
    # IEEE arithmetic: a NaN among one token's activations makes every output
    # of that token NaN (0 * NaN is NaN too), as in the oracle; the other
    # tokens are unaffected. Outputs start at a finite sentinel, so a NaN
    # below was written by the kernel.
    torch, q4, orc = env
    buf = _quantize_both(q4, orc, fmt, synth.weights(synth.seed_for(1300 + fmt, m), m, k))
    x = synth.activations(synth.seed_for(1300 + fmt, m, True), n, k)
    bad = n - 1
    x[bad, k // 3] = np.nan
    wd = torch.from_numpy(buf).cuda()
    xd = torch.from_numpy(x).cuda()
    yd = torch.full((n, m), 12345.0, dtype=torch.float32, device="cuda")
    say(f"nan activation fmt={fmt} m={m} k={k} n={n}")
    q4.q4_gemv(fmt, wd, xd, yd, m, k)
    torch.cuda.synchronize()
    y = yd.cpu().numpy()
    yr, ad = orc.matvec(fmt, buf, m, k, x, threads=threads(), absdot=True)
    assert np.isnan(yr[bad]).all() and np.isnan(y[bad]).all()
    if n > 1:
        check_tolerance(y[:bad], yr[:bad], ad[:bad], GEMV_TOL, what=f"fmt={fmt} tokens without the NaN")


def test_extreme_activation_scales(env):
    # Per-unit power-of-two scaling: results track x * 2^s exactly for large
    # and tiny s (fp16 alone would overflow at 65504 or flush tiny values).
    torch, q4, orc = env
    m, k = 96, 1024
    w = synth.weights(71, m, k)
    buf = q4.q4_quantize_ref(0, w)
    x = synth.activations(72, 2, k)
    y = _gemv(env, 0, buf, x, m, k)
    for s in (40, -40, 90):
        ys = _gemv(env, 0, buf, (x * np.float32(2.0 ** s)).astype(np.float32), m, k)
        assert np.array_equal(ys, (y.astype(np.float64) * 2.0 ** s).astype(np.float32)), s
    big = x.copy()
    big[0, 5] = 1e6
    yb = _gemv(env, 0, buf, big, m, k)
    yr, ad = orc.matvec(0, buf, m, k, big, absdot=True)
    check_tolerance(yb, yr, ad, GEMV_TOL, what="large activation")


def test_extreme_activation_q4_k(env):
    # Q4_K's value is the difference of two terms (d*sc*q and dmin*m); with an
    # outlier activation the elementwise error is bounded against the sum of
    # the term magnitudes (the oracle's termscale), and normwise as usual.
    torch, q4, orc = env
    m, k = 96, 1024
    buf = q4.q4_quantize_ref(1, synth.weights(73, m, k))
    x = synth.activations(74, 3, k)
    x[0, 5] = 1e6
    x[2, 700] = -3e4
    y = _gemv(env, 1, buf, x, m, k)
    yr = orc.matvec(1, buf, m, k, x)
    check_tolerance(y, yr, orc.termscale(1, buf, m, k, x), GEMV_TOL, what="q4_k outlier")


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("n", [1, 3])
def test_outlier_activation_single_fp16_path(env, fmt, n):
    # Products of 256 rows or more hold one fp16 per activation (the tests
    # above use 96 rows, the hi + lo form). An outlier sets its unit's
    # power-of-two scale, leaving the unit's other activations about 2^-20 of
    # it; where the outlier meets a zero weight (Q4_0 code 8) its term must
    # contribute exactly nothing, or the rounding of a running sum that holds
    # it swamps the unit's small terms. Each row's error is bounded against
    # its term magnitudes (about 15 % of the rows have code 8 at an outlier).
    from gpu_common import GEMV_TOL, check_tolerance

    torch, q4, orc = env
    m, k = 320, 1024
    buf = q4.q4_quantize_ref(fmt, synth.weights(75 + fmt, m, k))
    x = synth.activations(77, 3, k)
    x[0, 5] = 1e6
    x[1, 700] = -3e4
    x[2, ::97] = 1e5  # an outlier in each of eleven units
    x = x[:n]
    say(f"outlier activation single fp16 fmt={fmt} n={n}")
    y = _gemv(env, fmt, buf, x, m, k)
    if fmt == 0:
        yr, scale = orc.matvec(fmt, buf, m, k, x, absdot=True)
    else:
        yr, scale = orc.matvec(fmt, buf, m, k, x), orc.termscale(fmt, buf, m, k, x)
    check_tolerance(y, yr, scale, GEMV_TOL, what=f"outlier fmt={fmt} n={n}")


@pytest.mark.parametrize("fmt,k,parts", [(0, 960, (960, 320, 320)), (0, 960, (2560, 2560)), (1, 1024, (512, 256, 256))])
def test_stacked_projections_equal_separate_products(env, fmt, k, parts):
    # Shared-input projections (q|k|v, gate|up) row-stacked into one matrix:
    # blocks never cross rows, so the stacked weights quantize to the
    # concatenated rows and one launch reproduces the separate products
    # bit for bit (same tile geometry for every part).
    torch, q4, orc = env
    ws = [synth.weights(950 + i, m, k) for i, m in enumerate(parts)]
    x = synth.activations(960, 2, k)
    stacked = np.concatenate(ws, axis=0)
    ys = _gemv(env, fmt, q4.q4_quantize_ref(fmt, stacked), x, stacked.shape[0], k)
    r = 0
    for w in ws:
        y1 = _gemv(env, fmt, q4.q4_quantize_ref(fmt, w), x, w.shape[0], k)
        assert np.array_equal(ys[:, r:r + w.shape[0]].view(np.uint32), y1.view(np.uint32))
        r += w.shape[0]


@pytest.mark.parametrize("fmt,n", [(0, 2), (1, 2), (0, 8), (1, 8)])
def test_sequence_and_graph_match_single_calls(env, fmt, n):
    # At 8 tokens the 4096- and 11008-long rows stage their activations in
    # the opt-in LDS (whole row, or chunks larger than 64 KiB).
    torch, q4, _ = env
    if n == 8:
        shapes = [(4096, 300), (11008, 200), (768, 500)]
    else:
        shapes = [(768, 2304), (768, 768), (768, 3072), (3072, 768), (960, 320)] if fmt == 0 else \
                 [(1024, 512), (2560, 960), (4096, 257)]
    ops, refs = [], []
    for i, (k, m) in enumerate(shapes):
        w = synth.weights(800 + i, m, k)
        x = synth.activations(900 + i, n, k)
        wd = torch.from_numpy(q4.q4_quantize_ref(fmt, w)).cuda()
        xd = torch.from_numpy(x).cuda()
        ref = torch.empty((n, m), device="cuda")
        q4.q4_gemv(fmt, wd, xd, ref, m, k)
        refs.append(ref)
        ops.append((wd, xd, torch.full((n, m), float("nan"), device="cuda"), m, k))
    say(f"sequence fmt={fmt} n={n}")
    q4.q4_gemv_sequence(fmt, ops, n)
    torch.cuda.synchronize()
    for (_, _, y, _, _), ref in zip(ops, refs):
        assert torch.equal(y, ref)
    seq = q4.Q4Sequence(fmt, ops, n)  # marshalled once, launched twice
    for _ in range(2):
        for (_, _, y, _, _) in ops:
            y.fill_(float("nan"))
        seq.launch()
        torch.cuda.synchronize()
        for (_, _, y, _, _), ref in zip(ops, refs):
            assert torch.equal(y, ref)
    say(f"graph fmt={fmt} n={n}")
    g = q4.Q4Graph(fmt, ops, n)
    for rep in range(3):
        for (_, _, y, _, _) in ops:
            y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.launch()
        torch.cuda.synchronize()
        _ = torch.randn(1000, device="cuda").sum().item()  # eager work between replays
        for (_, _, y, _, _), ref in zip(ops, refs):
            assert torch.equal(y, ref), rep
    g.close()


# ---- gated product: silu(W_gate x) * (W_up x) from one stacked matrix ------------

def _glu(env, fmt, buf, x, m, k):
    torch, q4, _ = env
    wd = torch.from_numpy(buf).cuda()
    xd = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()
    yd = torch.full((x.shape[0], m), float("nan"), dtype=torch.float32, device="cuda")
    q4.q4_gemv_glu(fmt, wd, xd, yd, m, k)
    torch.cuda.synchronize()
    return yd.cpu().numpy()


def _silu_mul64(g, u):
    g = np.asarray(g, np.float64)
    return g / (1.0 + np.exp(-g)) * np.asarray(u, np.float64)


def _glu_plain_kernel(q4, fmt, n, m, k):
    """The kernel whose plain product of the stacked 2m-row matrix the gated
    product reproduces (q4.h, q4_gemv_glu): the matrix-core kernel for Q4_K
    where q4_gemv would pick it for the stacked matrix and the row has at most
    4096 weights, else the tiled kernel."""
    matrix = fmt == 1 and 2 * m >= 256 and k <= 4096 and (n >= 3 or (n == 2 and k <= 2048))
    return q4.Q4_GEMV_KERNEL_MATRIX if matrix else q4.Q4_GEMV_KERNEL_TILED


GLU_CASES = [
    (0, 1, 37, 96), (0, 3, 130, 960), (0, 1, 1280, 960), (0, 8, 200, 2560), (0, 1, 300, 4096), (0, 2, 70, 11008),
    (1, 1, 37, 256), (1, 4, 130, 1024), (1, 1, 300, 4096), (1, 8, 90, 4096), (1, 1, 70, 11008),
    (1, 2, 200, 2048), (1, 3, 130, 512), (1, 5, 300, 4096), (1, 8, 300, 4096),  # the matrix-core gated form
    (2, 1, 130, 960), (2, 4, 300, 4096),
    (3, 1, 130, 1024), (3, 4, 300, 4096),
    (4, 1, 130, 960), (4, 4, 300, 4096), (4, 1, 2560, 960),
    (0, 8, 300, 4096), (1, 4, 300, 4096), (1, 8, 70, 11008),  # 8-wave gated groups
    (0, 1, 11008, 4096), (1, 1, 11008, 4096), (1, 4, 11008, 4096), (1, 8, 11008, 4096),  # the 7B gate|up as benchmarked
]


@pytest.mark.parametrize("fmt,n,m,k", GLU_CASES)
def test_glu_matches_plain_product_of_stacked_matrix(env, fmt, n, m, k):
    # The gate and up sums are formed exactly as the plain product forms the
    # rows of the stacked matrix, so the gated output is silu(g) * u of the
    # plain product's rows, up to the fp32 epilogue (a few ulp).
    torch, q4, orc = env
    buf = q4.q4_quantize_ref(fmt, synth.weights(synth.seed_for(1100 + fmt, m), 2 * m, k))
    x = synth.activations(synth.seed_for(1100 + fmt, m, True), n, k)
    say(f"glu vs plain fmt={fmt} n={n} m={m} k={k}")
    # The plain product on the kernel the gated product shares (one token of
    # Q4_0 would otherwise take the streaming kernel).
    wd = torch.from_numpy(buf).cuda()
    xd = torch.from_numpy(x).cuda()
    ypd = torch.full((n, 2 * m), float("nan"), dtype=torch.float32, device="cuda")
    q4.q4_gemv_tuned(fmt, wd, xd, ypd, 2 * m, k, kernel=_glu_plain_kernel(q4, fmt, n, m, k))
    torch.cuda.synchronize()
    yp = ypd.cpu().numpy()
    yg = _glu(env, fmt, buf, x, m, k)
    ref = _silu_mul64(yp[:, :m], yp[:, m:])
    scale = np.abs(yp[:, :m].astype(np.float64) * yp[:, m:])
    assert np.all(np.isfinite(yg))
    assert np.all(np.abs(yg - ref) <= 4e-6 * scale + 1e-30), np.max(np.abs(yg - ref) / (scale + 1e-30))


@pytest.mark.parametrize("fmt,n,m,k", GLU_CASES)
def test_glu_parity_oracle(env, fmt, n, m, k):
    # Against the oracle's fp64 silu(g) * u: with |dg| <= tol * sum|w x| over
    # the gate row and |du| likewise over the up row (the decode product's
    # elementwise bound), and |silu'| <= 1.1, the gated output is within
    #   1.1 |u| tol A_g + |silu(g)| tol A_u + 1.1 tol^2 A_g A_u
    # plus the fp32 epilogue's few ulp.
    torch, q4, orc = env
    buf = q4.q4_quantize_ref(fmt, synth.weights(synth.seed_for(1200 + fmt, m), 2 * m, k))
    assert np.array_equal(buf, orc.quantize(fmt, synth.weights(synth.seed_for(1200 + fmt, m), 2 * m, k)))
    x = synth.activations(synth.seed_for(1200 + fmt, m, True), n, k)
    say(f"glu parity fmt={fmt} n={n} m={m} k={k}")
    yg = _glu(env, fmt, buf, x, m, k)
    yr, g, u = orc.matvec_silu_mul(fmt, buf, m, k, x, threads=threads(), parts=True)
    _, ad = orc.matvec(fmt, buf, 2 * m, k, x, threads=threads(), absdot=True)
    if fmt in (1, 3):  # the K-quants' elementwise bound is stated against their term scale
        ad = orc.termscale(fmt, buf, 2 * m, k, x, threads=threads())
    ag, au = ad[:, :m], ad[:, m:]
    silu = g / (1.0 + np.exp(-g))
    bound = (1.1 * np.abs(u) * GEMV_TOL * ag + np.abs(silu) * GEMV_TOL * au + 1.1 * GEMV_TOL ** 2 * ag * au
             + 4e-6 * np.abs(yr.astype(np.float64)) + 1e-30)
    err = np.abs(yg.astype(np.float64) - yr)
    assert np.all(np.isfinite(yg))
    bad = np.argwhere(err > bound)
    assert bad.size == 0, (bad[:5], err[tuple(bad[0])], bound[tuple(bad[0])])
    # Normwise as the decode product: within 2e-3 of the reference per token.
    for t in range(n):
        assert np.linalg.norm(yg[t] - yr[t]) <= GEMV_TOL * np.linalg.norm(yr[t])


def test_glu_noop_and_errors(env):
    torch, q4, _ = env
    lib = q4.raw()
    w = torch.zeros(4096, dtype=torch.uint8, device="cuda")
    x = torch.zeros(256, device="cuda")
    y = torch.full((8,), 5.0, device="cuda")
    assert lib.q4_gemv_glu(0, w.data_ptr(), x.data_ptr(), y.data_ptr(), 0, 32, 1, None) == q4.Q4_OK
    assert lib.q4_gemv_glu(0, w.data_ptr(), x.data_ptr(), y.data_ptr(), 4, 32, 0, None) == q4.Q4_OK
    assert lib.q4_gemv_glu(0, w.data_ptr(), x.data_ptr() + 2, y.data_ptr(), 4, 32, 1, None) == q4.Q4_EALIGN
    torch.cuda.synchronize()
    assert (y == 5.0).all()


@pytest.mark.parametrize("fmt", [0, 1])
def test_sequence_and_graph_with_gated_ops(env, fmt):
    # A SmolLM2-like fused layer: q|k|v stacked, o, gate|up gated, down; the
    # sequence and the replayed graph reproduce the single calls bit for bit.
    torch, q4, _ = env
    k0 = 960 if fmt == 0 else 1024
    k1 = 2560 if fmt == 0 else 2560 + 256 * 2
    shapes = [(k0, 1600, 0), (k0, k0, 0), (k0, 2560, 1), (k1, k0, 0)]
    n = 1
    ops, refs = [], []
    for i, (k, m, epi) in enumerate(shapes):
        rows = 2 * m if epi else m
        wd = torch.from_numpy(q4.q4_quantize_ref(fmt, synth.weights(1300 + i, rows, k))).cuda()
        xd = torch.from_numpy(synth.activations(1400 + i, n, k)).cuda()
        ref = torch.empty((n, m), device="cuda")
        (q4.q4_gemv_glu if epi else q4.q4_gemv)(fmt, wd, xd, ref, m, k)
        refs.append(ref)
        ops.append((wd, xd, torch.full((n, m), float("nan"), device="cuda"), m, k, epi))
    say(f"gated sequence fmt={fmt}")
    q4.q4_gemv_sequence(fmt, ops, n)
    torch.cuda.synchronize()
    for op, ref in zip(ops, refs):
        assert torch.equal(op[2], ref)
    say(f"gated graph fmt={fmt}")
    g = q4.Q4Graph(fmt, ops, n)
    for rep in range(3):
        for op in ops:
            op[2].fill_(float("nan"))
        torch.cuda.synchronize()
        g.launch()
        torch.cuda.synchronize()
        _ = torch.randn(1000, device="cuda").sum().item()
        for op, ref in zip(ops, refs):
            assert torch.equal(op[2], ref), rep
    g.close()
