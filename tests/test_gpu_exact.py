"""Decode products on inputs where every step of the arithmetic is exact.

* Exact sums: weights whose dequantized values are small integers (scale 1)
  and activations in {-1, 0, 1}. Every product, every 32-weight unit sum and
  every partial sum of a row is then an integer below 2^24, exact in fp32 in
  any order of summation, so the decode product must return the oracle's
  result bit for bit, at row lengths up to 2^20 and through every kernel the
  library picks (the one-token streaming kernel and the tiled kernel). A
  kernel that rounds a product or a partial sum -- as v_dot2c_f32_f16 does
  when fed fp16 subnormal operands on gfx950 -- fails this at once.
* Hand-built blocks: dequantization bit-exact through the public entry point
  (one-hot x = e_j returns column j of W_hat) for the codes and scales the
  quantizer never writes: Q4_0 code 0 (weight -8d), zero, subnormal,
  negative and largest-finite fp16 scales; Q4_K headers of the hand-worked
  super-block K-A and of all-63 fields, with those scales in d and dmin.
"""
import numpy as np
import pytest

import synth
from gpu_common import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch

    import oracle
    import q4_weight_gemv_amd as q4

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    oracle.lib()
    return torch, q4, oracle


def _run(env, fmt, buf, x, m, k, tuning=None):
    torch, q4, _ = env
    wd = torch.from_numpy(buf).cuda()
    xd = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()
    yd = torch.full((x.shape[0], m), float("nan"), dtype=torch.float32, device="cuda")
    if tuning is None:
        q4.q4_gemv(fmt, wd, xd, yd, m, k)
    else:
        q4.q4_gemv_tuned(fmt, wd, xd, yd, m, k, *tuning)
    torch.cuda.synchronize()
    return yd.cpu().numpy()


FP16_ONE = np.float16(1.0).view(np.uint16)


def _integer_buffer(q4, fmt, m, k, rng, small=False):
    """A valid m x k buffer whose dequantized weights are integers: every fp16
    scale is 1 (d and dmin for the K-quants), codes random. ``small`` keeps
    the K-quants' 6-bit fields below 8 so long rows stay below 2^24."""
    n = q4.q4_weight_bytes(fmt, m, k)
    buf = rng.integers(0, 256, size=n, dtype=np.uint8)
    one = np.array([FP16_ONE], np.uint16).view(np.uint8)
    if fmt in (0, 2, 4):  # code plane, then one fp16 scale per 32 weights
        nb = m * k // 32
        buf[n - 2 * nb:] = np.tile(one, nb)
    elif fmt == 1:  # 144-byte super-blocks: d, dmin, 12 bytes of 6-bit fields
        sb = buf.reshape(-1, 144)
        sb[:, 0:2] = one
        sb[:, 2:4] = one
        if small:
            sb[:, 4:16] &= 0x07  # every 6-bit field in 0..7
    else:  # Q2_K: codes, scale bytes (4-bit sc, 4-bit m), d and dmin
        ns = m * k // 256
        buf[n - 4 * ns:] = np.tile(np.concatenate([one, one]), ns)
    return buf


# (fmt, m, k): row lengths up to 2^20 (Q4_0: |w| <= 8; Q1_0: |w| = 1), and up
# to 2^16 for the formats whose integer weights are larger.
EXACT_CASES = [
    (0, 300, 4096), (0, 37, 11008), (0, 4096, 4096), (0, 11008, 4096), (0, 4096, 11008), (0, 70, 1 << 20),
    (0, 50257, 768), (0, 2304, 768),
    (1, 300, 4096), (1, 37, 11008), (1, 4096, 4096), (1, 90, 1 << 16),
    (2, 300, 4096), (2, 37, 11008), (2, 4096, 4096), (2, 50, 1 << 16),
    (3, 300, 4096), (3, 37, 11008), (3, 4096, 4096), (3, 50, 1 << 16),
    (4, 300, 4096), (4, 37, 11008), (4, 4096, 4096), (4, 70, 1 << 20),
]


@pytest.mark.parametrize("fmt,m,k", EXACT_CASES)
@pytest.mark.parametrize("n", [1, 3, 8])
def test_exact_integer_sums(env, fmt, m, k, n):
    torch, q4, orc = env
    rng = np.random.default_rng(fmt * 1000 + m + k + n)
    small = fmt == 1 and k > 8192
    buf = _integer_buffer(q4, fmt, m, k, rng, small=small)
    x = rng.integers(-1, 2, size=(n, k)).astype(np.float32)
    x[:, rng.integers(0, k, size=min(k, 64))] = 0.0
    say(f"exact sums fmt={fmt} m={m} k={k} n={n}")
    y = _run(env, fmt, buf, x, m, k)
    yr, ad = orc.matvec(fmt, buf, m, k, x, threads=16, absdot=True)
    # Every partial sum is bounded by the sum of the term magnitudes (for the
    # K-quants both terms of each weight, which the kernels sum apart).
    scale = orc.termscale(fmt, buf, m, k, x, threads=16) if fmt in (1, 3) else ad
    assert scale.max() < 2 ** 24, "case exceeds the exact range"
    bad = np.argwhere(y != yr)
    assert bad.size == 0, (bad[:5], y[tuple(bad[0])], yr[tuple(bad[0])])


def _geometry_list():
    import q4_weight_gemv_amd as q4

    return list(q4.GEMV_GEOMETRIES)


@pytest.mark.parametrize("geom", _geometry_list(), ids=lambda g: f"L{g[0]}R{g[1]}W{g[2]}")
@pytest.mark.parametrize("fmt", [0, 1, 2, 3, 4])
def test_exact_integer_sums_every_geometry(env, fmt, geom):
    torch, q4, orc = env
    m, k, n = 600, 2304, 2
    rng = np.random.default_rng(fmt * 77 + geom[0] + 10 * geom[1] + 100 * geom[2])
    buf = _integer_buffer(q4, fmt, m, k, rng)
    x = rng.integers(-1, 2, size=(n, k)).astype(np.float32)
    say(f"exact sums fmt={fmt} geometry {geom}")
    y = _run(env, fmt, buf, x, m, k, tuning=(geom[0], geom[1], geom[2], 1))
    yr = orc.matvec(fmt, buf, m, k, x, threads=16)
    assert np.array_equal(y, yr), np.argwhere(y != yr)[:5]


def _stream_geometry_list():
    import q4_weight_gemv_amd as q4

    return list(q4.GEMV_STREAM_GEOMETRIES)


@pytest.mark.parametrize("geom", _stream_geometry_list(), ids=lambda g: f"L{g[0]}W{g[1]}D{g[2]}")
@pytest.mark.parametrize("fmt", [0, 1, 2, 3, 4])
def test_exact_integer_sums_every_stream_geometry(env, fmt, geom):
    torch, q4, orc = env
    m, k = 600, 2304
    rng = np.random.default_rng(fmt * 91 + geom[0] + 10 * geom[1] + 100 * geom[2])
    buf = _integer_buffer(q4, fmt, m, k, rng)
    x = rng.integers(-1, 2, size=(1, k)).astype(np.float32)
    say(f"exact sums fmt={fmt} stream geometry {geom}")
    wd = torch.from_numpy(buf).cuda()
    xd = torch.from_numpy(x).cuda()
    yd = torch.full((1, m), float("nan"), dtype=torch.float32, device="cuda")
    q4.q4_gemv_tuned(fmt, wd, xd, yd, m, k, lanes_per_row=geom[0], waves_per_group=geom[1], groups_per_cu=1,
                     kernel=q4.Q4_GEMV_KERNEL_STREAM, depth=geom[2])
    torch.cuda.synchronize()
    y = yd.cpu().numpy()
    yr = orc.matvec(fmt, buf, m, k, x, threads=16)
    assert np.array_equal(y, yr), np.argwhere(y != yr)[:5]


# ---- hand-built blocks, one-hot columns ----------------------------------------

# fp16 scales the quantizer never writes, beside ordinary ones.
SPECIAL_SCALES = np.array([0.0, -0.0, 2.0 ** -24, 1023 * 2.0 ** -24, 2.0 ** -14, -0.0078125, -1.5,
                           65504.0, -65504.0, 0.0066, 1.0, 3.0], np.float16)


def _q4_0_hand_buffer(m, k, rng):
    """Q4_0 rows cycling through every code 0..15 in every nibble position and
    the special scales."""
    nb = m * k // 32
    codes = rng.integers(0, 16, size=(nb, 32), dtype=np.uint8)
    codes[0::5] = np.arange(32, dtype=np.uint8) % 16          # every code, both halves
    codes[1::5] = 0                                           # all -8
    codes[2::5, :16] = 15
    nib = (codes[:, :16] | (codes[:, 16:] << 4)).astype(np.uint8)
    scales = rng.uniform(0.001, 0.02, size=nb).astype(np.float16)
    scales[::3] = SPECIAL_SCALES[np.arange(len(scales[::3])) % len(SPECIAL_SCALES)]
    return np.concatenate([nib.reshape(-1), scales.view(np.uint8)])


def _q4_k_hand_buffer(orc, m, k, rng):
    """Q4_K super-blocks with the K-A header (tests/golden/q4_k_superblocks.txt),
    all-63 fields, all-zero fields and random fields, with special d and dmin."""
    ns = m * k // 256
    sb = rng.integers(0, 256, size=(ns, 144), dtype=np.uint8)
    ka = bytes.fromhex("010203c4000102c34556670f")
    all63 = orc.q4_k_pack_scales([63] * 8, [63] * 8)
    for i in range(ns):
        kind = i % 4
        if kind == 0:
            sb[i, 4:16] = np.frombuffer(ka, np.uint8)
        elif kind == 1:
            sb[i, 4:16] = all63
        elif kind == 2:
            sb[i, 4:16] = 0
        d = SPECIAL_SCALES[i % len(SPECIAL_SCALES)]
        dmin = SPECIAL_SCALES[(3 * i + 1) % len(SPECIAL_SCALES)]
        if i % 7 == 0:
            d, dmin = np.float16(1.0), np.float16(0.5)  # K-A's own scales
        sb[i, 0:2] = np.array([d], np.float16).view(np.uint8)
        sb[i, 2:4] = np.array([dmin], np.float16).view(np.uint8)
    sb[0::9, 16:] = 0xFF   # every code 15
    sb[1::9, 16:] = 0x00   # every code 0
    return sb.reshape(-1)


@pytest.mark.parametrize("fmt,m,k", [(0, 40, 1024), (0, 300, 1024), (0, 300, 4096), (1, 40, 1024), (1, 300, 1024),
                                     (1, 300, 4096)])
def test_hand_built_blocks_onehot(env, fmt, m, k):
    # Below and above 256 rows (activations as hi + lo fp16 pairs, or single
    # fp16 values); one token of Q4_0 takes the streaming kernel, several
    # tokens (and Q4_K) the tiled one.
    torch, q4, orc = env
    rng = np.random.default_rng(31 * m + k + fmt)
    buf = _q4_0_hand_buffer(m, k, rng) if fmt == 0 else _q4_k_hand_buffer(orc, m, k, rng)
    assert buf.size == q4.q4_weight_bytes(fmt, m, k)
    what = orc.dequantize(fmt, buf, m, k)
    cols = sorted(set([0, 1, 15, 16, 17, 31, 32, 33, 63, 64, 127, 128, 255, 256, k - 1, k - 16, k - 17]
                      + rng.integers(0, k, 40).tolist()))
    for n in (1, 8):
        for i in range(0, len(cols), n):
            group = cols[i:i + n]
            x = np.zeros((len(group), k), np.float32)
            for t, c in enumerate(group):
                x[t, c] = 1.0
            say(f"hand-built onehot fmt={fmt} m={m} k={k} cols={group}")
            y = _run(env, fmt, buf, x, m, k)
            for t, c in enumerate(group):
                assert np.array_equal(y[t], what[:, c]), (c, np.nonzero(y[t] != what[:, c])[0][:5])


@pytest.mark.parametrize("m,k", [(64, 1 << 22), (256, 1 << 21)])
def test_random_full_length_rows_unbiased(env, m, k):
    # Fully random rows of millions of weights (activations as hi + lo pairs
    # at 64 rows, as single fp16 values at 256): the fp32 sums carry no
    # same-sign drift, so even rows that cancel to ~1/sqrt(K) of their term
    # scale meet the normwise bound (a bias of 2^-22 of the term scale per
    # unit would exceed it several times over).
    from gpu_common import GEMV_TOL, check_tolerance

    torch, q4, orc = env
    n = 2
    buf = q4.q4_quantize_ref(0, synth.weights(97, m, k))
    x = synth.activations(98, n, k)
    say(f"random long rows m={m} k={k}")
    y = _run(env, 0, buf, x, m, k)
    yr, ad = orc.matvec(0, buf, m, k, x, threads=16, absdot=True)
    check_tolerance(y, yr, ad, GEMV_TOL, what="random long rows")
    # and the mean signed error is far below one part in 10^6 of the term scale
    assert abs(np.mean((y.astype(np.float64) - yr) / ad)) < 1e-7
