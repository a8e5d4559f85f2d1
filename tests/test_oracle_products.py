"""Pins for the oracle's matrix-vector and matrix-matrix products.

The dequantizers are pinned by the hand-worked blocks; these tests pin the
products built on them: exact rational brute force on tiny shapes, a library
float64 product, and closed forms that a transposed operand, a dropped term or
a wrong index would break.
"""
from fractions import Fraction

import numpy as np
import pytest

import synth


def _round_to_f32(fr: Fraction) -> np.float32:
    """Correctly rounded (nearest, ties to even) float32 of an exact rational."""
    approx = np.float32(float(fr))
    best = None
    cands = [approx, np.nextafter(approx, np.float32(np.inf)), np.nextafter(approx, np.float32(-np.inf))]
    for c in cands:
        dist = abs(Fraction(float(c)) - fr)
        key = (dist, int(np.array([c]).view(np.uint32)[0]) & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def _ulp_distance(a: np.float32, b: np.float32) -> int:
    ia = int(np.array([a], np.float32).view(np.int32)[0])
    ib = int(np.array([b], np.float32).view(np.int32)[0])
    ia = ia if ia >= 0 else -(ia & 0x7FFFFFFF)
    ib = ib if ib >= 0 else -(ib & 0x7FFFFFFF)
    return abs(ia - ib)


@pytest.mark.parametrize("fmt,m,k,n", [(0, 3, 32, 2), (0, 4, 64, 3), (1, 2, 256, 2), (1, 3, 256, 1), (2, 3, 64, 2),
                                       (3, 2, 256, 2), (4, 3, 64, 2)])
def test_brute_force_exact_rationals(orc, fmt, m, k, n):
    rng = np.random.default_rng(100 + m * k + n)
    w = (rng.standard_normal((m, k)) * 0.02).astype(np.float32)
    x = rng.standard_normal((n, k)).astype(np.float32)
    buf = orc.quantize(fmt, w)
    what = orc.dequantize(fmt, buf, m, k)
    y = orc.matvec(fmt, buf, m, k, x)
    exact_hits = 0
    for t in range(n):
        for i in range(m):
            fr = sum(Fraction(float(what[i, c])) * Fraction(float(x[t, c])) for c in range(k))
            ref = _round_to_f32(fr)
            dist = _ulp_distance(y[t, i], ref)
            assert dist <= 1, (t, i, y[t, i], ref)
            exact_hits += dist == 0
    assert exact_hits >= (m * n + 1) // 2


@pytest.mark.parametrize("fmt,m,k", [(0, 37, 320), (1, 19, 512), (0, 5, 2048), (2, 29, 416), (3, 13, 768),
                                     (4, 23, 320)])
def test_matches_numpy_float64(orc, fmt, m, k):
    w = synth.weights(21, m, k)
    x = synth.activations(22, 3, k)
    buf = orc.quantize(fmt, w)
    what = orc.dequantize(fmt, buf, m, k).astype(np.float64)
    y = orc.matvec(fmt, buf, m, k, x)
    ref = x.astype(np.float64) @ what.T
    assert np.allclose(y, ref.astype(np.float32), rtol=1e-6, atol=1e-9)
    # float64 result before rounding agrees closely
    v, ad = orc.matvec_one(fmt, buf, m, k, x, 2, m - 1)
    assert abs(v - ref[2, m - 1]) <= 1e-12 * ad


def test_closed_forms_q4_0(orc):
    m, k = 6, 96
    w = synth.weights(31, m, k)
    buf = orc.quantize(0, w)
    what = orc.dequantize(0, buf, m, k)
    # x = 1: row sums of the dequantized matrix (rows, not columns)
    y1 = orc.matvec(0, buf, m, k, np.ones((1, k), np.float32))[0]
    assert np.allclose(y1, what.astype(np.float64).sum(axis=1), rtol=1e-12, atol=0)
    assert not np.allclose(y1[:min(m, k)], what.astype(np.float64).sum(axis=0)[:min(m, k)])
    # one-hot x = e_j returns column j exactly
    for j in (0, 17, 31, 32, 95):
        e = np.zeros((1, k), np.float32)
        e[0, j] = 1.0
        assert np.array_equal(orc.matvec(0, buf, m, k, e)[0], what[:, j])
    # all codes 8 -> y = 0 exactly, whatever the scales and x
    allc8 = buf.copy()
    allc8[: m * k // 2] = 0x88
    x = synth.activations(32, 2, k)
    assert not orc.matvec(0, allc8, m, k, x).any()
    # scaling x by 2^k scales y exactly
    y = orc.matvec(0, buf, m, k, x)
    y8 = orc.matvec(0, buf, m, k, x * np.float32(8.0))
    assert np.array_equal(y8, y * np.float32(8.0))


def test_closed_forms_q4_k(orc):
    m, k = 3, 512
    w = synth.weights(41, m, k)
    buf = orc.quantize(1, w)
    what = orc.dequantize(1, buf, m, k)
    for j in (0, 33, 100, 255, 256, 511):
        e = np.zeros((1, k), np.float32)
        e[0, j] = 1.0
        assert np.array_equal(orc.matvec(1, buf, m, k, e)[0], what[:, j])
    # q = 0 everywhere and m = 0 everywhere -> y = 0
    z = buf.copy().reshape(-1, 144)
    z[:, 16:] = 0
    z[:, 4:16] = 0
    assert not orc.matvec(1, z.reshape(-1), m, k, synth.activations(42, 2, k)).any()


def test_closed_forms_q8_0(orc):
    m, k = 5, 128
    buf = orc.quantize(2, synth.weights(45, m, k))
    what = orc.dequantize(2, buf, m, k)
    # one-hot x = e_j returns column j exactly
    for j in (0, 31, 32, 127):
        e = np.zeros((1, k), np.float32)
        e[0, j] = 1.0
        assert np.array_equal(orc.matvec(2, buf, m, k, e)[0], what[:, j])
    # all codes 0 -> y = 0 exactly, whatever the scales and x
    z = buf.copy()
    z[: m * k] = 0
    assert not orc.matvec(2, z, m, k, synth.activations(46, 2, k)).any()
    # negating every code (two's complement) negates y exactly
    neg = buf.copy()
    neg[: m * k] = (-buf[: m * k].view(np.int8)).view(np.uint8)
    x = synth.activations(47, 2, k)
    assert np.array_equal(orc.matvec(2, neg, m, k, x), -orc.matvec(2, buf, m, k, x))


def test_closed_forms_q1_0(orc):
    m, k = 5, 128
    buf = orc.quantize(4, synth.weights(48, m, k))
    what = orc.dequantize(4, buf, m, k)
    nb = m * k // 32
    d = buf[m * k // 8:].view(np.float16).astype(np.float64).reshape(m, k // 32)
    # one-hot x = e_j returns column j exactly
    for j in (0, 31, 32, 127):
        e = np.zeros((1, k), np.float32)
        e[0, j] = 1.0
        assert np.array_equal(orc.matvec(4, buf, m, k, e)[0], what[:, j])
    # every bit set: y_i = sum over blocks of d_ib * (sum of the block's x)
    ones = buf.copy()
    ones[: nb * 4] = 0xFF
    x = synth.activations(49, 2, k)
    bsum = x.astype(np.float64).reshape(2, k // 32, 32).sum(axis=2)
    ref = (bsum[:, None, :] * d[None, :, :]).sum(axis=2)
    assert np.allclose(orc.matvec(4, ones, m, k, x), ref.astype(np.float32), rtol=1e-6, atol=1e-12)
    # flipping every bit negates y exactly
    flip = buf.copy()
    flip[: nb * 4] = ~buf[: nb * 4]
    assert np.array_equal(orc.matvec(4, flip, m, k, x), -orc.matvec(4, buf, m, k, x))


def test_threads_do_not_change_result(orc):
    m, k = 50, 256
    w = synth.weights(51, m, k)
    x = synth.activations(52, 2, k)
    buf = orc.quantize(0, w)
    assert np.array_equal(orc.matvec(0, buf, m, k, x, threads=1), orc.matvec(0, buf, m, k, x, threads=7))


def test_matmul_bf16(orc):
    torch = pytest.importorskip("torch")
    m, k, n = 9, 128, 5
    w = synth.weights(61, m, k)
    xb = synth.bf16_bits(synth.activations(62, n, k))
    buf = orc.quantize(0, w)
    what = orc.dequantize(0, buf, m, k)
    xf = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).double().numpy()
    y = orc.matmul(0, buf, m, k, xb)
    assert np.allclose(y, (xf @ what.astype(np.float64).T).astype(np.float32), rtol=1e-6, atol=1e-9)
    # bf16-rounded weights: against torch's bf16 cast of the dequantized matrix
    wb = torch.from_numpy(what).to(torch.bfloat16).double().numpy()
    yb = orc.matmul(0, buf, m, k, xb, round_w_bf16=True)
    assert np.allclose(yb, (xf @ wb.T).astype(np.float32), rtol=1e-6, atol=1e-9)
    # identity X gives bf16(W_hat)^T exactly
    eye = synth.bf16_bits(np.eye(k, dtype=np.float32))
    yi = orc.matmul(0, buf, m, k, eye, round_w_bf16=True)
    assert np.array_equal(yi, wb.T.astype(np.float32))
    yi = orc.matmul(0, buf, m, k, eye)
    assert np.array_equal(yi, what.T)


def test_termscale(orc):
    # Q4_0: the value is one term, so the scale is sum |w_hat x|.
    m, k = 7, 256
    w = synth.weights(71, m, k)
    x = synth.activations(72, 2, k)
    b0 = orc.quantize(0, w)
    _, ad0 = orc.matvec(0, b0, m, k, x, absdot=True)
    assert np.allclose(orc.termscale(0, b0, m, k, x), ad0, rtol=1e-12)
    # Q4_K: at least sum |w_hat x|, equal when every min is zero, and by hand
    # on K-A with one activation: |d*sc*q| + |dmin*m| for sub-block 7, q=15:
    # 945 + 24 = 969.
    b1 = orc.quantize(1, w)
    _, ad1 = orc.matvec(1, b1, m, k, x, absdot=True)
    ts = orc.termscale(1, b1, m, k, x)
    assert np.all(ts >= ad1 * (1 - 1e-12))
    z = b1.copy().reshape(-1, 144)
    z[:, 2:4] = 0  # dmin = 0
    _, adz = orc.matvec(1, z.reshape(-1), m, k, x, absdot=True)
    assert np.allclose(orc.termscale(1, z.reshape(-1), m, k, x), adz, rtol=1e-12)
    S = orc.q4_k_pack_scales([1, 2, 3, 4, 5, 6, 7, 63], [0, 1, 2, 3, 4, 5, 6, 48])
    sb = np.zeros(144, np.uint8)
    sb[0:2] = [0x00, 0x3C]
    sb[2:4] = [0x00, 0x38]
    sb[4:16] = S
    sb[16 + 32 * 3 + 32 - 32 + 0] |= 0xF0  # weight 224 = 64*3 + 32 + 0: high nibble of chunk 3 byte 0 -> sub-block 7
    e = np.zeros((1, 256), np.float32)
    e[0, 224] = 1.0
    assert orc.termscale(1, sb, 1, 256, e)[0, 0] == 969.0
    assert orc.matvec(1, sb, 1, 256, e)[0, 0] == 921.0
    # Q2_K: likewise at least sum |w_hat x|; by hand on a one-code super-block
    # (d = 1, dmin = 0.5, sub-block 12 with sc 12, m 3, element 200 with q 3):
    # |12*3| + |0.5*3| = 37.5 against the value 34.5.
    b3 = orc.quantize(3, w)
    _, ad3 = orc.matvec(3, b3, m, k, x, absdot=True)
    assert np.all(orc.termscale(3, b3, m, k, x) >= ad3 * (1 - 1e-12))
    hb = np.zeros(84, np.uint8)
    hb[40] = 0x30
    hb[64 + 12] = 12 | (3 << 4)
    hb[80:84] = [0x00, 0x3C, 0x00, 0x38]
    e = np.zeros((1, 256), np.float32)
    e[0, 200] = 1.0
    assert orc.termscale(3, hb, 1, 256, e)[0, 0] == 37.5
    assert orc.matvec(3, hb, 1, 256, e)[0, 0] == 34.5


# ---- gated product (gate and up rows of one stacked matrix, silu(g) * u) ----

@pytest.mark.parametrize("fmt,m,k,n", [(0, 6, 64, 2), (1, 3, 256, 2)])
def test_silu_mul_against_library_sigmoid(orc, fmt, m, k, n):
    # Reduces to the pinned products plus a library sigmoid: y = g * expit(g) * u
    # with g the gate row (first m rows) and u the up row (rows m..2m-1), each
    # the exact rational sum rounded once; swapping gate and up, dropping the
    # factor g, or reading the wrong half of the matrix fails here.
    from scipy.special import expit

    rng = np.random.default_rng(300 + m + k)
    w = (rng.standard_normal((2 * m, k)) * 0.05).astype(np.float32)
    x = rng.standard_normal((n, k)).astype(np.float32)
    buf = orc.quantize(fmt, w)
    what = orc.dequantize(fmt, buf, 2 * m, k).astype(np.float64)
    y, g, u = orc.matvec_silu_mul(fmt, buf, m, k, x, parts=True)
    for t in range(n):
        for i in range(m):
            gf = sum(Fraction(float(what[i, c])) * Fraction(float(x[t, c])) for c in range(k))
            uf = sum(Fraction(float(what[m + i, c])) * Fraction(float(x[t, c])) for c in range(k))
            assert abs(g[t, i] - float(gf)) <= 1e-12 * (abs(float(gf)) + 1e-30) + 1e-300
            assert abs(u[t, i] - float(uf)) <= 1e-12 * (abs(float(uf)) + 1e-30) + 1e-300
            ref = np.float32(float(gf) * expit(float(gf)) * float(uf))
            assert _ulp_distance(y[t, i], ref) <= 1, (t, i, y[t, i], ref)
    # The halves matter: silu(g) * u differs from silu(u) * g here.
    swapped = np.float32(u * expit(u) * g)
    assert not np.allclose(y, swapped, rtol=1e-3)


def test_silu_mul_closed_forms(orc):
    # Weights 7 * 2^j quantize exactly (d = 2^j, code 15 or 1), so the row
    # products below are exact small integers.
    k = 64
    x = np.ones((1, k), np.float32)
    # Gate rows of all-zero weights: g = 0, so y = 0 exactly, whatever u is.
    w = np.zeros((4, k), np.float32)
    w[2:] = 0.4375
    buf = orc.quantize(0, w)
    y, g, u = orc.matvec_silu_mul(0, buf, 2, k, x, parts=True)
    assert np.all(g == 0.0) and np.all(u == 28.0) and np.all(y == 0.0)
    # silu(g) -> g for large g: g = 7 * 64 = 448, exp(-448) is far below fp32
    # resolution, so y = fp32(448 * u).
    w = np.zeros((2, k), np.float32)
    w[0] = 7.0
    w[1] = 0.875
    buf = orc.quantize(0, w)
    y, g, u = orc.matvec_silu_mul(0, buf, 1, k, x, parts=True)
    assert g[0, 0] == 448.0 and u[0, 0] == 56.0 and y[0, 0] == np.float32(448.0 * 56.0)
    # silu(g) -> 0 for very negative g: -448 * e^-448 * 56 underflows fp32.
    w[0] = -7.0
    buf = orc.quantize(0, w)
    y = orc.matvec_silu_mul(0, buf, 1, k, x)
    assert y[0, 0] == 0.0
    # silu(g) - silu(-g) = g, for the same up row.
    w = np.zeros((4, k), np.float32)
    w[0] = 0.21875
    w[1] = -0.21875
    w[2:] = 0.875
    buf = orc.quantize(0, w)
    y, g, u = orc.matvec_silu_mul(0, buf, 2, k, x, parts=True)
    assert g[0, 0] == 14.0 and g[0, 1] == -14.0 and np.all(u == 56.0)
    assert abs((float(y[0, 0]) - float(y[0, 1])) / 56.0 - 14.0) < 1e-5
