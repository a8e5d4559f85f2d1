"""Pins for the oracle's Q1_0 quantizer, dequantizer and buffer layout.

Hand-worked blocks live in tests/golden/q1_0_blocks.txt; the invariants below
follow from the definition (d = fp16(mean |w|), b = [w >= 0], value
(2b - 1) d) without re-running it: every weight dequantizes to +-d with the
sign of w, d is the nearest fp16 to the mean magnitude (numpy's float16
conversion as an independent rounding), d minimises the squared error over
neighbouring fp16 scales, and quantizing a dequantized block is the identity.
"""
import numpy as np
import pytest

from golden import floats, hexbytes, load

G = load("q1_0_blocks.txt")


@pytest.mark.parametrize("name", sorted(G))
def test_golden_block(orc, name):
    sec = G[name]
    w = floats(sec["w"][0])
    assert w.shape == (32,)
    word, d = orc.quantize_q1_0_block(w)
    assert d == int(sec["d_bits"][0], 16)
    assert word.to_bytes(4, "little") == hexbytes(sec["codes"][0])
    # Through the matrix API (m=1, k=32): bit plane, then the scale plane.
    buf = orc.quantize(orc.Q1_0, w.reshape(1, 32))
    assert buf.size == 6
    assert bytes(buf[:4]) == hexbytes(sec["codes"][0])
    assert int(buf[4]) | (int(buf[5]) << 8) == d
    deq = orc.dequantize(orc.Q1_0, buf, 1, 32)[0]
    assert np.array_equal(deq, floats(sec["dequant"][0]))


def test_plane_layout_multi_block(orc):
    # m=2, k=64: bit plane = blocks in row-major order (4 bytes each), then
    # the scale plane in the same order.
    names = ("Q1-A", "Q1-B", "Q1-E", "Q1-F")
    blocks = [floats(G[n]["w"][0]) for n in names]
    w = np.stack([np.concatenate(blocks[0:2]), np.concatenate(blocks[2:4])])
    buf = orc.quantize(orc.Q1_0, w)
    assert buf.size == 2 * 64 * 3 // 16 == orc.weight_bytes(orc.Q1_0, 2, 64)
    for i, n in enumerate(names):
        assert bytes(buf[4 * i:4 * i + 4]) == hexbytes(G[n]["codes"][0])
        s = 16 + 2 * i
        assert int(buf[s]) | (int(buf[s + 1]) << 8) == int(G[n]["d_bits"][0], 16)
    deq = orc.dequantize(orc.Q1_0, buf, 2, 64)
    for i, n in enumerate(names):
        r, c = divmod(i, 2)
        assert np.array_equal(deq[r, 32 * c:32 * c + 32], floats(G[n]["dequant"][0]))


def test_errors(orc):
    for bad in (np.nan, np.inf, -np.inf):
        w = np.zeros(32, np.float32)
        w[7] = bad
        with pytest.raises(orc.OracleError) as e:
            orc.quantize_q1_0_block(w)
        assert e.value.status == orc.ENONFINITE
    # fp16's largest finite value is 65504; means from 65520 up round to inf.
    word, d = orc.quantize_q1_0_block(np.full(32, 65519.0, np.float32))
    assert d == 0x7BFF and word == 0xFFFFFFFF
    with pytest.raises(orc.OracleError) as e:
        orc.quantize_q1_0_block(np.full(32, -65520.0, np.float32))
    assert e.value.status == orc.ERANGE
    with pytest.raises(orc.OracleError) as e:
        orc.quantize(orc.Q1_0, np.zeros((2, 48), np.float32))  # k not a multiple of 32
    assert e.value.status == orc.EINVAL


def test_invariants_random_blocks(orc):
    rng = np.random.default_rng(11)
    n = 4000
    w = (rng.standard_normal((n, 32)) * np.exp(rng.uniform(-8, 8, (n, 1)))).astype(np.float32)
    w[::7, 3] = 0.0
    w[::11, 5] = -0.0
    buf = orc.quantize(orc.Q1_0, w.reshape(1, -1))
    deq = orc.dequantize(orc.Q1_0, buf, 1, 32 * n).reshape(n, 32)
    dh = buf[n * 4:].view(np.uint16)
    d = dh.view(np.float16).astype(np.float64)
    # Every weight is +-d with w's sign (zeros of either sign count as +).
    assert np.array_equal(np.abs(deq.astype(np.float64)), np.repeat(d[:, None], 32, 1))
    pos = ~np.signbit(w) | (w == 0)
    assert np.array_equal(deq >= 0, pos | (d[:, None] == 0))
    assert np.array_equal(np.signbit(deq), ~pos)
    # d is the nearest fp16 to the mean magnitude (numpy's conversion).
    mean = np.abs(w.astype(np.float64)).sum(axis=1) / 32.0
    assert np.array_equal(dh, mean.astype(np.float16).view(np.uint16))
    # Least squares among neighbouring fp16 scales, for the chosen signs.
    s = np.where(pos, 1.0, -1.0)
    err = lambda c: ((w - c[:, None] * s) ** 2).sum(axis=1)  # noqa: E731
    up = np.nextafter(d.astype(np.float16), np.float16(np.inf)).astype(np.float64)
    dn = np.nextafter(d.astype(np.float16), np.float16(0)).astype(np.float64)
    e0 = err(d)
    assert np.all(e0 <= err(up) * (1 + 1e-12)) and np.all(e0 <= err(dn) * (1 + 1e-12))
    # Quantizing a dequantized block returns the same bytes where d != 0 (a
    # zero scale dequantizes negative weights to -0, which re-quantize to 1).
    assert np.all(d > 0)
    buf2 = orc.quantize(orc.Q1_0, deq.reshape(1, -1))
    assert np.array_equal(buf, buf2)
