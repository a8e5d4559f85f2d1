"""Pins for the oracle's Q8_0 quantizer, dequantizer and buffer layout.

Hand-worked blocks live in tests/golden/q8_0_blocks.txt; the invariants below
follow from the definition (d = fp16(max|w|/127), q = round(w/d) clamped to
[-127, 127], value q d) without re-running it.
"""
import numpy as np
import pytest

from golden import floats, hexbytes, load

G = load("q8_0_blocks.txt")


@pytest.mark.parametrize("name", sorted(G))
def test_golden_block(orc, name):
    sec = G[name]
    w = floats(sec["w"][0])
    assert w.shape == (32,)
    q, d = orc.quantize_q8_0_block(w)
    assert d == int(sec["d_bits"][0], 16)
    assert q.tobytes() == hexbytes(sec["codes"][0])
    # Through the matrix API (m=1, k=32): code plane, then the scale plane.
    buf = orc.quantize(orc.Q8_0, w.reshape(1, 32))
    assert buf.size == 34
    assert bytes(buf[:32]) == hexbytes(sec["codes"][0])
    assert int(buf[32]) | (int(buf[33]) << 8) == d
    deq = orc.dequantize(orc.Q8_0, buf, 1, 32)[0]
    assert np.array_equal(deq, floats(sec["dequant"][0]))


def test_plane_layout_multi_block(orc):
    # m=2, k=64: code plane = blocks in row-major order (32 bytes each), then
    # the scale plane in the same order.
    names = ("Q8-A", "Q8-B", "Q8-D", "Q8-E")
    blocks = [floats(G[n]["w"][0]) for n in names]
    w = np.stack([np.concatenate(blocks[0:2]), np.concatenate(blocks[2:4])])
    buf = orc.quantize(orc.Q8_0, w)
    assert buf.size == 2 * 64 * 17 // 16
    for i, n in enumerate(names):
        assert bytes(buf[32 * i:32 * i + 32]) == hexbytes(G[n]["codes"][0])
        s = 128 + 2 * i
        assert int(buf[s]) | (int(buf[s + 1]) << 8) == int(G[n]["d_bits"][0], 16)
    deq = orc.dequantize(orc.Q8_0, buf, 2, 64)
    assert np.array_equal(deq[1, :32], floats(G["Q8-D"]["dequant"][0]))
    assert np.array_equal(deq[1, 32:], floats(G["Q8-E"]["dequant"][0]))


def test_code_minus_128_is_legal_input(orc):
    # The quantizer emits -127..127, but the byte 0x80 (-128) dequantizes as
    # -128 d: a hand-built block with d = 0.5.
    buf = np.array([0x80] + [0x01] * 31 + [0x00, 0x38], dtype=np.uint8)
    deq = orc.dequantize(orc.Q8_0, buf, 1, 32)[0]
    assert deq[0] == -64.0 and np.all(deq[1:] == 0.5)


def test_invariants_random_blocks(orc):
    rng = np.random.default_rng(8)
    n = 4000
    w = (rng.standard_normal((n, 32)) * np.exp(rng.uniform(-8, 8, (n, 1)))).astype(np.float32)
    buf = orc.quantize(orc.Q8_0, w.reshape(n // 4, 128))
    deq = orc.dequantize(orc.Q8_0, buf, n // 4, 128).reshape(n, 32)
    codes = buf[: n * 32].view(np.int8).reshape(n, 32)
    d = buf[n * 32:].view(np.float16).astype(np.float32)
    amax = np.abs(w).max(axis=1)
    # (i) d is the fp16 rounding of max|w| / 127 (numpy's float16 cast as the library routine).
    assert np.array_equal(d, (amax / np.float32(127)).astype(np.float16).astype(np.float32))
    # (ii) codes within [-127, 127]; the largest magnitude reaches 126..127.
    assert codes.min() >= -127 and codes.max() <= 127
    assert np.all(np.abs(codes).max(axis=1) >= 126)
    # (iii) every value is q * d; for a normal d it lies within d/2 of its
    # weight (a subnormal d carries fewer bits, and the clamp can engage).
    assert np.array_equal(deq, codes.astype(np.float32) * d[:, None])
    normal = d >= 2.0 ** -14
    assert 0 < normal.sum() < n
    assert np.all(np.abs(w - deq)[normal] <= d[normal, None] / 2 * (1 + 1e-6))
    # (iv) for a normal d, quantizing the dequantized block gives the same
    # bytes (its largest code is +-127, so the scale comes back unchanged).
    cnt = int(normal.sum())
    again = orc.quantize(orc.Q8_0, deq[normal])
    assert np.array_equal(again[: cnt * 32].view(np.int8).reshape(cnt, 32), codes[normal])
    assert np.array_equal(again[cnt * 32:].view(np.float16).astype(np.float32), d[normal])


def test_size_is_8p5_bits_per_weight(orc):
    assert orc.weight_bytes(orc.Q8_0, 4096, 4096) * 8 == 4096 * 4096 * 8.5


def test_errors(orc):
    with pytest.raises(orc.OracleError):
        orc.quantize(orc.Q8_0, np.full((1, 32), np.nan, np.float32))
    with pytest.raises(orc.OracleError):
        orc.quantize(orc.Q8_0, np.full((1, 32), 3e38, np.float32))  # d = 2.4e36 overflows fp16
