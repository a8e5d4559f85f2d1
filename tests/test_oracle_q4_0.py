"""Pins for the oracle's Q4_0 quantizer, dequantizer and buffer layout.

Hand-worked blocks live in tests/golden/q4_0_blocks.txt; the invariants below
follow from the definition (d = fp16(max|w|/7), q = round(w/d) + 8 clamped,
value (q - 8) d) without re-running it.
"""
import numpy as np
import pytest

from golden import floats, load

G = load("q4_0_blocks.txt")


@pytest.mark.parametrize("name", sorted(G))
def test_golden_block(orc, name):
    sec = G[name]
    w = floats(sec["w"][0])
    assert w.shape == (32,)
    nib, d = orc.quantize_q4_0_block(w)
    assert d == int(sec["d_bits"][0], 16)
    assert bytes(nib).hex() == sec["nibbles"][0]
    # Dequantize through the matrix API (m=1, k=32): plane-split buffer.
    buf = orc.quantize(orc.Q4_0, w.reshape(1, 32))
    assert bytes(buf[:16]).hex() == sec["nibbles"][0]
    assert int(buf[16]) | (int(buf[17]) << 8) == d
    deq = orc.dequantize(orc.Q4_0, buf, 1, 32)[0]
    assert np.array_equal(deq, floats(sec["dequant"][0]))


def test_code_zero_is_legal_input(orc):
    # Q0-E: a block built by hand with d = 1.0 and byte 0 = 0x80:
    # element 0 has code 0 -> -8, element 16 has code 8 -> 0.
    buf = np.array([0x80] + [0x88] * 15 + [0x00, 0x3C], dtype=np.uint8)
    deq = orc.dequantize(orc.Q4_0, buf, 1, 32)[0]
    assert deq[0] == -8.0 and deq[16] == 0.0 and np.all(deq[1:16] == 0)


def test_plane_layout_multi_block(orc):
    # Pins where each block's nibbles and scale land for m=2, k=64:
    # nibble plane = blocks in row-major order, then the scale plane in the same order.
    blocks = [floats(G[n]["w"][0]) for n in ("Q0-A", "Q0-B", "Q0-D", "Q0-F")]
    w = np.stack([np.concatenate(blocks[0:2]), np.concatenate(blocks[2:4])])
    buf = orc.quantize(orc.Q4_0, w)
    assert buf.size == 2 * 64 * 9 // 16
    names = ("Q0-A", "Q0-B", "Q0-D", "Q0-F")
    for i, n in enumerate(names):
        assert bytes(buf[16 * i:16 * i + 16]).hex() == G[n]["nibbles"][0]
        s = 64 + 2 * i
        assert int(buf[s]) | (int(buf[s + 1]) << 8) == int(G[n]["d_bits"][0], 16)
    deq = orc.dequantize(orc.Q4_0, buf, 2, 64)
    assert np.array_equal(deq[1, 32:], floats(G["Q0-F"]["dequant"][0]))


def test_aos_plane_bijection(orc):
    rng = np.random.default_rng(0)
    m, k = 7, 96
    buf = rng.integers(0, 256, size=m * k * 9 // 16, dtype=np.uint8)
    aos = orc.q4_0_planes_to_aos(buf, m, k)
    assert np.array_equal(orc.q4_0_aos_to_planes(aos, m, k), buf)
    # AoS block i = 2 scale bytes then its 16 nibble bytes.
    i = 5
    assert bytes(aos[18 * i:18 * i + 2]) == bytes(buf[m * k // 2 + 2 * i:m * k // 2 + 2 * i + 2])
    assert bytes(aos[18 * i + 2:18 * i + 18]) == bytes(buf[16 * i:16 * i + 16])


def _random_blocks(n, seed):
    rng = np.random.default_rng(seed)
    scales = 10.0 ** rng.uniform(-3, 3, size=(n, 1))
    return (rng.standard_normal((n, 32)) * scales).astype(np.float32)


def test_invariants_random_blocks(orc):
    w = _random_blocks(4000, 1)
    buf = orc.quantize(orc.Q4_0, w.reshape(1, -1))
    deq = orc.dequantize(orc.Q4_0, buf, 1, w.size).reshape(-1, 32)
    nb = w.shape[0]
    nib = buf[: nb * 16].reshape(nb, 16)
    codes = np.concatenate([nib & 15, nib >> 4], axis=1).astype(np.int32)
    d = buf[nb * 16:].view(np.uint16).view(np.float16).astype(np.float32)
    normal = d >= 2.0**-14
    assert normal.all()
    # (i) error at most half a step
    assert np.all(np.abs(w.astype(np.float64) - deq) <= d[:, None].astype(np.float64) / 2 * (1 + 1e-12))
    # (iii) codes in 1..15 for a normal scale
    assert codes.min() >= 1 and codes.max() <= 15
    # the largest-magnitude element maps to code 1 or 15
    amax_idx = np.argmax(np.abs(w), axis=1)
    c = codes[np.arange(nb), amax_idx]
    assert np.all((c == 1) | (c == 15))
    # (ii) quantize(dequantize(B)) == B
    buf2 = orc.quantize(orc.Q4_0, deq.reshape(1, -1))
    assert np.array_equal(buf2, buf)
    # scale is the fp16 rounding of max|w| / 7 (binary32 division)
    d_ref = (np.abs(w).max(axis=1) / np.float32(7)).astype(np.float32).astype(np.float16)
    assert np.array_equal(d_ref.view(np.uint16), buf[nb * 16:].view(np.uint16))


def test_size_is_4p5_bits_per_weight(orc):
    # GPT-2-124M matrices: 123,532,032 weights -> 69,486,768 bytes (falls within
    # the 50-84 MB the MicroLLM post gives for its 100M+ models).
    import synth
    total = sum(orc.weight_bytes(orc.Q4_0, m, k) for k, m in synth.gpt2_124m_step())
    assert total == 69_486_768
    assert 50e6 <= total <= 84e6


def test_errors(orc):
    w = np.zeros((1, 32), np.float32)
    w[0, 3] = np.nan
    with pytest.raises(orc.OracleError) as e:
        orc.quantize(orc.Q4_0, w)
    assert e.value.status == orc.ENONFINITE
    w[0, 3] = np.inf
    with pytest.raises(orc.OracleError):
        orc.quantize(orc.Q4_0, w)
    # max|w|/7 >= 65520 overflows the fp16 scale; 458632/7 = 65518.86 rounds to 65504.
    w = np.zeros((1, 32), np.float32)
    w[0, 0] = 458632.0
    buf = orc.quantize(orc.Q4_0, w)
    assert int(buf[16]) | (int(buf[17]) << 8) == 0x7BFF
    w[0, 0] = 458648.0
    with pytest.raises(orc.OracleError) as e:
        orc.quantize(orc.Q4_0, w)
    assert e.value.status == orc.ERANGE


def test_subnormal_scale_only_bytes_defined(orc):
    # A block whose scale is an fp16 subnormal still quantizes and dequantizes
    # within half a step (precision of d itself is then coarse).
    w = (np.linspace(-1, 1, 32) * 1e-5).astype(np.float32)
    buf = orc.quantize(orc.Q4_0, w.reshape(1, 32))
    d = float(buf[16:18].view(np.uint16).view(np.float16)[0])
    assert 0 < d < 2.0**-14
    deq = orc.dequantize(orc.Q4_0, buf, 1, 32)[0]
    q = np.concatenate([buf[:16] & 15, buf[:16] >> 4]).astype(np.int32)
    assert np.array_equal(deq, ((q - 8) * np.float32(d)).astype(np.float32))
