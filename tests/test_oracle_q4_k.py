"""Pins for the oracle's Q4_K super-block format (stretch format).

Hand-worked super-blocks live in tests/golden/q4_k_superblocks.txt.
"""
import itertools

import numpy as np
import pytest

from golden import floats, hexbytes, load

G = load("q4_k_superblocks.txt")


def _sb_with(d_bits, dmin_bits, S, qs):
    """Build one 144-byte super-block by hand from its fields (q per weight)."""
    out = np.zeros(144, np.uint8)
    out[0], out[1] = d_bits & 0xFF, d_bits >> 8
    out[2], out[3] = dmin_bits & 0xFF, dmin_bits >> 8
    out[4:16] = np.frombuffer(S, np.uint8)
    for c in range(4):
        for i in range(32):
            out[16 + 32 * c + i] = qs[64 * c + i] | (qs[64 * c + 32 + i] << 4)
    return out


def test_golden_ka_scales_and_values(orc):
    sec = G["K-A"]
    sc = [int(v) for v in sec["sc"][0].split()]
    mn = [int(v) for v in sec["m"][0].split()]
    S = hexbytes(sec["S"][0])
    assert bytes(orc.q4_k_pack_scales(sc, mn)) == S
    usc, umn = orc.q4_k_unpack_scales(np.frombuffer(S, np.uint8))
    assert list(usc) == sc and list(umn) == mn
    for probe in sec["probe"]:
        j, q, val = probe.split()
        j, q, val = int(j), int(q), float(val)
        qs = [0] * 256
        for i in range(32):
            qs[32 * j + i] = q
        sb = _sb_with(int(sec["d_bits"][0], 16), int(sec["dmin_bits"][0], 16), S, qs)
        deq = orc.dequantize(orc.Q4_K, sb, 1, 256)[0]
        assert np.all(deq[32 * j:32 * j + 32] == np.float32(val)), (j, q, deq[32 * j])


def test_golden_kb_quantize(orc):
    sec = G["K-B"]
    w = floats(sec["w"][0])
    assert w.shape == (256,)
    buf = orc.quantize(orc.Q4_K, w.reshape(1, 256))
    assert bytes(buf) == hexbytes(sec["bytes"][0])
    deq = orc.dequantize(orc.Q4_K, buf, 1, 256)[0]
    assert np.array_equal(deq, floats(sec["dequant"][0]))


def test_superblock_placement(orc):
    # K-B placed as super-block (row 1, column 1) of a 2 x 512 matrix of zeros.
    w = np.zeros((2, 512), np.float32)
    w[1, 256:] = floats(G["K-B"]["w"][0])
    buf = orc.quantize(orc.Q4_K, w)
    assert buf.size == 4 * 144
    assert bytes(buf[3 * 144:]) == hexbytes(G["K-B"]["bytes"][0])
    assert not buf[:3 * 144].any()


def test_pack_unpack_bijection_each_field(orc):
    # Exhaustive per field: every value 0..63 in every slot, others random.
    rng = np.random.default_rng(2)
    for slot, v in itertools.product(range(16), range(64)):
        fields = rng.integers(0, 64, size=16)
        fields[slot] = v
        S = orc.q4_k_pack_scales(fields[:8], fields[8:])
        sc, mn = orc.q4_k_unpack_scales(S)
        assert list(sc) == list(fields[:8]) and list(mn) == list(fields[8:])


def test_pack_unpack_random_headers(orc):
    rng = np.random.default_rng(4)
    for _ in range(20000):
        S = rng.integers(0, 256, size=12, dtype=np.uint8)
        sc, mn = orc.q4_k_unpack_scales(S)
        assert bytes(orc.q4_k_pack_scales(sc, mn)) == bytes(S)


def test_grid_and_dmin_zero(orc):
    rng = np.random.default_rng(7)
    w = (rng.standard_normal((3, 512)) * 0.02).astype(np.float32)
    buf = orc.quantize(orc.Q4_K, w)
    deq = orc.dequantize(orc.Q4_K, buf, 3, 512)
    for r in range(3):
        for s in range(2):
            sb = buf[(r * 2 + s) * 144:(r * 2 + s + 1) * 144]
            d = float(sb[0:2].view(np.float16)[0])
            dmin = float(sb[2:4].view(np.float16)[0])
            sc, mn = orc.q4_k_unpack_scales(sb[4:16])
            for j in range(8):
                vals = deq[r, 256 * s + 32 * j:256 * s + 32 * j + 32]
                grid = {np.float32(np.float32(d * sc[j] * q) - np.float32(dmin * mn[j])) for q in range(16)}
                assert set(vals.tolist()) <= grid
    # Gaussian data: quantization error bounded by one step per sub-block.
    err = np.abs(deq - w)
    assert err.max() < 0.02 * 4 / 15 * 1.5
    # dmin = 0 reduces the format to (d * sc) * q.
    S = orc.q4_k_pack_scales([3] * 8, [5] * 8)
    qs = list(range(16)) * 16
    sb = _sb_with(0x3C00, 0x0000, bytes(S), qs)
    deq = orc.dequantize(orc.Q4_K, sb, 1, 256)[0]
    expect = np.zeros(256, np.float32)
    for c in range(4):
        for i in range(32):
            expect[64 * c + i] = 3 * qs[64 * c + i]
            expect[64 * c + 32 + i] = 3 * qs[64 * c + 32 + i]
    assert np.array_equal(deq, expect)


def test_quantizer_reconstruction_bound(orc):
    # Each weight lies within half a code step (d*sc/2) of its value, up to the
    # 6-bit rounding of the step and offset; checked against the stored fields.
    rng = np.random.default_rng(9)
    w = (rng.standard_normal((1, 256 * 64)) * 0.02).astype(np.float32)
    buf = orc.quantize(orc.Q4_K, w)
    deq = orc.dequantize(orc.Q4_K, buf, 1, w.shape[1])[0]
    for s in range(64):
        sb = buf[s * 144:(s + 1) * 144]
        d = float(sb[0:2].view(np.float16)[0])
        dmin = float(sb[2:4].view(np.float16)[0])
        sc, mn = orc.q4_k_unpack_scales(sb[4:16])
        for j in range(8):
            seg = slice(256 * s + 32 * j, 256 * s + 32 * j + 32)
            lo = -dmin * mn[j]
            hi = lo + 15 * d * sc[j]
            inside = (w[0, seg] >= lo) & (w[0, seg] <= hi)
            e = np.abs(deq[seg] - w[0, seg])
            assert np.all(e[inside] <= d * sc[j] / 2 * (1 + 1e-6) + 1e-12)


def test_errors(orc):
    w = np.zeros((1, 256), np.float32)
    w[0, 100] = np.nan
    with pytest.raises(orc.OracleError) as e:
        orc.quantize(orc.Q4_K, w)
    assert e.value.status == orc.ENONFINITE
    w[0, 100] = 3e9  # (hi - lo)/15/63 overflows fp16
    with pytest.raises(orc.OracleError) as e:
        orc.quantize(orc.Q4_K, w)
    assert e.value.status == orc.ERANGE
    with pytest.raises(orc.OracleError):
        orc.quantize(orc.Q4_K, np.zeros((1, 128), np.float32))
