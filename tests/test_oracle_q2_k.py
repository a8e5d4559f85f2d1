"""Pins for the oracle's Q2_K quantizer, dequantizer and buffer layout.

A hand-worked super-block lives in tests/golden/q2_k_superblocks.txt; a
hand-built buffer pins the code bit positions, the sub-block indexing and the
plane order; the invariants follow from the definition (value d*sc*q - dmin*m
with 4-bit sc, m and 2-bit q) without re-running it.
"""
import numpy as np
import pytest

import synth
from golden import floats, hexbytes, load

G = load("q2_k_superblocks.txt")


def test_golden_superblock(orc):
    sec = G["K2-B"]
    w = floats(sec["w"][0]).reshape(1, 256)
    buf = orc.quantize(orc.Q2_K, w)
    assert buf.size == 84
    assert bytes(buf[:64]) == hexbytes(sec["codes"][0])
    assert bytes(buf[64:80]) == hexbytes(sec["scales"][0])
    assert bytes(buf[80:84]) == hexbytes(sec["dd"][0])
    deq = orc.dequantize(orc.Q2_K, buf, 1, 256)[0]
    assert np.array_equal(deq, np.tile(floats(sec["dequant_cycle"][0]), 64))


def _hand_buffer():
    # d = 1.0, dmin = 0.5; sub-block j has sc = j and m = 15 - j; every code 0
    # except: byte 40 bits 4-5 = 3 (h = 1, r = 8, j = 2: element 200),
    # byte 5 bits 6-7 = 3 (h = 0, r = 5, j = 3: element 101),
    # byte 37 bits 0-1 = 2 (h = 1, r = 5, j = 0: element 133).
    codes = np.zeros(64, np.uint8)
    codes[40] = 0x30
    codes[5] = 0xC0
    codes[37] = 0x02
    scales = np.array([j | ((15 - j) << 4) for j in range(16)], np.uint8)
    dd = np.array([0x00, 0x3C, 0x00, 0x38], np.uint8)
    return np.concatenate([codes, scales, dd])


def test_hand_built_layout(orc):
    deq = orc.dequantize(orc.Q2_K, _hand_buffer(), 1, 256)[0]
    # Element 200: sub-block 12 (sc 12, m 3): 12*3 - 0.5*3 = 34.5.
    # Element 101: sub-block 6 (sc 6, m 9): 6*3 - 4.5 = 13.5.
    # Element 133: sub-block 8 (sc 8, m 7): 8*2 - 3.5 = 12.5.
    # Every other element has q = 0: -0.5 * (15 - e/16).
    exp = np.array([-0.5 * (15 - e // 16) for e in range(256)], np.float32)
    exp[200], exp[101], exp[133] = 34.5, 13.5, 12.5
    assert np.array_equal(deq, exp)
    assert deq[255] == 0.0 and not np.signbit(deq[255])


def test_plane_layout_two_rows(orc):
    # m = 2, k = 512: code plane (4 super-blocks x 64 B), scale plane (4 x 16 B),
    # then d/dmin (4 x 4 B), each in row-major super-block order.
    w = synth.weights(5, 2, 512)
    w[1, 256:] = floats(G["K2-B"]["w"][0])
    buf = orc.quantize(orc.Q2_K, w)
    assert buf.size == 4 * 84
    assert bytes(buf[3 * 64:4 * 64]) == hexbytes(G["K2-B"]["codes"][0])
    assert bytes(buf[256 + 3 * 16:256 + 4 * 16]) == hexbytes(G["K2-B"]["scales"][0])
    assert bytes(buf[320 + 3 * 4:320 + 4 * 4]) == hexbytes(G["K2-B"]["dd"][0])
    # The same super-block alone quantizes to the same fields.
    one = orc.quantize(orc.Q2_K, w[:1, :256])
    assert bytes(buf[:64]) == bytes(one[:64]) and bytes(buf[256:272]) == bytes(one[64:80])
    assert bytes(buf[320:324]) == bytes(one[80:84])


def test_invariants_random_superblocks(orc):
    rng = np.random.default_rng(12)
    n = 300
    w = (rng.standard_normal((n, 256)) * np.exp(rng.uniform(-4, 4, (n, 1))) + rng.uniform(-1, 1, (n, 1))
         * np.exp(rng.uniform(-4, 4, (n, 1)))).astype(np.float32)
    buf = orc.quantize(orc.Q2_K, w)
    deq = orc.dequantize(orc.Q2_K, buf, n, 256)
    codes = buf[: n * 64].reshape(n, 64)
    scm = buf[n * 64: n * 80].reshape(n, 16)
    dd = buf[n * 80:].view(np.float16).astype(np.float64).reshape(n, 2)
    sc, mn = (scm & 15).astype(np.float64), (scm >> 4).astype(np.float64)
    e = np.arange(256)
    q = (codes[:, 32 * (e // 128) + e % 32] >> (2 * ((e % 128) // 32))) & 3
    j = e // 16
    step = dd[:, :1] * sc[:, j]
    off = dd[:, 1:] * mn[:, j]
    # (i) every value is d*sc*q - dmin*m, rounded once to fp32
    assert np.array_equal(deq, (step * q - off).astype(np.float32))
    # (ii) the error stays within half a step plus the rounding of the step and
    # offset to their 4-bit grids (a misplaced code would be a whole step off)
    lo = np.minimum(0, w.reshape(n, 16, 16).min(axis=2))[:, j]
    hi = w.reshape(n, 16, 16).max(axis=2)[:, j]
    s = (hi - lo) / 3
    bound = step / 2 + 3 * np.abs(s - step) + np.abs(-lo - off) + 1e-6 * np.abs(w)
    assert np.all(np.abs(w - deq) <= bound)
    # (iii) all-nonnegative sub-blocks: mu = 0 everywhere gives dmin = 0, m = 0
    pos = np.abs(w[:4])
    bpos = orc.quantize(orc.Q2_K, pos)
    assert not np.any(bpos[4 * 64: 4 * 80] >> 4) and not np.any(bpos[4 * 80:].view(np.uint16)[1::2])


def test_size_is_2p625_bits_per_weight(orc):
    assert orc.weight_bytes(orc.Q2_K, 4096, 4096) * 8 == 4096 * 4096 * 2.625


def test_errors(orc):
    with pytest.raises(orc.OracleError):
        orc.quantize(orc.Q2_K, np.full((1, 256), np.inf, np.float32))
    with pytest.raises(orc.OracleError):
        orc.quantize(orc.Q2_K, np.full((1, 256), -6e37, np.float32))  # dmin overflows fp16
