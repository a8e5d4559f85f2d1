"""Pins for the oracle's binary16 / bfloat16 conversions.

Both are written in the oracle from the IEEE-754 definitions; here they are
checked against library casts (numpy's float16, torch's bfloat16) and against
hand-built ties and overflow boundaries.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def test_fp16_to_fp32_exhaustive(orc):
    L = orc.lib()
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float32)
    got = np.array([L.oracle_fp16_to_fp32(int(b)) for b in bits], dtype=np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_fp16_roundtrip_exhaustive(orc):
    L = orc.lib()
    for b in range(65536):
        if (b & 0x7C00) == 0x7C00 and (b & 0x3FF):
            continue  # NaN payloads are not preserved
        f = L.oracle_fp16_to_fp32(b)
        assert L.oracle_fp32_to_fp16(f) == b, hex(b)


def test_fp32_to_fp16_matches_numpy_random(orc):
    L = orc.lib()
    rng = np.random.default_rng(11)
    # Random bit patterns over the whole binary32 range plus values near the
    # binary16 range, where rounding happens.
    u = rng.integers(0, 2**32, size=60000, dtype=np.uint64).astype(np.uint32)
    near = rng.uniform(-70000, 70000, size=60000).astype(np.float32)
    tiny = (rng.uniform(-1, 1, size=30000) * 2.0**-13).astype(np.float32)
    vals = np.concatenate([u.view(np.float32), near, tiny])
    vals = vals[~np.isnan(vals)]
    ref = vals.astype(np.float16).view(np.uint16)
    got = np.array([L.oracle_fp32_to_fp16(float(v)) for v in vals], dtype=np.uint16)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(vals[i]), hex(got[i]), hex(ref[i])) for i in bad[:5]]


@pytest.mark.parametrize("value,bits", [
    (65504.0, 0x7BFF),            # largest finite
    (65519.99609375, 0x7BFF),     # just below the overflow midpoint
    (65520.0, 0x7C00),            # midpoint 65504/65536 rounds to even -> overflow
    (-65520.0, 0xFC00),
    (2.0**-24, 0x0001),           # smallest subnormal
    (2.0**-25, 0x0000),           # tie between 0 and 2^-24 -> even (0)
    (3 * 2.0**-25, 0x0002),       # tie between 1 and 2 ulps -> even (2)
    (2.0**-14, 0x0400),           # smallest normal
    (1.0 + 2.0**-11, 0x3C00),     # tie -> even mantissa 0
    (1.0 + 3 * 2.0**-11, 0x3C02), # tie -> even mantissa 2
    (-0.0, 0x8000),
])
def test_fp16_boundaries(orc, value, bits):
    assert orc.fp32_to_fp16(value) == bits
    assert orc.f64_to_fp16(value) == bits


def test_f64_to_fp16_matches_numpy(orc):
    L = orc.lib()
    rng = np.random.default_rng(5)
    v = np.concatenate([rng.standard_normal(40000) * 10.0 ** rng.uniform(-8, 5, 40000)])
    ref = v.astype(np.float16).view(np.uint16)
    got = np.array([L.oracle_f64_to_fp16(float(x)) for x in v], dtype=np.uint16)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("in_bits,out_bits", [
    (0x3F808000, 0x3F80),  # exact tie, even neighbour below
    (0x3F818000, 0x3F82),  # exact tie, even neighbour above
    (0x3F808001, 0x3F81),  # just above the tie
    (0x3F807FFF, 0x3F80),  # just below the tie
    (0x7F7FFFFF, 0x7F80),  # largest float rounds to +inf
    (0x00008000, 0x0000),  # subnormal tie -> even (0)
    (0x00018000, 0x0002),  # subnormal tie -> even (2)
    (0x80000000, 0x8000),
])
def test_bf16_ties(orc, in_bits, out_bits):
    f = float(np.array([in_bits], dtype=np.uint32).view(np.float32)[0])
    assert orc.fp32_to_bf16(f) == out_bits


def test_bf16_matches_torch(orc):
    torch = pytest.importorskip("torch")
    L = orc.lib()
    rng = np.random.default_rng(3)
    u = rng.integers(0, 2**32, size=50000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    u = u[np.isfinite(u)]
    n = rng.standard_normal(20000).astype(np.float32)
    vals = np.concatenate([u, n])
    ref = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([L.oracle_fp32_to_bf16(float(v)) for v in vals], dtype=np.uint16)
    assert np.array_equal(got, ref)
    back = np.array([L.oracle_bf16_to_fp32(int(b)) for b in got[:2000]], dtype=np.float32)
    assert np.array_equal(back, torch.from_numpy(got[:2000].view(np.int16)).view(torch.bfloat16).float().numpy())
