"""CPU tests of the product library: exports, the host quantizer against the
oracle (two independent implementations, byte-identical output), and every
error status of the device entry points (validation precedes any HIP call,
so no GPU is needed)."""
import ctypes
import os
import re

import numpy as np
import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def q4():
    import q4_weight_gemv_amd as q4

    return q4


def _declared_functions():
    names = set()
    for h in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if h.endswith(".h"):
            text = open(os.path.join(ROOT, "include", h)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(q4_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_library_exports_every_declared_symbol(q4):
    declared = _declared_functions()
    assert set(declared) >= {"q4_weight_bytes", "q4_quantize_ref", "q4_gemv", "q4_gemm", "q4_strerror",
                             "q4_read_probe"}
    lib = ctypes.CDLL(q4.LIB_PATH)
    for name in declared:
        assert hasattr(lib, name), name
    assert set(declared) == set(q4.EXPORTS)


def test_weight_bytes(q4):
    assert q4.q4_weight_bytes(0, 768, 768) == 331_776
    assert q4.q4_weight_bytes(1, 4096, 11008) == 25_362_432
    assert q4.q4_weight_bytes(0, 4096, 11008) == 25_362_432
    assert q4.q4_weight_bytes(0, 3, 33) == 0
    assert q4.q4_weight_bytes(1, 3, 512 + 32) == 0
    assert q4.q4_weight_bytes(0, -1, 32) == 0
    assert q4.q4_weight_bytes(7, 1, 32) == 0
    assert q4.q4_weight_bytes(0, 0, 32) == 0
    total = sum(q4.q4_weight_bytes(0, m, k) for k, m in synth.gpt2_124m_step())
    assert total == 69_486_768
    total = sum(q4.q4_weight_bytes(0, m, k) for k, m in synth.smollm2_360m_step())
    assert total == 203_489_280
    total = sum(q4.q4_weight_bytes(1, m, k) for k, m in synth.llama7b_layer())
    assert total == 85_524_480
    # Q8_0: 34 bytes per 32 weights, k a multiple of 32.
    assert q4.q4_weight_bytes(2, 4096, 4096) == 4096 * 4096 * 34 // 32
    assert q4.q4_weight_bytes(2, 3, 33) == 0
    assert q4.q4_weight_bytes(2, 5, 96) == 5 * 3 * 34
    # Q2_K: 84 bytes per 256 weights, k a multiple of 256.
    assert q4.q4_weight_bytes(3, 4096, 11008) == 4096 * 43 * 84
    assert q4.q4_weight_bytes(3, 3, 288) == 0
    # Q1_0: 6 bytes per 32 weights (a code word and a scale), k a multiple of 32.
    assert q4.q4_weight_bytes(4, 4096, 11008) == 4096 * 11008 * 3 // 16
    assert q4.q4_weight_bytes(4, 3, 48) == 0
    assert q4.q4_weight_bytes(4, 5, 96) == 5 * 3 * 6


SHAPES = sorted(set(synth.gpt2_124m_step() + synth.smollm2_360m_step() + synth.llama7b_layer()))


@pytest.mark.parametrize("k,m", [s for s in SHAPES if s[1] * s[0] <= 12_000_000])
def test_quantize_ref_matches_oracle_q4_0(q4, orc, k, m):
    w = synth.weights(synth.seed_for(9, k % 97 + m % 89), m, k)
    assert np.array_equal(q4.q4_quantize_ref(0, w), orc.quantize(0, w))


@pytest.mark.parametrize("k,m", [(4096, 512), (11008, 128), (768, 64)])
def test_quantize_ref_matches_oracle_q4_k(q4, orc, k, m):
    if k % 256:
        k = 1024
    w = synth.weights(synth.seed_for(8, k % 97 + m % 89), m, k)
    assert np.array_equal(q4.q4_quantize_ref(1, w), orc.quantize(1, w))


@pytest.mark.parametrize("k,m", [(768, 768), (960, 320), (4096, 512), (11008, 96)])
def test_quantize_ref_matches_oracle_q8_0(q4, orc, k, m):
    w = synth.weights(synth.seed_for(7, k % 97 + m % 89), m, k)
    assert np.array_equal(q4.q4_quantize_ref(2, w), orc.quantize(2, w))


@pytest.mark.parametrize("k,m", [(768, 768), (1024, 320), (4096, 512), (11008, 96)])
def test_quantize_ref_matches_oracle_q2_k(q4, orc, k, m):
    w = synth.weights(synth.seed_for(6, k % 97 + m % 89), m, k)
    assert np.array_equal(q4.q4_quantize_ref(3, w), orc.quantize(3, w))


@pytest.mark.parametrize("k,m", [(768, 768), (960, 320), (4096, 512), (11008, 96)])
def test_quantize_ref_matches_oracle_q1_0(q4, orc, k, m):
    w = synth.weights(synth.seed_for(5, k % 97 + m % 89), m, k)
    assert np.array_equal(q4.q4_quantize_ref(4, w), orc.quantize(4, w))


def _edge_matrix(k):
    """Rows that exercise ties, subnormal scales, clamps, zeros and sign patterns."""
    rng = np.random.default_rng(17)
    rows = []
    d = np.float32(0.0078125)
    rows.append((rng.integers(-16, 17, size=k) * d / 2).astype(np.float32))   # many exact ties
    rows.append((rng.standard_normal(k) * 1e-6).astype(np.float32))          # subnormal fp16 scales
    rows.append(np.zeros(k, np.float32))
    rows.append(np.full(k, -3.0, np.float32))
    rows.append(np.full(k, 5.0, np.float32))
    r = rng.standard_normal(k).astype(np.float32)
    r[::7] *= 1000
    rows.append(r)
    rows.append((rng.standard_normal(k) * 60000).astype(np.float32))
    rows.append(np.abs(rng.standard_normal(k)).astype(np.float32))              # all positive (Q4_K min 0)
    rows.append(-np.abs(rng.standard_normal(k)).astype(np.float32) - 0.5)       # all negative
    return np.stack(rows)


@pytest.mark.parametrize("fmt", [0, 1, 2, 3, 4])
def test_quantize_ref_matches_oracle_edges(q4, orc, fmt):
    w = _edge_matrix(512)
    w[2, ::3] = -0.0  # signed zeros (the Q1_0 sign rule)
    assert np.array_equal(q4.q4_quantize_ref(fmt, w), orc.quantize(fmt, w))
    # Golden blocks through the product quantizer too.
    if fmt == 4:
        from golden import floats, hexbytes, load
        for name, sec in load("q1_0_blocks.txt").items():
            buf = q4.q4_quantize_ref(4, floats(sec["w"][0]).reshape(1, 32))
            assert bytes(buf[:4]) == hexbytes(sec["codes"][0]), name
            assert int(buf[4]) | (int(buf[5]) << 8) == int(sec["d_bits"][0], 16), name
    elif fmt == 3:
        from golden import floats, hexbytes, load
        sec = load("q2_k_superblocks.txt")["K2-B"]
        buf = q4.q4_quantize_ref(3, floats(sec["w"][0]).reshape(1, 256))
        assert bytes(buf) == hexbytes(sec["codes"][0]) + hexbytes(sec["scales"][0]) + hexbytes(sec["dd"][0])
    elif fmt == 2:
        from golden import floats, hexbytes, load
        for name, sec in load("q8_0_blocks.txt").items():
            buf = q4.q4_quantize_ref(2, floats(sec["w"][0]).reshape(1, 32))
            assert bytes(buf[:32]) == hexbytes(sec["codes"][0]), name
            assert int(buf[32]) | (int(buf[33]) << 8) == int(sec["d_bits"][0], 16), name
    elif fmt == 0:
        from golden import floats, load
        for name, sec in load("q4_0_blocks.txt").items():
            buf = q4.q4_quantize_ref(0, floats(sec["w"][0]).reshape(1, 32))
            assert bytes(buf[:16]).hex() == sec["nibbles"][0], name
    else:
        from golden import floats, hexbytes, load
        sec = load("q4_k_superblocks.txt")["K-B"]
        assert bytes(q4.q4_quantize_ref(1, floats(sec["w"][0]).reshape(1, 256))) == hexbytes(sec["bytes"][0])


def test_quantize_ref_status(q4, orc):
    w = synth.weights(3, 64, 256)
    w2 = w.copy()
    w2[40, 200] = np.nan
    w2[50, 3] = 1e9  # scale overflow in a later row: the first failing block decides
    with pytest.raises(q4.Q4Error) as e:
        q4.q4_quantize_ref(0, w2)
    assert e.value.status == q4.Q4_ENONFINITE
    with pytest.raises(orc.OracleError) as eo:
        orc.quantize(0, w2)
    assert eo.value.status == e.value.status
    w3 = w.copy()
    w3[10, 0] = 1e9
    w3[11, 0] = np.inf
    for fmt in (0, 1, 2, 3, 4):
        with pytest.raises(q4.Q4Error) as e:
            q4.q4_quantize_ref(fmt, w3)
        assert e.value.status == q4.Q4_ERANGE
    lib = q4.raw()
    out = np.zeros(16, np.uint8)
    assert lib.q4_quantize_ref(0, w.ctypes.data, 64, 255, out.ctypes.data, 16) == q4.Q4_EINVAL
    assert lib.q4_quantize_ref(0, w.ctypes.data, 64, 256, out.ctypes.data, 16) == q4.Q4_EINVAL  # short buffer
    assert lib.q4_quantize_ref(0, None, 64, 256, out.ctypes.data, 1 << 20) == q4.Q4_EINVAL
    assert lib.q4_quantize_ref(5, w.ctypes.data, 64, 256, out.ctypes.data, 1 << 20) == q4.Q4_EUNSUPPORTED
    assert lib.q4_quantize_ref(0, w.ctypes.data, 0, 256, out.ctypes.data, 0) == q4.Q4_OK


def test_quantize_ref_many_threads_same_bytes(q4, orc):
    # Large enough that the product quantizer splits rows across threads.
    w = synth.weights(77, 2048, 1024)
    assert np.array_equal(q4.q4_quantize_ref(0, w), orc.quantize(0, w))
    w[1500, 17] = np.nan
    w[100, 900] = 1e9
    with pytest.raises(q4.Q4Error) as e:
        q4.q4_quantize_ref(0, w)
    assert e.value.status == q4.Q4_ERANGE  # row 100 precedes row 1500


A16 = 1 << 20  # fake, 16-byte aligned addresses: validation rejects before any HIP call


@pytest.mark.parametrize("entry", ["q4_gemv", "q4_gemm"])
def test_product_argument_errors(q4, entry):
    f = getattr(q4.raw(), entry)
    ok = (A16, A16 * 2, A16 * 3)
    assert f(9, *ok, 64, 256, 1, None) == q4.Q4_EUNSUPPORTED          # unknown format
    assert f(0, *ok, 64, 48, 1, None) == q4.Q4_EINVAL                 # k not a multiple of 32
    assert f(1, *ok, 64, 288, 1, None) == q4.Q4_EINVAL                # k not a multiple of 256
    assert f(0, *ok, 64, 0, 1, None) == q4.Q4_EINVAL
    assert f(0, *ok, -1, 256, 1, None) == q4.Q4_EINVAL
    assert f(0, *ok, 64, 256, -1, None) == q4.Q4_EINVAL
    assert f(0, None, A16, A16, 64, 256, 1, None) == q4.Q4_EINVAL     # null pointers
    assert f(0, A16, None, A16, 64, 256, 1, None) == q4.Q4_EINVAL
    assert f(0, A16, A16, None, 64, 256, 1, None) == q4.Q4_EINVAL
    assert f(0, A16 + 2, A16, A16, 64, 256, 1, None) == q4.Q4_EALIGN  # misaligned w
    assert f(0, A16 + 8, A16, A16, 64, 256, 1, None) == q4.Q4_EALIGN  # w must be 16-byte aligned
    assert f(0, A16, A16 + 2, A16, 64, 256, 1, None) == q4.Q4_EALIGN  # misaligned x
    assert f(0, A16, A16, A16 + 2, 64, 256, 1, None) == q4.Q4_EALIGN  # misaligned y
    # A 4-byte-aligned x passes validation: the call reaches the HIP runtime,
    # which on a host without a GPU reports an error.
    assert f(0, A16, A16 + 4, A16, 64, 256, 1, None) == q4.Q4_EHIP
    assert f(0, None, None, None, 0, 256, 1, None) == q4.Q4_OK        # m == 0: no-op
    assert f(0, None, None, None, 64, 256, 0, None) == q4.Q4_OK       # n == 0: no-op
    assert f(0, *ok, 1 << 30, 1 << 10, 1, None) == q4.Q4_EUNSUPPORTED  # beyond 32-bit offsets
    assert f(0, *ok, 1 << 20, 4096, 1, None) == q4.Q4_EUNSUPPORTED    # weights of 2 GiB or more
    assert f(1, *ok, 1 << 20, 4096, 1, None) == q4.Q4_EUNSUPPORTED
    assert f(2, *ok, 64, 48, 1, None) == q4.Q4_EINVAL                 # Q8_0: k a multiple of 32
    assert f(2, *ok, 1 << 19, 4096, 1, None) == q4.Q4_EUNSUPPORTED    # Q8_0 weights of 2 GiB or more
    assert f(3, *ok, 64, 288, 1, None) == q4.Q4_EINVAL                # Q2_K: k a multiple of 256
    if entry == "q4_gemv":
        assert f(0, *ok, 64, 256, 9, None) == q4.Q4_EUNSUPPORTED       # decode batch is 1..8


def test_tuned_argument_errors(q4):
    f = q4.raw().q4_gemv_tuned
    ok = (A16, A16 * 2, A16 * 3)
    good = q4.q4_gemv_tuning(0, 0, 0, 0)
    assert f(0, *ok, 64, 256, 1, None, None) == q4.Q4_EINVAL
    assert f(0, *ok, 64, 256, 1, ctypes.byref(q4.q4_gemv_tuning(-1, 0, 0, 0)), None) == q4.Q4_EINVAL
    assert f(0, *ok, 64, 256, 1, ctypes.byref(q4.q4_gemv_tuning(0, 0, 0, 65)), None) == q4.Q4_EINVAL
    assert f(0, *ok, 64, 48, 1, ctypes.byref(good), None) == q4.Q4_EINVAL
    assert f(0, *ok, 64, 256, 9, ctypes.byref(good), None) == q4.Q4_EUNSUPPORTED
    assert f(0, A16 + 4, A16, A16, 64, 256, 1, ctypes.byref(good), None) == q4.Q4_EALIGN
    assert f(0, A16, A16 + 6, A16, 64, 256, 1, ctypes.byref(good), None) == q4.Q4_EALIGN
    assert f(0, None, None, None, 0, 256, 1, ctypes.byref(good), None) == q4.Q4_OK
    # kernel and depth fields: negative or unknown values are refused, and the
    # streaming kernel takes one token only.
    for t in (q4.q4_gemv_tuning(0, 0, 0, 0, -1, 0), q4.q4_gemv_tuning(0, 0, 0, 0, 4, 0),
              q4.q4_gemv_tuning(0, 0, 0, 0, 2, -1)):
        assert f(0, *ok, 64, 256, 1, ctypes.byref(t), None) == q4.Q4_EINVAL
    stream = q4.q4_gemv_tuning(0, 0, 0, 0, q4.Q4_GEMV_KERNEL_STREAM, 0)
    assert f(0, *ok, 64, 256, 2, ctypes.byref(stream), None) == q4.Q4_EUNSUPPORTED
    assert f(0, None, None, None, 0, 256, 1, ctypes.byref(stream), None) == q4.Q4_OK
    # The matrix-core kernel: Q4_K only, and groups_per_cu its only geometry field.
    matrix = q4.q4_gemv_tuning(0, 0, 0, 0, q4.Q4_GEMV_KERNEL_MATRIX, 0)
    assert f(0, *ok, 64, 256, 4, ctypes.byref(matrix), None) == q4.Q4_EUNSUPPORTED
    for t in (q4.q4_gemv_tuning(32, 0, 0, 0, q4.Q4_GEMV_KERNEL_MATRIX, 0),
              q4.q4_gemv_tuning(0, 2, 0, 0, q4.Q4_GEMV_KERNEL_MATRIX, 0),
              q4.q4_gemv_tuning(0, 0, 8, 0, q4.Q4_GEMV_KERNEL_MATRIX, 0),
              q4.q4_gemv_tuning(0, 0, 0, 0, q4.Q4_GEMV_KERNEL_MATRIX, 2)):
        assert f(1, *ok, 64, 256, 4, ctypes.byref(t), None) == q4.Q4_EUNSUPPORTED
    assert f(1, None, None, None, 0, 256, 4, ctypes.byref(matrix), None) == q4.Q4_OK
    assert f(1, None, None, None, 0, 256, 4,
             ctypes.byref(q4.q4_gemv_tuning(0, 0, 0, 2, q4.Q4_GEMV_KERNEL_MATRIX, 0)), None) == q4.Q4_OK


def test_gemm_tuned_argument_errors(q4):
    f = q4.raw().q4_gemm_tuned
    ok = (A16, A16 * 2, A16 * 3)
    assert f(0, *ok, 64, 256, 4, None, None) == q4.Q4_EINVAL
    assert f(0, *ok, 64, 256, 4, ctypes.byref(q4.q4_gemm_tuning(-1, 0, 0)), None) == q4.Q4_EINVAL
    assert f(0, *ok, 64, 48, 4, ctypes.byref(q4.q4_gemm_tuning(0, 0, 0)), None) == q4.Q4_EINVAL
    assert f(0, A16, A16 + 2, A16, 64, 256, 4, ctypes.byref(q4.q4_gemm_tuning(0, 0, 0)), None) == q4.Q4_EALIGN
    assert f(0, A16 + 4, A16, A16, 64, 256, 4, ctypes.byref(q4.q4_gemm_tuning(0, 0, 0)), None) == q4.Q4_EALIGN
    assert f(0, None, None, None, 0, 256, 4, ctypes.byref(q4.q4_gemm_tuning(0, 0, 0)), None) == q4.Q4_OK


def test_sequence_and_graph_argument_errors(q4):
    lib = q4.raw()
    ops = (q4.q4_gemv_op * 2)()
    ops[0] = q4.q4_gemv_op(A16, A16, A16, 64, 256)
    ops[1] = q4.q4_gemv_op(A16, A16 + 2, A16, 64, 256)  # misaligned x in the second op
    assert lib.q4_gemv_sequence(0, ops, 2, 1, None) == q4.Q4_EALIGN
    assert lib.q4_gemv_sequence(0, None, 2, 1, None) == q4.Q4_EINVAL
    assert lib.q4_gemv_sequence(0, ops, -1, 1, None) == q4.Q4_EINVAL
    assert lib.q4_gemv_sequence(0, ops, 1, 9, None) == q4.Q4_EUNSUPPORTED
    assert lib.q4_gemv_sequence(0, ops, 0, 1, None) == q4.Q4_OK
    h = ctypes.c_void_p(None)
    assert lib.q4_graph_create(0, ops, 2, 1, None, ctypes.byref(h)) == q4.Q4_EALIGN
    assert h.value is None
    assert lib.q4_graph_create(0, ops, 1, 1, None, None) == q4.Q4_EINVAL
    assert lib.q4_graph_launch(None, None) == q4.Q4_EINVAL
    assert lib.q4_graph_destroy(None) == q4.Q4_OK


def test_gated_product_argument_errors(q4):
    f = q4.raw().q4_gemv_glu
    ok = (A16, A16 * 2, A16 * 3)
    assert f(0, *ok, -1, 256, 1, None) == q4.Q4_EINVAL
    assert f(0, *ok, 64, 48, 1, None) == q4.Q4_EINVAL              # k not a multiple of 32
    assert f(1, *ok, 64, 288, 1, None) == q4.Q4_EINVAL             # Q4_K: k not a multiple of 256
    assert f(0, *ok, 64, 256, 9, None) == q4.Q4_EUNSUPPORTED       # tokens beyond 8
    assert f(9, *ok, 64, 256, 1, None) == q4.Q4_EUNSUPPORTED       # unknown format
    assert f(0, *ok, 1 << 29, 256, 1, None) == q4.Q4_EUNSUPPORTED  # 2m rows beyond the offset range
    assert f(0, A16 + 8, A16, A16, 64, 256, 1, None) == q4.Q4_EALIGN
    assert f(0, None, A16, A16, 64, 256, 1, None) == q4.Q4_EINVAL
    assert f(0, None, None, None, 0, 256, 1, None) == q4.Q4_OK      # m = 0: no-op
    # The weights of a gated product have 2m rows: a matrix of 2^31 bytes or
    # more is refused even when m rows alone would fit.
    m = (1 << 30) // (4096 * 9 // 16) + 1
    assert q4.q4_weight_bytes(0, m, 4096) < (1 << 31) <= q4.q4_weight_bytes(0, 2 * m, 4096)
    assert f(0, *ok, m, 4096, 1, None) == q4.Q4_EUNSUPPORTED


def test_addnorm_argument_errors(q4):
    f = q4.raw().q4_gemv_addnorm
    W, X, D, G, XO, Y = (A16 * i for i in range(1, 7))  # disjoint fake buffers
    assert f(0, W, X, D, None, 1e-5, XO, Y, 64, 256, 0, None) == q4.Q4_EINVAL       # no gain
    assert f(0, W, X, D, G + 4, 1e-5, XO, Y, 64, 256, 0, None) == q4.Q4_EALIGN     # misaligned gain
    assert f(0, W, X, D + 8, G, 1e-5, XO, Y, 64, 256, 0, None) == q4.Q4_EALIGN     # misaligned delta
    assert f(0, W, X, D, G, 1e-5, XO + 4, Y, 64, 256, 0, None) == q4.Q4_EALIGN     # misaligned x_out
    assert f(0, W, X + 2, D, G, 1e-5, XO, Y, 64, 256, 0, None) == q4.Q4_EALIGN     # misaligned x
    assert f(0, W, X, D, G, 1e-5, X, Y, 64, 256, 0, None) == q4.Q4_EINVAL          # x_out is x
    assert f(0, W, X, D, G, 1e-5, X + 512, Y, 64, 256, 0, None) == q4.Q4_EINVAL    # x_out overlaps x
    assert f(0, W, X, D, G, 1e-5, D - 16, Y, 64, 256, 0, None) == q4.Q4_EINVAL     # x_out overlaps delta
    assert f(0, W, X, D, G, 1e-5, Y + 64, Y, 64, 256, 0, None) == q4.Q4_EINVAL     # x_out overlaps y
    for eps in (-1e-6, float("inf"), float("nan")):
        assert f(0, W, X, D, G, eps, XO, Y, 64, 256, 0, None) == q4.Q4_EINVAL
    assert f(0, W, X, D, G, 1e-5, XO, Y, 64, 256, 7, None) == q4.Q4_EINVAL          # unknown epilogue
    assert f(9, W, X, D, G, 1e-5, XO, Y, 64, 256, 0, None) == q4.Q4_EUNSUPPORTED    # unknown format
    assert f(0, W, X, D, G, 1e-5, XO, Y, 64, 48, 0, None) == q4.Q4_EINVAL           # k not whole blocks
    assert f(1, W, X, D, G, 1e-5, XO, Y, 64, 288, 0, None) == q4.Q4_EINVAL          # Q4_K: k % 256
    assert f(0, W, X, D, G, 1e-5, XO, Y, 64, 14592, 0, None) == q4.Q4_EUNSUPPORTED  # row beyond LDS
    assert f(0, W, X, D, G, 1e-5, XO, Y, 1 << 29, 256, 1, None) == q4.Q4_EUNSUPPORTED  # 2m rows
    assert f(0, None, X, D, G, 1e-5, XO, Y, 64, 256, 0, None) == q4.Q4_EINVAL
    assert f(0, None, None, None, None, 1e-5, None, None, 0, 256, 0, None) == q4.Q4_OK  # m = 0: no-op


def test_addnorm_tuned_argument_errors(q4):
    f = q4.raw().q4_gemv_addnorm_tuned
    W, X, D, G, XO, Y = (A16 * i for i in range(1, 7))
    bad = q4.q4_gemv_tuning(-1, 0, 0, 0)
    assert f(0, W, X, D, G, 1e-5, XO, Y, 64, 256, 0, None, None) == q4.Q4_EINVAL          # no tuning
    assert f(0, W, X, D, G, 1e-5, XO, Y, 64, 256, 0, ctypes.byref(bad), None) == q4.Q4_EINVAL
    big = q4.q4_gemv_tuning(0, 0, 0, 65)
    assert f(0, W, X, D, G, 1e-5, XO, Y, 64, 256, 0, ctypes.byref(big), None) == q4.Q4_EINVAL
    ok = q4.q4_gemv_tuning(0, 0, 0, 0)
    assert f(0, W, X, D, None, 1e-5, XO, Y, 64, 256, 0, ctypes.byref(ok), None) == q4.Q4_EINVAL  # no gain
    assert f(0, W, X, D, G, 1e-5, X, Y, 64, 256, 0, ctypes.byref(ok), None) == q4.Q4_EINVAL     # x_out is x
    assert f(0, W, X, D, G, 1e-5, XO, Y, 64, 14592, 0, ctypes.byref(ok), None) == q4.Q4_EUNSUPPORTED
    assert f(0, None, None, None, None, 1e-5, None, None, 0, 256, 0, ctypes.byref(ok), None) == q4.Q4_OK
    stream = q4.q4_gemv_tuning(0, 0, 0, 0, q4.Q4_GEMV_KERNEL_STREAM, 0)  # the fused norm is tiled only
    assert f(0, W, X, D, G, 1e-5, XO, Y, 64, 256, 0, ctypes.byref(stream), None) == q4.Q4_EUNSUPPORTED
    matrix = q4.q4_gemv_tuning(0, 0, 0, 0, q4.Q4_GEMV_KERNEL_MATRIX, 0)
    assert f(1, W, X, D, G, 1e-5, XO, Y, 64, 256, 0, ctypes.byref(matrix), None) == q4.Q4_EUNSUPPORTED
    unknown = q4.q4_gemv_tuning(0, 0, 0, 0, 5, 0)
    assert f(0, W, X, D, G, 1e-5, XO, Y, 64, 256, 0, ctypes.byref(unknown), None) == q4.Q4_EINVAL


def test_sequence_epilogue_field(q4):
    lib = q4.raw()
    ops = (q4.q4_gemv_op * 1)()
    ops[0] = q4.q4_gemv_op(A16, A16, A16, 64, 256, 7)  # unknown epilogue
    assert lib.q4_gemv_sequence(0, ops, 1, 1, None) == q4.Q4_EINVAL
    ops[0] = q4.q4_gemv_op(A16, A16 + 2, A16, 64, 256, q4.Q4_EPILOGUE_SILU_MUL)
    assert lib.q4_gemv_sequence(0, ops, 1, 1, None) == q4.Q4_EALIGN
    ops[0] = q4.q4_gemv_op(A16, A16, A16, 1 << 29, 256, q4.Q4_EPILOGUE_SILU_MUL)
    assert lib.q4_gemv_sequence(0, ops, 1, 1, None) == q4.Q4_EUNSUPPORTED


def test_llama_step_argument_errors(q4):
    lib = q4.raw()
    cfg = q4.q4_llama_config(2, 128, 4, 2, 32, 256, 384, 16, 1e4, 1e-5)
    layers = (q4.q4_llama_layer * 2)()
    for i in range(2):
        layers[i] = q4.q4_llama_layer(A16, A16, A16, A16, A16, A16)
    st = q4.q4_llama_state(*([A16] * 11))
    f = lib.q4_llama_step
    ok = lambda c=cfg, s=st: f(0, ctypes.byref(c), A16, A16, layers, ctypes.byref(s), None)  # noqa: E731
    assert f(0, None, A16, A16, layers, ctypes.byref(st), None) == q4.Q4_EINVAL
    assert f(0, ctypes.byref(cfg), None, A16, layers, ctypes.byref(st), None) == q4.Q4_EINVAL
    assert f(9, ctypes.byref(cfg), A16, A16, layers, ctypes.byref(st), None) == q4.Q4_EUNSUPPORTED
    bad = q4.q4_llama_config(2, 128, 4, 3, 32, 256, 384, 16, 1e4, 1e-5)       # heads % kv_heads
    assert ok(bad) == q4.Q4_EINVAL
    bad = q4.q4_llama_config(2, 128, 4, 2, 48, 256, 384, 16, 1e4, 1e-5)       # head_dim not 32, 64, 128
    assert ok(bad) == q4.Q4_EUNSUPPORTED
    bad = q4.q4_llama_config(2, 128, 4, 2, 32, 256, 384, 9000, 1e4, 1e-5)     # cache beyond the LDS scores
    assert ok(bad) == q4.Q4_EUNSUPPORTED
    bad = q4.q4_llama_config(2, 100, 4, 2, 32, 256, 384, 16, 1e4, 1e-5)       # hidden not whole blocks
    assert ok(bad) == q4.Q4_EINVAL
    bad = q4.q4_llama_config(2, 128, 4, 2, 32, 256, 384, 16, -1.0, 1e-5)      # theta
    assert ok(bad) == q4.Q4_EINVAL
    st2 = q4.q4_llama_state(*([A16] * 10 + [None]))                            # no position buffer
    assert ok(cfg, st2) == q4.Q4_EINVAL
    st3 = q4.q4_llama_state(*([A16] + [A16 + 4] + [A16] * 9))                  # misaligned h (a product input)
    assert ok(cfg, st3) == q4.Q4_EALIGN
    st4 = q4.q4_llama_state(*([A16] * 7 + [A16 + 8] + [A16] * 3))              # misaligned key cache
    assert ok(cfg, st4) == q4.Q4_EALIGN
    # The allocation-free step validates the same way before any HIP call; its
    # state's workspace pointers are ignored (null here), and a model whose
    # intermediate vectors exceed its 65536-float array is refused.
    g = lib.q4_llama_step_noalloc
    st0 = q4.q4_llama_state(*([A16] * 2 + [None] * 4 + [A16] * 5))
    ok0 = lambda c=cfg, s=st0: g(0, ctypes.byref(c), A16, A16, layers, ctypes.byref(s), None)  # noqa: E731
    assert g(0, None, A16, A16, layers, ctypes.byref(st0), None) == q4.Q4_EINVAL
    assert g(0, ctypes.byref(cfg), A16, A16, layers, None, None) == q4.Q4_EINVAL
    assert g(9, ctypes.byref(cfg), A16, A16, layers, ctypes.byref(st0), None) == q4.Q4_EUNSUPPORTED
    for c, code in ((q4.q4_llama_config(2, 128, 4, 3, 32, 256, 384, 16, 1e4, 1e-5), q4.Q4_EINVAL),
                    (q4.q4_llama_config(2, 128, 4, 2, 48, 256, 384, 16, 1e4, 1e-5), q4.Q4_EUNSUPPORTED),
                    (q4.q4_llama_config(2, 100, 4, 2, 32, 256, 384, 16, 1e4, 1e-5), q4.Q4_EINVAL)):
        assert ok0(c) == code
    st5 = q4.q4_llama_state(*([A16] * 10 + [None]))                            # no position buffer
    assert ok0(cfg, st5) == q4.Q4_EINVAL
    st6 = q4.q4_llama_state(*([A16] * 7 + [A16 + 8] + [A16] * 3))              # misaligned key cache
    assert ok0(cfg, st6) == q4.Q4_EALIGN
    # Distinct buffers pass every other check; an ffn of 65536 floats alone
    # exceeds the array (a fitting model would go on to the device lookup).
    a = lambda i: A16 + (i << 16)  # noqa: E731
    lay = (q4.q4_llama_layer * 2)()
    for i in range(2):
        lay[i] = q4.q4_llama_layer(a(1), a(2), a(3), a(4), a(5), a(6))
    sd = q4.q4_llama_state(a(10), a(11), None, None, None, None, a(16), a(17), a(18), a(19), a(20))
    for ffn in (65536, 131072):
        big = q4.q4_llama_config(2, 128, 4, 2, 32, ffn, 384, 16, 1e4, 1e-5)
        assert g(0, ctypes.byref(big), a(30), a(31), lay, ctypes.byref(sd), None) == q4.Q4_EUNSUPPORTED
    h = ctypes.c_void_p(None)
    assert lib.q4_llama_graph_create(0, None, A16, A16, layers, ctypes.byref(st), None, ctypes.byref(h)) == q4.Q4_EINVAL
    assert h.value is None
    assert lib.q4_llama_graph_launch(None, None) == q4.Q4_EINVAL
    assert lib.q4_llama_graph_destroy(None) == q4.Q4_OK


def test_strerror(q4):
    for st in (0, -1, -2, -3, -4, -5, -6):
        assert q4.q4_strerror(st) and q4.q4_strerror(st) != "unknown status"
    assert q4.q4_strerror(-99) == "unknown status"


def test_geometry_lists_match_header(q4):
    """The binding's geometry lists are the ones the header documents."""
    import re

    text = open(os.path.join(ROOT, "include", "q4.h")).read()
    tiled_doc = text[text.index("Q4_GEMV_KERNEL_TILED: workgroups"):text.index("Q4_GEMV_KERNEL_STREAM: one token")]
    stream_doc = text[text.index("Q4_GEMV_KERNEL_STREAM: one token"):text.index("With kernel Q4_GEMV_KERNEL_AUTO")]
    gemm_doc = text[text.index("/* Tile geometry of the prefill product"):text.index("int tile_rows;")]
    triples = lambda t: tuple(tuple(int(v) for v in m) for m in re.findall(r"\((\d+),(\d+),(\d+)\)", t))
    assert triples(tiled_doc) == q4.GEMV_GEOMETRIES
    assert triples(stream_doc) == q4.GEMV_STREAM_GEOMETRIES
    assert triples(gemm_doc) == q4.GEMM_TILES
    src = open(os.path.join(ROOT, "q4_weight_gemv_amd", "csrc", "q4_gemv_stream.hip")).read()
    listed = tuple(tuple(int(v) for v in m) for m in re.findall(r"X\((\d+), (\d+), (\d+)\)", src))
    assert listed == q4.GEMV_STREAM_GEOMETRIES


def test_binding_loads_torch_runtime_first():
    """The binding imports torch before loading the library, so the library's
    HIP runtime is torch's (same soname; the first copy loaded wins)."""
    import subprocess
    import sys

    code = ("import q4_weight_gemv_amd as q4, sys; "
            "maps = open('/proc/self/maps').read(); "
            "hip = sorted({l.split()[-1] for l in maps.splitlines() if 'libamdhip64' in l}); "
            "print(hip); assert len(hip) == 1 and '/torch/lib/' in hip[0], hip; "
            "assert q4.raw().q4_last_hip_error() == b'hipSuccess'")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr


def test_read_probe_argument_errors(q4):
    f = q4.raw().q4_read_probe
    assert f(None, 1 << 20, A16, 64, None) == q4.Q4_EINVAL
    assert f(A16, 0, A16, 64, None) == q4.Q4_EINVAL
    assert f(A16, 1 << 20, A16, 0, None) == q4.Q4_EINVAL
    assert f(A16, 1 << 20, A16 + 2, 64, None) == q4.Q4_EALIGN  # sink not 4-byte aligned (NULL is allowed)
    assert f(A16, 1 << 20, A16, 65537, None) == q4.Q4_EINVAL
    assert f(A16 + 8, 1 << 20, A16, 64, None) == q4.Q4_EALIGN
    assert f(A16, (1 << 20) + 8, A16, 64, None) == q4.Q4_EALIGN
