"""GPU parity of the fused residual add + RMSNorm decode product (q4_gemv_addnorm).

Reference: v = x + delta in float32 (the one rounding the kernel also makes),
h = rmsnorm(v) * gain in float64 (oracle.llama.rmsnorm), rounded to float32
as the oracle's products take it, then the oracle's product of h (or its
gated product). The updated residual x_out must equal v bit for bit; y is
held to the decode product's tolerance relative to the normalised input.
Shapes cover every one-token geometry the library picks for the four
formats (short and long rows, tall LM-head-like products, ragged tails) and
both epilogues.
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


def _inputs(seed, k, with_delta=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(k).astype(np.float32)
    delta = (0.5 * rng.standard_normal(k)).astype(np.float32) if with_delta else None
    gain = (1.0 + 0.25 * rng.standard_normal(k)).astype(np.float32)
    return x, delta, gain


def _normed(x, delta, gain, eps):
    from oracle import llama

    v = x + delta if delta is not None else x.copy()  # float32 add
    return v, llama.rmsnorm(v, gain, eps).astype(np.float32)


def _run(env, fmt, buf, x, delta, gain, eps, m, k, epilogue, want_out=True):
    torch, q4, _ = env
    dev = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    wd, xd, dd, gd = dev(buf), dev(x), dev(delta), dev(gain)
    xo = torch.full((k,), float("nan"), device="cuda") if want_out else None
    y = torch.full((m,), float("nan"), device="cuda")
    q4.q4_gemv_addnorm(fmt, wd, xd, dd, gd, eps, xo, y, m, k, epilogue)
    torch.cuda.synchronize()
    # The inputs are left as they were.
    assert np.array_equal(xd.cpu().numpy(), x)
    return y.cpu().numpy(), None if xo is None else xo.cpu().numpy()


# (fmt, m, k): one-token geometries of the plain product per format.
PLAIN = [
    (0, 37, 96), (0, 1600, 960), (0, 16500, 768), (0, 130, 2560), (0, 300, 4096), (0, 77, 14560),
    (1, 37, 256), (1, 300, 4096), (1, 9000, 4096), (1, 70, 8192), (1, 130, 1024),
    (2, 37, 320), (2, 130, 960), (2, 300, 4096), (2, 8200, 4096),
    (3, 130, 1024), (3, 300, 4096), (3, 70, 8192),
    (4, 37, 320), (4, 1600, 960), (4, 300, 4096), (4, 16500, 768),
]


@pytest.mark.parametrize("fmt,m,k", PLAIN)
def test_addnorm_parity(env, fmt, m, k):
    torch, q4, orc = env
    seed = synth.seed_for(3000 + fmt, m + k)
    buf = q4.q4_quantize_ref(fmt, synth.weights(seed, m, k))
    x, delta, gain = _inputs(seed + 1, k)
    eps = 1e-5
    say(f"addnorm fmt={fmt} m={m} k={k}")
    y, xo = _run(env, fmt, buf, x, delta, gain, eps, m, k, q4.Q4_EPILOGUE_NONE)
    v, h = _normed(x, delta, gain, eps)
    assert np.array_equal(xo, v), np.nonzero(xo != v)[0][:5]
    yr, ad = orc.matvec(fmt, buf, m, k, h, threads=threads(), absdot=True)
    check_tolerance(y[None, :], yr, ad, GEMV_TOL, what=f"addnorm fmt={fmt} {m}x{k}")


def test_addnorm_without_delta_or_output(env):
    # delta NULL: the input is rmsnorm(x) * gain and x_out = x; x_out NULL:
    # nothing written, same y.
    torch, q4, orc = env
    fmt, m, k = 0, 300, 960
    buf = q4.q4_quantize_ref(fmt, synth.weights(3101, m, k))
    x, _, gain = _inputs(3102, k, with_delta=False)
    say("addnorm no delta")
    y, xo = _run(env, fmt, buf, x, None, gain, 1e-5, m, k, q4.Q4_EPILOGUE_NONE)
    assert np.array_equal(xo, x)
    y2, _ = _run(env, fmt, buf, x, None, gain, 1e-5, m, k, q4.Q4_EPILOGUE_NONE, want_out=False)
    assert np.array_equal(y, y2)
    _, h = _normed(x, None, gain, 1e-5)
    yr, ad = orc.matvec(fmt, buf, m, k, h, threads=threads(), absdot=True)
    check_tolerance(y[None, :], yr, ad, GEMV_TOL, what="addnorm no delta")


def test_addnorm_scale_invariance(env):
    # rmsnorm(c v) = rmsnorm(v) for eps = 0: scaling x and delta by a power of
    # two (exact) leaves y unchanged bit for bit, since the kernel's staging
    # already removes a power of two per unit and the sum of squares scales
    # exactly.
    torch, q4, _ = env
    fmt, m, k = 0, 200, 768
    buf = q4.q4_quantize_ref(fmt, synth.weights(3201, m, k))
    x, delta, gain = _inputs(3202, k)
    say("addnorm scale invariance")
    y1, _ = _run(env, fmt, buf, x, delta, gain, 0.0, m, k, q4.Q4_EPILOGUE_NONE)
    y2, _ = _run(env, fmt, buf, x * 64, delta * 64, gain, 0.0, m, k, q4.Q4_EPILOGUE_NONE)
    assert np.array_equal(y1, y2)


# (fmt, m, k) for the gated epilogue: the gated geometries.
GLU = [(0, 37, 96), (0, 2560, 960), (0, 130, 2560), (0, 300, 4096), (1, 130, 1024), (1, 300, 4096),
       (2, 300, 4096), (3, 130, 1024), (3, 300, 4096), (4, 2560, 960), (4, 300, 4096)]


@pytest.mark.parametrize("fmt,m,k", GLU)
def test_addnorm_glu_parity(env, fmt, m, k):
    # Bound as for the gated product: |dg| <= tol A_g, |du| <= tol A_u, and
    # |silu'| <= 1.1 give 1.1 |u| tol A_g + |silu(g)| tol A_u + 1.1 tol^2 A_g A_u.
    torch, q4, orc = env
    seed = synth.seed_for(3300 + fmt, m + k)
    buf = q4.q4_quantize_ref(fmt, synth.weights(seed, 2 * m, k))
    x, delta, gain = _inputs(seed + 1, k)
    eps = 1e-5
    say(f"addnorm glu fmt={fmt} m={m} k={k}")
    y, xo = _run(env, fmt, buf, x, delta, gain, eps, m, k, q4.Q4_EPILOGUE_SILU_MUL)
    v, h = _normed(x, delta, gain, eps)
    assert np.array_equal(xo, v)
    yr, g, u = orc.matvec_silu_mul(fmt, buf, m, k, h[None, :], threads=threads(), parts=True)
    if fmt in (1, 3):
        ad = orc.termscale(fmt, buf, 2 * m, k, h[None, :], threads=threads())
    else:
        _, ad = orc.matvec(fmt, buf, 2 * m, k, h[None, :], threads=threads(), absdot=True)
    ag, au = ad[:, :m], ad[:, m:]
    silu = g / (1.0 + np.exp(-g))
    bound = (1.1 * np.abs(u) * GEMV_TOL * ag + np.abs(silu) * GEMV_TOL * au + 1.1 * GEMV_TOL ** 2 * ag * au
             + 4e-6 * np.abs(yr) + 1e-30)
    err = np.abs(y[None, :].astype(np.float64) - yr)
    assert np.all(np.isfinite(y))
    bad = np.argwhere(err > bound)
    assert bad.size == 0, (bad[:5], err[tuple(bad[0])], bound[tuple(bad[0])])
    assert np.linalg.norm(y - yr[0]) <= GEMV_TOL * np.linalg.norm(yr[0])


def test_addnorm_matches_unfused(env):
    # The fused launch against the two-step form: the plain product of the
    # float32 normalised input (rounded once more, so within the product's
    # tolerance rather than bit for bit).
    torch, q4, orc = env
    fmt, m, k = 0, 1600, 960
    buf = q4.q4_quantize_ref(fmt, synth.weights(3401, m, k))
    x, delta, gain = _inputs(3402, k)
    say("addnorm vs unfused")
    y, _ = _run(env, fmt, buf, x, delta, gain, 1e-5, m, k, q4.Q4_EPILOGUE_NONE)
    _, h = _normed(x, delta, gain, 1e-5)
    yd = torch.empty(1, m, device="cuda")
    q4.q4_gemv(fmt, torch.from_numpy(buf).cuda(), torch.from_numpy(h[None, :]).cuda(), yd, m, k)
    torch.cuda.synchronize()
    _, ad = orc.matvec(fmt, buf, m, k, h, threads=threads(), absdot=True)
    check_tolerance(y[None, :], yd.cpu().numpy(), ad, GEMV_TOL, what="fused vs unfused")


NORM_GEOMS = [(8, 1, 1), (8, 2, 1), (16, 1, 1), (16, 1, 4), (32, 1, 4), (32, 1, 8), (32, 2, 1), (32, 2, 4),
              (64, 1, 4)]
NORM_GLU_GEOMS = [(16, 2, 1), (16, 2, 4), (32, 2, 1), (32, 2, 4), (32, 2, 8), (64, 2, 4)]


@pytest.mark.parametrize("fmt", [0, 1, 2, 3, 4])
@pytest.mark.parametrize("glu", [False, True])
def test_addnorm_every_geometry(env, fmt, glu):
    # Every instantiated fused-norm geometry through the tuned entry point,
    # at two grid sizes (one workgroup per CU: several tiles per workgroup).
    torch, q4, orc = env
    m, k = (133, 960) if fmt in (0, 2, 4) else (133, 1024)
    rows = 2 * m if glu else m
    buf = q4.q4_quantize_ref(fmt, synth.weights(synth.seed_for(3500 + fmt, glu), rows, k))
    x, delta, gain = _inputs(3501 + fmt, k)
    v, h = _normed(x, delta, gain, 1e-5)
    if glu:
        yr = orc.matvec_silu_mul(fmt, buf, m, k, h[None, :], threads=threads())
    else:
        yr = orc.matvec(fmt, buf, m, k, h[None, :], threads=threads())
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    wd, xd, dd, gd = dev(buf), dev(x), dev(delta), dev(gain)
    epi = q4.Q4_EPILOGUE_SILU_MUL if glu else q4.Q4_EPILOGUE_NONE
    for geom in (NORM_GLU_GEOMS if glu else NORM_GEOMS):
        for gpc in (0, 1):
            say(f"addnorm geometry fmt={fmt} glu={glu} {geom} groups_per_cu={gpc}")
            xo = torch.full((k,), float("nan"), device="cuda")
            y = torch.full((m,), float("nan"), device="cuda")
            q4.q4_gemv_addnorm_tuned(fmt, wd, xd, dd, gd, 1e-5, xo, y, m, k, epi, *geom, gpc)
            torch.cuda.synchronize()
            yc = y.cpu().numpy().astype(np.float64)
            assert np.array_equal(xo.cpu().numpy(), v), geom
            assert np.all(np.isfinite(yc)), geom
            assert np.linalg.norm(yc - yr[0]) <= GEMV_TOL * np.linalg.norm(yr[0]), (geom, gpc)


def test_addnorm_noop_and_errors(env):
    torch, q4, _ = env
    lib = q4.raw()
    w = torch.zeros(4096, dtype=torch.uint8, device="cuda")
    x = torch.zeros(256, device="cuda")
    g = torch.ones(256, device="cuda")
    xo = torch.full((256,), 7.0, device="cuda")
    y = torch.full((8,), 5.0, device="cuda")
    p = lambda t, off=0: t.data_ptr() + off  # noqa: E731
    assert lib.q4_gemv_addnorm(0, p(w), p(x), None, p(g), 1e-5, p(xo), p(y), 0, 32, 0, None) == q4.Q4_OK
    assert lib.q4_gemv_addnorm(0, p(w), p(x), None, p(g, 4), 1e-5, p(xo), p(y), 4, 32, 0, None) == q4.Q4_EALIGN
    assert lib.q4_gemv_addnorm(0, p(w), p(x), None, p(g), 1e-5, p(x), p(y), 4, 32, 0, None) == q4.Q4_EINVAL
    torch.cuda.synchronize()
    assert (y == 5.0).all() and (xo == 7.0).all()


@pytest.mark.parametrize("geom,glu", [((32, 1, 4), False), ((32, 1, 8), False), ((64, 1, 4), False),
                                      ((32, 2, 4), True), ((32, 2, 8), True)])
def test_addnorm_longest_row(env, geom, glu):
    # The longest row the fused norm stages (455 units, 14560 weights: 65520
    # bytes of activations, plus one sum of squares per wave), with 4- and
    # 8-wave groups: the per-wave sums take the workgroup past 64 KiB, which
    # the launch covers with the device's opt-in LDS.
    torch, q4, orc = env
    fmt, m, k = 0, 300, 14560
    rows = 2 * m if glu else m
    buf = q4.q4_quantize_ref(fmt, synth.weights(synth.seed_for(3600, glu), rows, k))
    x, delta, gain = _inputs(3601, k)
    v, h = _normed(x, delta, gain, 1e-5)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    wd, xd, dd, gd = dev(buf), dev(x), dev(delta), dev(gain)
    xo = torch.full((k,), float("nan"), device="cuda")
    y = torch.full((m,), float("nan"), device="cuda")
    epi = q4.Q4_EPILOGUE_SILU_MUL if glu else q4.Q4_EPILOGUE_NONE
    say(f"addnorm longest row geometry {geom} glu={glu}")
    q4.q4_gemv_addnorm_tuned(fmt, wd, xd, dd, gd, 1e-5, xo, y, m, k, epi, *geom, 0)
    torch.cuda.synchronize()
    assert np.array_equal(xo.cpu().numpy(), v)
    if glu:
        yr = orc.matvec_silu_mul(fmt, buf, m, k, h[None, :], threads=threads())
    else:
        yr = orc.matvec(fmt, buf, m, k, h[None, :], threads=threads())
    yc = y.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(yc))
    assert np.linalg.norm(yc - yr[0]) <= GEMV_TOL * np.linalg.norm(yr[0]), geom
