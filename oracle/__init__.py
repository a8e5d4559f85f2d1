"""CPU oracle for the Q4 products -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the bench's CPU-baseline leg may import
this package.  The product library (``q4_weight_gemv_amd``) never imports,
links or executes anything here, and this package imports nothing from it.

Thin ctypes marshalling over ``liboracle.so`` (built from ``q4_oracle.c`` with
gcc; see ``build()``).  Every function takes and returns numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "q4_oracle.c")
# Q4_ORACLE_LIB names another build of the oracle to load (the mutation tests
# point it at copies of the source with planted mistakes).
LIB = os.environ.get("Q4_ORACLE_LIB") or os.path.join(HERE, "liboracle.so")

Q4_0 = 0
Q4_K = 1
Q8_0 = 2
Q2_K = 3
Q1_0 = 4

OK, EINVAL, ENONFINITE, ERANGE = 0, -1, -4, -5


def build(force: bool = True, src: str | None = None, out: str | None = None) -> str:
    """Compile the oracle with gcc (IEEE semantics: no contraction, no fast-math):
    ``src`` (default q4_oracle.c) into ``out`` (default the library loaded here)."""
    src, out = src or SRC, out or LIB
    if force or not os.path.exists(out):
        tmp = out + ".tmp"
        cmd = ["gcc", "-std=c99", "-O2", "-fPIC", "-shared", "-ffp-contract=off",
               "-fno-fast-math", "-Wall", "-Wextra", "-o", tmp, src, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, out)
    return out


_lib = None
_lock = threading.Lock()

_u8p = ctypes.POINTER(ctypes.c_uint8)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)
_i64 = ctypes.c_int64


def lib():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB):
                build(force=False)
            L = ctypes.CDLL(LIB)
            sigs = {
                "oracle_fp16_to_fp32": (ctypes.c_float, [ctypes.c_uint16]),
                "oracle_f64_to_fp16": (ctypes.c_uint16, [ctypes.c_double]),
                "oracle_fp32_to_fp16": (ctypes.c_uint16, [ctypes.c_float]),
                "oracle_bf16_to_fp32": (ctypes.c_float, [ctypes.c_uint16]),
                "oracle_fp32_to_bf16": (ctypes.c_uint16, [ctypes.c_float]),
                "oracle_q4_0_bytes": (ctypes.c_size_t, [_i64, _i64]),
                "oracle_q4_k_bytes": (ctypes.c_size_t, [_i64, _i64]),
                "oracle_q8_0_bytes": (ctypes.c_size_t, [_i64, _i64]),
                "oracle_q2_k_bytes": (ctypes.c_size_t, [_i64, _i64]),
                "oracle_q1_0_bytes": (ctypes.c_size_t, [_i64, _i64]),
                "oracle_q1_0_quantize_block": (ctypes.c_int, [_f32p, ctypes.POINTER(ctypes.c_uint32), _u16p]),
                "oracle_q1_0_quantize": (ctypes.c_int, [_f32p, _i64, _i64, _u8p]),
                "oracle_q1_0_dequantize": (None, [_u8p, _i64, _i64, _f32p]),
                "oracle_q2_k_quantize": (ctypes.c_int, [_f32p, _i64, _i64, _u8p]),
                "oracle_q2_k_dequantize": (None, [_u8p, _i64, _i64, _f32p]),
                "oracle_q8_0_quantize_block": (ctypes.c_int, [_f32p, ctypes.POINTER(ctypes.c_int8), _u16p]),
                "oracle_q8_0_quantize": (ctypes.c_int, [_f32p, _i64, _i64, _u8p]),
                "oracle_q8_0_dequantize": (None, [_u8p, _i64, _i64, _f32p]),
                "oracle_q4_0_quantize_block": (ctypes.c_int, [_f32p, _u8p, _u16p]),
                "oracle_q4_0_quantize": (ctypes.c_int, [_f32p, _i64, _i64, _u8p]),
                "oracle_q4_0_dequantize": (None, [_u8p, _i64, _i64, _f32p]),
                "oracle_q4_0_planes_to_aos": (None, [_u8p, _i64, _i64, _u8p]),
                "oracle_q4_0_aos_to_planes": (None, [_u8p, _i64, _i64, _u8p]),
                "oracle_q4_k_unpack_scales": (None, [_u8p, _u8p, _u8p]),
                "oracle_q4_k_pack_scales": (None, [_u8p, _u8p, _u8p]),
                "oracle_q4_k_quantize": (ctypes.c_int, [_f32p, _i64, _i64, _u8p]),
                "oracle_q4_k_dequantize": (None, [_u8p, _i64, _i64, _f32p]),
                "oracle_matvec": (None, [ctypes.c_int, _u8p, _i64, _i64, _f32p, _i64, _f32p, _i64, _i64]),
                "oracle_matvec_absdot": (None, [ctypes.c_int, _u8p, _i64, _i64, _f32p, _i64, _f32p, _f64p, _i64, _i64]),
                "oracle_matmul": (None, [ctypes.c_int, _u8p, _i64, _i64, _u16p, _i64, _f32p, ctypes.c_int, _f64p, _i64, _i64]),
                "oracle_matvec_termscale": (None, [ctypes.c_int, _u8p, _i64, _i64, _f32p, _i64, _f64p, _i64, _i64]),
                "oracle_matvec_one": (ctypes.c_double, [ctypes.c_int, _u8p, _i64, _i64, _f32p, _i64, _i64, _f64p]),
                "oracle_matvec_silu_mul": (None, [ctypes.c_int, _u8p, _i64, _i64, _f32p, _i64, _f32p, _f64p, _f64p,
                                                  _i64, _i64]),
            }
            for name, (res, args) in sigs.items():
                fn = getattr(L, name)
                fn.restype = res
                fn.argtypes = args
            _lib = L
    return _lib


def _p(a: np.ndarray, t):
    return a.ctypes.data_as(t)


class OracleError(RuntimeError):
    def __init__(self, status: int):
        super().__init__(f"oracle status {status}")
        self.status = status


# --------------------------------------------------------------------------- formats

def fp16_to_fp32(h: int) -> float:
    return lib().oracle_fp16_to_fp32(h)


def fp32_to_fp16(f: float) -> int:
    return lib().oracle_fp32_to_fp16(f)


def f64_to_fp16(v: float) -> int:
    return lib().oracle_f64_to_fp16(v)


def fp32_to_bf16(f: float) -> int:
    return lib().oracle_fp32_to_bf16(f)


def bf16_to_fp32(b: int) -> float:
    return lib().oracle_bf16_to_fp32(b)


def weight_bytes(fmt: int, m: int, k: int) -> int:
    L = lib()
    return {Q4_0: L.oracle_q4_0_bytes, Q4_K: L.oracle_q4_k_bytes, Q8_0: L.oracle_q8_0_bytes,
            Q2_K: L.oracle_q2_k_bytes, Q1_0: L.oracle_q1_0_bytes}[fmt](m, k)


def quantize(fmt: int, w: np.ndarray) -> np.ndarray:
    """float32 W[m][k] -> packed bytes (plane-split Q4_0 or Q8_0, or Q4_K super-blocks)."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    m, k = w.shape
    out = np.zeros(weight_bytes(fmt, m, k), dtype=np.uint8)
    L = lib()
    fn = {Q4_0: L.oracle_q4_0_quantize, Q4_K: L.oracle_q4_k_quantize, Q8_0: L.oracle_q8_0_quantize,
          Q2_K: L.oracle_q2_k_quantize, Q1_0: L.oracle_q1_0_quantize}[fmt]
    st = fn(_p(w, _f32p), m, k, _p(out, _u8p))
    if st != OK:
        raise OracleError(st)
    return out


def quantize_q4_0_block(w32: np.ndarray):
    w32 = np.ascontiguousarray(w32, dtype=np.float32)
    assert w32.shape == (32,)
    nib = np.zeros(16, dtype=np.uint8)
    d = ctypes.c_uint16(0)
    st = lib().oracle_q4_0_quantize_block(_p(w32, _f32p), _p(nib, _u8p), ctypes.byref(d))
    if st != OK:
        raise OracleError(st)
    return nib, d.value


def quantize_q8_0_block(w32: np.ndarray):
    w32 = np.ascontiguousarray(w32, dtype=np.float32)
    assert w32.shape == (32,)
    q = np.zeros(32, dtype=np.int8)
    d = ctypes.c_uint16(0)
    st = lib().oracle_q8_0_quantize_block(_p(w32, _f32p), q.ctypes.data_as(ctypes.POINTER(ctypes.c_int8)),
                                          ctypes.byref(d))
    if st != OK:
        raise OracleError(st)
    return q, d.value


def quantize_q1_0_block(w32: np.ndarray):
    w32 = np.ascontiguousarray(w32, dtype=np.float32)
    assert w32.shape == (32,)
    bits = ctypes.c_uint32(0)
    d = ctypes.c_uint16(0)
    st = lib().oracle_q1_0_quantize_block(_p(w32, _f32p), ctypes.byref(bits), ctypes.byref(d))
    if st != OK:
        raise OracleError(st)
    return bits.value, d.value


def dequantize(fmt: int, buf: np.ndarray, m: int, k: int) -> np.ndarray:
    buf = np.ascontiguousarray(buf, dtype=np.uint8)
    assert buf.size == weight_bytes(fmt, m, k)
    out = np.empty((m, k), dtype=np.float32)
    L = lib()
    fn = {Q4_0: L.oracle_q4_0_dequantize, Q4_K: L.oracle_q4_k_dequantize, Q8_0: L.oracle_q8_0_dequantize,
          Q2_K: L.oracle_q2_k_dequantize, Q1_0: L.oracle_q1_0_dequantize}[fmt]
    fn(_p(buf, _u8p), m, k, _p(out, _f32p))
    return out


def q4_0_planes_to_aos(buf: np.ndarray, m: int, k: int) -> np.ndarray:
    out = np.empty(weight_bytes(Q4_0, m, k), dtype=np.uint8)
    lib().oracle_q4_0_planes_to_aos(_p(np.ascontiguousarray(buf), _u8p), m, k, _p(out, _u8p))
    return out


def q4_0_aos_to_planes(buf: np.ndarray, m: int, k: int) -> np.ndarray:
    out = np.empty(weight_bytes(Q4_0, m, k), dtype=np.uint8)
    lib().oracle_q4_0_aos_to_planes(_p(np.ascontiguousarray(buf), _u8p), m, k, _p(out, _u8p))
    return out


def q4_k_pack_scales(sc, mn) -> np.ndarray:
    sc = np.ascontiguousarray(sc, dtype=np.uint8)
    mn = np.ascontiguousarray(mn, dtype=np.uint8)
    out = np.zeros(12, dtype=np.uint8)
    lib().oracle_q4_k_pack_scales(_p(sc, _u8p), _p(mn, _u8p), _p(out, _u8p))
    return out


def q4_k_unpack_scales(S):
    S = np.ascontiguousarray(S, dtype=np.uint8)
    sc = np.zeros(8, dtype=np.uint8)
    mn = np.zeros(8, dtype=np.uint8)
    lib().oracle_q4_k_unpack_scales(_p(S, _u8p), _p(sc, _u8p), _p(mn, _u8p))
    return sc, mn


# --------------------------------------------------------------------------- products

def _row_split(m: int, threads: int):
    threads = max(1, min(threads, m)) if m > 0 else 1
    step = (m + threads - 1) // threads if m > 0 else 0
    return [(r, min(m, r + step)) for r in range(0, m, step)] if m > 0 else []


def matvec(fmt: int, buf: np.ndarray, m: int, k: int, x: np.ndarray, threads: int = 1,
           absdot: bool = False, rows=None):
    """y[n][m] = fp32(sum_k w_hat * x) in float64; rows split over ``threads`` threads.

    Returns y, or (y, sum_k |w_hat*x|) with ``absdot``. ``rows`` (a list of
    (r0, r1) ranges) restricts the work to those rows; the others stay 0.
    """
    buf = np.ascontiguousarray(buf, dtype=np.uint8)
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.ndim == 1:
        x = x.reshape(1, -1)
    n = x.shape[0]
    assert x.shape[1] == k and buf.size == weight_bytes(fmt, m, k)
    y = np.zeros((n, m), dtype=np.float32)
    ad = np.zeros((n, m), dtype=np.float64) if absdot else None
    L = lib()

    def run(r0, r1):
        if absdot:
            L.oracle_matvec_absdot(fmt, _p(buf, _u8p), m, k, _p(x, _f32p), n, _p(y, _f32p),
                                   _p(ad, _f64p), r0, r1)
        else:
            L.oracle_matvec(fmt, _p(buf, _u8p), m, k, _p(x, _f32p), n, _p(y, _f32p), r0, r1)

    ranges = _row_split(m, threads) if rows is None else _split_ranges(rows, threads)
    _parallel(run, ranges)
    return (y, ad) if absdot else y


def matvec_silu_mul(fmt: int, buf: np.ndarray, m: int, k: int, x: np.ndarray, threads: int = 1,
                    parts: bool = False):
    """Gated product over the stacked (2m) x k matrix: y[n][m] = fp32(silu(g) * u) in float64.

    With ``parts`` also returns the float64 row products g and u.
    """
    buf = np.ascontiguousarray(buf, dtype=np.uint8)
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.ndim == 1:
        x = x.reshape(1, -1)
    n = x.shape[0]
    assert x.shape[1] == k and buf.size == weight_bytes(fmt, 2 * m, k)
    y = np.zeros((n, m), dtype=np.float32)
    g = np.zeros((n, m), dtype=np.float64)
    u = np.zeros((n, m), dtype=np.float64)
    L = lib()

    def run(r0, r1):
        L.oracle_matvec_silu_mul(fmt, _p(buf, _u8p), m, k, _p(x, _f32p), n, _p(y, _f32p), _p(g, _f64p),
                                 _p(u, _f64p), r0, r1)

    _parallel(run, _row_split(m, threads))
    return (y, g, u) if parts else y


def _split_ranges(rows, threads):
    out = []
    per = max(1, sum(r1 - r0 for r0, r1 in rows) // max(1, threads))
    for r0, r1 in rows:
        for a in range(r0, r1, per):
            out.append((a, min(r1, a + per)))
    return out


def matmul(fmt: int, buf: np.ndarray, m: int, k: int, x_bf16: np.ndarray, round_w_bf16: bool = False,
           threads: int = 1, absdot: bool = False, rows=None):
    """Y[n][m] = fp32(sum_k w_eff * X) in float64, X given as bf16 bit patterns."""
    buf = np.ascontiguousarray(buf, dtype=np.uint8)
    x_bf16 = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    n = x_bf16.shape[0]
    assert x_bf16.shape[1] == k and buf.size == weight_bytes(fmt, m, k)
    y = np.zeros((n, m), dtype=np.float32)
    ad = np.zeros((n, m), dtype=np.float64) if absdot else None
    L = lib()

    def run(r0, r1):
        L.oracle_matmul(fmt, _p(buf, _u8p), m, k, _p(x_bf16, _u16p), n, _p(y, _f32p),
                        1 if round_w_bf16 else 0, _p(ad, _f64p) if absdot else None, r0, r1)

    ranges = _row_split(m, threads) if rows is None else _split_ranges(rows, threads)
    _parallel(run, ranges)
    return (y, ad) if absdot else y


def termscale(fmt: int, buf: np.ndarray, m: int, k: int, x: np.ndarray, threads: int = 1, rows=None):
    """sum_k (term magnitudes of w_hat[i][k]) * |x[t][k]| per output (see q4_oracle.c)."""
    buf = np.ascontiguousarray(buf, dtype=np.uint8)
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.ndim == 1:
        x = x.reshape(1, -1)
    n = x.shape[0]
    out = np.zeros((n, m), dtype=np.float64)
    L = lib()

    def run(r0, r1):
        L.oracle_matvec_termscale(fmt, _p(buf, _u8p), m, k, _p(x, _f32p), n, _p(out, _f64p), r0, r1)

    _parallel(run, _row_split(m, threads) if rows is None else _split_ranges(rows, threads))
    return out


def matvec_one(fmt: int, buf: np.ndarray, m: int, k: int, x: np.ndarray, t: int, i: int):
    """One output y[t][i] (float64 sum, before the final fp32 rounding) and its |.| scale."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.ndim == 1:
        x = x.reshape(1, -1)
    ad = ctypes.c_double(0.0)
    v = lib().oracle_matvec_one(fmt, _p(buf, _u8p), m, k, _p(x, _f32p), t, i, ctypes.byref(ad))
    return v, ad.value


def _parallel(fn, ranges):
    if len(ranges) <= 1:
        for r0, r1 in ranges:
            fn(r0, r1)
        return
    # ctypes releases the GIL for the duration of each foreign call.
    ths = [threading.Thread(target=fn, args=rr) for rr in ranges]
    for t in ths:
        t.start()
    for t in ths:
        t.join()
