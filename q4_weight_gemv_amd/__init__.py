"""Python binding of the Q4 weight-matrix product library (gfx950 / MI355X).

Argument marshalling only: every entry point forwards to the C ABI declared
in ``include/q4.h`` (the in-tree ``libq4gemv.so``), which runs the products in
hand-written HIP kernels. PyTorch supplies device memory and streams. There
is no fallback path: if the library is missing, import fails.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
# Q4_GEMV_LIB names another build of the library (the host-sanitizer test
# tier loads one); by default the in-tree build.
LIB_PATH = os.environ.get("Q4_GEMV_LIB") or os.path.join(HERE, "libq4gemv.so")

Q4_FMT_Q4_0 = 0
Q4_FMT_Q4_K = 1
Q4_FMT_Q8_0 = 2
Q4_FMT_Q2_K = 3
Q4_FMT_Q1_0 = 4

Q4_OK = 0
Q4_EINVAL = -1
Q4_EUNSUPPORTED = -2
Q4_EALIGN = -3
Q4_ENONFINITE = -4
Q4_ERANGE = -5
Q4_EHIP = -6

Q4_EPILOGUE_NONE = 0
Q4_EPILOGUE_SILU_MUL = 1

BLOCK = {Q4_FMT_Q4_0: 32, Q4_FMT_Q4_K: 256, Q4_FMT_Q8_0: 32, Q4_FMT_Q2_K: 256, Q4_FMT_Q1_0: 32}

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python q4_weight_gemv_amd/build.py`")

# The library must run on the same HIP runtime as the torch tensors and
# streams it is handed. torch ships its own libamdhip64 under the same soname
# as the system one this library links to, and the dynamic linker keeps the
# first copy loaded; importing torch first makes that copy torch's. (Loaded
# the other way round, the two end up on different runtimes and the library
# finds no device.)
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(LIB_PATH)


Q4_GEMV_KERNEL_AUTO = 0
Q4_GEMV_KERNEL_TILED = 1
Q4_GEMV_KERNEL_STREAM = 2
Q4_GEMV_KERNEL_MATRIX = 3


class q4_gemv_tuning(ctypes.Structure):
    _fields_ = [("lanes_per_row", ctypes.c_int), ("rows_per_lane", ctypes.c_int),
                ("waves_per_group", ctypes.c_int), ("groups_per_cu", ctypes.c_int),
                ("kernel", ctypes.c_int), ("depth", ctypes.c_int)]


class q4_gemm_tuning(ctypes.Structure):
    _fields_ = [("tile_rows", ctypes.c_int), ("tile_tokens", ctypes.c_int), ("stage_k", ctypes.c_int)]


class q4_gemv_op(ctypes.Structure):
    _fields_ = [("w", ctypes.c_void_p), ("x", ctypes.c_void_p), ("y", ctypes.c_void_p),
                ("m", ctypes.c_int64), ("k", ctypes.c_int64), ("epilogue", ctypes.c_int)]


class q4_llama_config(ctypes.Structure):
    _fields_ = [("layers", ctypes.c_int), ("hidden", ctypes.c_int), ("heads", ctypes.c_int), ("kv_heads", ctypes.c_int),
                ("head_dim", ctypes.c_int), ("ffn", ctypes.c_int), ("vocab", ctypes.c_int), ("max_pos", ctypes.c_int),
                ("rope_theta", ctypes.c_float), ("norm_eps", ctypes.c_float)]


class q4_llama_layer(ctypes.Structure):
    _fields_ = [("qkv", ctypes.c_void_p), ("o", ctypes.c_void_p), ("gate_up", ctypes.c_void_p),
                ("down", ctypes.c_void_p), ("norm_attn", ctypes.c_void_p), ("norm_mlp", ctypes.c_void_p)]


class q4_llama_state(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("x", "h", "qkv", "att", "delta", "act", "logits", "k_cache", "v_cache",
                                               "token", "pos")]


_i64 = ctypes.c_int64
_vp = ctypes.c_void_p
_SIGS = {
    "q4_weight_bytes": (ctypes.c_size_t, [ctypes.c_int, _i64, _i64]),
    "q4_quantize_ref": (ctypes.c_int, [ctypes.c_int, _vp, _i64, _i64, _vp, ctypes.c_size_t]),
    "q4_gemv": (ctypes.c_int, [ctypes.c_int, _vp, _vp, _vp, _i64, _i64, _i64, _vp]),
    "q4_gemv_glu": (ctypes.c_int, [ctypes.c_int, _vp, _vp, _vp, _i64, _i64, _i64, _vp]),
    "q4_gemv_addnorm": (ctypes.c_int, [ctypes.c_int, _vp, _vp, _vp, _vp, ctypes.c_float, _vp, _vp, _i64, _i64,
                                        ctypes.c_int, _vp]),
    "q4_gemv_addnorm_tuned": (ctypes.c_int, [ctypes.c_int, _vp, _vp, _vp, _vp, ctypes.c_float, _vp, _vp, _i64, _i64,
                                              ctypes.c_int, ctypes.POINTER(q4_gemv_tuning), _vp]),
    "q4_gemv_tuned": (ctypes.c_int, [ctypes.c_int, _vp, _vp, _vp, _i64, _i64, _i64,
                                      ctypes.POINTER(q4_gemv_tuning), _vp]),
    "q4_gemm": (ctypes.c_int, [ctypes.c_int, _vp, _vp, _vp, _i64, _i64, _i64, _vp]),
    "q4_gemm_tuned": (ctypes.c_int, [ctypes.c_int, _vp, _vp, _vp, _i64, _i64, _i64,
                                      ctypes.POINTER(q4_gemm_tuning), _vp]),
    "q4_gemv_sequence": (ctypes.c_int, [ctypes.c_int, ctypes.POINTER(q4_gemv_op), ctypes.c_int, _i64, _vp]),
    "q4_graph_create": (ctypes.c_int, [ctypes.c_int, ctypes.POINTER(q4_gemv_op), ctypes.c_int, _i64, _vp,
                                        ctypes.POINTER(_vp)]),
    "q4_graph_launch": (ctypes.c_int, [_vp, _vp]),
    "q4_graph_destroy": (ctypes.c_int, [_vp]),
    "q4_llama_step": (ctypes.c_int, [ctypes.c_int, ctypes.POINTER(q4_llama_config), _vp, _vp,
                                      ctypes.POINTER(q4_llama_layer), ctypes.POINTER(q4_llama_state), _vp]),
    "q4_llama_step_noalloc": (ctypes.c_int, [ctypes.c_int, ctypes.POINTER(q4_llama_config), _vp, _vp,
                                              ctypes.POINTER(q4_llama_layer), ctypes.POINTER(q4_llama_state), _vp]),
    "q4_llama_graph_create": (ctypes.c_int, [ctypes.c_int, ctypes.POINTER(q4_llama_config), _vp, _vp,
                                              ctypes.POINTER(q4_llama_layer), ctypes.POINTER(q4_llama_state), _vp,
                                              ctypes.POINTER(_vp)]),
    "q4_llama_graph_launch": (ctypes.c_int, [_vp, _vp]),
    "q4_llama_graph_destroy": (ctypes.c_int, [_vp]),
    "q4_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "q4_last_hip_error": (ctypes.c_char_p, []),
    "q4_read_probe": (ctypes.c_int, [_vp, ctypes.c_size_t, _vp, ctypes.c_int, _vp]),
}
for _name, (_res, _args) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args

EXPORTS = tuple(_SIGS)


class Q4Error(RuntimeError):
    def __init__(self, status: int, where: str):
        detail = f", {_lib.q4_last_hip_error().decode()}" if status == Q4_EHIP else ""
        super().__init__(f"{where}: {q4_strerror(status)} (status {status}{detail})")
        self.status = status


def _check(status: int, where: str) -> None:
    if status != Q4_OK:
        raise Q4Error(status, where)


def q4_strerror(status: int) -> str:
    return _lib.q4_strerror(status).decode()


def q4_weight_bytes(fmt: int, m: int, k: int) -> int:
    return int(_lib.q4_weight_bytes(fmt, m, k))


def q4_quantize_ref(fmt: int, w: np.ndarray) -> np.ndarray:
    """Host quantizer: float32 W[m][k] -> packed uint8 buffer (layout in include/q4.h)."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    if w.ndim != 2:
        raise ValueError("w must be 2-D [m][k]")
    m, k = w.shape
    nbytes = q4_weight_bytes(fmt, m, k)
    out = np.zeros(max(nbytes, 1), dtype=np.uint8)
    _check(_lib.q4_quantize_ref(fmt, w.ctypes.data, m, k, out.ctypes.data, nbytes), "q4_quantize_ref")
    return out[:nbytes]


def _stream_ptr(stream):
    if stream is None:
        import torch

        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def q4_gemv(fmt: int, w, x, y, m: int, k: int, stream=None) -> None:
    """y[n][m] = W_hat x for n = x.shape[0] tokens (1..8); torch device tensors."""
    n = x.shape[0] if x.dim() == 2 else 1
    _check(_lib.q4_gemv(fmt, w.data_ptr(), x.data_ptr(), y.data_ptr(), m, k, n, _stream_ptr(stream)), "q4_gemv")


def q4_gemv_glu(fmt: int, w, x, y, m: int, k: int, stream=None) -> None:
    """y[n][m] = silu(W_gate x) * (W_up x), w the quantized stacked (2m) x k matrix."""
    n = x.shape[0] if x.dim() == 2 else 1
    _check(_lib.q4_gemv_glu(fmt, w.data_ptr(), x.data_ptr(), y.data_ptr(), m, k, n, _stream_ptr(stream)),
           "q4_gemv_glu")


def q4_gemv_addnorm(fmt: int, w, x, delta, gain, eps: float, x_out, y, m: int, k: int,
                    epilogue: int = 0, stream=None) -> None:
    """One token: v = x + delta (delta may be None), x_out = v (if given), and
    y = W rmsnorm(v) * gain, or silu(W_gate .) * (W_up .) with Q4_EPILOGUE_SILU_MUL."""
    ptr = lambda t: None if t is None else t.data_ptr()  # noqa: E731
    _check(_lib.q4_gemv_addnorm(fmt, w.data_ptr(), x.data_ptr(), ptr(delta), ptr(gain), eps, ptr(x_out),
                                y.data_ptr(), m, k, epilogue, _stream_ptr(stream)), "q4_gemv_addnorm")


def q4_gemv_addnorm_tuned(fmt: int, w, x, delta, gain, eps: float, x_out, y, m: int, k: int, epilogue: int,
                          lanes_per_row=0, rows_per_lane=0, waves_per_group=0, groups_per_cu=0, stream=None) -> None:
    """q4_gemv_addnorm with an explicit tile geometry (0 keeps the library's choice)."""
    ptr = lambda t: None if t is None else t.data_ptr()  # noqa: E731
    t = q4_gemv_tuning(lanes_per_row, rows_per_lane, waves_per_group, groups_per_cu)
    _check(_lib.q4_gemv_addnorm_tuned(fmt, w.data_ptr(), x.data_ptr(), ptr(delta), ptr(gain), eps, ptr(x_out),
                                      y.data_ptr(), m, k, epilogue, ctypes.byref(t), _stream_ptr(stream)),
           "q4_gemv_addnorm_tuned")


# The instantiated tile geometries, as the header lists them.
# Decode, tiled kernel: (lanes_per_row, rows_per_lane, waves_per_group).
GEMV_GEOMETRIES = ((8, 1, 1), (8, 2, 1), (8, 4, 1), (16, 1, 1), (16, 2, 1), (32, 1, 1), (32, 2, 1), (64, 1, 1),
                   (16, 1, 4), (32, 1, 4), (32, 2, 4), (64, 1, 4), (64, 2, 4), (64, 4, 4), (32, 1, 8))
# Decode, one-token streaming kernel: (lanes_per_row, waves_per_group, depth).
GEMV_STREAM_GEOMETRIES = ((8, 16, 2), (16, 16, 2), (16, 1, 2), (32, 1, 2), (32, 8, 2), (32, 16, 2), (64, 4, 2),
                          (64, 8, 2), (64, 16, 2), (64, 8, 3), (64, 16, 4))
# Prefill: (tile_rows, tile_tokens, stage_k).
GEMM_TILES = ((16, 64, 512), (16, 64, 1024), (32, 64, 256), (32, 64, 512), (32, 64, 1024), (32, 128, 512),
              (64, 64, 256), (64, 64, 512))


def q4_gemv_tuned(fmt: int, w, x, y, m: int, k: int, lanes_per_row=0, rows_per_lane=0, waves_per_group=0,
                  groups_per_cu=0, stream=None, kernel=Q4_GEMV_KERNEL_AUTO, depth=0) -> None:
    """q4_gemv with an explicit kernel and geometry (0 keeps the library's choice)."""
    n = x.shape[0] if x.dim() == 2 else 1
    t = q4_gemv_tuning(lanes_per_row, rows_per_lane, waves_per_group, groups_per_cu, kernel, depth)
    _check(_lib.q4_gemv_tuned(fmt, w.data_ptr(), x.data_ptr(), y.data_ptr(), m, k, n, ctypes.byref(t),
                              _stream_ptr(stream)), "q4_gemv_tuned")


def q4_gemm(fmt: int, w, x_bf16, y, m: int, k: int, stream=None) -> None:
    """Y[n][m] = bf16(W_hat) X for bf16 X[n][k] (torch bfloat16/int16 device tensor)."""
    n = x_bf16.shape[0]
    _check(_lib.q4_gemm(fmt, w.data_ptr(), x_bf16.data_ptr(), y.data_ptr(), m, k, n, _stream_ptr(stream)),
           "q4_gemm")


def q4_gemm_tuned(fmt: int, w, x_bf16, y, m: int, k: int, tile_rows=0, tile_tokens=0, stage_k=0,
                  stream=None) -> None:
    """q4_gemm with an explicit tile geometry (0 keeps the library's choice)."""
    n = x_bf16.shape[0]
    t = q4_gemm_tuning(tile_rows, tile_tokens, stage_k)
    _check(_lib.q4_gemm_tuned(fmt, w.data_ptr(), x_bf16.data_ptr(), y.data_ptr(), m, k, n, ctypes.byref(t),
                              _stream_ptr(stream)), "q4_gemm_tuned")


def q4_read_probe(buf, sink, groups: int = 2048, stream=None) -> None:
    """Stream-read a device buffer once (measured HBM ceiling; not a product).
    ``sink`` None: a pure read; else (device, 4-byte elements, at least
    4 * ``groups`` of them) it receives one XOR fold per wave."""
    if sink is not None and sink.numel() * sink.element_size() < 16 * groups:
        raise Q4Error(Q4_EINVAL, "q4_read_probe: sink holds fewer than 4 * `groups` 4-byte words")
    _check(_lib.q4_read_probe(buf.data_ptr(), buf.numel() * buf.element_size(),
                              None if sink is None else sink.data_ptr(), groups,
                              _stream_ptr(stream)), "q4_read_probe")


def _ops_array(ops):
    arr = (q4_gemv_op * len(ops))()
    for i, op in enumerate(ops):
        w, x, y, m, k = op[:5]
        epilogue = op[5] if len(op) > 5 else Q4_EPILOGUE_NONE
        arr[i] = q4_gemv_op(w.data_ptr(), x.data_ptr(), y.data_ptr(), m, k, epilogue)
    return arr


def q4_gemv_sequence(fmt: int, ops, n: int, stream=None) -> None:
    """Enqueue decode products back-to-back; ops = [(w, x, y, m, k[, epilogue]), ...]."""
    arr = _ops_array(ops)
    _check(_lib.q4_gemv_sequence(fmt, arr, len(ops), n, _stream_ptr(stream)), "q4_gemv_sequence")


class Q4Sequence:
    """A layer stack marshalled once for q4_gemv_sequence: each launch() enqueues
    the products back-to-back on the stream (no graph), with no per-call
    argument building on the Python side."""

    def __init__(self, fmt: int, ops, n: int):
        self._ops = list(ops)  # keep the tensors alive: their pointers are in the array
        self._arr = _ops_array(self._ops)
        self._fmt, self._n = fmt, n

    def launch(self, stream=None) -> None:
        _check(_lib.q4_gemv_sequence(self._fmt, self._arr, len(self._ops), self._n, _stream_ptr(stream)),
               "q4_gemv_sequence")


class Q4Graph:
    """A captured decode step: q4_graph_create / q4_graph_launch / q4_graph_destroy."""

    def __init__(self, fmt: int, ops, n: int, stream=None):
        self._ops = list(ops)  # keep the tensors alive: their pointers are in the graph
        arr = _ops_array(self._ops)
        h = ctypes.c_void_p(None)
        _check(_lib.q4_graph_create(fmt, arr, len(self._ops), n, _stream_ptr(stream), ctypes.byref(h)),
               "q4_graph_create")
        self._h = h

    def launch(self, stream=None) -> None:
        _check(_lib.q4_graph_launch(self._h, _stream_ptr(stream)), "q4_graph_launch")

    def close(self) -> None:
        if self._h is not None and self._h.value:
            _check(_lib.q4_graph_destroy(self._h), "q4_graph_destroy")
        self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def raw():
    """The ctypes library handle (tests call entry points with raw pointers)."""
    return _lib


class LlamaStep:
    """A Llama-family decode step over caller-owned device tensors
    (q4_llama_step, and q4_llama_graph_* for the captured form).

    cfg: dict with layers, hidden, heads, kv_heads, head_dim, ffn, vocab,
    max_pos, theta, eps. w: dict of device tensors: emb, norm_final, and per
    layer i qkv{i}, o{i}, gu{i}, down{i} (quantized, fmt), norm_attn{i},
    norm_mlp{i} (float32). The state buffers are allocated here once.
    """

    def __init__(self, fmt: int, cfg: dict, w: dict):
        import torch as _t

        self.fmt, self.cfg, self.w = fmt, cfg, w
        c = cfg
        qkv_n = (c["heads"] + 2 * c["kv_heads"]) * c["head_dim"]
        f32 = dict(dtype=_t.float32, device="cuda")
        self.buf = {
            "x": _t.zeros(c["hidden"], **f32), "h": _t.zeros(c["hidden"], **f32), "qkv": _t.zeros(qkv_n, **f32),
            "att": _t.zeros(c["heads"] * c["head_dim"], **f32), "delta": _t.zeros(c["hidden"], **f32),
            "act": _t.zeros(c["ffn"], **f32), "logits": _t.zeros(c["vocab"], **f32),
            "k_cache": _t.zeros(c["layers"] * c["kv_heads"] * c["max_pos"] * c["head_dim"], **f32),
            "v_cache": _t.zeros(c["layers"] * c["kv_heads"] * c["max_pos"] * c["head_dim"], **f32),
            "token": _t.zeros(1, dtype=_t.int32, device="cuda"), "pos": _t.zeros(1, dtype=_t.int32, device="cuda"),
        }
        self._cfg = q4_llama_config(c["layers"], c["hidden"], c["heads"], c["kv_heads"], c["head_dim"], c["ffn"],
                                    c["vocab"], c["max_pos"], c["theta"], c["eps"])
        self._layers = (q4_llama_layer * c["layers"])()
        for i in range(c["layers"]):
            self._layers[i] = q4_llama_layer(w[f"qkv{i}"].data_ptr(), w[f"o{i}"].data_ptr(), w[f"gu{i}"].data_ptr(),
                                             w[f"down{i}"].data_ptr(), w[f"norm_attn{i}"].data_ptr(),
                                             w[f"norm_mlp{i}"].data_ptr())
        self._state = q4_llama_state(*[self.buf[n].data_ptr() for n in
                                       ("x", "h", "qkv", "att", "delta", "act", "logits", "k_cache", "v_cache",
                                        "token", "pos")])
        self._graph = None

    def set(self, token: int, pos: int) -> None:
        self.buf["token"].fill_(token)
        self.buf["pos"].fill_(pos)

    def step(self, stream=None) -> None:
        _check(_lib.q4_llama_step(self.fmt, ctypes.byref(self._cfg), self.w["emb"].data_ptr(),
                                  self.w["norm_final"].data_ptr(), self._layers, ctypes.byref(self._state),
                                  _stream_ptr(stream)), "q4_llama_step")

    def step_noalloc(self, stream=None) -> None:
        """The same step through q4_llama_step_noalloc (intermediate vectors in
        the library's static device array; this object's qkv, att, delta and
        act buffers are not used)."""
        _check(_lib.q4_llama_step_noalloc(self.fmt, ctypes.byref(self._cfg), self.w["emb"].data_ptr(),
                                          self.w["norm_final"].data_ptr(), self._layers, ctypes.byref(self._state),
                                          _stream_ptr(stream)), "q4_llama_step_noalloc")

    def capture(self, stream=None) -> None:
        h = ctypes.c_void_p(None)
        _check(_lib.q4_llama_graph_create(self.fmt, ctypes.byref(self._cfg), self.w["emb"].data_ptr(),
                                          self.w["norm_final"].data_ptr(), self._layers, ctypes.byref(self._state),
                                          _stream_ptr(stream), ctypes.byref(h)), "q4_llama_graph_create")
        self._graph = h

    def replay(self, stream=None) -> None:
        _check(_lib.q4_llama_graph_launch(self._graph, _stream_ptr(stream)), "q4_llama_graph_launch")

    def close(self) -> None:
        if self._graph is not None:
            _lib.q4_llama_graph_destroy(self._graph)
            self._graph = None
