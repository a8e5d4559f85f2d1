"""Plain float64 reference for a whole synthetic decode step -- TEST INFRASTRUCTURE ONLY.

The decode step of a Llama-family model (the SmolLM2 models the MicroLLM Lab
post runs, "Seven models, all in Q4") around the quantized matrix products:
the token's embedding, then per layer a residual add and RMSNorm, the stacked
q|k|v product, rotary position embedding of q and k, a KV-cache append,
grouped-query attention over the cached positions, the output projection, a
second residual add and RMSNorm, the gated MLP silu(W_gate h) * (W_up h) and
the down projection; then the final residual add and norm, the LM head (the
embedding matrix, tied) and the greedy next token. Keeping keys and values
cached between steps, and running the selection on the device, are items of
the WebGPT README's "Roadmap"; the technical summary of Llamas on the Web
allocates every intermediate buffer statically up front (Methodology
section 1), as the GPU step here does.

The pages define none of these operators; the definitions below are the
standard ones of that model family, each written out plainly:
  * rmsnorm(x) = x / sqrt(mean(x^2) + eps) * g;
  * rotary embedding, rotate-half form: for each head and i < d/2, with
    a = pos * theta^(-2i/d): x'[i] = x[i] cos a - x[i+d/2] sin a,
    x'[i+d/2] = x[i+d/2] cos a + x[i] sin a;
  * attention: query head h reads key/value head h // (H / H_kv); scores
    q . k_t / sqrt(d) for t <= pos, softmax, output sum_t w_t v_t;
  * silu(g) = g / (1 + e^-g).
Weights are the dequantized matrices of the quantized buffers the GPU reads
(``oracle.dequantize``); every step is evaluated in float64 with numpy (the
matrix products as plain ``@``). This module imports nothing from the product
library.
"""
from __future__ import annotations

import math

import numpy as np

from . import dequantize


def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    x = np.asarray(x, np.float64)
    return x / math.sqrt(float(np.mean(x * x)) + eps) * np.asarray(g, np.float64)


def rope(v: np.ndarray, pos: int, theta: float, head_dim: int) -> np.ndarray:
    """Rotate every head of v (a flat vector of heads of head_dim) to position pos."""
    v = np.asarray(v, np.float64).reshape(-1, head_dim)
    half = head_dim // 2
    i = np.arange(half, dtype=np.float64)
    a = pos * theta ** (-2.0 * i / head_dim)
    c, s = np.cos(a), np.sin(a)
    out = np.empty_like(v)
    out[:, :half] = v[:, :half] * c - v[:, half:] * s
    out[:, half:] = v[:, half:] * c + v[:, :half] * s
    return out.reshape(-1)


def attention(q: np.ndarray, kcache: np.ndarray, vcache: np.ndarray, pos: int, heads: int) -> np.ndarray:
    """q: [heads * d]; kcache, vcache: [kv_heads, T, d] holding positions 0..pos."""
    kv_heads, _, d = kcache.shape
    group = heads // kv_heads
    q = np.asarray(q, np.float64).reshape(heads, d)
    out = np.empty((heads, d))
    for h in range(heads):
        k = kcache[h // group, : pos + 1]
        v = vcache[h // group, : pos + 1]
        s = k @ q[h] / math.sqrt(d)
        w = np.exp(s - s.max())
        w /= w.sum()
        out[h] = w @ v
    return out.reshape(-1)


def silu(g: np.ndarray) -> np.ndarray:
    g = np.asarray(g, np.float64)
    return g / (1.0 + np.exp(-g))


class Model:
    """Dequantized weights and a float64 KV cache for one sequence.

    cfg: dict with layers, hidden, heads, kv_heads, head_dim, ffn, vocab,
    max_pos, theta, eps. bufs: dict of quantized host buffers (numpy uint8)
    keyed qkv{i}, o{i}, gu{i} (stacked gate then up rows), down{i}, emb; and
    float32 norm weights norm_attn{i}, norm_mlp{i}, norm_final.
    """

    def __init__(self, fmt: int, cfg: dict, bufs: dict):
        self.cfg = c = cfg
        hd, q_n, kv_n = c["hidden"], c["heads"] * c["head_dim"], c["kv_heads"] * c["head_dim"]
        deq = lambda name, m, k: dequantize(fmt, bufs[name], m, k).astype(np.float64)  # noqa: E731
        self.emb = deq("emb", c["vocab"], hd)
        self.layers = []
        for i in range(c["layers"]):
            self.layers.append({
                "qkv": deq(f"qkv{i}", q_n + 2 * kv_n, hd),
                "o": deq(f"o{i}", hd, q_n),
                "gu": deq(f"gu{i}", 2 * c["ffn"], hd),
                "down": deq(f"down{i}", hd, c["ffn"]),
                "norm_attn": np.asarray(bufs[f"norm_attn{i}"], np.float64),
                "norm_mlp": np.asarray(bufs[f"norm_mlp{i}"], np.float64),
            })
        self.norm_final = np.asarray(bufs["norm_final"], np.float64)
        shape = (c["layers"], c["kv_heads"], c["max_pos"], c["head_dim"])
        self.kcache = np.zeros(shape)
        self.vcache = np.zeros(shape)

    def step(self, token: int, pos: int):
        """One decode step: returns (logits, next token), and appends to the cache."""
        c = self.cfg
        d, hq, hkv = c["head_dim"], c["heads"], c["kv_heads"]
        q_n, kv_n = hq * d, hkv * d
        x = self.emb[token].copy()
        delta = np.zeros_like(x)
        for i, L in enumerate(self.layers):
            x = x + delta
            h = rmsnorm(x, L["norm_attn"], c["eps"])
            qkv = L["qkv"] @ h
            q = rope(qkv[:q_n], pos, c["theta"], d)
            k = rope(qkv[q_n:q_n + kv_n], pos, c["theta"], d)
            v = qkv[q_n + kv_n:]
            self.kcache[i, :, pos] = k.reshape(hkv, d)
            self.vcache[i, :, pos] = v.reshape(hkv, d)
            att = attention(q, self.kcache[i], self.vcache[i], pos, hq)
            x = x + L["o"] @ att
            h2 = rmsnorm(x, L["norm_mlp"], c["eps"])
            gu = L["gu"] @ h2
            delta = L["down"] @ (silu(gu[: c["ffn"]]) * gu[c["ffn"]:])
        x = x + delta
        logits = self.emb @ rmsnorm(x, self.norm_final, c["eps"])
        return logits, int(np.argmax(logits))
