"""Seeded synthetic inputs shared by the tests, the bench and the oracle timing leg.

This module holds no part of the quantization or product arithmetic: it only
draws numbers.  Both the HIP path and the CPU oracle are fed the identical
host arrays it returns, so the two sides never need a common RNG.

Generator (counter-based, so any slice can be regenerated independently):
  * SplitMix64 finalizer applied to ``seed_key + (i + 1) * 0x9E3779B97F4A7C15``
    for counter ``i`` (Steele, Lea and Flood, "Fast splittable pseudorandom
    number generators", OOPSLA 2014);
  * the top 53 bits give a uniform in [0, 1);
  * Box-Muller in float64 turns each pair of uniforms into two normals;
  * the normals are scaled by sigma and rounded to float32 (round to nearest even).

Workload shapes are those of the models the pages run (GPT-2-124M, SmolLM2-360M,
a 7B-class Llama layer); weights ~ N(0, 0.02) with 0.02 read as the standard
deviation, activations ~ N(0, 1).  No trained checkpoint is used anywhere.
"""
from __future__ import annotations

import numpy as np

_GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_CHUNK = 1 << 22


def _splitmix64(counter: np.ndarray, key: np.uint64) -> np.ndarray:
    z = key + (counter + np.uint64(1)) * _GOLDEN
    z = (z ^ (z >> np.uint64(30))) * _M1
    z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def _seed_key(seed: int) -> np.uint64:
    # Decorrelate nearby seeds by passing the seed itself through the mixer once.
    return _splitmix64(np.array([seed], dtype=np.uint64), np.uint64(0x5851F42D4C957F2D))[0]


def uniform53(seed: int, start: int, count: int) -> np.ndarray:
    """Uniforms in [0, 1) for counters start .. start+count-1 (float64)."""
    key = _seed_key(seed)
    ctr = np.arange(start, start + count, dtype=np.uint64)
    with np.errstate(over="ignore"):
        bits = _splitmix64(ctr, key)
    return (bits >> np.uint64(11)).astype(np.float64) * (1.0 / 9007199254740992.0)


def normal_f32(seed: int, count: int, sigma: float = 1.0) -> np.ndarray:
    """``count`` float32 samples of N(0, sigma^2); element i depends only on (seed, i)."""
    out = np.empty(count, dtype=np.float32)
    npairs = (count + 1) // 2
    for p0 in range(0, npairs, _CHUNK):
        p1 = min(npairs, p0 + _CHUNK)
        u = uniform53(seed, 2 * p0, 2 * (p1 - p0))
        u1 = u[0::2]
        u2 = u[1::2]
        r = np.sqrt(-2.0 * np.log1p(-u1))
        th = 2.0 * np.pi * u2
        z = np.empty(2 * (p1 - p0), dtype=np.float64)
        z[0::2] = r * np.cos(th)
        z[1::2] = r * np.sin(th)
        z *= sigma
        lo = 2 * p0
        hi = min(count, 2 * p1)
        out[lo:hi] = z[: hi - lo].astype(np.float32)
    return out


def weights(seed: int, m: int, k: int, sigma: float = 0.02) -> np.ndarray:
    """Row-major float32 W[m][k] ~ N(0, sigma^2)."""
    return normal_f32(seed, m * k, sigma).reshape(m, k)


def activations(seed: int, n: int, k: int, sigma: float = 1.0) -> np.ndarray:
    """Token-major float32 x[n][k] ~ N(0, sigma^2)."""
    return normal_f32(seed, n * k, sigma).reshape(n, k)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns via torch's CPU cast (round to nearest even).

    Only turns drawn float32 activations into the bf16 inputs the prefill
    product takes; a library cast, so no rounding code lives here.
    """
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def seed_for(config: int, tensor_index: int, is_x: bool = False) -> int:
    """Seed convention: 1000*config + 10*tensor_index (+1 for the activation)."""
    return 1000 * config + 10 * tensor_index + (1 if is_x else 0)


# ---------------------------------------------------------------------------
# Workload shapes: (K -> M) per matrix, in the order a decode step runs them.
# ---------------------------------------------------------------------------

def gpt2_124m_step():
    """GPT-2-124M decode step: 12 layers of QKV, attn-out, MLP-up, MLP-down, then the LM head."""
    d = 768
    layer = [(d, 3 * d), (d, d), (d, 4 * d), (4 * d, d)]
    return [s for _ in range(12) for s in layer] + [(d, 50257)]


def smollm2_360m_step():
    """SmolLM2-360M decode step: 32 Llama layers (q, k, v, o, gate, up, down), then the LM head."""
    h = 960
    layer = [(h, h), (h, 320), (h, 320), (h, h), (h, 2560), (h, 2560), (2560, h)]
    return [s for _ in range(32) for s in layer] + [(h, 49152)]


def smollm2_360m_step_fused():
    """SmolLM2-360M decode step with the shared-input projections stacked by
    rows: q|k|v 960->1600, o 960->960, gate|up 960->5120, down 2560->960
    (x 32 layers), then the LM head. Same weight bytes, 129 products."""
    h = 960
    layer = [(h, 1600), (h, h), (h, 5120), (2560, h)]
    return [s for _ in range(32) for s in layer] + [(h, 49152)]


def smollm2_360m_step_gated():
    """SmolLM2-360M decode step with q|k|v stacked and gate|up as one gated
    product (silu(gate) * up, 2 x 2560 weight rows, 2560 outputs): entries
    (K, M, gated) with gated = 1 for the gated product. 129 products."""
    h = 960
    layer = [(h, 1600, 0), (h, h, 0), (h, 2560, 1), (2560, h, 0)]
    return [s for _ in range(32) for s in layer] + [(h, 49152, 0)]


def smollm2_360m_layer():
    """The 7 matrices of one SmolLM2-360M layer (prefill GEMM workload)."""
    h = 960
    return [(h, h), (h, 320), (h, 320), (h, h), (h, 2560), (h, 2560), (2560, h)]


def smollm2_360m_layer_stacked():
    """The same layer with q|k|v and gate|up stacked: 4 matrices (prefill GEMM)."""
    h = 960
    return [(h, 1600), (h, h), (h, 5120), (2560, h)]


def llama7b_layer():
    """7B-class layer as listed: 4096->4096, 4096->11008 (gate, up) and 11008->4096."""
    return [(4096, 4096), (4096, 11008), (4096, 11008), (11008, 4096)]


# ---------------------------------------------------------------------------
# A whole Llama-family model (float weights only; quantization happens elsewhere).
# ---------------------------------------------------------------------------

SMOLLM2_360M = dict(layers=32, hidden=960, heads=15, kv_heads=5, head_dim=64, ffn=2560, vocab=49152, max_pos=1024,
                    theta=100000.0, eps=1e-5)


def llama_float_weights(cfg: dict, seed: int = 5000):
    """Seeded float32 weights for every matrix of a Llama-family model (keys as
    the decode-step runners use them: emb, qkv{i}, o{i}, gu{i} (gate rows then
    up rows), down{i}) and its norm gains (norm_attn{i}, norm_mlp{i},
    norm_final: 1 + N(0, 0.1)). Matrices ~ N(0, 0.02), the embedding N(0, 0.5)
    so that a token's row is of order one."""
    c = cfg
    qn, kvn = c["heads"] * c["head_dim"], c["kv_heads"] * c["head_dim"]
    out = {"emb": weights(seed, c["vocab"], c["hidden"], 0.5)}
    for i in range(c["layers"]):
        s = seed + 10 * (i + 1)
        out[f"qkv{i}"] = weights(s + 1, qn + 2 * kvn, c["hidden"])
        out[f"o{i}"] = weights(s + 2, c["hidden"], qn)
        out[f"gu{i}"] = weights(s + 3, 2 * c["ffn"], c["hidden"])
        out[f"down{i}"] = weights(s + 4, c["hidden"], c["ffn"])
        out[f"norm_attn{i}"] = (1.0 + activations(s + 5, 1, c["hidden"], 0.1)[0]).astype(np.float32)
        out[f"norm_mlp{i}"] = (1.0 + activations(s + 6, 1, c["hidden"], 0.1)[0]).astype(np.float32)
    out["norm_final"] = (1.0 + activations(seed + 7, 1, c["hidden"], 0.1)[0]).astype(np.float32)
    return out
