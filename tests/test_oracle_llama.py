"""Pins for the float64 decode-step reference (oracle/llama.py).

Each operator is checked against what mathematics fixes independently of the
code: closed forms, invariances, special cases that reduce to a library
routine (scipy's softmax), and the composition of the step from its parts.
"""
import math

import numpy as np
import pytest

import synth


@pytest.fixture(scope="module")
def L():
    from oracle import llama

    return llama


def test_rmsnorm_closed_forms(L):
    g = np.linspace(0.5, 2.0, 64)
    # constant vector c: x / sqrt(c^2 + eps) = sign(c) / sqrt(1 + eps/c^2)
    h = L.rmsnorm(np.full(64, -3.0), g, 1e-5)
    assert np.allclose(h, -g / math.sqrt(1 + 1e-5 / 9), rtol=1e-15)
    # scale invariance (eps = 0), and the mean square of the output is 1 with g = 1
    x = synth.activations(1, 1, 64)[0].astype(np.float64)
    assert np.allclose(L.rmsnorm(x * 37.0, g, 0.0), L.rmsnorm(x, g, 0.0), rtol=1e-14)
    assert abs(np.mean(L.rmsnorm(x, np.ones(64), 0.0) ** 2) - 1.0) < 1e-14


def test_rope_closed_forms(L):
    d = 64
    v = synth.activations(2, 1, 3 * d)[0].astype(np.float64)
    # position 0 is the identity; rotation keeps each pair's length
    assert np.array_equal(L.rope(v, 0, 1e4, d), v)
    r = L.rope(v, 17, 1e4, d).reshape(3, d)
    vv = v.reshape(3, d)
    assert np.allclose(r[:, :32] ** 2 + r[:, 32:] ** 2, vv[:, :32] ** 2 + vv[:, 32:] ** 2, rtol=1e-13)
    # pair 0 turns by exactly pos radians (theta^0 = 1): e_0 -> (cos p, sin p) in slots 0 and 32
    e = np.zeros(d)
    e[0] = 1.0
    r = L.rope(e, 5, 1e4, d)
    assert r[0] == math.cos(5.0) and r[32] == math.sin(5.0) and not np.any(np.delete(r, [0, 32]))
    # pair i turns by pos * theta^(-2i/d): i = 16 with theta = 100 gives pos / 10
    e = np.zeros(d)
    e[16 + 32] = 1.0
    r = L.rope(e, 3, 100.0, d)
    assert np.isclose(r[16 + 32], math.cos(0.3), rtol=1e-15) and np.isclose(r[16], -math.sin(0.3), rtol=1e-15)
    # rotations compose: position a then b equals position a + b
    assert np.allclose(L.rope(L.rope(v, 4, 1e4, d), 9, 1e4, d), L.rope(v, 13, 1e4, d), rtol=1e-12, atol=1e-14)


def test_attention_special_cases(L):
    from scipy.special import softmax

    rng = np.random.default_rng(3)
    heads, kvh, d, T = 6, 2, 16, 9
    q = rng.standard_normal(heads * d)
    kc = rng.standard_normal((kvh, T, d))
    vc = rng.standard_normal((kvh, T, d))
    # one position: every head returns its group's v_0 exactly
    out = L.attention(q, kc, vc, 0, heads).reshape(heads, d)
    for h in range(heads):
        assert np.array_equal(out[h], vc[h // 3, 0])
    # equal keys: uniform weights, the mean of the values
    kc2 = np.repeat(kc[:, :1], T, axis=1)
    out = L.attention(q, kc2, vc, 5, heads).reshape(heads, d)
    assert np.allclose(out[4], vc[1, :6].mean(axis=0), rtol=1e-13)
    # against scipy's softmax, and only positions <= pos and the right group are read
    pos = 6
    out = L.attention(q, kc, vc, pos, heads).reshape(heads, d)
    for h in range(heads):
        g = h // 3
        w = softmax(kc[g, : pos + 1] @ q.reshape(heads, d)[h] / math.sqrt(d))
        assert np.allclose(out[h], w @ vc[g, : pos + 1], rtol=1e-12)
    kc3, vc3 = kc.copy(), vc.copy()
    kc3[:, pos + 1:] = 1e3
    vc3[:, pos + 1:] = 1e3
    assert np.array_equal(L.attention(q, kc3, vc3, pos, heads), out.reshape(-1))


def _tiny_model(fmt=0, layers=2):
    import oracle

    cfg = dict(layers=layers, hidden=128, heads=4, kv_heads=2, head_dim=32, ffn=256, vocab=384, max_pos=16,
               theta=1e4, eps=1e-5)
    c = cfg
    qn, kvn = c["heads"] * c["head_dim"], c["kv_heads"] * c["head_dim"]
    bufs = {"emb": oracle.quantize(fmt, synth.weights(10, c["vocab"], c["hidden"], 0.5))}
    for i in range(layers):
        bufs[f"qkv{i}"] = oracle.quantize(fmt, synth.weights(20 + i, qn + 2 * kvn, c["hidden"], 0.1))
        bufs[f"o{i}"] = oracle.quantize(fmt, synth.weights(30 + i, c["hidden"], qn, 0.1))
        bufs[f"gu{i}"] = oracle.quantize(fmt, synth.weights(40 + i, 2 * c["ffn"], c["hidden"], 0.1))
        bufs[f"down{i}"] = oracle.quantize(fmt, synth.weights(50 + i, c["hidden"], c["ffn"], 0.1))
        bufs[f"norm_attn{i}"] = 1.0 + synth.activations(60 + i, 1, c["hidden"], 0.1)[0]
        bufs[f"norm_mlp{i}"] = 1.0 + synth.activations(70 + i, 1, c["hidden"], 0.1)[0]
    bufs["norm_final"] = 1.0 + synth.activations(80, 1, c["hidden"], 0.1)[0]
    return cfg, bufs


def test_step_is_the_composition_of_its_parts(L):
    # One layer written out by hand from the operators (and numpy's own
    # sigmoid form of silu) reproduces Model.step over three positions, each
    # step reading the earlier steps' cache entries. The tokens are given,
    # not chained, and distinct: a model that repeats its input token would
    # cache the same value at every position, and attention's output would
    # then not depend on its weights (nor on the keys' rotation).
    import oracle

    cfg, bufs = _tiny_model(layers=1)
    m = L.Model(0, cfg, bufs)
    tokens = (7, 11, 3)
    ref = [m.step(t, pos) for pos, t in enumerate(tokens)]
    c = cfg
    d, H, Hk = c["head_dim"], c["heads"], c["kv_heads"]
    emb = oracle.dequantize(0, bufs["emb"], c["vocab"], c["hidden"]).astype(np.float64)
    W = {n: oracle.dequantize(0, bufs[f"{n}0"], *shape).astype(np.float64) for n, shape in
         (("qkv", (H * d + 2 * Hk * d, c["hidden"])), ("o", (c["hidden"], H * d)),
          ("gu", (2 * c["ffn"], c["hidden"])), ("down", (c["hidden"], c["ffn"])))}
    kc = np.zeros((Hk, len(tokens), d))
    vc = np.zeros((Hk, len(tokens), d))
    for pos, tok in enumerate(tokens):
        x = emb[tok]
        h = x / np.sqrt(np.mean(x * x) + c["eps"]) * bufs["norm_attn0"]
        qkv = W["qkv"] @ h
        q = L.rope(qkv[:H * d], pos, c["theta"], d)
        kc[:, pos] = L.rope(qkv[H * d:H * d + Hk * d], pos, c["theta"], d).reshape(Hk, d)
        vc[:, pos] = qkv[H * d + Hk * d:].reshape(Hk, d)
        x = x + W["o"] @ L.attention(q, kc, vc, pos, H)
        h2 = x / np.sqrt(np.mean(x * x) + c["eps"]) * bufs["norm_mlp0"]
        gu = W["gu"] @ h2
        gate = gu[: c["ffn"]]
        x = x + W["down"] @ (gate * (1.0 / (1.0 + np.exp(-gate))) * gu[c["ffn"]:])
        logits = emb @ (x / np.sqrt(np.mean(x * x) + c["eps"]) * bufs["norm_final"])
        assert np.allclose(logits, ref[pos][0], rtol=1e-12, atol=1e-12), pos
        assert int(np.argmax(logits)) == ref[pos][1]
