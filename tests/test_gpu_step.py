"""GPU parity of the whole decode step (q4_llama_step / the captured graph)
against the float64 reference oracle.llama.Model.

Small Llama-family models run several steps on the device (given tokens, or
chained through the device's own selection, which the oracle then follows);
each step's logits are compared
(normwise, and elementwise against the logits' term scale), the device token
must be a maximum of the reference logits within that error, and the KV cache
must hold the reference's rotated keys and values. The captured graph
reproduces the eager steps bit for bit.
"""
import numpy as np
import pytest

import synth
from gpu_common import say

pytestmark = pytest.mark.gpu

TINY = dict(layers=2, hidden=128, heads=4, kv_heads=2, head_dim=32, ffn=256, vocab=384, max_pos=16, theta=1e4,
            eps=1e-5)
TINY_K = dict(layers=2, hidden=256, heads=8, kv_heads=2, head_dim=32, ffn=512, vocab=300, max_pos=16, theta=1e4,
              eps=1e-5)
LOGIT_TOL = 1e-2  # normwise, per step, after the layers' fp16-activation products compound


@pytest.fixture(scope="module")
def env():
    import torch

    import oracle
    import q4_weight_gemv_amd as q4

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    oracle.lib()
    return torch, q4, oracle


def _build(env, fmt, cfg, seed=5000):
    torch, q4, orc = env
    from oracle import llama

    fw = synth.llama_float_weights(cfg, seed)
    host, dev = {}, {}
    for k, v in fw.items():
        if k.startswith("norm"):
            host[k] = v
            dev[k] = torch.from_numpy(v).cuda()
        else:
            buf = q4.q4_quantize_ref(fmt, v)
            assert np.array_equal(buf, orc.quantize(fmt, v))
            host[k] = buf
            dev[k] = torch.from_numpy(buf).cuda()
    return q4.LlamaStep(fmt, cfg, dev), llama.Model(fmt, cfg, host)


def _check_step(gpu_logits, ref_logits, gpu_token, what):
    rel = np.linalg.norm(gpu_logits - ref_logits) / np.linalg.norm(ref_logits)
    assert rel <= LOGIT_TOL, f"{what}: logits normwise {rel:.2e}"
    err = np.linalg.norm(gpu_logits - ref_logits, np.inf)
    assert ref_logits[gpu_token] >= ref_logits.max() - 2 * err - 1e-6, f"{what}: token {gpu_token} not a maximum"


HD64 = dict(TINY, hidden=256, heads=4, kv_heads=2, head_dim=64, ffn=512)
HD128 = dict(TINY, hidden=256, heads=2, kv_heads=1, head_dim=128, ffn=512)


@pytest.mark.parametrize("fmt,cfg", [(0, TINY), (2, TINY), (1, TINY_K), (3, TINY_K), (4, TINY), (0, HD64), (0, HD128)],
                         ids=["q4_0", "q8_0", "q4_k", "q2_k", "q1_0", "q4_0-d64", "q4_0-d128"])
def test_steps_match_reference(env, fmt, cfg):
    # Six steps with given, distinct tokens: these small random models tend
    # to repeat their input token, and a cache holding the same value at
    # every position would hide the attention weights. The device's own
    # selection and position advance are checked at every step; the chained
    # generation loop is covered by the graph and long-context tests.
    torch, q4, _ = env
    gpu, ref = _build(env, fmt, cfg)
    for pos, token in enumerate((7, 11, 3, 250, 42, 99)):
        gpu.set(token=token, pos=pos)
        say(f"step fmt={fmt} pos={pos}")
        gpu.step()
        torch.cuda.synchronize()
        lg = gpu.buf["logits"].cpu().numpy().astype(np.float64)
        tok = int(gpu.buf["token"].item())
        ref_lg, _ = ref.step(token, pos)
        _check_step(lg, ref_lg, tok, f"fmt {fmt} pos {pos}")
        assert int(gpu.buf["pos"].item()) == pos + 1
    c = cfg
    kc = gpu.buf["k_cache"].cpu().numpy().reshape(c["layers"], c["kv_heads"], c["max_pos"], c["head_dim"])
    vc = gpu.buf["v_cache"].cpu().numpy().reshape(c["layers"], c["kv_heads"], c["max_pos"], c["head_dim"])
    for cache, refc in ((kc, ref.kcache), (vc, ref.vcache)):
        a, b = cache[:, :, :6].astype(np.float64), refc[:, :, :6]
        assert np.linalg.norm(a - b) <= 1e-2 * np.linalg.norm(b)
        assert not np.any(cache[:, :, 6:])  # positions not reached are untouched


def test_graph_replays_match_eager_steps(env):
    torch, q4, _ = env
    eager, _ = _build(env, 0, TINY)
    graph, _ = _build(env, 0, TINY)
    eager.set(token=11, pos=0)
    graph.set(token=11, pos=0)
    say("llama graph capture")
    graph.capture()
    for pos in range(5):
        eager.step()
        graph.replay()
        torch.cuda.synchronize()
        _ = torch.randn(1000, device="cuda").sum().item()  # eager work between replays
        for name in ("logits", "token", "pos", "x", "h"):
            assert torch.equal(eager.buf[name], graph.buf[name]), (pos, name)
    assert torch.equal(eager.buf["k_cache"], graph.buf["k_cache"])
    graph.close()


def test_long_context(env):
    # 100 chained steps; the attention then spans 100 cached positions.
    torch, q4, _ = env
    cfg = dict(TINY, layers=1, max_pos=128)
    gpu, ref = _build(env, 0, cfg, seed=6000)
    gpu.set(token=3, pos=0)
    gpu.capture()
    token = 3
    for pos in range(100):
        gpu.replay()
        torch.cuda.synchronize()
        tok = int(gpu.buf["token"].item())
        ref_lg, _ = ref.step(token, pos)
        if pos % 11 == 0 or pos == 99:
            say(f"long context pos={pos}")
            _check_step(gpu.buf["logits"].cpu().numpy().astype(np.float64), ref_lg, tok, f"pos {pos}")
        token = tok
    assert int(gpu.buf["pos"].item()) == 100
    gpu.close()


def test_smollm2_360m_graph_as_benchmarked(env):
    # The whole SmolLM2-360M step at full size, as the benchmark's generation
    # loop runs it: the same seeded float weights (seed 5000), Q4_0, one
    # captured graph replayed from token 1 at position 0, the tokens chaining
    # on the device. Every one of the first 40 positions is checked against
    # the float64 model.
    torch, q4, _ = env
    cfg = dict(synth.SMOLLM2_360M)
    say("smollm2-360m step: building")
    gpu, ref = _build(env, 0, cfg)
    gpu.set(token=1, pos=0)
    say("smollm2-360m step: capture")
    gpu.capture()
    token = 1
    for pos in range(40):
        gpu.replay()
        torch.cuda.synchronize()
        tok = int(gpu.buf["token"].item())
        ref_lg, _ = ref.step(token, pos)
        _check_step(gpu.buf["logits"].cpu().numpy().astype(np.float64), ref_lg, tok, f"smollm2 pos {pos}")
        token = tok
    say("smollm2-360m step: 40 positions checked")
    assert int(gpu.buf["pos"].item()) == 40
    gpu.close()


def test_position_past_the_cache_is_refused_on_device(env):
    # pos = max_pos: the attention writes NaN, no cache entry is written, the
    # step completes (no fault), and the selection falls back to token 0.
    torch, q4, _ = env
    gpu, _ = _build(env, 0, TINY)
    gpu.set(token=5, pos=TINY["max_pos"])
    gpu.step()
    torch.cuda.synchronize()
    assert torch.isnan(gpu.buf["att"]).all()
    assert not gpu.buf["k_cache"].any() and not gpu.buf["v_cache"].any()
    assert int(gpu.buf["token"].item()) == 0


# Positions on the attention kernel's boundaries: rounds of 512 / 256 / 128
# positions (head_dim 32 / 64 / 128) for keys and values alike, the row
# slices of 32 / 16 / 8 positions inside them (skipped past pos), and the
# last position the scores' LDS holds (8191).
ATT_POSITIONS = [0, 1, 127, 128, 129, 255, 256, 257, 511, 512, 513, 1000, 4097, 8191]


@pytest.mark.parametrize("head_dim,heads,kv_heads", [(32, 8, 2), (64, 4, 2), (128, 2, 1)])
def test_attention_at_long_positions(env, head_dim, heads, kv_heads):
    # One layer; the caches hold random rows (keys scaled so the softmax is
    # far from uniform). After one step at pos, the attention output must be
    # the float64 attention (oracle.llama) of the step's own q|k|v, rotated to
    # pos, over those rows with row pos replaced by the new key and value;
    # and the caches must hold the new rotated key and value at pos.
    # theta = 1 makes every rotation angle the position itself, exact in
    # fp32, so the comparison isolates the attention's reductions (fp32
    # angles pos * theta^(-2i/d) drift by up to ~4e-4 rad at pos 8191, which
    # alone moves the output by ~1e-3; the step tests cover theta = 1e4).
    torch, q4, _ = env
    from oracle import llama

    cfg = dict(TINY, layers=1, hidden=256, heads=heads, kv_heads=kv_heads, head_dim=head_dim, ffn=512,
               max_pos=8192, theta=1.0)
    gpu, _ = _build(env, 0, cfg, seed=6100 + head_dim)
    rng = np.random.default_rng(head_dim)
    shape = (kv_heads, cfg["max_pos"], head_dim)
    kc0 = (10.0 * rng.standard_normal(shape)).astype(np.float32)
    vc0 = rng.standard_normal(shape).astype(np.float32)
    qn, kvn = heads * head_dim, kv_heads * head_dim
    for pos in ATT_POSITIONS:
        gpu.buf["k_cache"].copy_(torch.from_numpy(kc0.reshape(-1)))
        gpu.buf["v_cache"].copy_(torch.from_numpy(vc0.reshape(-1)))
        gpu.set(token=11, pos=pos)
        say(f"attention head_dim={head_dim} pos={pos}")
        gpu.step()
        torch.cuda.synchronize()
        qkv = gpu.buf["qkv"].cpu().numpy().astype(np.float64)
        q = llama.rope(qkv[:qn], pos, cfg["theta"], head_dim)
        k = llama.rope(qkv[qn:qn + kvn], pos, cfg["theta"], head_dim).reshape(kv_heads, head_dim)
        v = qkv[qn + kvn:].reshape(kv_heads, head_dim)
        kc = kc0.astype(np.float64)
        vc = vc0.astype(np.float64)
        kc[:, pos] = k
        vc[:, pos] = v
        ref = llama.attention(q, kc, vc, pos, heads).reshape(heads, head_dim)
        att = gpu.buf["att"].cpu().numpy().astype(np.float64).reshape(heads, head_dim)
        for h in range(heads):
            rel = np.linalg.norm(att[h] - ref[h]) / np.linalg.norm(ref[h])
            assert rel <= 3e-5, (pos, h, rel)
        kg = gpu.buf["k_cache"].cpu().numpy().reshape(shape)
        vg = gpu.buf["v_cache"].cpu().numpy().reshape(shape)
        assert np.allclose(kg[:, pos], k, rtol=1e-5, atol=1e-5 * np.abs(k).max()), pos
        assert np.array_equal(vg[:, pos], v.astype(np.float32)), pos
        others = np.ones(cfg["max_pos"], bool)
        others[pos] = False
        assert np.array_equal(kg[:, others], kc0[:, others]) and np.array_equal(vg[:, others], vc0[:, others])
    gpu.close()
