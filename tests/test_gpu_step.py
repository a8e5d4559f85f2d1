"""GPU parity of the whole decode step (q4_llama_step / the captured graph)
against the float64 reference oracle.llama.Model.

Small Llama-family models run several chained steps on the device; the oracle
follows the tokens the device picks, and each step's logits are compared
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


@pytest.mark.parametrize("fmt,cfg", [(0, TINY), (2, TINY), (1, TINY_K), (3, TINY_K), (4, TINY)],
                         ids=["q4_0", "q8_0", "q4_k", "q2_k", "q1_0"])
def test_steps_match_reference(env, fmt, cfg):
    torch, q4, _ = env
    gpu, ref = _build(env, fmt, cfg)
    gpu.set(token=7, pos=0)
    token = 7
    for pos in range(6):
        say(f"step fmt={fmt} pos={pos}")
        gpu.step()
        torch.cuda.synchronize()
        lg = gpu.buf["logits"].cpu().numpy().astype(np.float64)
        tok = int(gpu.buf["token"].item())
        ref_lg, _ = ref.step(token, pos)
        _check_step(lg, ref_lg, tok, f"fmt {fmt} pos {pos}")
        assert int(gpu.buf["pos"].item()) == pos + 1
        token = tok
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
