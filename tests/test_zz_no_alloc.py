"""GPU test of q4_llama_step_noalloc, the decode step whose intermediate
vectors live in the library's static device array, against q4_llama_step with
caller-owned buffers: the same model, token and positions must give the same
logits, token, position, residual stream and caches bit for bit (the two run
the same kernels). Two models in a row, the second smaller, so the second
call reuses the array after the first left its contents there; and a model
too large for the array is refused before anything is enqueued.
"""
import numpy as np
import pytest

import synth
from gpu_common import say

pytestmark = pytest.mark.gpu

LARGER = dict(layers=2, hidden=256, heads=4, kv_heads=2, head_dim=64, ffn=512, vocab=384, max_pos=16, theta=1e4,
              eps=1e-5)
SMALLER = dict(layers=2, hidden=128, heads=4, kv_heads=2, head_dim=32, ffn=256, vocab=300, max_pos=16, theta=1e4,
               eps=1e-5)


@pytest.fixture(scope="module")
def env():
    import torch

    import q4_weight_gemv_amd as q4

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch, q4


def _weights(torch, q4, cfg, seed):
    dev = {}
    for name, v in synth.llama_float_weights(cfg, seed).items():
        dev[name] = torch.from_numpy(v if name.startswith("norm") else q4.q4_quantize_ref(0, v)).cuda()
    return dev


def test_noalloc_step_matches_step(env):
    torch, q4 = env
    for cfg, seed, token in ((LARGER, 7100, 11), (SMALLER, 7200, 5)):
        w = _weights(torch, q4, cfg, seed)
        ref = q4.LlamaStep(0, cfg, w)
        got = q4.LlamaStep(0, cfg, w)
        ref.set(token=token, pos=0)
        got.set(token=token, pos=0)
        for pos in range(3):
            say(f"noalloc step hidden={cfg['hidden']} pos={pos}")
            ref.step()
            got.step_noalloc()
            torch.cuda.synchronize()
            for name in ("logits", "token", "pos", "x", "h", "k_cache", "v_cache"):
                assert torch.equal(ref.buf[name], got.buf[name]), (cfg["hidden"], pos, name)
        assert np.isfinite(got.buf["logits"].cpu().numpy()).all()
        # The caller's workspace buffers were not used.
        for name in ("qkv", "att", "delta", "act"):
            assert not torch.any(got.buf[name]), name


def test_noalloc_step_refuses_a_model_beyond_its_array(env):
    torch, q4 = env
    w = _weights(torch, q4, LARGER, 7100)
    # (4 + 4) * 64 + 4 * 64 + 256 + 65536 floats > 65536.
    big = q4.LlamaStep(0, dict(LARGER, ffn=65536), w)
    big.set(token=1, pos=0)
    torch.cuda.synchronize()
    with pytest.raises(q4.Q4Error) as e:
        big.step_noalloc()
    assert e.value.status == q4.Q4_EUNSUPPORTED
    torch.cuda.synchronize()
    assert int(big.buf["pos"].item()) == 0  # nothing was enqueued
    assert not torch.any(big.buf["k_cache"])


def test_noalloc_step_under_caller_graph_capture(env):
    # The callers it is for: one call on the device outside capture (the
    # array's address is looked up then), then the step captured into the
    # caller's own graph (torch's, on its capture stream) and replayed as a
    # generation loop: every replay, with eager work and synchronizations
    # between them, equals q4_llama_step on an identical model bit for bit.
    torch, q4 = env
    cfg = SMALLER
    w = _weights(torch, q4, cfg, 7300)
    first = q4.LlamaStep(0, cfg, w)
    first.set(token=1, pos=0)
    first.step_noalloc()
    ref = q4.LlamaStep(0, cfg, w)
    got = q4.LlamaStep(0, cfg, w)
    ref.set(token=9, pos=0)
    got.set(token=9, pos=0)
    torch.cuda.synchronize()
    say("noalloc step under caller capture")
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        got.step_noalloc()
    torch.cuda.synchronize()
    # Capture enqueues nothing to run: the state is as set.
    assert int(got.buf["pos"].item()) == 0
    for pos in range(4):
        ref.step()
        graph.replay()
        torch.cuda.synchronize()
        _ = torch.randn(1000, device="cuda").sum().item()  # eager work between replays
        for name in ("logits", "token", "pos", "x", "h", "k_cache", "v_cache"):
            assert torch.equal(ref.buf[name], got.buf[name]), (pos, name)
    assert int(got.buf["pos"].item()) == 4
    del graph
