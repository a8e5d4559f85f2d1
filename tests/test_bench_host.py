"""Host-side pieces of bench.py that its reported figures rest on (CPU only):
the algorithmic bytes that GB/s and the roofline divide by, the cold-cache
rotation, the rule that HBM traffic is reported only from counters taken on
the current kernel sources, and the refusal of more than one GPU."""
import os
import subprocess
import sys

import pytest

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def q4():
    import q4_weight_gemv_amd as q4

    return q4


def test_gpt2_step_algorithmic_bytes(q4):
    # Per product: Q4_0 weights (a 16-byte code block and a 2-byte scale per
    # 32 weights: M*K*9/16 bytes), fp32 x in, fp32 y out.
    shapes = synth.gpt2_124m_step()
    assert len(shapes) == 49
    total = sum(bench.gemv_bytes(q4, 0, m, k, 1) for k, m in shapes)
    assert total == sum(m * k * 9 // 16 + 4 * (k + m) for k, m in shapes)
    assert total == 70_280_692


def test_batched_and_gated_product_bytes(q4):
    # n tokens read n activation rows and write n output rows; a gated
    # product reads 2m weight rows and writes m outputs.
    assert bench.gemv_bytes(q4, 0, 4096, 4096, 8) == 4096 * 4096 * 9 // 16 + 4 * 8 * (4096 + 4096)
    assert bench.gemv_bytes(q4, 0, 2560, 960, 1, gated=1) == 2 * 2560 * 960 * 9 // 16 + 4 * (960 + 2560)
    assert bench.gemv_bytes(q4, 1, 4096, 4096, 1) == 4096 * 4096 // 256 * 144 + 4 * (4096 + 4096)


def test_cold_rotation_reads_past_the_caches():
    # Between two reads of one weight copy, the other copies (at least 512
    # MiB, twice the 256 MB memory-side cache) pass through.
    for nbytes in (1 << 20, 9_437_184, 70_280_692, 203_489_280, 1 << 30):
        c = bench.copies_for(nbytes)
        assert c >= 2 and (c - 1) * nbytes >= 512 << 20, (nbytes, c)


def test_headline_layer_bytes(q4):
    # The headline step: the 7B-class layer as listed (4096->4096,
    # 4096->11008 x2, 11008->4096) in Q4_0 at one token.
    shapes = synth.llama7b_layer()
    assert shapes == [(4096, 4096), (4096, 11008), (4096, 11008), (11008, 4096)]
    weights = sum(m * k * 9 // 16 for k, m in shapes)
    assert weights == 85_524_480
    assert sum(bench.gemv_bytes(q4, 0, m, k, 1) for k, m in shapes) == weights + 4 * sum(k + m for k, m in shapes)
    k, m = bench.DOMINANT
    assert (k, m) in shapes and bench.gemv_bytes(q4, 0, m, k, 1) == 25_362_432 + 4 * (4096 + 11008)


def test_profile_figures_reported_only_for_matching_sources(tmp_path):
    h = bench.kernel_source_hash()
    good = tmp_path / "good.txt"
    good.write_text(f"kernel_source_sha256: {h}\nhbm_bytes_per_launch: 1570923\nmedian_us: 7.125\n")
    assert bench.traffic_from_profile(str(good)) == 1570923.0
    assert bench.trace_median_from_profile(str(good)) == 7.125
    other = "0" * 16 if h != "0" * 16 else "1" * 16
    stale = tmp_path / "stale.txt"
    stale.write_text(f"kernel_source_sha256: {other}\nhbm_bytes_per_launch: 1570923\nmedian_us: 7.125\n")
    assert bench.traffic_from_profile(str(stale)) is None
    assert bench.trace_median_from_profile(str(stale)) is None
    assert bench.traffic_from_profile(str(tmp_path / "missing.txt")) is None
    good.write_text(f"kernel_source_sha256: {h}\nkernel_us_per_step: 125.0\n")
    stale.write_text(f"kernel_source_sha256: {other}\nkernel_us_per_step: 125.0\n")
    busy = bench.device_busy("good.txt", str(good))
    assert busy["kernel_us_per_step"] == 125.0 and busy["tokens_per_s"] == 8000.0
    assert bench.device_busy("stale.txt", str(stale)) is None


def test_source_hash_covers_the_headline_kernel():
    # The one-token decode kernels (streaming and tiled), their Q4_0
    # instantiation units and the host code that picks between them.
    for f in ("q4_gemv_kernel.h", "q4_gemv_stream.h", "q4_gemv.hip", "q4_gemv_stream.hip", "q4_gemv_q4_0_a.hip",
              "q4_gemv_q4_0_b.hip"):
        assert f in bench.KERNEL_SOURCES
        assert os.path.exists(os.path.join(ROOT, "q4_weight_gemv_amd", "csrc", f))


def test_cpu_share_and_host_description():
    cores, model = bench.host_cpu()
    assert cores >= 1 and isinstance(model, str) and model
    assert bench.CPU_SHARE == 16


def test_more_than_one_gpu_is_refused():
    for args, env in ((["--gpus", "2"], {}), (["--gpus", "1"], {"WORLD_SIZE": "2"})):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args, capture_output=True, text=True,
                           timeout=120, env=dict(os.environ, **env))
        assert r.returncode == 2, r.stderr
        assert "one GPU" in r.stdout
