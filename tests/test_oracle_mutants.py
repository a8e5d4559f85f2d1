"""The oracle's pins catch plausible mistakes (CPU only).

Each case plants one mistake in a copy of the oracle's C source: a wrong
rounding rule, a dropped or mis-signed term, a wrong index, offset or
operand, a swapped field. The copy is built with the oracle's own flags and
the oracle's pin suites (tests/test_oracle_*.py) run against it in a
subprocess; at least one pin must fail. The float64 decode-step reference
(oracle/llama.py) gets the same treatment: a copy of the oracle package with
one mistake in it is imported in place of the original, and its pins must
fail. The pins compare the oracle with
values fixed from outside it (hand-worked blocks, exact rationals, closed
forms, library routines), so a mistake that none of them notices would be
one the oracle could carry into every parity test.
"""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PINS = sorted(p for p in glob.glob(os.path.join(ROOT, "tests", "test_oracle_*.py")) if not p.endswith("_mutants.py"))

# (name, exact text of the oracle source, planted replacement)
MUTANTS = [
    ("fp16_ties_away",
     "    if (frac > 0.5 || (frac == 0.5 && fmod(nf, 2.0) != 0.0)) nf += 1.0;\n    /* nf * 2^(E-10)",
     "    if (frac >= 0.5) nf += 1.0;\n    /* nf * 2^(E-10)"),
    ("fp16_subnormal_binade", "if (E < -14) E = -14;", "if (E < -15) E = -15;"),
    ("bf16_truncates",
     "    if (frac > 0.5 || (frac == 0.5 && fmod(nf, 2.0) != 0.0)) nf += 1.0;\n    double r = ldexp(nf, E - 7);",
     "    double r = ldexp(nf, E - 7);"),
    ("q4_0_scale_divisor", "float d32 = amax / 7.0f;", "float d32 = amax / 8.0f;"),
    ("q4_0_round_half_up", "q[i] = clampi((int)round_half_away(t) + 8, 0, 15);",
     "q[i] = clampi((int)floor(t + 0.5) + 8, 0, 15);"),
    ("q4_0_interleaved_nibbles", "nib[j] = (uint8_t)(q[j] | (q[j + 16] << 4));",
     "nib[j] = (uint8_t)(q[2 * j] | (q[2 * j + 1] << 4));"),
    ("q4_0_offset", "return (float)(q - 8) * d;", "return (float)(q - 7) * d;"),
    ("q4_0_nibbles_swapped", "int q = (e < 16) ? (blk[e] & 0x0F) : (blk[e - 16] >> 4);",
     "int q = (e < 16) ? (blk[e] >> 4) : (blk[e - 16] & 0x0F);"),
    ("q4_0_scale_plane_transposed", "const uint8_t *s = buf + (size_t)(m * k / 2) + (r * nb + b) * 2;",
     "const uint8_t *s = buf + (size_t)(m * k / 2) + (b * m + r) * 2;"),
    ("q4_k_min_sign", "    float b = dmin * (float)mn[j];\n    return a - b;",
     "    float b = dmin * (float)mn[j];\n    return a + b;"),
    ("q4_k_upper_scale_field", "sc[j] = (uint8_t)((S[j + 4] & 15) | ((S[j - 4] >> 6) << 4));",
     "sc[j] = (uint8_t)((S[j + 4] >> 4) | ((S[j - 4] >> 6) << 4));"),
    ("q4_k_nibble_halves", "int q = hi ? (byte >> 4) : (byte & 15);", "int q = hi ? (byte & 15) : (byte >> 4);"),
    ("q4_k_min_offset_sign",
     "q[32 * j + i] = (uint8_t)(step == 0.0 ? 0 : clampi((int)round_half_away((v + off) / step), 0, 15));",
     "q[32 * j + i] = (uint8_t)(step == 0.0 ? 0 : clampi((int)round_half_away((v - off) / step), 0, 15));"),
    ("q8_0_asymmetric_clamp", "clampi((int)round_half_away(t), -127, 127)", "clampi((int)round_half_away(t), -128, 127)"),
    ("q2_k_min_field", "float b = dmin * (float)(scm >> 4);", "float b = dmin * (float)(scm & 15);"),
    ("q1_0_zero_sign", "if (w[i] >= 0.0f) word |= (uint32_t)1 << i;", "if (w[i] > 0.0f) word |= (uint32_t)1 << i;"),
    ("q1_0_scale_via_fp32", "uint16_t dh = oracle_f64_to_fp16(sum / 32.0);",
     "uint16_t dh = oracle_fp32_to_fp16((float)(sum / 32.0));"),
    ("matvec_fp32_accumulation",
     "            double acc = 0.0;\n            for (int64_t c = 0; c < k; c++)\n"
     "                acc += (double)weight_at(fmt, w, m, k, i, c) * (double)x[t * k + c];",
     "            float acc = 0.0f;\n            for (int64_t c = 0; c < k; c++)\n"
     "                acc += (float)weight_at(fmt, w, m, k, i, c) * x[t * k + c];"),
    ("matvec_token_index",
     "                acc += (double)weight_at(fmt, w, m, k, i, c) * (double)x[t * k + c];\n            y[t * m + i]",
     "                acc += (double)weight_at(fmt, w, m, k, i, c) * (double)x[c * n + t];\n            y[t * m + i]"),
    ("matmul_bf16_flag_inverted", "if (round_w_bf16) wv = oracle_bf16_to_fp32(oracle_fp32_to_bf16(wv));",
     "if (!round_w_bf16) wv = oracle_bf16_to_fp32(oracle_fp32_to_bf16(wv));"),
    ("silu_sign", "double silu = g / (1.0 + exp(-g));", "double silu = g / (1.0 + exp(g));"),
]


def _run_pins(tmp_path, source):
    import oracle

    copy = tmp_path / "q4_oracle_copy.c"
    copy.write_text(source)
    lib = oracle.build(force=True, src=str(copy), out=str(tmp_path / "liboracle_copy.so"))
    return subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu", "-p", "no:cacheprovider"] + PINS,
                          cwd=ROOT, env=dict(os.environ, Q4_ORACLE_LIB=lib), capture_output=True, text=True,
                          timeout=600)


def test_unmutated_copy_passes(tmp_path):
    # The harness itself: the unchanged source, built and loaded the same
    # way, passes every pin (so a failure below is the planted mistake's).
    import oracle

    r = _run_pins(tmp_path, open(oracle.SRC).read())
    assert r.returncode == 0, r.stdout[-1500:]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_fails_a_pin(tmp_path, name, old, new):
    import oracle

    src = open(oracle.SRC).read()
    assert src.count(old) == 1, f"{name}: the text to mutate must occur exactly once"
    r = _run_pins(tmp_path, src.replace(old, new))
    assert r.returncode == 1 and " failed" in r.stdout, f"{name} was not caught:\n{r.stdout[-1500:]}\n{r.stderr[-500:]}"


# Mistakes in the float64 decode step (oracle/llama.py).
LLAMA_MUTANTS = [
    ("rmsnorm_eps_outside_root", "x / math.sqrt(float(np.mean(x * x)) + eps)",
     "x / (math.sqrt(float(np.mean(x * x))) + eps)"),
    ("rope_sign", "out[:, :half] = v[:, :half] * c - v[:, half:] * s", "out[:, :half] = v[:, :half] * c + v[:, half:] * s"),
    ("rope_frequency", "a = pos * theta ** (-2.0 * i / head_dim)", "a = pos * theta ** (-1.0 * i / head_dim)"),
    ("attention_scale", "s = k @ q[h] / math.sqrt(d)", "s = k @ q[h] / d"),
    ("attention_group_map", "k = kcache[h // group, : pos + 1]\n        v = vcache[h // group, : pos + 1]",
     "k = kcache[h % kv_heads, : pos + 1]\n        v = vcache[h % kv_heads, : pos + 1]"),
    ("attention_reads_one_past", "k = kcache[h // group, : pos + 1]", "k = kcache[h // group, : pos + 2]"),
    ("step_mlp_norm_weight", "h2 = rmsnorm(x, L[\"norm_mlp\"], c[\"eps\"])", "h2 = rmsnorm(x, L[\"norm_attn\"], c[\"eps\"])"),
    ("step_gate_up_swapped", "delta = L[\"down\"] @ (silu(gu[: c[\"ffn\"]]) * gu[c[\"ffn\"]:])",
     "delta = L[\"down\"] @ (silu(gu[c[\"ffn\"]:]) * gu[: c[\"ffn\"]])"),
    ("step_value_not_rotated_key", "k = rope(qkv[q_n:q_n + kv_n], pos, c[\"theta\"], d)", "k = qkv[q_n:q_n + kv_n]"),
]


def _run_llama_pins(tmp_path, source):
    import oracle

    pkg = tmp_path / "oracle"
    shutil.copytree(os.path.dirname(oracle.SRC), pkg, ignore=shutil.ignore_patterns("__pycache__"))
    (pkg / "llama.py").write_text(source)
    env = dict(os.environ, PYTHONPATH=ROOT)
    env.pop("Q4_ORACLE_LIB", None)
    where = subprocess.run([sys.executable, "-c", "import oracle.llama as m; print(m.__file__)"], cwd=tmp_path, env=env,
                           capture_output=True, text=True, timeout=120)
    assert where.stdout.strip() == str(pkg / "llama.py"), where.stdout + where.stderr  # the copy is what runs
    return subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu", "-p", "no:cacheprovider",
                           os.path.join(ROOT, "tests", "test_oracle_llama.py")],
                          cwd=tmp_path, env=env, capture_output=True, text=True, timeout=600)


def test_unmutated_llama_copy_passes(tmp_path):
    import oracle

    r = _run_llama_pins(tmp_path, open(os.path.join(os.path.dirname(oracle.SRC), "llama.py")).read())
    assert r.returncode == 0, r.stdout[-1500:]


@pytest.mark.parametrize("name,old,new", LLAMA_MUTANTS, ids=[m[0] for m in LLAMA_MUTANTS])
def test_planted_llama_mistake_fails_a_pin(tmp_path, name, old, new):
    import oracle

    src = open(os.path.join(os.path.dirname(oracle.SRC), "llama.py")).read()
    assert src.count(old) == 1, f"{name}: the text to mutate must occur exactly once"
    r = _run_llama_pins(tmp_path, src.replace(old, new))
    assert r.returncode == 1 and " failed" in r.stdout, f"{name} was not caught:\n{r.stdout[-1500:]}\n{r.stderr[-500:]}"
