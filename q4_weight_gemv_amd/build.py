"""Build the in-tree shared library ``libq4gemv.so`` for gfx950 with hipcc.

Every .hip source is compiled for gfx950 only; the host quantizer (.cpp) is
compiled as plain C++ with floating-point contraction off. Run as a script
(``python q4_weight_gemv_amd/build.py``) or through ``__graft_entry__.build()``;
it does not import the package (which would load the library being rebuilt).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJ = os.path.join(ROOT, "_build", "obj")
LIB = os.path.join(HERE, "libq4gemv.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = ["-std=c++17", "-fPIC", "-Wall", "-Wextra", "-Wno-unused-parameter", f"-I{INCLUDE}", f"-I{CSRC}"]
# Packed fp32 VALU forms are kept out of the device code.
DEVICE = ["-O3", f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-ffp-contract=fast", "-munsafe-fp-atomics"]
# -O2 for the host quantizer: clang's -O3 loop passes take many minutes on it.
HOST_ONLY = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-pthread"]

SOURCES = [
    ("q4_host.cpp", "host"),
    ("q4_gemv.hip", "device"),
    ("q4_gemv_q4_0_a.hip", "device"),
    ("q4_gemv_q4_0_b.hip", "device"),
    ("q4_gemv_q4_k_a.hip", "device"),
    ("q4_gemv_q4_k_b.hip", "device"),
    ("q4_gemv_q8_0_a.hip", "device"),
    ("q4_gemv_q8_0_b.hip", "device"),
    ("q4_gemv_q2_k_a.hip", "device"),
    ("q4_gemv_q2_k_b.hip", "device"),
    ("q4_gemv_q1_0_a.hip", "device"),
    ("q4_gemv_q1_0_b.hip", "device"),
    ("q4_gemv_norm_a.hip", "device"),
    ("q4_gemv_norm_b.hip", "device"),
    ("q4_gemv_stream.hip", "device"),
    ("q4_gemv_mfma.hip", "device"),
    ("q4_gemm.hip", "device"),
    ("q4_stack.hip", "device"),
    ("q4_step.hip", "device"),
    ("q4_bench.hip", "device"),
]


# Host sanitizers for a test build (sanitize="address,undefined"): the host
# code of every unit is instrumented, the device code is built as usual.
def _host_sanitizer_flags(sanitize: str | None, device_unit: bool) -> list:
    if not sanitize:
        return []
    if device_unit:
        return ["-Xarch_host", f"-fsanitize={sanitize}", "-Xarch_host", "-fno-omit-frame-pointer"]
    return [f"-fsanitize={sanitize}", "-fno-omit-frame-pointer"]


def _compile(src: str, kind: str, obj_dir: str = OBJ, sanitize: str | None = None) -> str:
    out = os.path.join(obj_dir, os.path.splitext(src)[0] + ".o")
    path = os.path.join(CSRC, src)
    if kind == "host":
        cmd = [HIPCC, "-x", "c++"] + COMMON + HOST_ONLY + _host_sanitizer_flags(sanitize, False) + ["-c", path, "-o", out]
    else:
        cmd = [HIPCC, "-x", "hip"] + COMMON + DEVICE + _host_sanitizer_flags(sanitize, True) + ["-c", path, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return out


def build(verbose: bool = False, sanitize: str | None = None, out: str | None = None) -> str:
    """Build the library (``out``, default the in-tree libq4gemv.so). With
    ``sanitize`` (e.g. "address,undefined") the host code is instrumented and
    the objects go to their own folder; load such a build by pointing
    Q4_GEMV_LIB at it, with the sanitizer runtime preloaded."""
    lib = out or LIB
    obj_dir = OBJ if not sanitize else os.path.join(ROOT, "_build", "obj_" + sanitize.replace(",", "_"))
    os.makedirs(obj_dir, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda s: _compile(*s, obj_dir=obj_dir, sanitize=sanitize), SOURCES))
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-pthread", "-o", tmp] + objs
    if sanitize:
        cmd += ["-Xarch_host", f"-fsanitize={sanitize}", "-shared-libsan"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


if __name__ == "__main__":
    if not shutil.which(HIPCC) and not os.path.exists(HIPCC):
        sys.exit("hipcc not found")
    build(verbose=True)
