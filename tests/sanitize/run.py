"""Host sanitizer tier of the CPU tests.

    python tests/sanitize/run.py asan   # address + undefined-behaviour sanitizers
    python tests/sanitize/run.py tsan   # thread sanitizer on the threaded host quantizer
    python tests/sanitize/run.py        # both

asan: builds the library with its host code instrumented
(-fsanitize=address,undefined on the host side of every unit; the device code
is built as usual) and the C oracle with the same sanitizers, both with
clang, then runs the CPU test suite (pytest -m "not gpu") against them, with
the sanitizer runtime preloaded into Python. Any report fails the run.
tsan: builds the host quantizer with a thread-sanitized driver
(host_threads.cpp) and runs it. Builds go to _build/san/.
"""
from __future__ import annotations

import glob
import importlib.util
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
OUT = os.path.join(ROOT, "_build", "san")
CLANG = "/opt/rocm/llvm/bin/clang"
CLANGXX = "/opt/rocm/llvm/bin/clang++"


def _run(cmd, env=None):
    print("+", " ".join(cmd), flush=True)
    r = subprocess.run(cmd, env=env)
    if r.returncode != 0:
        sys.exit(f"failed ({r.returncode}): {' '.join(cmd)}")


def _runtime(name):
    found = glob.glob(f"/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.{name}-x86_64.so")
    if not found:
        sys.exit(f"no {name} runtime found")
    return found[0]


def asan():
    os.makedirs(OUT, exist_ok=True)
    spec = importlib.util.spec_from_file_location("q4_build", os.path.join(ROOT, "q4_weight_gemv_amd", "build.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    lib = b.build(verbose=True, sanitize="address,undefined", out=os.path.join(OUT, "libq4gemv_asan.so"))
    olib = os.path.join(OUT, "liboracle_asan.so")
    _run([CLANG, "-std=c99", "-O1", "-g", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
          "-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-shared-libsan", "-o", olib,
          os.path.join(ROOT, "oracle", "q4_oracle.c"), "-lm"])
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": _runtime("asan"),
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:halt_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "Q4_GEMV_LIB": lib,
        "Q4_ORACLE_LIB": olib,
    })
    _run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests"), "-q", "-x", "-m", "not gpu",
          "-p", "no:cacheprovider"], env=env)


def tsan():
    os.makedirs(OUT, exist_ok=True)
    exe = os.path.join(OUT, "host_threads_tsan")
    _run([CLANGXX, "-std=c++17", "-O1", "-g", "-fsanitize=thread", "-ffp-contract=off", "-pthread",
          f"-I{os.path.join(ROOT, 'include')}", "-o", exe, os.path.join(HERE, "host_threads.cpp"),
          os.path.join(ROOT, "q4_weight_gemv_amd", "csrc", "q4_host.cpp")])
    env = dict(os.environ, TSAN_OPTIONS="halt_on_error=1")
    _run([exe], env=env)


if __name__ == "__main__":
    what = sys.argv[1] if len(sys.argv) > 1 else "all"
    if what in ("tsan", "all"):
        tsan()
    if what in ("asan", "all"):
        asan()
    print("sanitizer runs clean", flush=True)
