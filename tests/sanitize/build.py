"""Sanitizer builds for the CPU test suites (AddressSanitizer and
UndefinedBehaviorSanitizer, host code only):

* the C oracle, ``oracle/fp8_oracle.c``, with the oracle's own IEEE flags;
* the C ABI layer, ``csrc/api.cpp``, compiled by g++ as host code and linked
  with ``launch_stubs.cpp`` in place of the GPU kernels (its validation is
  what runs without a GPU).

``python tests/sanitize/build.py OUT_DIR`` writes ``liboracle_asan.so`` and
``libfp8q_host_asan.so`` there and prints the environment that makes the
oracle and the binding load them (``FP8Q_ORACLE_LIBRARY``,
``FP8Q_LIBRARY``) with the ASan runtime preloaded.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
CSRC = os.path.join(ROOT, "fine_grained_fp8_quantize_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g", "-O1"]


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("%s\n%s%s" % (" ".join(cmd), res.stdout, res.stderr))


def build(out_dir: str) -> dict:
    os.makedirs(out_dir, exist_ok=True)
    oracle_so = os.path.join(out_dir, "liboracle_asan.so")
    _run(["gcc", *SAN, "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared",
          "-Wall", "-Wextra", os.path.join(ROOT, "oracle", "fp8_oracle.c"), "-o", oracle_so, "-lm"])
    api_so = os.path.join(out_dir, "libfp8q_host_asan.so")
    _run(["g++", *SAN, "-std=c++17", "-fPIC", "-shared", "-Wall", "-D__HIP_PLATFORM_AMD__",
          "-I", "/opt/rocm/include", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
          os.path.join(CSRC, "api.cpp"), os.path.join(HERE, "launch_stubs.cpp"), "-o", api_so,
          "-L", "/opt/rocm/lib", "-Wl,-rpath,/opt/rocm/lib", "-lamdhip64"])
    asan_rt = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True,
                             check=True).stdout.strip()
    return {
        "LD_PRELOAD": asan_rt,
        "ASAN_OPTIONS": "detect_leaks=0:detect_odr_violation=0:alloc_dealloc_mismatch=0:"
                        "abort_on_error=1:verify_asan_link_order=0",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "FP8Q_ORACLE_LIBRARY": oracle_so,
        "FP8Q_LIBRARY": api_so,
    }


if __name__ == "__main__":
    for k, v in build(sys.argv[1] if len(sys.argv) > 1 else os.path.join(ROOT, "_build", "asan")).items():
        print("%s=%s" % (k, v))
