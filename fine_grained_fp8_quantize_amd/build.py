"""Build ``libfp8q.so`` (the gfx950 HIP library) in-tree with hipcc.

Usage: ``python -m fine_grained_fp8_quantize_amd.build``. Every HIP source is
compiled for gfx950 only. Packed FP32 instructions are disabled
(``-packed-fp32-ops``): the promotion FMAs and the quantizer arithmetic are
plain ``v_fma_f32``/``v_mul_f32``. No fast-math flags, so fp32 division is
IEEE and denormals are kept.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libfp8q.so")

SOURCES = ["api.cpp", "quant.hip", "gemm.hip"]
HEADERS = ["fp8q_device.h", "gemm_common.h", "launch.h"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950",
    "-mcode-object-version=5",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-command-line-argument",
]


def sources() -> list[str]:
    return [os.path.join(CSRC, s) for s in SOURCES]


def build(force: bool = True, verbose: bool = False) -> str:
    deps = sources() + [os.path.join(CSRC, h) for h in HEADERS] + [os.path.join(INCLUDE, "fp8q.h")]
    if not force and os.path.exists(LIB) and all(os.path.getmtime(LIB) >= os.path.getmtime(d) for d in deps):
        return LIB
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *FLAGS, "-I", INCLUDE, "-I", CSRC, *sources(), "-o", tmp]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so; keep
    # every other diagnostic.
    noise = "'-packed-fp32-ops' is not a recognized feature"
    msgs = [l for l in (res.stdout + res.stderr).splitlines() if noise not in l]
    if msgs:
        print("\n".join(msgs), file=sys.stderr)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed with status %d" % res.returncode)
    # A shared library links with unresolved symbols; bind every symbol now
    # so that a missing kernel stub fails the build, not the first call.
    try:
        ctypes.CDLL(tmp, mode=os.RTLD_NOW | os.RTLD_LOCAL)
    except OSError as e:
        os.unlink(tmp)
        raise RuntimeError("built library does not load: %s" % e) from None
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(force=True, verbose=True))
