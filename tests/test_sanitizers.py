"""The CPU suites of the oracle and of the C ABI's host-side validation, run
again under AddressSanitizer and UndefinedBehaviorSanitizer: both C/C++
libraries are rebuilt with the sanitizers (tests/sanitize/build.py; the ABI
layer is host code, linked with launcher stubs that fail as a machine
without a GPU does) and the two test files run in a child process that loads
those builds with the ASan runtime preloaded. Any sanitizer report aborts the
child, which fails this test."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "sanitize"))

PROBE = ("import fine_grained_fp8_quantize_amd as fq, oracle;"
         "fq._load(); oracle.lib();"
         "maps = open('/proc/self/maps').read();"
         "assert 'libasan' in maps, 'ASan runtime not loaded';"
         "assert 'liboracle_asan.so' in maps and 'libfp8q_host_asan.so' in maps, 'sanitizer builds not loaded';"
         "print('sanitized builds loaded')")


@pytest.mark.skipif(shutil.which("gcc") is None or shutil.which("g++") is None, reason="needs gcc and g++")
def test_oracle_and_abi_suites_under_asan_ubsan(tmp_path):
    import build as san_build
    env = dict(os.environ)
    env.update(san_build.build(str(tmp_path)))
    root = os.path.dirname(HERE)
    env["PYTHONPATH"] = os.pathsep.join([root, HERE] + [p for p in env.get("PYTHONPATH", "").split(os.pathsep) if p])
    probe = subprocess.run([sys.executable, "-c", PROBE], cwd=root, env=env, capture_output=True, text=True,
                           timeout=300)
    assert probe.returncode == 0, probe.stdout + probe.stderr
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                          os.path.join(HERE, "test_abi.py"), os.path.join(HERE, "test_oracle.py")],
                         cwd=root, env=env, capture_output=True, text=True, timeout=1200)
    tail = (res.stdout + res.stderr)[-4000:]
    assert res.returncode == 0, tail
    assert "passed" in res.stdout and "ERROR: AddressSanitizer" not in tail and "runtime error" not in tail, tail
