"""The C ABI's host code under AddressSanitizer (CPU only).

build() also links libgq_asan.so, the same library with AddressSanitizer on its host
code (argument checks, workspace sizing, the error string, the static entry point's
size checks, timing reads).  This test runs the CPU ABI tests (tests/test_abi.py) in a
child process that preloads the sanitizer runtime and loads that library instead of
libgq.so, so an invalid host memory access on any of those paths ends the child with a
sanitizer report.  GPU code is not sanitized.
"""
import os
import subprocess
import sys

import pytest

from post_weight_quantization_gq_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _env(rt):
    env = os.environ.copy()
    env["LD_PRELOAD"] = rt
    env["GQ_LIBRARY"] = B.LIB_ASAN
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1"
    env["PYTHONPATH"] = ROOT + os.pathsep + env.get("PYTHONPATH", "")
    return env


def test_abi_checks_under_address_sanitizer():
    rt = B.asan_runtime()
    if rt is None:
        pytest.skip("this ROCm install has no AddressSanitizer runtime")
    if not os.path.exists(B.LIB_ASAN):
        B.build(asan=True)
    env = _env(rt)
    # the child really runs the sanitized library under the runtime
    probe = subprocess.run(
        [sys.executable, "-c",
         "import ctypes, post_weight_quantization_gq_amd as gq\n"
         "lib = gq.library()\n"
         "assert lib._name.endswith('libgq_asan.so'), lib._name\n"
         "assert hasattr(ctypes.CDLL(None), '__asan_init')\n"
         "print('loaded', lib._name)\n"],
        cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert probe.returncode == 0, probe.stdout + probe.stderr
    run = subprocess.run(
        [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
         os.path.join(ROOT, "tests", "test_abi.py")],
        cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = run.stdout + run.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert run.returncode == 0, out[-4000:]
    assert " passed" in out, out[-2000:]
