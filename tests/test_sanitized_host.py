"""The C ABI's host logic under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

libllama_layer_asan.so is the same library with its host code instrumented (``python -m
transformer_layer_forward_amd.build --sanitize``; built here when missing or older than the sources). The
C-ABI checks of tests/test_abi.py (symbol exports, struct layouts, every argument-validation path, workspace
size queries and the no-allocation entry point's limit) run against it in a child process that preloads
the compiler's ASan runtime; any sanitizer report fails the child and this test. No device code runs.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "transformer_layer_forward_amd")
ASAN_LIB = os.path.join(PKG, "libllama_layer_asan.so")


def _stale():
    if not os.path.exists(ASAN_LIB):
        return True
    t = os.path.getmtime(ASAN_LIB)
    srcs = glob.glob(os.path.join(PKG, "csrc", "*")) + glob.glob(os.path.join(ROOT, "include", "*.h"))
    return any(os.path.getmtime(p) > t for p in srcs)


def test_abi_checks_under_asan_and_ubsan():
    if os.environ.get("LD_PRELOAD"):
        pytest.skip("a preload is already configured in this environment; it is left untouched")
    from transformer_layer_forward_amd import build
    try:
        runtime = build.asan_runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    if _stale():
        build.build(sanitize=True)
    env = dict(os.environ, LLAMA_LAYER_LIB=ASAN_LIB, LD_PRELOAD=runtime,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    probe = ("import transformer_layer_forward_amd as L; L.load(); "
             "print([l.split()[-1] for l in open('/proc/self/maps') if 'libllama_layer' in l][0])")
    p = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert p.returncode == 0 and p.stdout.strip().endswith("libllama_layer_asan.so"), p.stdout + p.stderr
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert " passed" in out
