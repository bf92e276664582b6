"""Host-side logic of the library checked on the CPU with a plain C++ compiler (no GPU, no HIP runtime).

The balanced decode partition (csrc/decode_partition.h) and the RoPE table bookkeeping (transformer_layer_forward_amd/csrc/rope_cache.h) is built together with a
driver that replaces device memory and the table kernel by counters, under AddressSanitizer and
UndefinedBehaviorSanitizer, and run: one slot per (RoPE parameters, head size, device, stream), geometric
growth, in-place regeneration of a dynamic-NTK table whose length changes, everything freed on release.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "transformer_layer_forward_amd", "csrc")
CPP = os.path.join(ROOT, "tests", "cpp")


def _build_and_run(src, tmp_path, sanitize=True):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path / "check")
    flags = ["-std=c++17", "-O1", "-g"]
    if sanitize:
        flags += ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
    r = subprocess.run([gxx, *flags, f"-I{CSRC}", os.path.join(CPP, src), "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    return r.stdout


def test_rope_table_cache_policy(tmp_path):
    out = _build_and_run("rope_cache_check.cpp", tmp_path)
    assert "all checks passed" in out


def test_balanced_decode_partition(tmp_path):
    """The balanced decode kernel's work split (csrc/decode_partition.h), replayed for 3000 random batches:
    every tile of every (sequence, head group) processed exactly once, record indices unique, and the
    combine finds exactly the records each segment's pieces wrote."""
    out = _build_and_run("decode_partition_check.cpp", tmp_path)
    assert "all checks passed" in out
