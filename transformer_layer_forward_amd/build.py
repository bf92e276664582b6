"""Build the gfx950 HIP library ``libllama_layer.so`` in-tree with hipcc.

Every call recompiles all sources, so a stale library is never reused.
Usage: python -m transformer_layer_forward_amd.build
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libllama_layer.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
SOURCES = ["api.hip", "norm_rope.hip", "gemm.hip", "attn.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-mcode-object-version=5",
    # keep the compiler from forming packed fp32 vector ops (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the gfx950 library)")


def build(verbose: bool = False) -> str:
    hipcc = _hipcc()
    tmp = tempfile.mkdtemp(prefix="llbuild_")
    try:
        def compile_one(src):
            obj = os.path.join(tmp, src + ".o")
            cmd = [hipcc, *HIPCC_FLAGS, f"-I{INCLUDE}", f"-I{CSRC}", "-c", os.path.join(CSRC, src), "-o", obj]
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
            # the host pass does not know the packed-fp32 target feature and says so: not a problem
            noise = "'-packed-fp32-ops' is not a recognized feature"
            msg = "\n".join(l for l in r.stderr.splitlines() if noise not in l and l.strip())
            if verbose and msg:
                print(msg, file=sys.stderr)
            return obj

        with concurrent.futures.ThreadPoolExecutor(max_workers=min(4, len(SOURCES))) as ex:
            objs = list(ex.map(compile_one, SOURCES))
        out_tmp = LIB_PATH + ".tmp"
        cmd = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", out_tmp, *objs]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed:\n{r.stderr}")
        os.replace(out_tmp, LIB_PATH)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
