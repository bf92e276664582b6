"""Llama decoder-layer forward for AMD Instinct MI355X (gfx950): hand-written HIP kernels behind a C ABI.

The C ABI is declared in include/llama_layer.h; this package holds its sources (csrc/), the in-tree
build (build.py) and a thin ctypes binding with the same entry-point names.
"""
from ._lib import (  # noqa: F401
    LayerConfig,
    Rope,
    gqa_attn_decode,
    gqa_attn_prefill,
    gqa_attn_prefill_chunk,
    gqa_attn_prefill_varlen,
    layer_workspace_bytes,
    last_error,
    llama_layer_forward,
    llama_layer_forward_chunk,
    llama_layer_forward_noalloc,
    llama_layer_forward_varlen,
    llama_model_forward,
    load,
    profile_begin,
    profile_end,
    release_caches,
    rmsnorm,
    rope_apply,
    swiglu_mlp,
    version,
)
