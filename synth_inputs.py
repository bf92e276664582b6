"""Seeded synthetic inputs for the Llama decoder-layer forward.

This module draws the random tensors that both the GPU path's tests/bench and
the CPU oracle consume. It holds none of the layer's arithmetic: only shapes,
distributions, seeds and the storage format (bf16 bit patterns or float32).

Distributions (the workload statement of the layer shapes):
  hidden states N(0,1); projection weights N(0,0.02); RMSNorm gains 1+N(0,0.1);
  decode positions integer-uniform on [1024, 8191]; KV caches N(0,1).
Tensor k is drawn from ``numpy.random.default_rng([seed, k])``; cache rows use
``default_rng([seed, k, b])`` so one batch row can be regenerated alone.

bf16 tensors are produced by rounding the float32 draw to bfloat16 with
round-to-nearest-even on the bit pattern, and are carried as uint16 arrays.
Both sides see exactly the same values: the GPU gets the uint16 bits, the
oracle upcasts those bits exactly.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

# tensor stream ids
K_HIDDEN, K_WQKV, K_WO, K_WGU, K_WDOWN, K_GATTN, K_GMLP, K_POS, K_KCACHE, K_VCACHE = range(10)
K_EMB, K_GFINAL, K_LMHEAD, K_TOKENS = 30, 31, 32, 33


@dataclasses.dataclass(frozen=True)
class RopeCfg:
    type: str = "default"          # default | linear | dynamic_ntk | llama3
    theta: float = 10000.0
    factor: float = 1.0
    low_freq_factor: float = 1.0
    high_freq_factor: float = 4.0
    original_max_pos: int = 8192
    interleaved: bool = False


@dataclasses.dataclass(frozen=True)
class LayerCfg:
    name: str
    B: int
    S: int
    hidden: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    intermediate: int
    eps: float
    rope: RopeCfg
    dtype: str                      # "f32" | "bf16"
    decode: bool = False
    ctx: int = 0                    # KV-cache slots per sequence (decode)

    @property
    def qkv_dim(self) -> int:
        return (self.n_heads + 2 * self.n_kv_heads) * self.head_dim

    @property
    def M(self) -> int:
        return self.B * self.S


# The five workloads: a tiny fp32 layer, a Llama-3.2-1B-shaped prefill, a
# Llama-3-8B-shaped prefill, an 8B-shaped decode step against a KV cache and an
# 8B-shaped 32k prefill with Llama3 frequency scaling.
CONFIGS = {
    "tiny_f32": LayerCfg("tiny_f32", B=1, S=32, hidden=64, n_heads=4, n_kv_heads=2, head_dim=16,
                         intermediate=176, eps=1e-5, rope=RopeCfg(theta=10000.0), dtype="f32"),
    "llama32_1b_prefill": LayerCfg("llama32_1b_prefill", B=4, S=2048, hidden=2048, n_heads=32, n_kv_heads=8,
                                   head_dim=64, intermediate=8192, eps=1e-5, rope=RopeCfg(theta=500000.0),
                                   dtype="bf16"),
    "llama3_8b_prefill": LayerCfg("llama3_8b_prefill", B=2, S=4096, hidden=4096, n_heads=32, n_kv_heads=8,
                                  head_dim=128, intermediate=14336, eps=1e-5, rope=RopeCfg(theta=500000.0),
                                  dtype="bf16"),
    "llama3_8b_decode": LayerCfg("llama3_8b_decode", B=64, S=1, hidden=4096, n_heads=32, n_kv_heads=8,
                                 head_dim=128, intermediate=14336, eps=1e-5, rope=RopeCfg(theta=500000.0),
                                 dtype="bf16", decode=True, ctx=8192),
    "llama3_8b_long_llama3rope": LayerCfg(
        "llama3_8b_long_llama3rope", B=1, S=32768, hidden=4096, n_heads=32, n_kv_heads=8, head_dim=128,
        intermediate=14336, eps=1e-5,
        rope=RopeCfg(type="llama3", theta=500000.0, factor=8.0, low_freq_factor=1.0, high_freq_factor=4.0,
                     original_max_pos=8192),
        dtype="bf16"),
}


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bit patterns."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def to_f64(t: np.ndarray, dtype: str) -> np.ndarray:
    """Exact fp64 view of a stored tensor (uint16 bf16 bits or float32)."""
    if dtype == "bf16":
        return bf16_bits_to_f32(t).astype(np.float64)
    return np.asarray(t, dtype=np.float32).astype(np.float64)


def _draw(seed, k, shape, std, mean, dtype, extra=()):
    rng = np.random.default_rng([seed, k, *extra])
    x = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    if mean != 0.0:
        x += np.float32(mean)
    return f32_to_bf16_bits(x) if dtype == "bf16" else x


def make_weights(cfg: LayerCfg, seed: int = 0) -> dict:
    """Projection weights stored [out_features, in_features]; fused rows Q|K|V and gate|up."""
    d = cfg.dtype
    return {
        "w_qkv": _draw(seed, K_WQKV, (cfg.qkv_dim, cfg.hidden), 0.02, 0.0, d),
        "w_o": _draw(seed, K_WO, (cfg.hidden, cfg.n_heads * cfg.head_dim), 0.02, 0.0, d),
        "w_gate_up": _draw(seed, K_WGU, (2 * cfg.intermediate, cfg.hidden), 0.02, 0.0, d),
        "w_down": _draw(seed, K_WDOWN, (cfg.hidden, cfg.intermediate), 0.02, 0.0, d),
        "g_attn": _draw(seed, K_GATTN, (cfg.hidden,), 0.1, 1.0, d),
        "g_mlp": _draw(seed, K_GMLP, (cfg.hidden,), 0.1, 1.0, d),
    }


def make_model_weights(cfg: LayerCfg, n_layers: int, vocab: int, seed: int = 0) -> dict:
    """A synthetic model stack: layer l gets make_weights(cfg, seed * 1000 + l); token embeddings
    [vocab, H] ~ N(0,1) (the hidden-state distribution of the layer workloads), final RMSNorm gain
    1+N(0,0.1), output projection [vocab, H] ~ N(0,0.02)."""
    d = cfg.dtype
    return {
        "layers": [make_weights(cfg, seed * 1000 + l) for l in range(n_layers)],
        "tok_embeddings": _draw(seed, K_EMB, (vocab, cfg.hidden), 1.0, 0.0, d),
        "g_final": _draw(seed, K_GFINAL, (cfg.hidden,), 0.1, 1.0, d),
        "lm_head": _draw(seed, K_LMHEAD, (vocab, cfg.hidden), 0.02, 0.0, d),
    }


def make_tokens(cfg: LayerCfg, vocab: int, seed: int = 0) -> np.ndarray:
    """Token ids [B, S] integer-uniform on [0, vocab) (int64)."""
    rng = np.random.default_rng([seed, K_TOKENS])
    return rng.integers(0, vocab, size=(cfg.B, cfg.S), dtype=np.int64)


def make_hidden(cfg: LayerCfg, seed: int = 0) -> np.ndarray:
    return _draw(seed, K_HIDDEN, (cfg.B, cfg.S, cfg.hidden), 1.0, 0.0, cfg.dtype)


def make_prefill_positions(cfg: LayerCfg) -> np.ndarray:
    """position_ids[b, s] = s (int64)."""
    return np.broadcast_to(np.arange(cfg.S, dtype=np.int64), (cfg.B, cfg.S)).copy()


def make_decode_positions(cfg: LayerCfg, seed: int = 0, lo: int = 1024, hi: Optional[int] = None) -> np.ndarray:
    """One position per sequence, integer-uniform on [lo, hi) with hi defaulting to the cache length."""
    hi = cfg.ctx if hi is None else hi
    rng = np.random.default_rng([seed, K_POS])
    return rng.integers(lo, hi, size=(cfg.B,), dtype=np.int64)


def make_cache_row(cfg: LayerCfg, which: str, b: int, seed: int = 0) -> np.ndarray:
    """One batch row [ctx, n_kv, d] of the K or V cache, N(0,1)."""
    k = K_KCACHE if which == "k" else K_VCACHE
    return _draw(seed, k, (cfg.ctx, cfg.n_kv_heads, cfg.head_dim), 1.0, 0.0, cfg.dtype, extra=(b,))


def make_cache(cfg: LayerCfg, which: str, seed: int = 0) -> np.ndarray:
    out = np.empty((cfg.B, cfg.ctx, cfg.n_kv_heads, cfg.head_dim),
                   dtype=np.uint16 if cfg.dtype == "bf16" else np.float32)
    for b in range(cfg.B):
        out[b] = make_cache_row(cfg, which, b, seed)
    return out


def normal(seed: int, stream: int, shape, dtype: str, std: float = 1.0, mean: float = 0.0) -> np.ndarray:
    """A seeded N(mean, std) tensor for kernel-level cases (stream ids >= 100 by convention)."""
    return _draw(seed, stream, tuple(shape), std, mean, dtype)


def scaled(cfg: LayerCfg, **kw) -> LayerCfg:
    """A copy of a config with some fields replaced (smaller parity cases of the same family)."""
    return dataclasses.replace(cfg, **kw)
