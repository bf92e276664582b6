"""ctypes binding of libllama_layer.so (the gfx950 HIP library declared in include/llama_layer.h).

Argument marshalling only: every step of the layer runs in the library's kernels. torch is used for
device memory and the current stream. The library must be built (``python -m
transformer_layer_forward_amd.build``); there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

import torch  # loaded first so the library binds to the HIP runtime torch already holds

_PKG = os.path.dirname(os.path.abspath(__file__))
# LLAMA_LAYER_LIB selects another build of the same library (the CPU checks load the host-sanitized one)
LIB_PATH = os.environ.get("LLAMA_LAYER_LIB") or os.path.join(_PKG, "libllama_layer.so")

LL_OK, LL_EINVAL, LL_EUNSUPPORTED, LL_EHIP, LL_ENOMEM = range(5)
LL_F32, LL_BF16 = 0, 1
ROPE_TYPES = {"default": 0, "linear": 1, "dynamic_ntk": 2, "llama3": 3}
STATUS_NAMES = {0: "LL_OK", 1: "LL_EINVAL", 2: "LL_EUNSUPPORTED", 3: "LL_EHIP", 4: "LL_ENOMEM"}

EXPORTED = (
    "llama_layer_workspace_bytes", "llama_layer_forward", "llama_layer_forward_noalloc", "llama_layer_forward_chunk", "llama_layer_forward_varlen",
    "llama_model_workspace_bytes", "llama_model_forward",
    "rmsnorm", "rope_apply", "gqa_attn_prefill", "gqa_attn_prefill_chunk_workspace_bytes", "gqa_attn_prefill_chunk",
    "gqa_attn_prefill_varlen",
    "gqa_attn_decode_workspace_bytes", "gqa_attn_decode", "swiglu_mlp_workspace_bytes", "swiglu_mlp",
    "ll_last_error", "ll_release_caches", "ll_profile_begin", "ll_profile_begin_stages", "ll_profile_end",
    "ll_profile_stage_name",
    "ll_version",
)


class LLRope(ctypes.Structure):
    _fields_ = [("type", ctypes.c_int32), ("interleaved", ctypes.c_int32), ("theta", ctypes.c_double),
                ("factor", ctypes.c_double), ("low_freq_factor", ctypes.c_double),
                ("high_freq_factor", ctypes.c_double), ("original_max_pos", ctypes.c_int64)]


class LLLayerCfg(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int64), ("n_heads", ctypes.c_int64), ("n_kv_heads", ctypes.c_int64),
                ("head_dim", ctypes.c_int64), ("intermediate", ctypes.c_int64), ("eps", ctypes.c_double),
                ("rope", LLRope), ("dtype", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class LLLayerWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("w_qkv", "w_o", "w_gate_up", "w_down", "g_attn", "g_mlp")]


@dataclasses.dataclass(frozen=True)
class Rope:
    type: str = "default"
    theta: float = 10000.0
    factor: float = 1.0
    low_freq_factor: float = 1.0
    high_freq_factor: float = 4.0
    original_max_pos: int = 8192
    interleaved: bool = False

    def to_c(self) -> LLRope:
        return LLRope(ROPE_TYPES[self.type], int(bool(self.interleaved)), float(self.theta), float(self.factor),
                      float(self.low_freq_factor), float(self.high_freq_factor), int(self.original_max_pos))


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    hidden: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    intermediate: int
    eps: float = 1e-5
    rope: Rope = Rope()
    dtype: torch.dtype = torch.bfloat16

    def to_c(self) -> LLLayerCfg:
        return LLLayerCfg(self.hidden, self.n_heads, self.n_kv_heads, self.head_dim, self.intermediate,
                          float(self.eps), self.rope.to_c(), _dtype_code(self.dtype), 0)


_lib = None


def _single_hip_runtime() -> None:
    """The library must share torch's HIP runtime (streams and pointers are runtime objects)."""
    try:
        with open("/proc/self/maps") as fh:
            paths = {line.split()[-1] for line in fh if "libamdhip64" in line}
    except OSError:
        return
    real = {os.path.realpath(p) for p in paths}
    if len(real) > 1:
        raise RuntimeError(f"two HIP runtimes are loaded in this process: {sorted(real)}")


def load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m transformer_layer_forward_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    _single_hip_runtime()
    c_i64, c_i32, c_vp, c_sz, c_d = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_double
    sig = {
        "llama_layer_workspace_bytes": (c_sz, [ctypes.POINTER(LLLayerCfg), c_i64, c_i64, c_i64]),
        "llama_layer_forward": (c_i32, [ctypes.POINTER(LLLayerCfg), ctypes.POINTER(LLLayerWeights), c_vp, c_vp, c_i64,
                                        c_i64, c_i64, c_vp, c_vp, c_i64, c_vp, c_vp, c_sz, c_vp]),
        "llama_layer_forward_noalloc": (c_i32, [ctypes.POINTER(LLLayerCfg), ctypes.POINTER(LLLayerWeights), c_vp, c_vp,
                                                c_i64, c_i64, c_i64, c_vp, c_vp, c_i64, c_vp, c_vp]),
        "llama_layer_forward_chunk": (c_i32, [ctypes.POINTER(LLLayerCfg), ctypes.POINTER(LLLayerWeights), c_vp, c_vp,
                                              c_i64, c_i64, c_i64, c_vp, c_vp, c_i64, c_vp, c_vp, c_sz, c_vp]),
        "llama_layer_forward_varlen": (c_i32, [ctypes.POINTER(LLLayerCfg), ctypes.POINTER(LLLayerWeights), c_vp,
                                               c_vp, c_vp, c_i64, c_i64, c_i64, c_i64, c_vp, c_vp, c_sz, c_vp]),
        "llama_model_workspace_bytes": (c_sz, [ctypes.POINTER(LLLayerCfg), c_i64, c_i64, c_i64]),
        "llama_model_forward": (c_i32, [ctypes.POINTER(LLLayerCfg), c_i64, ctypes.POINTER(LLLayerWeights), c_vp, c_vp,
                                        c_vp, c_i64, c_vp, c_vp, c_i64, c_i64, c_i64, c_vp, c_vp, c_sz, c_vp]),
        "rmsnorm": (c_i32, [c_vp, c_vp, c_vp, c_i64, c_i64, c_d, c_i32, c_vp]),
        "rope_apply": (c_i32, [ctypes.POINTER(LLRope), c_vp, c_vp, c_i64, c_i64, c_i64, c_i64, c_i64, c_i64, c_i32,
                               c_vp]),
        "gqa_attn_prefill": (c_i32, [c_vp, ctypes.POINTER(LLRope), c_vp, c_i64, c_vp, c_vp, c_vp, c_i64, c_i64, c_i64,
                                     c_i64, c_i64, c_i64, c_i32, c_vp]),
        "gqa_attn_prefill_chunk_workspace_bytes": (c_sz, [c_i64, c_i64, c_i64, c_i64, c_i64, c_i64, c_i32]),
        "gqa_attn_prefill_chunk": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_i64, c_i64, c_i64, c_i64, c_i64, c_i64,
                                           c_i32, c_vp, c_sz, c_vp]),
        "gqa_attn_prefill_varlen": (c_i32, [c_vp, c_vp, c_i64, c_i64, c_i64, c_vp, c_i64, c_i64, c_i64, c_i32, c_vp]),
        "gqa_attn_decode_workspace_bytes": (c_sz, [c_i64, c_i64, c_i64, c_i64]),
        "gqa_attn_decode": (c_i32, [c_vp, ctypes.POINTER(LLRope), c_vp, c_i64, c_vp, c_vp, c_i64, c_vp, c_i64, c_i64,
                                    c_i64, c_i64, c_i32, c_vp, c_sz, c_vp]),
        "swiglu_mlp_workspace_bytes": (c_sz, [c_i64, c_i64, c_i64, c_i32]),
        "swiglu_mlp": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_i64, c_i64, c_i64, c_i32, c_vp, c_sz, c_vp]),
        "ll_last_error": (ctypes.c_char_p, []),
        "ll_release_caches": (None, []),
        "ll_profile_begin": (c_i32, [c_i32]),
        "ll_profile_begin_stages": (c_i32, [c_i32, ctypes.c_uint32]),
        "ll_profile_end": (c_i32, [ctypes.POINTER(c_d), ctypes.POINTER(c_i64), c_i32]),
        "ll_profile_stage_name": (ctypes.c_char_p, [c_i32]),
        "ll_version": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


# ------------------------------------------------------------------ helpers
def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.bfloat16:
        return LL_BF16
    if dt == torch.float32:
        return LL_F32
    raise TypeError(f"unsupported dtype {dt} (bfloat16 or float32)")


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _check(status: int, name: str) -> None:
    if status != LL_OK:
        msg = load().ll_last_error().decode(errors="replace")
        raise RuntimeError(f"{name} failed with {STATUS_NAMES.get(status, status)}: {msg}")


def last_error() -> str:
    return load().ll_last_error().decode(errors="replace")


def version() -> str:
    return load().ll_version().decode()


def release_caches() -> None:
    load().ll_release_caches()


# ------------------------------------------------------------------ entry points
def rmsnorm(x: torch.Tensor, gain: torch.Tensor, eps: float, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    lib = load()
    H = x.shape[-1]
    rows = x.numel() // H
    y = torch.empty_like(x) if out is None else out
    _check(lib.rmsnorm(_ptr(x), _ptr(gain), _ptr(y), rows, H, float(eps), _dtype_code(x.dtype), _stream(x)), "rmsnorm")
    return y


def rope_apply(rope: Rope, qkv: torch.Tensor, position_ids: torch.Tensor, n_heads: int, n_kv_heads: int,
               head_dim: int, kv_seq_len: int) -> torch.Tensor:
    lib = load()
    B, S = position_ids.shape
    r = rope.to_c()
    _check(lib.rope_apply(ctypes.byref(r), _ptr(qkv), _ptr(position_ids), B, S, n_heads, n_kv_heads, head_dim,
                          int(kv_seq_len), _dtype_code(qkv.dtype), _stream(qkv)), "rope_apply")
    return qkv


def gqa_attn_prefill(qkv: torch.Tensor, position_ids: Optional[torch.Tensor], n_heads: int, n_kv_heads: int,
                     head_dim: int, rope: Optional[Rope] = None, kv_seq_len: int = 0,
                     k_cache: Optional[torch.Tensor] = None, v_cache: Optional[torch.Tensor] = None,
                     out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """qkv [B, S, (n_h + 2 n_kv) d] -> o [B, S, n_h d]."""
    lib = load()
    B, S = qkv.shape[0], qkv.shape[1]
    o = out if out is not None else torch.empty((B, S, n_heads * head_dim), dtype=qkv.dtype, device=qkv.device)
    r = rope.to_c() if rope is not None else None
    ctx = k_cache.shape[1] if k_cache is not None else 0
    _check(lib.gqa_attn_prefill(_ptr(qkv), ctypes.byref(r) if r is not None else None, _ptr(position_ids),
                                int(kv_seq_len), _ptr(o), _ptr(k_cache), _ptr(v_cache), ctx, B, S, n_heads, n_kv_heads,
                                head_dim, _dtype_code(qkv.dtype), _stream(qkv)), "gqa_attn_prefill")
    return o


def gqa_attn_prefill_chunk(qkv: torch.Tensor, position_ids: torch.Tensor, k_cache: torch.Tensor,
                           v_cache: torch.Tensor, n_heads: int, n_kv_heads: int, head_dim: int,
                           out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                           split_keys: bool = True) -> torch.Tensor:
    """qkv [B, S, (n_h + 2 n_kv) d] with q, k rotated; stores K/V at slots position_ids[b, s], then each
    query attends over cache slots 0 .. its position -> o [B, S, n_h d]. With split_keys (default) a
    workspace for the key-split records is used (allocated here if not given); without, none is passed."""
    lib = load()
    B, S = qkv.shape[0], qkv.shape[1]
    ctx = k_cache.shape[1]
    o = out if out is not None else torch.empty((B, S, n_heads * head_dim), dtype=qkv.dtype, device=qkv.device)
    dt = _dtype_code(qkv.dtype)
    ws = None
    if split_keys:
        need = lib.gqa_attn_prefill_chunk_workspace_bytes(B, S, n_heads, n_kv_heads, head_dim, ctx, dt)
        ws = workspace if workspace is not None else (
            torch.empty(need, dtype=torch.uint8, device=qkv.device) if need > 0 else None)
    _check(lib.gqa_attn_prefill_chunk(_ptr(qkv), _ptr(position_ids), _ptr(o), _ptr(k_cache), _ptr(v_cache),
                                      ctx, B, S, n_heads, n_kv_heads, head_dim, dt, _ptr(ws),
                                      ws.numel() if ws is not None else 0, _stream(qkv)), "gqa_attn_prefill_chunk")
    return o


def gqa_attn_prefill_varlen(qkv: torch.Tensor, cu_seqlens: torch.Tensor, max_seqlen: int, n_heads: int,
                            n_kv_heads: int, head_dim: int, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Packed qkv [T, (n_h + 2 n_kv) d] (q, k rotated), cu_seqlens [n+1] int32 -> o [T, n_h d], causal
    within each sequence."""
    lib = load()
    T = qkv.shape[0]
    if cu_seqlens.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    o = out if out is not None else torch.empty((T, n_heads * head_dim), dtype=qkv.dtype, device=qkv.device)
    _check(lib.gqa_attn_prefill_varlen(_ptr(qkv), _ptr(cu_seqlens), cu_seqlens.numel() - 1, int(max_seqlen), T,
                                       _ptr(o), n_heads, n_kv_heads, head_dim, _dtype_code(qkv.dtype), _stream(qkv)),
           "gqa_attn_prefill_varlen")
    return o


def gqa_attn_decode(qkv: torch.Tensor, pos: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, n_heads: int,
                    n_kv_heads: int, head_dim: int, rope: Optional[Rope] = None, kv_seq_len: int = 0,
                    out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """qkv [B, (n_h + 2 n_kv) d] (one token per sequence), pos [B] -> o [B, n_h d]; writes slot pos[b]."""
    lib = load()
    B = qkv.shape[0]
    ctx = k_cache.shape[1]
    o = out if out is not None else torch.empty((B, n_heads * head_dim), dtype=qkv.dtype, device=qkv.device)
    need = lib.gqa_attn_decode_workspace_bytes(B, n_heads, head_dim, ctx)
    ws = workspace if workspace is not None else torch.empty(max(need, 1), dtype=torch.uint8, device=qkv.device)
    r = rope.to_c() if rope is not None else None
    _check(lib.gqa_attn_decode(_ptr(qkv), ctypes.byref(r) if r is not None else None, _ptr(pos), int(kv_seq_len),
                               _ptr(k_cache), _ptr(v_cache), ctx, _ptr(o), B, n_heads, n_kv_heads, head_dim,
                               _dtype_code(qkv.dtype), _ptr(ws), ws.numel(), _stream(qkv)), "gqa_attn_decode")
    return o


def swiglu_mlp(x: torch.Tensor, w_gate_up: torch.Tensor, w_down: torch.Tensor,
               residual: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
               workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    lib = load()
    H = x.shape[-1]
    M = x.numel() // H
    I = w_down.shape[1]
    dt = _dtype_code(x.dtype)
    y = out if out is not None else torch.empty_like(x)
    need = lib.swiglu_mlp_workspace_bytes(M, H, I, dt)
    ws = workspace if workspace is not None else torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    _check(lib.swiglu_mlp(_ptr(x), _ptr(w_gate_up), _ptr(w_down), _ptr(residual), _ptr(y), M, H, I, dt, _ptr(ws),
                          ws.numel(), _stream(x)), "swiglu_mlp")
    return y


def layer_workspace_bytes(cfg: LayerConfig, B: int, S: int, ctx: int = 0) -> int:
    c = cfg.to_c()
    n = load().llama_layer_workspace_bytes(ctypes.byref(c), B, S, ctx)
    if n == 0:
        raise ValueError(f"invalid layer configuration: {last_error()}")
    return n


def llama_layer_forward(cfg: LayerConfig, weights: dict, hidden: torch.Tensor, position_ids: torch.Tensor,
                        kv_seq_len: Optional[int] = None, k_cache: Optional[torch.Tensor] = None,
                        v_cache: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                        workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """hidden [B, S, H]; position_ids [B, S] int64; weights: w_qkv, w_o, w_gate_up, w_down, g_attn, g_mlp.

    kv_seq_len defaults to the cache length (when caches are given) or S."""
    lib = load()
    B, S = hidden.shape[0], hidden.shape[1]
    ctx = k_cache.shape[1] if k_cache is not None else 0
    if kv_seq_len is None:
        kv_seq_len = ctx if ctx else S
    c = cfg.to_c()
    w = LLLayerWeights(*(weights[k].data_ptr() for k in ("w_qkv", "w_o", "w_gate_up", "w_down", "g_attn", "g_mlp")))
    for k in ("w_qkv", "w_o", "w_gate_up", "w_down", "g_attn", "g_mlp"):
        _ptr(weights[k])
    need = lib.llama_layer_workspace_bytes(ctypes.byref(c), B, S, ctx)
    if need == 0:
        raise ValueError(f"invalid layer configuration: {last_error()}")
    ws = workspace if workspace is not None else torch.empty(need, dtype=torch.uint8, device=hidden.device)
    y = out if out is not None else torch.empty_like(hidden)
    _check(lib.llama_layer_forward(ctypes.byref(c), ctypes.byref(w), _ptr(hidden), _ptr(position_ids), B, S,
                                   int(kv_seq_len), _ptr(k_cache), _ptr(v_cache), ctx, _ptr(y), _ptr(ws), ws.numel(),
                                   _stream(hidden)), "llama_layer_forward")
    return y


def llama_layer_forward_noalloc(cfg: LayerConfig, weights: dict, hidden: torch.Tensor, position_ids: torch.Tensor,
                                kv_seq_len: Optional[int] = None, k_cache: Optional[torch.Tensor] = None,
                                v_cache: Optional[torch.Tensor] = None, out: torch.Tensor = None) -> torch.Tensor:
    """llama_layer_forward whose workspace and RoPE table live in the library's static device scratch: the
    library allocates nothing. ``out`` must be given (this wrapper allocates nothing either)."""
    lib = load()
    B, S = hidden.shape[0], hidden.shape[1]
    ctx = k_cache.shape[1] if k_cache is not None else 0
    if kv_seq_len is None:
        kv_seq_len = ctx if ctx else S
    if out is None:
        raise ValueError("llama_layer_forward_noalloc needs a preallocated out tensor")
    c = cfg.to_c()
    w = LLLayerWeights(*(weights[k].data_ptr() for k in ("w_qkv", "w_o", "w_gate_up", "w_down", "g_attn", "g_mlp")))
    for k in ("w_qkv", "w_o", "w_gate_up", "w_down", "g_attn", "g_mlp"):
        _ptr(weights[k])
    _check(lib.llama_layer_forward_noalloc(ctypes.byref(c), ctypes.byref(w), _ptr(hidden), _ptr(position_ids), B, S,
                                           int(kv_seq_len), _ptr(k_cache), _ptr(v_cache), ctx, _ptr(out),
                                           _stream(hidden)), "llama_layer_forward_noalloc")
    return out


def llama_layer_forward_varlen(cfg: LayerConfig, weights: dict, hidden: torch.Tensor, position_ids: torch.Tensor,
                               cu_seqlens: torch.Tensor, max_seqlen: int, kv_seq_len: Optional[int] = None,
                               out: Optional[torch.Tensor] = None,
                               workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Packed sequences: hidden [T, H], position_ids [T] int64, cu_seqlens [n+1] int32 (device);
    kv_seq_len (RoPE table length) defaults to max_seqlen."""
    lib = load()
    T = hidden.shape[0]
    if cu_seqlens.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    if kv_seq_len is None:
        kv_seq_len = max(int(max_seqlen), 1)
    c = cfg.to_c()
    w = LLLayerWeights(*(weights[k].data_ptr() for k in ("w_qkv", "w_o", "w_gate_up", "w_down", "g_attn", "g_mlp")))
    for k in ("w_qkv", "w_o", "w_gate_up", "w_down", "g_attn", "g_mlp"):
        _ptr(weights[k])
    need = lib.llama_layer_workspace_bytes(ctypes.byref(c), 1, T, 0)
    if need == 0:
        raise ValueError(f"invalid layer configuration: {last_error()}")
    ws = workspace if workspace is not None else torch.empty(need, dtype=torch.uint8, device=hidden.device)
    y = out if out is not None else torch.empty_like(hidden)
    _check(lib.llama_layer_forward_varlen(ctypes.byref(c), ctypes.byref(w), _ptr(hidden), _ptr(position_ids),
                                          _ptr(cu_seqlens), cu_seqlens.numel() - 1, int(max_seqlen), T,
                                          int(kv_seq_len), _ptr(y), _ptr(ws), ws.numel(), _stream(hidden)),
           "llama_layer_forward_varlen")
    return y


def llama_layer_forward_chunk(cfg: LayerConfig, weights: dict, hidden: torch.Tensor, position_ids: torch.Tensor,
                              k_cache: torch.Tensor, v_cache: torch.Tensor, kv_seq_len: Optional[int] = None,
                              out: Optional[torch.Tensor] = None,
                              workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Chunked prefill on a cache prefix: hidden [B, S, H] at positions position_ids [B, S]; the chunk's
    K/V are stored in the caches and attention reads cache slots 0 .. each token's position.
    kv_seq_len defaults to the cache length."""
    lib = load()
    B, S = hidden.shape[0], hidden.shape[1]
    ctx = k_cache.shape[1]
    if kv_seq_len is None:
        kv_seq_len = ctx
    c = cfg.to_c()
    w = LLLayerWeights(*(weights[k].data_ptr() for k in ("w_qkv", "w_o", "w_gate_up", "w_down", "g_attn", "g_mlp")))
    for k in ("w_qkv", "w_o", "w_gate_up", "w_down", "g_attn", "g_mlp"):
        _ptr(weights[k])
    # sized with the cache length: includes room for key-split attention records on small chunks
    need = lib.llama_layer_workspace_bytes(ctypes.byref(c), B, S, ctx)
    if need == 0:
        raise ValueError(f"invalid layer configuration: {last_error()}")
    ws = workspace if workspace is not None else torch.empty(need, dtype=torch.uint8, device=hidden.device)
    y = out if out is not None else torch.empty_like(hidden)
    _check(lib.llama_layer_forward_chunk(ctypes.byref(c), ctypes.byref(w), _ptr(hidden), _ptr(position_ids), B, S,
                                         int(kv_seq_len), _ptr(k_cache), _ptr(v_cache), ctx, _ptr(y), _ptr(ws),
                                         ws.numel(), _stream(hidden)), "llama_layer_forward_chunk")
    return y


def llama_model_forward(cfg: LayerConfig, model: dict, tokens: torch.Tensor, position_ids: torch.Tensor,
                        kv_seq_len: Optional[int] = None, out: Optional[torch.Tensor] = None,
                        workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """model: "layers" (list of layer weight dicts), "tok_embeddings" [vocab, H], "g_final" [H],
    "lm_head" [vocab, H]; tokens, position_ids [B, S] int64 -> logits [B, S, vocab]."""
    lib = load()
    B, S = tokens.shape
    vocab = model["lm_head"].shape[0]
    if kv_seq_len is None:
        kv_seq_len = S
    c = cfg.to_c()
    names = ("w_qkv", "w_o", "w_gate_up", "w_down", "g_attn", "g_mlp")
    n = len(model["layers"])
    arr = (LLLayerWeights * max(n, 1))()
    for i, W in enumerate(model["layers"]):
        arr[i] = LLLayerWeights(*(_ptr(W[k]) for k in names))
    need = lib.llama_model_workspace_bytes(ctypes.byref(c), vocab, B, S)
    if need == 0:
        raise ValueError(f"invalid model configuration: {last_error()}")
    ws = workspace if workspace is not None else torch.empty(need, dtype=torch.uint8, device=tokens.device)
    y = out if out is not None else torch.empty((B, S, vocab), dtype=model["lm_head"].dtype, device=tokens.device)
    _check(lib.llama_model_forward(ctypes.byref(c), n, arr, _ptr(model["tok_embeddings"]), _ptr(model["g_final"]),
                                   _ptr(model["lm_head"]), vocab, _ptr(tokens), _ptr(position_ids), B, S,
                                   int(kv_seq_len), _ptr(y), _ptr(ws), ws.numel(), _stream(tokens)),
           "llama_model_forward")
    return y


# ------------------------------------------------------------------ stage timing
def profile_begin(reserve_calls: int = 64, stages=None) -> None:
    """Time the stages of later llama_layer_forward calls on this thread: all of them, or only those named
    in `stages` (names as profile_end reports them)."""
    lib = load()
    if stages is None:
        _check(lib.ll_profile_begin(int(reserve_calls)), "ll_profile_begin")
        return
    names = [lib.ll_profile_stage_name(i).decode() for i in range(7)]
    mask = 0
    for st in stages:
        if st not in names:
            raise ValueError(f"unknown stage {st!r}; stages are {names}")
        mask |= 1 << names.index(st)
    _check(lib.ll_profile_begin_stages(int(reserve_calls), mask), "ll_profile_begin_stages")


def profile_end() -> dict:
    """{stage name: (summed ms, calls)} for the timed stages."""
    lib = load()
    ms = (ctypes.c_double * 8)()
    n = (ctypes.c_int64 * 8)()
    k = lib.ll_profile_end(ms, n, 8)
    if k < 0:
        raise RuntimeError(f"ll_profile_end failed: {last_error()}")
    return {lib.ll_profile_stage_name(i).decode(): (ms[i], n[i]) for i in range(k) if n[i] > 0}
