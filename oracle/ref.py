"""fp64 CPU oracle of the Llama decoder-layer forward.

TEST INFRASTRUCTURE ONLY. Only tests/, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of bench.py may import this package. The GPU library never
calls it, and it shares no code, tables or constants with the GPU library.

Every function is the plain definition of its step, computed in float64 with
NumPy (BLAS matmuls as the only library primitive), with no blocking, fusion or
reordering beyond a query-block loop that bounds memory. Inputs are the exact
fp64 widening of the values the GPU receives.

Sources (the pages, cited by title and section):
  [nanotron]  "模型层：从 Embedding 到 Loss 的实现" (nanotron tutorial ch. 9):
              §9.3 CausalSelfAttention, §9.4 MLP, §9.5 LlamaDecoderLayer.
  [verl]      "parallel_attention.py — LLaMA 并行注意力" (verl docs):
              §1 RoPE (LlamaRotaryEmbedding and its linear / dynamic-NTK / Llama3
              variants), §2 ParallelLlamaAttention (eager attention).
  [llama3]    "llama3 结构详解": §3.1 RMSNorm, §3.2 Attention (GQA, KV cache).
  [meta-qa]   the CSDN answer explaining Meta's model.py: "#### 1. RMSNorm",
              "#### 2. 旋转位置编码", "#### 3. 注意力机制", "#### 4. 前馈网络",
              "#### 5. Transformer整体结构".
  [nju]       NJU LLM course lecture 5: "编码实现RMSNorm", "RoPE公式",
              "RoPE高效实现", "SwiGLU模块", "LlamaDecoderLayer内部结构".

Readings taken where the pages are silent or ambiguous (each listed in the
design notes): RoPE pairs are half-split (j, j+d/2) unless ``interleaved``;
q head h reads kv head floor(h / (n_heads / n_kv_heads)); dynamic-NTK uses the
NTK-aware base rescaling with L = kv_seq_len; Llama3 scaling is the piecewise
form with linear interpolation in orig/wavelength; eps sits inside the square
root; the causal mask is by token index; decode treats cached slots as already
rotated and overwrites slot pos_b with the new token.

No function is parity unpinned. The three readings the pages leave open (dynamic-NTK
frequencies for L > original_max_pos, the Llama3 middle band, and the repeat_kv head
mapping) are pinned against the Hugging Face Llama modules that the verl and nanotron
pages build on, run in float64 (tests/test_oracle_library_pins.py).
"""
from __future__ import annotations

import math

import numpy as np

F64 = np.float64


# ---------------------------------------------------------------- RMSNorm
def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """y = x / sqrt(mean(x^2) + eps) * g over the last axis.

    [llama3] §3.1: a_i / RMS(a) * g_i with RMS(a) = sqrt(mean a^2); the Meta code
    there (and [nju] "编码实现RMSNorm") adds eps to the mean inside rsqrt.
    """
    x = np.asarray(x, dtype=F64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(g, dtype=F64)


# ---------------------------------------------------------------- RoPE
def rope_frequencies(head_dim: int, rope, kv_seq_len: int) -> np.ndarray:
    """Per-pair angular frequencies f'_i, i = 0 .. head_dim/2 - 1.

    Base: f_i = theta^(-2i/d)  ([verl] §1 inv_freq = 1/(base^(arange(0,dim,2)/dim));
    [meta-qa] #### 2 precompute_freqs_cis).
    linear:      f'_i = f_i / factor ([verl] §1: positions divided by the scaling factor).
    dynamic_ntk: if L > original_max_pos the base becomes
                 theta * (factor*L/orig - (factor-1))^(d/(d-2)), else unchanged
                 ([verl] §1 "dynamically adjust base"; the formula is the reading).
    llama3:      wavelength lam_i = 2*pi/f_i; lam < orig/high_freq_factor keeps f;
                 lam > orig/low_freq_factor divides by factor; between, linear
                 interpolation with s = (orig/lam - lff)/(hff - lff)
                 ([verl] §1 Llama3 variant; [meta-qa] think §3 apply_scaling).
    """
    d = int(head_dim)
    i = np.arange(d // 2, dtype=F64)
    theta = float(rope.theta)
    t = rope.type
    if t == "dynamic_ntk":
        L = float(kv_seq_len)
        orig = float(rope.original_max_pos)
        if L > orig:
            theta = theta * (rope.factor * L / orig - (rope.factor - 1.0)) ** (d / (d - 2.0))
    f = theta ** (-(2.0 * i) / d)
    if t == "default" or t == "dynamic_ntk":
        return f
    if t == "linear":
        return f / rope.factor
    if t == "llama3":
        orig = float(rope.original_max_pos)
        lam = 2.0 * math.pi / f
        lam_hi = orig / rope.high_freq_factor
        lam_lo = orig / rope.low_freq_factor
        out = np.empty_like(f)
        for j in range(f.size):
            if lam[j] < lam_hi:
                out[j] = f[j]
            elif lam[j] > lam_lo:
                out[j] = f[j] / rope.factor
            else:
                s = (orig / lam[j] - rope.low_freq_factor) / (rope.high_freq_factor - rope.low_freq_factor)
                out[j] = (1.0 - s) * f[j] / rope.factor + s * f[j]
        return out
    raise ValueError(f"unknown rope type {t!r}")


def rope_rotate(x: np.ndarray, positions: np.ndarray, freqs: np.ndarray, interleaved: bool = False) -> np.ndarray:
    """Rotate each pair of x[..., d] by angle pos * f'_j.

    Half-split pairs (j, j+d/2): x'_j = x_j cos - x_{j+d/2} sin,
    x'_{j+d/2} = x_{j+d/2} cos + x_j sin  ([nju] "RoPE高效实现" rotate_half:
    q*cos + rotate_half(q)*sin with cos = cat(cos, cos) as in [verl] §1).
    Interleaved pairs (2j, 2j+1): multiplication of x_{2j} + i x_{2j+1} by
    e^{i phi} ([meta-qa] #### 2, torch.polar and complex multiply).
    ``positions`` broadcasts against x[..., 0].
    """
    x = np.asarray(x, dtype=F64)
    d = x.shape[-1]
    h = d // 2
    phi = np.asarray(positions, dtype=F64)[..., None] * np.asarray(freqs, dtype=F64)  # [..., d/2]
    c, s = np.cos(phi), np.sin(phi)
    out = np.empty_like(x)
    if interleaved:
        a, b = x[..., 0::2], x[..., 1::2]
        out[..., 0::2] = a * c - b * s
        out[..., 1::2] = b * c + a * s
    else:
        a, b = x[..., :h], x[..., h:]
        out[..., :h] = a * c - b * s
        out[..., h:] = b * c + a * s
    return out


# ---------------------------------------------------------------- projections
def linear(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """y = x W^T with W stored [out_features, in_features] (nn.Linear, bias=False:
    [nju] "LlamaDecoderLayer内部结构")."""
    return np.asarray(x, dtype=F64) @ np.asarray(w, dtype=F64).T


def split_qkv(qkv: np.ndarray, n_heads: int, n_kv_heads: int, head_dim: int):
    """Packed rows Q|K|V ([nanotron] §9.3 fused qkv_proj of width hidden + 2*n_kv*d;
    [verl] §2 split([q_size, k_size, v_size])), each viewed [..., heads, d]."""
    qd, kd = n_heads * head_dim, n_kv_heads * head_dim
    lead = qkv.shape[:-1]
    q = qkv[..., :qd].reshape(*lead, n_heads, head_dim)
    k = qkv[..., qd:qd + kd].reshape(*lead, n_kv_heads, head_dim)
    v = qkv[..., qd + kd:].reshape(*lead, n_kv_heads, head_dim)
    return q, k, v


# ---------------------------------------------------------------- attention
def _softmax_rows(s: np.ndarray) -> np.ndarray:
    """softmax over the last axis, max-subtracted ([verl] §2 softmax in float32 there; exact here)."""
    m = np.max(s, axis=-1, keepdims=True)
    p = np.exp(s - m)
    return p / np.sum(p, axis=-1, keepdims=True)


def attention_prefill(q: np.ndarray, k: np.ndarray, v: np.ndarray, causal: bool = True,
                      q_block: int = 512) -> np.ndarray:
    """Grouped-query scaled-dot-product attention over one call's tokens.

    q [B,S,n_h,d], k/v [B,S,n_kv,d] -> o [B,S,n_h*d] (heads concatenated, [llama3]
    §3.2 transpose(1,2).view(bsz, seqlen, -1)).
    o_i = sum_{j<=i} softmax_j(q_i . k_j / sqrt(d)) v_j  ([verl] §2: matmul / sqrt(head_dim),
    softmax, matmul; causal mask triu(-inf, diagonal=1) by index, [meta-qa] #### 5).
    q head h uses kv head h // (n_h/n_kv): each group of consecutive query heads
    shares one K/V head ([llama3] §3.2 GQA; repeat_kv in [nanotron] §9.3).
    """
    B, S, nh, d = q.shape
    nkv = k.shape[2]
    g = nh // nkv
    out = np.empty((B, S, nh, d), dtype=F64)
    scale = 1.0 / math.sqrt(d)
    for b in range(B):
        for h in range(nh):
            c = h // g
            kk = np.asarray(k[b, :, c, :], dtype=F64)
            vv = np.asarray(v[b, :, c, :], dtype=F64)
            for i0 in range(0, S, q_block):
                i1 = min(S, i0 + q_block)
                qq = np.asarray(q[b, i0:i1, h, :], dtype=F64)
                kmax = i1 if causal else S
                s = (qq @ kk[:kmax].T) * scale                  # [i1-i0, kmax]
                if causal:
                    rows = np.arange(i0, i1)[:, None]
                    cols = np.arange(kmax)[None, :]
                    s = np.where(cols > rows, -np.inf, s)
                out[b, i0:i1, h, :] = _softmax_rows(s) @ vv[:kmax]
    return out.reshape(B, S, nh * d)


def attention_one_query(q: np.ndarray, keys: np.ndarray, values: np.ndarray) -> np.ndarray:
    """One query position against L keys: q [n_h,d], keys/values [L,n_kv,d] -> [n_h*d].

    Used for decode (keys = cache slots 0..pos_b, [llama3] §3.2 cache_k[:bsz, :start_pos+seqlen])
    and for sampled rows of a prefill (keys = tokens 0..i)."""
    nh, d = q.shape
    nkv = keys.shape[1]
    g = nh // nkv
    out = np.empty((nh, d), dtype=F64)
    for h in range(nh):
        c = h // g
        s = (keys[:, c, :] @ q[h]) / math.sqrt(d)
        p = np.exp(s - np.max(s))
        out[h] = (p / np.sum(p)) @ values[:, c, :]
    return out.reshape(nh * d)


def attention_chunk(q: np.ndarray, k_new: np.ndarray, v_new: np.ndarray, positions: np.ndarray,
                    cache_k: np.ndarray, cache_v: np.ndarray):
    """Chunked prefill on a cache prefix ([llama3] §3.2: cache_k[:bsz, start_pos : start_pos + seqlen] = xk,
    then keys = cache_k[:bsz, : start_pos + seqlen]; [meta-qa] #### 5: for start_pos > 0 the mask is the
    causal triangle preceded by start_pos zero columns).

    q [B,S,n_h,d] and k_new [B,S,n_kv,d] already rotated, v_new [B,S,n_kv,d], positions [B,S];
    cache_k/cache_v [B,ctx,n_kv,d] before the write. The chunk's keys and values are written at their
    positions first; query (b, s) then attends over cache slots 0 .. positions[b, s].
    Returns o [B,S,n_h*d] and the caches after the write.
    """
    K = np.array(cache_k, dtype=F64, copy=True)
    V = np.array(cache_v, dtype=F64, copy=True)
    B, S = positions.shape
    for b in range(B):
        for s in range(S):
            K[b, int(positions[b, s])] = k_new[b, s]
            V[b, int(positions[b, s])] = v_new[b, s]
    nh, d = q.shape[2], q.shape[3]
    o = np.empty((B, S, nh * d), dtype=F64)
    for b in range(B):
        for s in range(S):
            p = int(positions[b, s])
            o[b, s] = attention_one_query(np.asarray(q[b, s], dtype=F64), K[b, :p + 1], V[b, :p + 1])
    return o, K, V


def attention_varlen(q: np.ndarray, k: np.ndarray, v: np.ndarray, cu_seqlens) -> np.ndarray:
    """Padding-free (packed) causal attention ([verl] §3 ParallelLlamaAttentionRmPad:
    flash_attn_varlen_func with cu_seqlens_q = cu_seqlens_k = cu_seqlens, causal=True).

    q [T,n_h,d], k/v [T,n_kv,d] hold the tokens of several sequences back to back; sequence i is tokens
    cu_seqlens[i] .. cu_seqlens[i+1]-1. Each token attends causally to the earlier tokens of its own
    sequence only. Returns o [T, n_h*d].
    """
    T, nh, d = q.shape
    out = np.empty((T, nh * d), dtype=F64)
    cu = [int(c) for c in cu_seqlens]
    for i in range(len(cu) - 1):
        a, b = cu[i], cu[i + 1]
        if b > a:
            out[a:b] = attention_prefill(q[None, a:b], k[None, a:b], v[None, a:b])[0]
    return out


# ---------------------------------------------------------------- MLP
def silu(z: np.ndarray) -> np.ndarray:
    """silu(z) = z * sigmoid(z) = z / (1 + e^-z) ([nju] "SwiGLU模块")."""
    z = np.asarray(z, dtype=F64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu_act(x: np.ndarray, w_gate_up: np.ndarray, intermediate: int) -> np.ndarray:
    """act = silu(x W_gate^T) * (x W_up^T) with W_gate_up rows gate|up
    ([nanotron] §9.4: gate_up_proj, chunk(2), F.silu(gate) * up)."""
    gu = linear(x, w_gate_up)
    return silu(gu[..., :intermediate]) * gu[..., intermediate:]


# ---------------------------------------------------------------- the layer
def _rope_qk(cfg, q, k, positions, kv_seq_len):
    f = rope_frequencies(cfg.head_dim, cfg.rope, kv_seq_len)
    il = bool(cfg.rope.interleaved)
    # positions [..] broadcast over heads
    qr = rope_rotate(q, positions[..., None], f, il)
    kr = rope_rotate(k, positions[..., None], f, il)
    return qr, kr


def layer_prefill(cfg, W: dict, x: np.ndarray, position_ids: np.ndarray, kv_seq_len: int) -> dict:
    """Full decoder-layer forward over B sequences of S tokens ([nanotron] §9.5):
        h   = x + o_proj(attn(rmsnorm(x; g_attn)))
        out = h + down(silu(gate(hn)) * up(hn)),  hn = rmsnorm(h; g_mlp)
    Returns out and the residual-free branch outputs for separate comparison.
    W holds fp64 arrays (w_qkv, w_o, w_gate_up, w_down, g_attn, g_mlp); x [B,S,H].
    """
    x = np.asarray(x, dtype=F64)
    xn = rmsnorm(x, W["g_attn"], cfg.eps)
    qkv = linear(xn, W["w_qkv"])
    q, k, v = split_qkv(qkv, cfg.n_heads, cfg.n_kv_heads, cfg.head_dim)
    qr, kr = _rope_qk(cfg, q, k, np.asarray(position_ids), kv_seq_len)
    o = attention_prefill(qr, kr, v, causal=True)
    attn_proj = linear(o, W["w_o"])
    h = x + attn_proj
    hn = rmsnorm(h, W["g_mlp"], cfg.eps)
    act = swiglu_act(hn, W["w_gate_up"], cfg.intermediate)
    mlp_out = linear(act, W["w_down"])
    out = h + mlp_out
    return {"xn": xn, "qkv": qkv, "q_rot": qr, "k_rot": kr, "v": v, "o": o, "attn_proj": attn_proj,
            "h": h, "hn": hn, "act": act, "mlp_out": mlp_out, "out": out}


def layer_prefill_rows(cfg, W: dict, x: np.ndarray, position_ids: np.ndarray, kv_seq_len: int,
                       rows) -> dict:
    """The same layer, evaluated only at the token rows ``rows`` = [(b, i), ...].

    Each sampled row still attends over the full keys/values of tokens 0..i of
    its sequence, so K and V are formed for every token of the sequences
    involved. Returns arrays indexed like ``rows``.
    """
    x = np.asarray(x, dtype=F64)
    f = rope_frequencies(cfg.head_dim, cfg.rope, kv_seq_len)
    il = bool(cfg.rope.interleaved)
    nh, nkv, d = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
    res = {k: [] for k in ("o", "attn_proj", "h", "act", "mlp_out", "out", "k_rot", "v")}
    by_b = {}
    for r, (b, i) in enumerate(rows):
        by_b.setdefault(b, []).append((r, i))
    out_rows = [None] * len(rows)
    for b, items in by_b.items():
        xb = x[b]
        xn = rmsnorm(xb, W["g_attn"], cfg.eps)
        imax = max(i for _, i in items) + 1
        qkv = linear(xn[:imax], W["w_qkv"])
        q, k, v = split_qkv(qkv, nh, nkv, d)
        pos = np.asarray(position_ids[b, :imax])
        kr = rope_rotate(k, pos[:, None], f, il)
        for r, i in items:
            qr = rope_rotate(q[i], np.full((nh,), pos[i]), f, il)
            o = attention_one_query(qr, kr[:i + 1], v[:i + 1])
            attn_proj = linear(o, W["w_o"])
            h = xb[i] + attn_proj
            hn = rmsnorm(h, W["g_mlp"], cfg.eps)
            act = swiglu_act(hn, W["w_gate_up"], cfg.intermediate)
            mlp_out = linear(act, W["w_down"])
            out_rows[r] = {"o": o, "attn_proj": attn_proj, "h": h, "act": act, "mlp_out": mlp_out,
                           "out": h + mlp_out, "k_rot": kr[i].reshape(-1), "v": v[i].reshape(-1)}
    for key in res:
        res[key] = np.stack([row[key] for row in out_rows])
    return res


def layer_prefill_chunk(cfg, W: dict, x: np.ndarray, position_ids: np.ndarray, kv_seq_len: int,
                        cache_k: np.ndarray, cache_v: np.ndarray) -> dict:
    """The decoder layer over a chunk of S tokens per sequence that continues a cached prefix
    ([llama3] §3.2 with start_pos > 0 and seqlen > 1; [meta-qa] #### 5 mask with start_pos zero
    columns): as layer_prefill, except that attention is attention_chunk over the caches
    (cache_k/cache_v [B,ctx,n_kv,d] before the call). Returns the layer outputs and the caches after."""
    x = np.asarray(x, dtype=F64)
    xn = rmsnorm(x, W["g_attn"], cfg.eps)
    qkv = linear(xn, W["w_qkv"])
    q, k, v = split_qkv(qkv, cfg.n_heads, cfg.n_kv_heads, cfg.head_dim)
    qr, kr = _rope_qk(cfg, q, k, np.asarray(position_ids), kv_seq_len)
    o, K, V = attention_chunk(qr, kr, v, np.asarray(position_ids), cache_k, cache_v)
    attn_proj = linear(o, W["w_o"])
    h = attn_proj + x
    hn = rmsnorm(h, W["g_mlp"], eps=cfg.eps)
    act = swiglu_act(hn, W["w_gate_up"], cfg.intermediate)
    mlp_out = linear(act, W["w_down"])
    return {"o": o, "attn_proj": attn_proj, "h": h, "act": act, "mlp_out": mlp_out, "out": h + mlp_out,
            "k_rot": kr, "v": v, "cache_k": K, "cache_v": V}


def layer_prefill_varlen(cfg, W: dict, x: np.ndarray, position_ids: np.ndarray, cu_seqlens, kv_seq_len: int) -> dict:
    """The decoder layer over packed tokens ([verl] §3 ParallelLlamaAttentionRmPad): x [T,H] holds several
    sequences back to back (boundaries cu_seqlens); the projections, norms and MLP act per token, RoPE
    rotates token t at position_ids[t] (the rmpad path rotates by the index within the sequence, which
    is what callers pass), and attention is attention_varlen."""
    x = np.asarray(x, dtype=F64)
    xn = rmsnorm(x, W["g_attn"], cfg.eps)
    qkv = linear(xn, W["w_qkv"])
    q, k, v = split_qkv(qkv, cfg.n_heads, cfg.n_kv_heads, cfg.head_dim)
    qr, kr = _rope_qk(cfg, q, k, np.asarray(position_ids), kv_seq_len)
    o = attention_varlen(qr, kr, v, cu_seqlens)
    attn_proj = linear(o, W["w_o"])
    h = np.add(x, attn_proj)
    hn = rmsnorm(h, g=W["g_mlp"], eps=cfg.eps)
    act = swiglu_act(hn, W["w_gate_up"], cfg.intermediate)
    mlp_out = linear(act, W["w_down"])
    return {"o": o, "attn_proj": attn_proj, "h": h, "act": act, "mlp_out": mlp_out, "out": mlp_out + h}


def layer_decode(cfg, W: dict, x: np.ndarray, pos: np.ndarray, kv_seq_len: int, cache_row_k, cache_row_v,
                 batch_rows=None) -> dict:
    """One decode step: S = 1 new token per sequence b at position pos[b] ([llama3] §3.2 with
    start_pos = pos[b], seqlen = 1; [meta-qa] #### 3 KV cache).

    The rotated new key and the new value overwrite cache slot pos[b]; the query
    attends over slots 0..pos[b], earlier slots taken as stored (already rotated).
    ``cache_row_k(b)`` / ``cache_row_v(b)`` return the fp64 cache row [ctx, n_kv, d]
    before the write. ``batch_rows`` limits the evaluation to some sequences.
    """
    x = np.asarray(x, dtype=F64)                       # [B, 1, H]
    f = rope_frequencies(cfg.head_dim, cfg.rope, kv_seq_len)
    il = bool(cfg.rope.interleaved)
    nh, nkv, d = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
    bs = range(x.shape[0]) if batch_rows is None else batch_rows
    outs = {k: [] for k in ("o", "attn_proj", "h", "act", "mlp_out", "out", "k_new", "v_new")}
    for b in bs:
        xb = x[b, 0]
        xn = rmsnorm(xb, W["g_attn"], cfg.eps)
        qkv = linear(xn, W["w_qkv"])
        q, k, v = split_qkv(qkv, nh, nkv, d)
        p = int(pos[b])
        qr = rope_rotate(q, np.full((nh,), p), f, il)
        kr = rope_rotate(k, np.full((nkv,), p), f, il)
        K = cache_row_k(b)[:p + 1].copy()
        V = cache_row_v(b)[:p + 1].copy()
        K[p] = kr
        V[p] = v
        o = attention_one_query(qr, K, V)
        attn_proj = linear(o, W["w_o"])
        h = xb + attn_proj
        hn = rmsnorm(h, W["g_mlp"], cfg.eps)
        act = swiglu_act(hn, W["w_gate_up"], cfg.intermediate)
        mlp_out = linear(act, W["w_down"])
        for key, val in (("o", o), ("attn_proj", attn_proj), ("h", h), ("act", act), ("mlp_out", mlp_out),
                         ("out", h + mlp_out), ("k_new", kr.reshape(-1)), ("v_new", v.reshape(-1))):
            outs[key].append(val)
    return {k: np.stack(v) for k, v in outs.items()}


# ---------------------------------------------------------------- the model stack
def embedding(table: np.ndarray, tokens: np.ndarray) -> np.ndarray:
    """nn.Embedding lookup ([meta-qa] #### 5 tok_embeddings(tokens)): row tokens[b, s] of table [vocab, H]."""
    return np.asarray(table, dtype=F64)[np.asarray(tokens)]


def model_prefill(cfg, M: dict, tokens: np.ndarray, position_ids: np.ndarray, kv_seq_len: int) -> dict:
    """The model driver of [meta-qa] #### 5 (Transformer.forward at start_pos = 0): token embeddings,
    the decoder layers in order, the final RMSNorm, then the output projection to vocabulary logits
    (output(norm(h)), no bias). M holds fp64 "layers" (list of layer weight dicts), "tok_embeddings"
    [vocab, H], "g_final" [H] and "lm_head" [vocab, H]. Returns the last hidden state and the logits."""
    h = embedding(M["tok_embeddings"], tokens)
    for W in M["layers"]:
        h = layer_prefill(cfg, W, h, position_ids, kv_seq_len)["out"]
    hn = rmsnorm(h, M["g_final"], cfg.eps)
    return {"h": h, "logits": linear(hn, M["lm_head"])}


# ---------------------------------------------------------------- comparison metric
def max_rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """Normwise max relative error: max|got - ref| / max|ref| (the reading of "max relative
    error" used for every parity threshold)."""
    got = np.asarray(got, dtype=F64)
    ref = np.asarray(ref, dtype=F64)
    den = float(np.max(np.abs(ref))) if ref.size else 0.0
    num = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    if den == 0.0:
        return num
    return num / den
