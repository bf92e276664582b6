"""GPU parity of llama_layer_forward at the workloads' full sizes, whole outputs and separated branches.

* The Llama-3.2-1B (B=4, S=2048) and Llama-3-8B (B=2, S=4096) prefill layers are compared element by
  element over the whole output with the oracle's full layer.
* Each residual branch is also checked alone, at the same full sizes: the hidden input is scaled by 2^-12
  (exact in bf16) and eps set to 0, so both RMSNorms see the same normalised rows as the unscaled input
  while the residual stream becomes negligible next to the branch; then
    - W_down = 0 leaves out = x + o W_o^T (the attention branch, nanotron §9.5 first residual),
    - W_o = 0 leaves out = x + act W_down^T (the MLP branch alone),
    - W_o = identity and W_down = 0 leaves out = x + o, the attention output itself (llama3 结构详解 §3.2).
  Each is compared normwise with the oracle's own result for those weights, so a branch error can no longer
  hide under the N(0,1) residual stream or cancel between the two branches.
* The 32k Llama3-RoPE prefill is compared on 256 rows: the first and last row of each 256-row tile.
* The 8B decode step is compared on all 64 sequences, with both appended cache slots (K and V).
* Decode with B = 128 (more than 64 rows: the projections take their many-row plan) on a short cache.
* Dynamic-NTK RoPE over 50 decode steps whose kv_seq_len grows past original_max_pos, each step against
  the oracle, with device memory flat across the steps (the RoPE table is regenerated in place).
"""
import dataclasses

import numpy as np
import pytest
import torch

import transformer_layer_forward_amd as L
from oracle import ref
from synth_inputs import (CONFIGS, RopeCfg, make_cache, make_cache_row, make_decode_positions, make_hidden,
                          make_prefill_positions, make_weights, scaled, to_f64 as bits_to_f64, f32_to_bf16_bits)
from tests.gpu_util import DEV, require_gpu, tol, to_dev, to_f64
from tests.test_gpu_layer import check, dev_weights, layer_cfg, w64

pytestmark = pytest.mark.gpu


def _run_prefill(cfg, W, x, pos):
    out = L.llama_layer_forward(layer_cfg(cfg), dev_weights(W, cfg.dtype), to_dev(x, cfg.dtype),
                                torch.from_numpy(pos).to(DEV), kv_seq_len=cfg.S)
    return to_f64(out)


@pytest.mark.parametrize("name", ["llama32_1b_prefill", "llama3_8b_prefill"])
def test_layer_full_size_whole_output(name):
    """Every element of out (and of out - hidden) against the oracle's full layer."""
    require_gpu()
    cfg = CONFIGS[name]
    print(f"case {name} whole output", flush=True)
    W = make_weights(cfg, seed=0)
    x = make_hidden(cfg, seed=0)
    pos = make_prefill_positions(cfg)
    got = _run_prefill(cfg, W, x, pos)
    x64 = bits_to_f64(x, cfg.dtype)
    want = ref.layer_prefill(cfg, w64(W, cfg.dtype), x64, pos, cfg.S)
    check(got, x64, want["out"], want["attn_proj"] + want["mlp_out"], cfg.dtype, name)


def _scale_bits(bits, k):
    """Multiply bf16 values (uint16 bits) by 2^k exactly (exponent shift; no value here under/overflows)."""
    f = bits_to_f64(bits, "bf16").astype(np.float32) * np.float32(2.0 ** k)
    out = f32_to_bf16_bits(f)
    assert np.array_equal(bits_to_f64(out, "bf16"), bits_to_f64(bits, "bf16") * 2.0 ** k)
    return out


def _identity_bits(n):
    return f32_to_bf16_bits(np.eye(n, dtype=np.float32))


@pytest.mark.parametrize("branch", ["attention", "mlp", "attention_output"])
@pytest.mark.parametrize("name", ["llama32_1b_prefill", "llama3_8b_prefill"])
def test_layer_branch_alone_full_size(name, branch):
    require_gpu()
    cfg = dataclasses.replace(CONFIGS[name], eps=0.0)
    print(f"case {name} branch {branch}", flush=True)
    W = make_weights(cfg, seed=0)
    if branch in ("attention", "attention_output"):
        W["w_down"] = np.zeros_like(W["w_down"])
    if branch == "mlp":
        W["w_o"] = np.zeros_like(W["w_o"])
    if branch == "attention_output":
        assert cfg.n_heads * cfg.head_dim == cfg.hidden
        W["w_o"] = _identity_bits(cfg.hidden)
    x = _scale_bits(make_hidden(cfg, seed=0), -12)
    pos = make_prefill_positions(cfg)
    got = _run_prefill(cfg, W, x, pos)
    x64 = bits_to_f64(x, cfg.dtype)
    want = ref.layer_prefill(cfg, w64(W, cfg.dtype), x64, pos, cfg.S)
    target = {"attention": want["attn_proj"], "mlp": want["mlp_out"], "attention_output": want["o"]}[branch]
    # the scaled residual is below a bf16 step of the branch: out is the branch to within tolerance
    assert np.max(np.abs(x64)) < 2.0 ** -7 * np.max(np.abs(target))
    e = ref.max_rel_err(got, want["out"])
    e_branch = ref.max_rel_err(got - x64, target)
    print(f"{name} {branch}: out err {e:.3e}, branch err {e_branch:.3e}", flush=True)
    assert e <= tol(cfg.dtype)
    assert e_branch <= tol(cfg.dtype)


def test_layer_long_llama3rope_tile_edge_rows():
    """32k prefill with Llama3 RoPE: the first and last row of every 256-row tile of the sequence."""
    require_gpu()
    cfg = CONFIGS["llama3_8b_long_llama3rope"]
    print("case llama3_8b_long_llama3rope tile-edge rows", flush=True)
    W = make_weights(cfg, seed=0)
    x = make_hidden(cfg, seed=0)
    pos = make_prefill_positions(cfg)
    got = _run_prefill(cfg, W, x, pos)
    rows = sorted({(0, t) for t0 in range(0, cfg.S, 256) for t in (t0, t0 + 255)})
    assert len(rows) == 256
    x64 = bits_to_f64(x, cfg.dtype)
    want = ref.layer_prefill_rows(cfg, w64(W, cfg.dtype), x64, pos, cfg.S, rows)
    g = np.stack([got[b, i] for b, i in rows])
    xs = np.stack([x64[b, i] for b, i in rows])
    check(g, xs, want["out"], want["attn_proj"] + want["mlp_out"], cfg.dtype, cfg.name)


def _decode_case(cfg, seed, lo):
    W = make_weights(cfg, seed=seed)
    x = make_hidden(cfg, seed=seed)
    pos = make_decode_positions(cfg, seed=seed, lo=lo)
    return W, x, pos


def _check_decode_all(cfg, W, x, pos, tk, tv, out, krow, vrow):
    got = to_f64(out)[:, 0]
    x64 = bits_to_f64(x, cfg.dtype)
    want = ref.layer_decode(cfg, w64(W, cfg.dtype), x64, pos, cfg.ctx, krow, vrow)
    check(got, x64[:, 0], want["out"], want["attn_proj"] + want["mlp_out"], cfg.dtype, cfg.name)
    idx = torch.from_numpy(pos).to(DEV)
    ar = torch.arange(cfg.B, device=DEV)
    gk = to_f64(tk[ar, idx]).reshape(cfg.B, -1)
    gv = to_f64(tv[ar, idx]).reshape(cfg.B, -1)
    for b in range(cfg.B):
        assert ref.max_rel_err(gk[b], want["k_new"][b]) <= tol(cfg.dtype), b
        assert ref.max_rel_err(gv[b], want["v_new"][b]) <= tol(cfg.dtype), b


def test_layer_full_size_decode_all_sequences():
    """The 8B decode step (B = 64 against [64, 8192, 8, 128] caches): every sequence's output and both
    appended cache slots."""
    require_gpu()
    cfg = CONFIGS["llama3_8b_decode"]
    print("case llama3_8b_decode all sequences", flush=True)
    W, x, pos = _decode_case(cfg, 0, 1024)
    tk = to_dev(make_cache(cfg, "k", seed=0), cfg.dtype)
    tv = to_dev(make_cache(cfg, "v", seed=0), cfg.dtype)
    out = L.llama_layer_forward(layer_cfg(cfg), dev_weights(W, cfg.dtype), to_dev(x, cfg.dtype),
                                torch.from_numpy(pos).to(DEV), kv_seq_len=cfg.ctx, k_cache=tk, v_cache=tv)
    _check_decode_all(cfg, W, x, pos, tk, tv, out,
                      lambda b: bits_to_f64(make_cache_row(cfg, "k", b, 0), cfg.dtype),
                      lambda b: bits_to_f64(make_cache_row(cfg, "v", b, 0), cfg.dtype))


@pytest.mark.parametrize("B", [96, 128])
def test_layer_decode_many_sequences(B):
    """Decode with more than 64 sequences: the projections leave the skinny path (their many-row plan and its
    cache append); every sequence's output and both appended slots."""
    require_gpu()
    cfg = scaled(CONFIGS["llama3_8b_decode"], B=B, ctx=300)
    print(f"case decode B={B}", flush=True)
    W, x, pos = _decode_case(cfg, 5, 1)
    pos[0], pos[-1] = 0, cfg.ctx - 1
    kc, vc = make_cache(cfg, "k", seed=5), make_cache(cfg, "v", seed=5)
    tk, tv = to_dev(kc, cfg.dtype), to_dev(vc, cfg.dtype)
    out = L.llama_layer_forward(layer_cfg(cfg), dev_weights(W, cfg.dtype), to_dev(x, cfg.dtype),
                                torch.from_numpy(pos).to(DEV), kv_seq_len=cfg.ctx, k_cache=tk, v_cache=tv)
    _check_decode_all(cfg, W, x, pos, tk, tv, out, lambda b: bits_to_f64(kc[b], cfg.dtype),
                      lambda b: bits_to_f64(vc[b], cfg.dtype))


def test_layer_decode_dynamic_ntk_growing_length():
    """verl "parallel_attention.py" §1-§2: dynamic-NTK recomputes the RoPE base from kv_seq_len. 50 decode
    steps with kv_seq_len = 8193 .. 8242 past original_max_pos = 8192 (each step's token at position
    kv_seq_len - 1), each against the oracle at that length; the oracle carries its own cache forward
    (its rotated keys and values), the GPU its own. Device memory stays flat: the table (8242 rows of 64
    cos/sin pairs, 4 MiB per length) is regenerated in place, not reallocated per length."""
    require_gpu()
    cfg = scaled(CONFIGS["llama3_8b_decode"], B=3, ctx=8256, hidden=1024, n_heads=8, n_kv_heads=2,
                 intermediate=2048, rope=RopeCfg(type="dynamic_ntk", theta=500000.0, factor=4.0,
                                                 original_max_pos=8192))
    print("case dynamic-NTK growing decode", flush=True)
    W = make_weights(cfg, seed=8)
    Wd = dev_weights(W, cfg.dtype)
    W64 = w64(W, cfg.dtype)
    lc = layer_cfg(cfg)
    kc, vc = make_cache(cfg, "k", seed=8), make_cache(cfg, "v", seed=8)
    tk, tv = to_dev(kc, cfg.dtype), to_dev(vc, cfg.dtype)
    K64 = [bits_to_f64(kc[b], cfg.dtype) for b in range(cfg.B)]
    V64 = [bits_to_f64(vc[b], cfg.dtype) for b in range(cfg.B)]
    free0 = None
    for step in range(50):
        Lq = 8193 + step
        x = make_hidden(cfg, seed=100 + step)
        pos = np.full((cfg.B,), Lq - 1, dtype=np.int64)
        out = L.llama_layer_forward(lc, Wd, to_dev(x, cfg.dtype), torch.from_numpy(pos).to(DEV), kv_seq_len=Lq,
                                    k_cache=tk, v_cache=tv)
        torch.cuda.synchronize()
        if step == 0:
            free0 = torch.cuda.mem_get_info()[0]
        x64 = bits_to_f64(x, cfg.dtype)
        want = ref.layer_decode(cfg, W64, x64, pos, Lq, lambda b: K64[b], lambda b: V64[b])
        got = to_f64(out)[:, 0]
        e = ref.max_rel_err(got, want["out"])
        eb = ref.max_rel_err(got - x64[:, 0], want["attn_proj"] + want["mlp_out"])
        assert e <= tol(cfg.dtype) and eb <= 3e-2, (step, e, eb)
        for b in range(cfg.B):
            K64[b][Lq - 1] = want["k_new"][b].reshape(cfg.n_kv_heads, cfg.head_dim)
            V64[b][Lq - 1] = want["v_new"][b].reshape(cfg.n_kv_heads, cfg.head_dim)
            assert ref.max_rel_err(to_f64(tk[b, Lq - 1]).reshape(-1), want["k_new"][b]) <= tol(cfg.dtype)
    print(f"free memory after step 0: {free0}, after step 49: {torch.cuda.mem_get_info()[0]}", flush=True)
    assert torch.cuda.mem_get_info()[0] == free0
