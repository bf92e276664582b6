"""GPU parity of llama_layer_forward against the fp64 oracle.

Small members of each workload family are compared in full; the full-size workloads are compared on
seeded sampled rows the oracle evaluates one by one (rows 0 and S-1 always included). Besides the
output, out - hidden (the two residual branches together, o_proj + MLP) is compared, since the
N(0,1) residual stream would otherwise hide branch errors."""
import dataclasses
import os

import numpy as np
import pytest
import torch

import transformer_layer_forward_amd as L
from oracle import ref
from synth_inputs import (CONFIGS, RopeCfg, make_cache, make_cache_row, make_decode_positions, make_hidden,
                          make_prefill_positions, make_weights, normal, scaled, to_f64 as bits_to_f64)
from tests.gpu_util import DEV, require_gpu, tol, to_dev, to_f64

pytestmark = pytest.mark.gpu

TD = {"bf16": torch.bfloat16, "f32": torch.float32}


def layer_cfg(cfg) -> L.LayerConfig:
    rc = cfg.rope
    rope = L.Rope(type=rc.type, theta=rc.theta, factor=rc.factor, low_freq_factor=rc.low_freq_factor,
                  high_freq_factor=rc.high_freq_factor, original_max_pos=rc.original_max_pos,
                  interleaved=rc.interleaved)
    return L.LayerConfig(cfg.hidden, cfg.n_heads, cfg.n_kv_heads, cfg.head_dim, cfg.intermediate, cfg.eps, rope,
                         TD[cfg.dtype])


def dev_weights(W, dtype):
    return {k: to_dev(v, dtype) for k, v in W.items()}


def w64(W, dtype):
    return {k: bits_to_f64(v, dtype) for k, v in W.items()}


def check(got_out, x64, want_out, want_branch, dtype, label=""):
    e_out = ref.max_rel_err(got_out, want_out)
    e_br = ref.max_rel_err(got_out - x64, want_branch)
    print(f"{label} out err {e_out:.3e} branch err {e_br:.3e}", flush=True)
    assert e_out <= tol(dtype), label
    # out - hidden inherits out's own rounding (half an ulp: 2^-9 |out| in bf16), so the branch bound is
    # the tolerance on the branch plus that rounding
    ulp = 2.0 ** -8 if dtype == "bf16" else 1e-6
    bound = tol(dtype) * np.max(np.abs(want_branch)) + ulp * np.max(np.abs(got_out))
    assert np.max(np.abs(got_out - x64 - want_branch)) <= bound, label


SMALL = [
    CONFIGS["tiny_f32"],
    scaled(CONFIGS["tiny_f32"], B=2, S=45, rope=RopeCfg(type="llama3", theta=10000.0, factor=8.0,
                                                        original_max_pos=16, interleaved=True)),
    scaled(CONFIGS["llama32_1b_prefill"], B=2, S=160),
    scaled(CONFIGS["llama3_8b_prefill"], B=1, S=100),
    scaled(CONFIGS["llama3_8b_prefill"], B=2, S=70, rope=RopeCfg(type="dynamic_ntk", theta=500000.0, factor=2.0,
                                                                 original_max_pos=32)),
    scaled(CONFIGS["llama3_8b_prefill"], B=1, S=129, rope=RopeCfg(type="linear", theta=500000.0, factor=4.0,
                                                                  interleaved=True)),
    scaled(CONFIGS["llama3_8b_long_llama3rope"], S=300),
    scaled(CONFIGS["llama32_1b_prefill"], B=1, S=90, rope=RopeCfg(type="llama3", theta=500000.0, factor=32.0,
                                                                  original_max_pos=64, interleaved=True)),
    # d = 64 with (n_h + n_kv) odd: the rotated q/k columns end half-way through a 128-column block
    scaled(CONFIGS["llama32_1b_prefill"], name="d64_odd_heads", B=1, S=150, hidden=384, n_heads=6, n_kv_heads=3,
           intermediate=512),
]


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: f"{c.name}-B{c.B}-S{c.S}-{c.rope.type}")
def test_layer_prefill_small(cfg):
    require_gpu()
    W = make_weights(cfg, seed=0)
    x = make_hidden(cfg, seed=0)
    pos = make_prefill_positions(cfg)
    out = L.llama_layer_forward(layer_cfg(cfg), dev_weights(W, cfg.dtype), to_dev(x, cfg.dtype),
                                torch.from_numpy(pos).to(DEV), kv_seq_len=cfg.S)
    got = to_f64(out)
    x64 = bits_to_f64(x, cfg.dtype)
    want = ref.layer_prefill(cfg, w64(W, cfg.dtype), x64, pos, cfg.S)
    check(got, x64, want["out"], want["attn_proj"] + want["mlp_out"], cfg.dtype, cfg.name)


def test_profile_selected_stages_only():
    """Stage timing restricted to one stage reports that stage alone, once per call, and leaves the output
    bit-identical to an untimed call."""
    require_gpu()
    cfg = scaled(CONFIGS["llama3_8b_prefill"], B=1, S=100)
    W = dev_weights(make_weights(cfg, seed=6), cfg.dtype)
    x = to_dev(make_hidden(cfg, seed=6), cfg.dtype)
    pos = torch.from_numpy(make_prefill_positions(cfg)).to(DEV)
    lc = layer_cfg(cfg)
    plain = L.llama_layer_forward(lc, W, x, pos, kv_seq_len=cfg.S)
    L.profile_begin(4, stages=["gate_up_silu"])
    outs = [L.llama_layer_forward(lc, W, x, pos, kv_seq_len=cfg.S) for _ in range(3)]
    st = L.profile_end()
    assert set(st) == {"gate_up_silu"}
    ms, n = st["gate_up_silu"]
    assert n == 3 and ms > 0.0
    for o in outs:
        assert torch.equal(o, plain)


def test_layer_in_place_and_causality():
    """out may equal hidden; perturbing later tokens leaves earlier rows bit-identical."""
    require_gpu()
    cfg = scaled(CONFIGS["llama32_1b_prefill"], B=1, S=200)
    W = dev_weights(make_weights(cfg, seed=1), cfg.dtype)
    x = to_dev(make_hidden(cfg, seed=1), cfg.dtype)
    pos = torch.from_numpy(make_prefill_positions(cfg)).to(DEV)
    lc = layer_cfg(cfg)
    a = L.llama_layer_forward(lc, W, x, pos)
    x2 = x.clone()
    x2[:, 120:] = -x2[:, 120:]
    b = L.llama_layer_forward(lc, W, x2, pos)
    inplace = x.clone()
    L.llama_layer_forward(lc, W, inplace, pos, out=inplace)
    torch.cuda.synchronize()
    assert torch.equal(a[:, :120], b[:, :120])
    assert not torch.equal(a[:, 120:], b[:, 120:])
    assert torch.equal(inplace, a)


def test_layer_zero_branches_is_identity():
    """W_o = W_down = 0 makes both branches exactly zero: out == hidden bit for bit (nanotron §9.5)."""
    require_gpu()
    cfg = scaled(CONFIGS["llama3_8b_prefill"], B=1, S=80)
    W = dev_weights(make_weights(cfg, seed=2), cfg.dtype)
    W["w_o"].zero_()
    W["w_down"].zero_()
    x = to_dev(make_hidden(cfg, seed=2), cfg.dtype)
    out = L.llama_layer_forward(layer_cfg(cfg), W, x, torch.from_numpy(make_prefill_positions(cfg)).to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(out, x)


# Decode shapes of the bf16 projections that sum their K ranges in the kernel (arrival groups of one
# 64-row block, of two blocks per 128-wide half-split RoPE head, single-range RoPE partials) and of the
# fp32 path.
DECODE_SMALL = [
    scaled(CONFIGS["llama3_8b_decode"], B=5, ctx=1300),
    scaled(CONFIGS["llama3_8b_decode"], name="8b_decode_interleaved", B=3, ctx=700,
           rope=RopeCfg(type="llama3", theta=500000.0, factor=8.0, original_max_pos=256, interleaved=True)),
    scaled(CONFIGS["llama32_1b_prefill"], name="1b_decode", B=7, S=1, ctx=900, decode=True),
    scaled(CONFIGS["llama32_1b_prefill"], name="d64_odd_heads_decode", B=4, S=1, ctx=300, decode=True, hidden=384,
           n_heads=6, n_kv_heads=3, intermediate=512),
    scaled(CONFIGS["tiny_f32"], B=3, S=1, ctx=40, decode=True),
]


@pytest.mark.parametrize("cfg", DECODE_SMALL, ids=lambda c: c.name)
def test_layer_decode_small(cfg):
    require_gpu()
    W = make_weights(cfg, seed=3)
    x = make_hidden(cfg, seed=3)
    lo = 1 if cfg.ctx < 1024 else 1024
    pos = make_decode_positions(cfg, seed=3, lo=lo)
    pos[0] = cfg.ctx - 1
    kc, vc = make_cache(cfg, "k", seed=3), make_cache(cfg, "v", seed=3)
    tk, tv = to_dev(kc, cfg.dtype), to_dev(vc, cfg.dtype)
    out = L.llama_layer_forward(layer_cfg(cfg), dev_weights(W, cfg.dtype), to_dev(x, cfg.dtype),
                                torch.from_numpy(pos).to(DEV), kv_seq_len=cfg.ctx, k_cache=tk, v_cache=tv)
    got = to_f64(out)[:, 0]
    x64 = bits_to_f64(x, cfg.dtype)
    want = ref.layer_decode(cfg, w64(W, cfg.dtype), x64, pos, cfg.ctx, lambda b: bits_to_f64(kc[b], cfg.dtype),
                            lambda b: bits_to_f64(vc[b], cfg.dtype))
    check(got, x64[:, 0], want["out"], want["attn_proj"] + want["mlp_out"], cfg.dtype, cfg.name)
    gk, gv = to_f64(tk), to_f64(tv)
    for b in range(cfg.B):
        assert ref.max_rel_err(gk[b, pos[b]].reshape(-1), want["k_new"][b]) <= tol(cfg.dtype)
        assert ref.max_rel_err(gv[b, pos[b]].reshape(-1), want["v_new"][b]) <= tol(cfg.dtype)


def test_layer_decode_matches_prefill_row():
    """Prefill of tokens 0..P-1 fills the cache; a decode step for token P must reproduce row P of a
    prefill over tokens 0..P (llama3 结构详解 §3.2; CSDN answer "#### 3.": the cache avoids recompute)."""
    require_gpu()
    P = 150
    cfg = scaled(CONFIGS["llama3_8b_prefill"], B=2, S=P + 1)
    W = dev_weights(make_weights(cfg, seed=4), cfg.dtype)
    x = to_dev(make_hidden(cfg, seed=4), cfg.dtype)
    lc = layer_cfg(cfg)
    ctx = 256
    pos = torch.from_numpy(make_prefill_positions(cfg)).to(DEV)
    full = L.llama_layer_forward(lc, W, x, pos, kv_seq_len=ctx)
    kc = torch.zeros((2, ctx, cfg.n_kv_heads, cfg.head_dim), device=DEV, dtype=torch.bfloat16)
    vc = torch.zeros_like(kc)
    L.llama_layer_forward(lc, W, x[:, :P].contiguous(), pos[:, :P].contiguous(), kv_seq_len=ctx, k_cache=kc,
                          v_cache=vc)
    step = L.llama_layer_forward(lc, W, x[:, P:P + 1].contiguous(), pos[:, P:P + 1].contiguous(), kv_seq_len=ctx,
                                 k_cache=kc, v_cache=vc)
    torch.cuda.synchronize()
    a, b = to_f64(step)[:, 0], to_f64(full)[:, P]
    xb = to_f64(x)[:, P]
    assert ref.max_rel_err(a, b) <= 2e-2
    assert ref.max_rel_err(a - xb, b - xb) <= 3e-2


# ------------------------------------------------------------------ chunked prefill on a cache prefix
CHUNK_LAYER = [
    # config, chunk length S, prefix length per sequence, ctx
    (scaled(CONFIGS["llama3_8b_prefill"], B=2, S=90), (0, 130), 256),
    (scaled(CONFIGS["llama32_1b_prefill"], B=1, S=70), (200,), 300),
    (scaled(CONFIGS["tiny_f32"], B=2, S=9), (5, 20), 40),
]


@pytest.mark.parametrize("case", CHUNK_LAYER, ids=lambda c: f"{c[0].name}-S{c[0].S}-P{'_'.join(map(str, c[1]))}")
def test_layer_chunk_small(case):
    """llama_layer_forward_chunk against the oracle's layer_prefill_chunk: a chunk at positions
    P..P+S-1 over seeded caches whose slots below P stand for an earlier prefix."""
    require_gpu()
    cfg, starts, ctx = case
    W = make_weights(cfg, seed=2)
    x = make_hidden(cfg, seed=2)
    pos = np.stack([np.arange(P, P + cfg.S) for P in starts]).astype(np.int64)
    kc = normal_cache(cfg, ctx, 160)
    vc = normal_cache(cfg, ctx, 161)
    x64 = bits_to_f64(x, cfg.dtype)
    K0, V0 = bits_to_f64(kc, cfg.dtype), bits_to_f64(vc, cfg.dtype)
    want = ref.layer_prefill_chunk(cfg, w64(W, cfg.dtype), x64, pos, ctx, K0, V0)
    tk, tv = to_dev(kc, cfg.dtype), to_dev(vc, cfg.dtype)
    out = L.llama_layer_forward_chunk(layer_cfg(cfg), dev_weights(W, cfg.dtype), to_dev(x, cfg.dtype),
                                      torch.from_numpy(pos).to(DEV), tk, tv, kv_seq_len=ctx)
    got = to_f64(out)
    check(got, x64, want["out"], want["attn_proj"] + want["mlp_out"], cfg.dtype, cfg.name)
    gk, gv = to_f64(tk), to_f64(tv)
    for b, P in enumerate(starts):
        assert ref.max_rel_err(gk[b, P:P + cfg.S], want["cache_k"][b, P:P + cfg.S]) <= tol(cfg.dtype)
        assert ref.max_rel_err(gv[b, P:P + cfg.S], want["cache_v"][b, P:P + cfg.S]) <= tol(cfg.dtype)
        np.testing.assert_array_equal(gk[b, :P], K0[b, :P])
        np.testing.assert_array_equal(gv[b, P + cfg.S:], V0[b, P + cfg.S:])


def normal_cache(cfg, ctx, k):
    return normal(2, k, (cfg.B, ctx, cfg.n_kv_heads, cfg.head_dim), cfg.dtype)


def test_layer_chunk_matches_one_shot():
    """Prefill of tokens 0..P-1 into the caches, then a chunk of tokens P..P+S-1, reproduces rows P.. of
    one prefill over all P+S tokens (llama3 结构详解 §3.2 start_pos; CSDN answer "#### 5.")."""
    require_gpu()
    P, S = 150, 100
    cfg = scaled(CONFIGS["llama3_8b_prefill"], B=2, S=P + S)
    W = dev_weights(make_weights(cfg, seed=5), cfg.dtype)
    x = to_dev(make_hidden(cfg, seed=5), cfg.dtype)
    lc = layer_cfg(cfg)
    ctx = 320
    pos = torch.from_numpy(make_prefill_positions(cfg)).to(DEV)
    full = L.llama_layer_forward(lc, W, x, pos, kv_seq_len=ctx)
    kc = torch.zeros((2, ctx, cfg.n_kv_heads, cfg.head_dim), device=DEV, dtype=torch.bfloat16)
    vc = torch.zeros_like(kc)
    L.llama_layer_forward(lc, W, x[:, :P].contiguous(), pos[:, :P].contiguous(), kv_seq_len=ctx, k_cache=kc,
                          v_cache=vc)
    chunk = L.llama_layer_forward_chunk(lc, W, x[:, P:].contiguous(), pos[:, P:].contiguous(), kc, vc,
                                        kv_seq_len=ctx)
    torch.cuda.synchronize()
    a, b = to_f64(chunk), to_f64(full)[:, P:]
    xb = to_f64(x)[:, P:]
    assert ref.max_rel_err(a, b) <= 2e-2
    assert ref.max_rel_err(a - xb, b - xb) <= 3e-2


# ------------------------------------------------------------------ varlen packed prefill
VARLEN_LAYER = [
    (scaled(CONFIGS["llama3_8b_prefill"], B=1, S=1), (90, 130, 1)),
    (scaled(CONFIGS["llama32_1b_prefill"], B=1, S=1), (64, 100)),
    (scaled(CONFIGS["tiny_f32"], B=1, S=1), (7, 12, 1)),
]


@pytest.mark.parametrize("case", VARLEN_LAYER, ids=lambda c: f"{c[0].name}-{'_'.join(map(str, c[1]))}")
def test_layer_varlen_small(case):
    """llama_layer_forward_varlen against the oracle's layer_prefill_varlen, RoPE at in-sequence positions
    (the rmpad convention of parallel_attention.py §4)."""
    require_gpu()
    base, lens = case
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    cfg = scaled(base, B=1, S=T)
    W = make_weights(cfg, seed=3)
    x = make_hidden(cfg, seed=3)[0]
    pos = np.concatenate([np.arange(n) for n in lens]).astype(np.int64)
    kv = max(lens)
    x64 = bits_to_f64(x, cfg.dtype)
    want = ref.layer_prefill_varlen(cfg, w64(W, cfg.dtype), x64, pos, cu, kv)
    out = L.llama_layer_forward_varlen(layer_cfg(cfg), dev_weights(W, cfg.dtype), to_dev(x, cfg.dtype),
                                       torch.from_numpy(pos).to(DEV), torch.from_numpy(cu).to(DEV), max(lens),
                                       kv_seq_len=kv)
    check(to_f64(out), x64, want["out"], want["attn_proj"] + want["mlp_out"], cfg.dtype, cfg.name)


@pytest.mark.parametrize("base", ["tiny_f32", "llama3_8b_prefill"])
def test_layer_varlen_equals_separate_calls(base):
    """Packing changes nothing per token: the varlen layer equals one llama_layer_forward per sequence.
    fp32: bit for bit (its kernels compute each row alone). bf16: a projection with few 256 x 256
    tiles splits K into a number of ranges that depends on the token count, so the packed and the
    separate runs may round differently; they must agree to within a few bf16 steps, where a token
    that saw another sequence's keys would be off by the size of the output itself."""
    require_gpu()
    lens = (130, 257, 65)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    cfg = scaled(CONFIGS[base], B=1, S=T)
    W = dev_weights(make_weights(cfg, seed=6), cfg.dtype)
    x = to_dev(make_hidden(cfg, seed=6), cfg.dtype)[0]
    pos = torch.from_numpy(np.concatenate([np.arange(n) for n in lens]).astype(np.int64)).to(DEV)
    lc = layer_cfg(cfg)
    kv = max(lens)
    packed = L.llama_layer_forward_varlen(lc, W, x, pos, torch.from_numpy(cu).to(DEV), kv, kv_seq_len=kv)
    for i, n in enumerate(lens):
        a, b = int(cu[i]), int(cu[i + 1])
        one = L.llama_layer_forward(lc, W, x[None, a:b].contiguous(), pos[None, a:b].contiguous(), kv_seq_len=kv)
        torch.cuda.synchronize()
        if cfg.dtype == "f32":
            assert torch.equal(packed[a:b], one[0]), i
        else:
            # the residual stream (|x| up to ~4) dominates the output: compare the layer's increment
            got, want, xin = packed[a:b].float(), one[0].float(), x[a:b].float()
            diff = (got - want).abs().max().item()
            scale = (want - xin).abs().max().item()
            print(f"seq {i}: max |packed - separate| {diff:.3e}, max |layer increment| {scale:.3e}")
            assert diff <= 2.0 ** -7 * want.abs().max().item() + 2.0 ** -6 * scale, (i, diff, scale)


# ------------------------------------------------------------------ full-size workloads, sampled rows
def _sample_rows(cfg, n, seed=7):
    rng = np.random.default_rng([seed, 99])
    rows = {(0, 0), (cfg.B - 1, cfg.S - 1)}
    while len(rows) < n:
        rows.add((int(rng.integers(0, cfg.B)), int(rng.integers(0, cfg.S))))
    return sorted(rows)


@pytest.mark.parametrize("name", ["llama32_1b_prefill", "llama3_8b_prefill", "llama3_8b_long_llama3rope"])
def test_layer_full_size_sampled(name):
    require_gpu()
    cfg = CONFIGS[name]
    W = make_weights(cfg, seed=0)
    x = make_hidden(cfg, seed=0)
    pos = make_prefill_positions(cfg)
    out = L.llama_layer_forward(layer_cfg(cfg), dev_weights(W, cfg.dtype), to_dev(x, cfg.dtype),
                                torch.from_numpy(pos).to(DEV), kv_seq_len=cfg.S)
    got = to_f64(out)
    rows = _sample_rows(cfg, 12 if cfg.S > 10000 else 24)
    x64 = bits_to_f64(x, cfg.dtype)
    want = ref.layer_prefill_rows(cfg, w64(W, cfg.dtype), x64, pos, cfg.S, rows)
    g = np.stack([got[b, i] for b, i in rows])
    xs = np.stack([x64[b, i] for b, i in rows])
    check(g, xs, want["out"], want["attn_proj"] + want["mlp_out"], cfg.dtype, name)


def test_layer_full_size_decode_sampled():
    require_gpu()
    cfg = CONFIGS["llama3_8b_decode"]
    W = make_weights(cfg, seed=0)
    x = make_hidden(cfg, seed=0)
    pos = make_decode_positions(cfg, seed=0)
    kc, vc = make_cache(cfg, "k", seed=0), make_cache(cfg, "v", seed=0)
    tk, tv = to_dev(kc, cfg.dtype), to_dev(vc, cfg.dtype)
    del kc, vc
    out = L.llama_layer_forward(layer_cfg(cfg), dev_weights(W, cfg.dtype), to_dev(x, cfg.dtype),
                                torch.from_numpy(pos).to(DEV), kv_seq_len=cfg.ctx, k_cache=tk, v_cache=tv)
    got = to_f64(out)[:, 0]
    bs = [0, 17, 63]
    x64 = bits_to_f64(x, cfg.dtype)
    want = ref.layer_decode(cfg, w64(W, cfg.dtype), x64, pos, cfg.ctx,
                            lambda b: bits_to_f64(make_cache_row(cfg, "k", b, 0), cfg.dtype),
                            lambda b: bits_to_f64(make_cache_row(cfg, "v", b, 0), cfg.dtype), batch_rows=bs)
    check(got[bs], x64[bs, 0], want["out"], want["attn_proj"] + want["mlp_out"], cfg.dtype, cfg.name)
    for i, b in enumerate(bs):
        krow = to_f64(tk[b, int(pos[b])]).reshape(-1)
        assert ref.max_rel_err(krow, want["k_new"][i]) <= tol(cfg.dtype)
