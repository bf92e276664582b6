"""Pins of the fp64 oracle to facts fixed by the pages and by mathematics (CPU only).

Each test names the property it pins and the passage it comes from. Together
they are chosen so that a dropped term, a wrong sign, a wrong index or a
transposed operand anywhere in oracle/ref.py fails at least one of them.
"""
import dataclasses
import math
import os

import numpy as np
import pytest
import torch

from oracle import brute, ref
from synth_inputs import CONFIGS, RopeCfg, make_hidden, make_prefill_positions, make_weights, scaled, to_f64

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(1234)


def _w64(cfg, seed=0):
    return {k: to_f64(v, cfg.dtype) for k, v in make_weights(cfg, seed).items()}


# ------------------------------------------------------------------ RMSNorm
def test_rmsnorm_constant_vector_returns_gain():
    """llama3 结构详解 §3.1: a_i / RMS(a) * g_i; for a = c*1, RMS = |c|, so y = g*sign(c)
    up to eps: y_i = g_i * c / sqrt(c^2 + eps) exactly."""
    H, eps = 64, 1e-5
    g = RNG.normal(1.0, 0.1, H)
    for c in (3.0, -0.5, 7.25):
        y = ref.rmsnorm(np.full(H, c), g, eps)
        np.testing.assert_allclose(y, g * c / math.sqrt(c * c + eps), rtol=1e-15, atol=0)
        np.testing.assert_allclose(y, g * np.sign(c), rtol=eps / (c * c))
    assert np.all(ref.rmsnorm(np.zeros(H), g, eps) == 0.0)


def test_rmsnorm_scale_invariance_without_eps():
    """With eps = 0 the norm divides by RMS, so rmsnorm(alpha x) = sign(alpha) rmsnorm(x)."""
    x = RNG.standard_normal((5, 96))
    g = RNG.normal(1.0, 0.1, 96)
    y = ref.rmsnorm(x, g, 0.0)
    for a in (1e-3, 17.0, -2.5):
        np.testing.assert_allclose(ref.rmsnorm(a * x, g, 0.0), np.sign(a) * y, rtol=1e-13, atol=1e-15)


def test_rmsnorm_matches_torch_nn_rmsnorm():
    """NJU lecture 5 "RMSNorm": torch.nn.RMSNorm is the library form of the same norm."""
    x = RNG.standard_normal((7, 64))
    g = RNG.normal(1.0, 0.1, 64)
    m = torch.nn.RMSNorm(64, eps=1e-5, dtype=torch.float64)
    with torch.no_grad():
        m.weight.copy_(torch.from_numpy(g))
        want = m(torch.from_numpy(x)).numpy()
    np.testing.assert_allclose(ref.rmsnorm(x, g, 1e-5), want, rtol=1e-14, atol=1e-15)


# ------------------------------------------------------------------ RoPE
ROPES = [
    RopeCfg(theta=10000.0),
    RopeCfg(type="linear", theta=10000.0, factor=4.0),
    RopeCfg(type="dynamic_ntk", theta=10000.0, factor=2.0, original_max_pos=64),
    RopeCfg(type="llama3", theta=500000.0, factor=8.0, low_freq_factor=1.0, high_freq_factor=4.0,
            original_max_pos=8192),
]


def test_rope_base_frequency_literals():
    """parallel_attention.py §1: inv_freq = 1/base^(2i/dim). Hand values: d=4, theta=1e4 gives
    [1, 0.01]; d=128, theta=5e5 gives f_0 = 1 and f_32 = 5e5^(-1/2) = sqrt(2)/1000."""
    np.testing.assert_allclose(ref.rope_frequencies(4, RopeCfg(theta=1e4), 10), [1.0, 0.01], rtol=1e-15)
    f = ref.rope_frequencies(128, RopeCfg(theta=5e5), 10)
    assert f.shape == (64,)
    assert f[0] == 1.0
    np.testing.assert_allclose(f[32], 0.0014142135623730951, rtol=1e-14)
    assert np.all(np.diff(f) < 0)


def test_rope_rotation_direction_literal():
    """d = 2: the single pair is rotated by +pos rad (x' = x cos - y sin, y' = y cos + x sin),
    NJU lecture 5 "RoPE高效实现": q*cos + rotate_half(q)*sin with rotate_half = cat(-x2, x1)."""
    f = ref.rope_frequencies(2, RopeCfg(theta=10000.0), 4)
    y = ref.rope_rotate(np.array([1.0, 0.0]), np.array(1.0), f)
    np.testing.assert_allclose(y, [0.5403023058681398, 0.8414709848078965], rtol=1e-15)
    y = ref.rope_rotate(np.array([0.0, 1.0]), np.array(1.0), f)
    np.testing.assert_allclose(y, [-0.8414709848078965, 0.5403023058681398], rtol=1e-15)


def test_rope_position_zero_is_identity():
    x = RNG.standard_normal((3, 5, 16))
    for rc in ROPES:
        f = ref.rope_frequencies(16, rc, 100)
        np.testing.assert_array_equal(ref.rope_rotate(x, np.zeros((3, 5)), f, rc.interleaved), x)


@pytest.mark.parametrize("interleaved", [False, True])
def test_rope_preserves_pair_norms(interleaved):
    """NJU lecture 5 "RoPE公式": the rotation keeps the norm (here: of every pair)."""
    d = 64
    x = RNG.standard_normal((40, d))
    pos = RNG.integers(0, 40000, 40).astype(float)
    f = ref.rope_frequencies(d, ROPES[3], 40000)
    y = ref.rope_rotate(x, pos, f, interleaved)
    if interleaved:
        nx, ny = x[:, 0::2] ** 2 + x[:, 1::2] ** 2, y[:, 0::2] ** 2 + y[:, 1::2] ** 2
    else:
        nx, ny = x[:, :d // 2] ** 2 + x[:, d // 2:] ** 2, y[:, :d // 2] ** 2 + y[:, d // 2:] ** 2
    np.testing.assert_allclose(ny, nx, rtol=1e-13)


@pytest.mark.parametrize("rc", ROPES, ids=lambda r: r.type)
@pytest.mark.parametrize("interleaved", [False, True])
def test_rope_relative_position(rc, interleaved):
    """CSDN model.py answer "#### 2. 旋转位置编码": RoPE is a relative encoding, so
    <R_m q, R_n k> depends only on m - n (frequencies fixed within one call)."""
    d = 32
    f = ref.rope_frequencies(d, rc, 200)
    q, k = RNG.standard_normal(d), RNG.standard_normal(d)
    for m, n, delta in ((5, 2, 11), (0, 7, 100), (150, 149, 33)):
        a = ref.rope_rotate(q, np.array(m), f, interleaved) @ ref.rope_rotate(k, np.array(n), f, interleaved)
        b = ref.rope_rotate(q, np.array(m + delta), f, interleaved) @ \
            ref.rope_rotate(k, np.array(n + delta), f, interleaved)
        np.testing.assert_allclose(a, b, rtol=1e-11, atol=1e-12)


def test_rope_interleaved_is_complex_multiplication():
    """CSDN answer "#### 2.": freqs_cis = polar(1, t*f) and the rotation is a complex multiply of
    (x_{2j} + i x_{2j+1}). numpy's complex exp/multiply is the library form."""
    d = 16
    x = RNG.standard_normal((9, d))
    pos = np.arange(9, dtype=float) * 37.0
    f = ref.rope_frequencies(d, RopeCfg(theta=10000.0), 1000)
    z = (x[:, 0::2] + 1j * x[:, 1::2]) * np.exp(1j * pos[:, None] * f[None, :])
    y = ref.rope_rotate(x, pos, f, interleaved=True)
    np.testing.assert_allclose(y[:, 0::2], z.real, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(y[:, 1::2], z.imag, rtol=1e-13, atol=1e-14)


def test_rope_halfsplit_is_permuted_interleaved():
    """Half-split pairs (j, j+d/2) are the interleaved pairs (2j, 2j+1) under one fixed permutation."""
    d = 16
    perm = np.empty(d, dtype=int)
    perm[0::2] = np.arange(d // 2)
    perm[1::2] = np.arange(d // 2) + d // 2          # interleaved slot -> half-split slot
    x = RNG.standard_normal((6, d))
    pos = np.arange(6) * 3.0
    f = ref.rope_frequencies(d, ROPES[0], 100)
    half = ref.rope_rotate(x, pos, f, interleaved=False)
    inter = ref.rope_rotate(x[:, perm], pos, f, interleaved=True)
    np.testing.assert_array_equal(inter, half[:, perm])


def test_rope_linear_is_default_at_scaled_position():
    """parallel_attention.py §1 linear variant: t = t / scaling_factor."""
    d = 32
    x = RNG.standard_normal((4, d))
    pos = np.array([0.0, 3.0, 100.0, 5001.0])
    lin = ref.rope_rotate(x, pos, ref.rope_frequencies(d, ROPES[1], 6000))
    dft = ref.rope_rotate(x, pos / 4.0, ref.rope_frequencies(d, ROPES[0], 6000))
    np.testing.assert_allclose(lin, dft, rtol=1e-13, atol=1e-14)


def test_rope_dynamic_ntk_reading():
    """parallel_attention.py §1 dynamic-NTK ("dynamically adjust base"). Under the NTK-aware reading:
    L <= original_max_pos leaves the default frequencies; L = orig is continuous with it; and
    d=4, theta=1e4, factor=2, orig=100, L=200 gives base 1e4 * (2*2 - 1)^(4/2) = 9e4, f_1 = 1/300."""
    rc = RopeCfg(type="dynamic_ntk", theta=1e4, factor=2.0, original_max_pos=100)
    dft = ref.rope_frequencies(4, RopeCfg(theta=1e4), 0)
    for L in (1, 50, 99, 100):                           # the threshold is L > orig, not L >= orig - 1
        np.testing.assert_array_equal(ref.rope_frequencies(4, rc, L), dft)
    # first length past the threshold: base 1e4 * (2*101/100 - 1)^2 = 1e4 * 1.02^2, f_1 = 1/102
    np.testing.assert_allclose(ref.rope_frequencies(4, rc, 101), [1.0, 1.0 / 102.0], rtol=1e-14)
    np.testing.assert_allclose(ref.rope_frequencies(4, rc, 200), [1.0, 1.0 / 300.0], rtol=1e-14)
    np.testing.assert_allclose(brute.inv_freq(4, rc, 200), [1.0, 1.0 / 300.0], rtol=1e-14)


def test_rope_llama3_bands():
    """parallel_attention.py §1 Llama3 variant (high frequencies kept, low divided, middle
    interpolated) with factor 8, low 1, high 4, orig 8192, theta 5e5, d = 128.
    Hand derivation: lambda_i = 2 pi 5e5^(i/64) < 2048 iff i <= 28 (29 kept); > 8192 iff
    i >= 35 (29 divided by 8); i = 29..34 interpolated (6)."""
    rc = ROPES[3]
    f0 = ref.rope_frequencies(128, RopeCfg(theta=5e5), 0)
    f3 = ref.rope_frequencies(128, rc, 0)
    r = f3 / f0
    assert np.sum(r == 1.0) == 29 and np.all(r[:29] == 1.0)
    np.testing.assert_allclose(r[35:], 1.0 / 8.0, rtol=1e-15)
    assert np.all((r[29:35] < 1.0) & (r[29:35] > 1.0 / 8.0))
    assert np.all(np.diff(r[28:36]) < 0)                 # interpolation weight falls with wavelength
    assert np.all(np.diff(f3) < 0)                       # scaled frequencies stay monotone
    # continuity at both band edges: s = 1 at lambda = orig/hff and s = 0 at lambda = orig/lff
    for lam, want in ((8192 / 4.0, 1.0), (8192 / 1.0, 1.0 / 8.0)):
        fr = 2 * math.pi / lam
        theta_eff = fr ** (-64.0)                        # puts f_1 = theta^(-2/128) on that band edge
        rc1 = dataclasses.replace(rc, theta=theta_eff)
        got = ref.rope_frequencies(128, rc1, 0)[1] / fr
        np.testing.assert_allclose(got, want, rtol=1e-9)
    # factor = 1 is the identity
    np.testing.assert_allclose(ref.rope_frequencies(128, dataclasses.replace(rc, factor=1.0), 0), f0, rtol=1e-15)
    np.testing.assert_allclose(brute.inv_freq(128, rc, 0), f3, rtol=1e-14)


# ------------------------------------------------------------------ attention
def _qkv(B, S, nh, nkv, d):
    return (RNG.standard_normal((B, S, nh, d)), RNG.standard_normal((B, S, nkv, d)),
            RNG.standard_normal((B, S, nkv, d)))


def test_attention_single_key_returns_value():
    """A query whose visible prefix is one key returns that key's value (row 0 of a causal call, or S = 1)."""
    q, k, v = _qkv(2, 7, 4, 2, 16)
    o = ref.attention_prefill(q, k, v).reshape(2, 7, 4, 16)
    for h in range(4):
        np.testing.assert_allclose(o[:, 0, h], v[:, 0, h // 2], rtol=1e-15)
    o1 = ref.attention_prefill(q[:, :1], k[:, :1], v[:, :1]).reshape(2, 1, 4, 16)
    np.testing.assert_allclose(o1[:, 0, 3], v[:, 0, 1], rtol=1e-15)


def test_attention_equal_keys_gives_prefix_mean():
    """All keys equal: the softmax is uniform over the visible prefix, so row i = mean(v_0..v_i)."""
    q, k, v = _qkv(1, 9, 2, 1, 8)
    k[:] = k[:, :1]
    o = ref.attention_prefill(q, k, v).reshape(1, 9, 2, 8)
    for i in range(9):
        np.testing.assert_allclose(o[0, i, 1], v[0, :i + 1, 0].mean(axis=0), rtol=1e-13, atol=1e-15)


def test_gqa_equals_mha_on_repeated_kv():
    """llama3 结构详解 §3.2: each group of query heads shares one K/V head; with K/V heads repeated
    (torch.repeat_interleave, the library form of repeat_kv) it is plain multi-head attention, and
    with n_kv = n_h it is MHA itself."""
    q, k, v = _qkv(2, 11, 8, 2, 16)
    gqa = ref.attention_prefill(q, k, v)
    kr = torch.from_numpy(k).repeat_interleave(4, dim=2).numpy()
    vr = torch.from_numpy(v).repeat_interleave(4, dim=2).numpy()
    np.testing.assert_allclose(ref.attention_prefill(q, kr, vr), gqa, rtol=1e-14, atol=1e-15)


def test_attention_matches_torch_sdpa():
    """parallel_attention.py §2 eager attention and nanotron §9.3 flash_attn_func(causal=True) compute
    softmax(q k^T / sqrt(d)) v with a causal mask; torch's scaled_dot_product_attention in float64 is
    the library form."""
    B, S, nh, nkv, d = 2, 37, 8, 2, 32
    q, k, v = _qkv(B, S, nh, nkv, d)
    tq = torch.from_numpy(q).transpose(1, 2)
    tk = torch.from_numpy(k).repeat_interleave(nh // nkv, dim=2).transpose(1, 2)
    tv = torch.from_numpy(v).repeat_interleave(nh // nkv, dim=2).transpose(1, 2)
    want = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True)
    want = want.transpose(1, 2).reshape(B, S, nh * d).numpy()
    np.testing.assert_allclose(ref.attention_prefill(q, k, v, q_block=8), want, rtol=1e-12, atol=1e-13)


def test_attention_causality_bitwise():
    """CSDN answer "#### 5." causal mask triu(-inf, diagonal=1): tokens after i cannot change row i."""
    q, k, v = _qkv(1, 20, 4, 2, 16)
    o = ref.attention_prefill(q, k, v)
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    q2[:, 13:] += 5.0
    k2[:, 13:] *= -3.0
    v2[:, 13:] += 100.0
    o2 = ref.attention_prefill(q2, k2, v2)
    np.testing.assert_array_equal(o2[:, :13], o[:, :13])
    assert not np.array_equal(o2[:, 13:], o[:, 13:])


# ------------------------------------------------------------------ MLP
def test_silu_special_values():
    assert ref.silu(np.array(0.0)) == 0.0
    np.testing.assert_allclose(ref.silu(np.array(40.0)), 40.0, rtol=1e-15)
    assert abs(ref.silu(np.array(-40.0))) < 1e-15
    z = RNG.standard_normal(50) * 4
    np.testing.assert_allclose(ref.silu(z), torch.nn.functional.silu(torch.from_numpy(z)).numpy(), rtol=1e-14)


def test_fused_gate_up_equals_separate_projections():
    """nanotron §9.4 fused gate_up_proj + chunk(2) vs NJU lecture 5 "SwiGLU实现"
    down_proj(act_fn(gate_proj(x)) * up_proj(x)) with separate linears (torch F.linear float64)."""
    H, I = 24, 40
    x = RNG.standard_normal((6, H))
    wgu = RNG.standard_normal((2 * I, H)) * 0.2
    wd = RNG.standard_normal((H, I)) * 0.2
    F = torch.nn.functional
    tx = torch.from_numpy(x)
    want = F.linear(F.silu(F.linear(tx, torch.from_numpy(wgu[:I]))) * F.linear(tx, torch.from_numpy(wgu[I:])),
                    torch.from_numpy(wd)).numpy()
    got = ref.linear(ref.swiglu_act(x, wgu, I), wd)
    np.testing.assert_allclose(got, want, rtol=1e-13, atol=1e-15)


# ------------------------------------------------------------------ whole layer
def _tiny_variants():
    base = CONFIGS["tiny_f32"]
    out = [base]
    for rc in ROPES:
        for il in (False, True):
            out.append(scaled(base, S=8, rope=dataclasses.replace(rc, interleaved=il, original_max_pos=4
                                                                  if rc.type == "dynamic_ntk" else
                                                                  rc.original_max_pos)))
    return out


@pytest.mark.parametrize("cfg", _tiny_variants(), ids=lambda c: f"S{c.S}-{c.rope.type}-il{int(c.rope.interleaved)}")
def test_layer_matches_brute_force(cfg):
    """Whole layer (nanotron §9.5) against the scalar-loop twin, every RoPE type and pairing."""
    W = _w64(cfg)
    x = to_f64(make_hidden(cfg), cfg.dtype)
    pos = make_prefill_positions(cfg) * (3 if cfg.S == 8 else 1)   # spread positions past orig_max_pos
    L = int(pos.max()) + 1
    got = ref.layer_prefill(cfg, W, x, pos, L)
    Wl = {k: v.tolist() for k, v in W.items()}
    bout, bo = brute.layer_prefill(cfg, Wl, x.tolist(), pos.tolist(), L)
    np.testing.assert_allclose(got["out"], np.array(bout), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(got["o"], np.array(bo), rtol=1e-12, atol=1e-12)


def test_layer_zero_projections_is_identity():
    """nanotron §9.5: out = h + mlp(norm(h)), h = x + attn(norm(x)); with W_o = W_down = 0 both
    branches add exact zeros, so out equals the input bit for bit."""
    cfg = CONFIGS["tiny_f32"]
    W = _w64(cfg)
    W["w_o"] = np.zeros_like(W["w_o"])
    W["w_down"] = np.zeros_like(W["w_down"])
    x = to_f64(make_hidden(cfg), cfg.dtype)
    got = ref.layer_prefill(cfg, W, x, make_prefill_positions(cfg), cfg.S)
    np.testing.assert_array_equal(got["out"], x)


def test_layer_causality_bitwise():
    cfg = CONFIGS["tiny_f32"]
    W = _w64(cfg)
    x = to_f64(make_hidden(cfg), cfg.dtype)
    pos = make_prefill_positions(cfg)
    a = ref.layer_prefill(cfg, W, x, pos, cfg.S)["out"]
    x2 = x.copy()
    x2[:, 20:] = RNG.standard_normal(x2[:, 20:].shape)
    b = ref.layer_prefill(cfg, W, x2, pos, cfg.S)["out"]
    np.testing.assert_array_equal(a[:, :20], b[:, :20])


def test_sampled_rows_equal_full_layer():
    cfg = scaled(CONFIGS["tiny_f32"], B=2, S=24)
    W = _w64(cfg)
    x = to_f64(make_hidden(cfg), cfg.dtype)
    pos = make_prefill_positions(cfg)
    full = ref.layer_prefill(cfg, W, x, pos, cfg.S)
    rows = [(0, 0), (1, 23), (0, 11), (1, 5)]
    part = ref.layer_prefill_rows(cfg, W, x, pos, cfg.S, rows)
    for r, (b, i) in enumerate(rows):
        np.testing.assert_allclose(part["out"][r], full["out"][b, i], rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(part["o"][r], full["o"][b, i], rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(part["k_rot"][r], full["k_rot"][b, i].reshape(-1), rtol=1e-13, atol=1e-13)


def test_decode_equals_prefill_last_row():
    """llama3 结构详解 §3.2 / CSDN answer "#### 3.": the KV cache stores rotated keys and values so a
    decode step at position p over a cache filled from tokens 0..p-1 reproduces prefill row p."""
    base = CONFIGS["tiny_f32"]
    cfg = scaled(base, B=2, S=13)
    W = _w64(cfg)
    x = to_f64(make_hidden(cfg), cfg.dtype)
    pos = make_prefill_positions(cfg)
    full = ref.layer_prefill(cfg, W, x, pos, 64)
    ctx = 16
    dcfg = scaled(base, B=2, S=1, ctx=ctx, decode=True)
    caches = {}
    for name in ("k", "v"):
        c = RNG.standard_normal((2, ctx, cfg.n_kv_heads, cfg.head_dim))   # junk beyond the prefix
        src = full["k_rot"] if name == "k" else full["v"]
        c[:, :12] = src[:, :12]
        caches[name] = c
    p = np.array([12, 12])
    dec = ref.layer_decode(dcfg, W, x[:, 12:13], p, 64, lambda b: caches["k"][b], lambda b: caches["v"][b])
    np.testing.assert_allclose(dec["out"], full["out"][:, 12], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(dec["k_new"], full["k_rot"][:, 12].reshape(2, -1), rtol=1e-13, atol=1e-14)


# ------------------------------------------------------------------ chunked prefill on a cache prefix
def test_attention_chunk_empty_prefix_equals_prefill():
    """llama3 结构详解 §3.2 with start_pos = 0: a chunk at positions 0..S-1 writes its own keys to the
    cache and attends over them causally, exactly the one-call prefill (junk in other slots unused)."""
    B, S, nh, nkv, d, ctx = 2, 9, 4, 2, 16, 13
    q, k, v = _qkv(B, S, nh, nkv, d)
    ck, cv = RNG.standard_normal((B, ctx, nkv, d)), RNG.standard_normal((B, ctx, nkv, d))
    pos = np.broadcast_to(np.arange(S), (B, S))
    o, K, V = ref.attention_chunk(q, k, v, pos, ck, cv)
    np.testing.assert_allclose(o, ref.attention_prefill(q, k, v), rtol=1e-13, atol=1e-14)
    np.testing.assert_array_equal(K[:, :S], k)
    np.testing.assert_array_equal(V[:, S:], cv[:, S:])


@pytest.mark.parametrize("starts", [(5, 9), (0, 7), (16, 1)])
def test_attention_chunk_continues_one_shot_prefill(starts):
    """CSDN answer "#### 5." start_pos > 0: the chunk's rows equal rows start_pos.. of one causal
    prefill over prefix + chunk, when the cache holds the prefix's keys and values (one-shot reference:
    attention_prefill, itself pinned to torch's scaled_dot_product_attention)."""
    B, S, nh, nkv, d, ctx = 2, 6, 4, 2, 16, 32
    ck, cv = RNG.standard_normal((B, ctx, nkv, d)), RNG.standard_normal((B, ctx, nkv, d))
    pos = np.stack([np.arange(P, P + S) for P in starts])
    q = RNG.standard_normal((B, S, nh, d))
    k = RNG.standard_normal((B, S, nkv, d))
    v = RNG.standard_normal((B, S, nkv, d))
    o, K, V = ref.attention_chunk(q, k, v, pos, ck, cv)
    for b, P in enumerate(starts):
        qq = np.concatenate([RNG.standard_normal((1, P, nh, d)), q[b:b + 1]], axis=1)
        kk = np.concatenate([ck[b:b + 1, :P], k[b:b + 1]], axis=1)
        vv = np.concatenate([cv[b:b + 1, :P], v[b:b + 1]], axis=1)
        full = ref.attention_prefill(qq, kk, vv)
        np.testing.assert_allclose(o[b], full[0, P:], rtol=1e-12, atol=1e-13)
        np.testing.assert_array_equal(K[b, P:P + S], k[b])
        np.testing.assert_array_equal(K[b, :P], ck[b, :P])


def test_attention_chunk_reads_only_slots_up_to_its_position():
    """Slots after a query's position (later cache contents) cannot change it; a prefix slot can."""
    B, S, nh, nkv, d, ctx = 1, 4, 2, 1, 8, 20
    q, k, v = _qkv(B, S, nh, nkv, d)
    ck, cv = RNG.standard_normal((B, ctx, nkv, d)), RNG.standard_normal((B, ctx, nkv, d))
    pos = np.array([[7, 8, 9, 10]])
    o, _, _ = ref.attention_chunk(q, k, v, pos, ck, cv)
    ck2, cv2 = ck.copy(), cv.copy()
    ck2[:, 11:] += 3.0
    cv2[:, 11:] -= 7.0
    o2, _, _ = ref.attention_chunk(q, k, v, pos, ck2, cv2)
    np.testing.assert_array_equal(o2, o)
    cv2[:, 3] += 1.0
    o3, _, _ = ref.attention_chunk(q, k, v, pos, ck2, cv2)
    assert not np.array_equal(o3, o)


def test_layer_chunk_continues_one_shot_prefill():
    """The decoder layer over a chunk at positions P..P+S-1 on top of a cache filled from tokens
    0..P-1 reproduces rows P.. of the one-call layer over all P+S tokens (llama3 结构详解 §3.2)."""
    base = CONFIGS["tiny_f32"]
    P, S, ctx = 11, 6, 24
    cfg = scaled(base, B=2, S=P + S)
    W = _w64(cfg)
    x = to_f64(make_hidden(cfg), cfg.dtype)
    pos = make_prefill_positions(cfg)
    full = ref.layer_prefill(cfg, W, x, pos, 64)
    ck = RNG.standard_normal((2, ctx, cfg.n_kv_heads, cfg.head_dim))
    cv = RNG.standard_normal((2, ctx, cfg.n_kv_heads, cfg.head_dim))
    ck[:, :P] = full["k_rot"][:, :P]
    cv[:, :P] = full["v"][:, :P]
    ch = ref.layer_prefill_chunk(scaled(base, B=2, S=S), W, x[:, P:], pos[:, P:], 64, ck, cv)
    np.testing.assert_allclose(ch["out"], full["out"][:, P:], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(ch["cache_k"][:, P:P + S], full["k_rot"][:, P:], rtol=1e-13, atol=1e-14)


# ------------------------------------------------------------------ varlen packed prefill
def test_attention_varlen_equals_per_sequence_prefill():
    """parallel_attention.py §3: flash_attn_varlen_func(cu_seqlens, causal=True) over packed tokens is
    causal attention within each sequence; it equals attention_prefill run on each sequence alone, and
    tokens of one sequence cannot change another's rows."""
    lens = [5, 1, 0, 9, 3]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T, nh, nkv, d = int(cu[-1]), 4, 2, 16
    q, k, v = RNG.standard_normal((T, nh, d)), RNG.standard_normal((T, nkv, d)), RNG.standard_normal((T, nkv, d))
    o = ref.attention_varlen(q, k, v, cu)
    for i in range(len(lens)):
        a, b = int(cu[i]), int(cu[i + 1])
        if b > a:
            want = ref.attention_prefill(q[None, a:b], k[None, a:b], v[None, a:b])[0]
            np.testing.assert_array_equal(o[a:b], want)
    k2, v2 = k.copy(), v.copy()
    k2[cu[3]:cu[4]] += 2.0
    v2[cu[3]:cu[4]] -= 4.0
    o2 = ref.attention_varlen(q, k2, v2, cu)
    np.testing.assert_array_equal(o2[:cu[3]], o[:cu[3]])
    np.testing.assert_array_equal(o2[cu[4]:], o[cu[4]:])
    assert not np.array_equal(o2[cu[3]:cu[4]], o[cu[3]:cu[4]])


def test_layer_varlen_equals_per_sequence_layer():
    """The packed layer with in-sequence positions (the rmpad RoPE convention) equals the one-call layer
    run on each sequence separately."""
    base = CONFIGS["tiny_f32"]
    lens = [7, 12, 1]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T = int(cu[-1])
    cfg = scaled(base, B=1, S=T)
    W = _w64(cfg)
    x = to_f64(make_hidden(cfg), cfg.dtype)[0]
    pos = np.concatenate([np.arange(n) for n in lens]).astype(np.int64)
    got = ref.layer_prefill_varlen(cfg, W, x, pos, cu, 64)
    for i, n in enumerate(lens):
        a, b = int(cu[i]), int(cu[i + 1])
        one = ref.layer_prefill(scaled(base, B=1, S=n), W, x[None, a:b], pos[None, a:b], 64)
        np.testing.assert_allclose(got["out"][a:b], one["out"][0], rtol=1e-13, atol=1e-13)


# ------------------------------------------------------------------ model stack
def test_embedding_is_one_hot_product():
    """nn.Embedding(vocab, dim)(tokens) equals one_hot(tokens) @ table (the lookup as a matrix product)."""
    table = RNG.standard_normal((11, 6))
    tok = np.array([[3, 0, 10], [7, 7, 1]])
    one_hot = np.eye(11)[tok]
    np.testing.assert_array_equal(ref.embedding(table, tok), one_hot @ table)


def _model64(cfg, n_layers, vocab, seed=0):
    from synth_inputs import make_model_weights
    M = make_model_weights(cfg, n_layers, vocab, seed)
    return {"layers": [{k: to_f64(v, cfg.dtype) for k, v in W.items()} for W in M["layers"]],
            "tok_embeddings": to_f64(M["tok_embeddings"], cfg.dtype), "g_final": to_f64(M["g_final"], cfg.dtype),
            "lm_head": to_f64(M["lm_head"], cfg.dtype)}


def test_model_stack_causality_and_layer_order():
    """Logits of token i depend only on tokens 0..i (bitwise), and the layers apply in order (swapping two
    different layers changes the result)."""
    cfg = scaled(CONFIGS["tiny_f32"], B=1, S=9)
    M = _model64(cfg, 2, 31)
    pos = make_prefill_positions(cfg)
    tok = np.array([[4, 8, 15, 16, 23, 30, 2, 7, 1]])
    a = ref.model_prefill(cfg, M, tok, pos, 16)["logits"]
    tok2 = tok.copy()
    tok2[0, 6:] = [0, 0, 0]
    b = ref.model_prefill(cfg, M, tok2, pos, 16)["logits"]
    np.testing.assert_array_equal(a[:, :6], b[:, :6])
    assert not np.array_equal(a[:, 6:], b[:, 6:])
    M2 = dict(M, layers=M["layers"][::-1])
    assert not np.allclose(ref.model_prefill(cfg, M2, tok, pos, 16)["logits"], a)


# ------------------------------------------------------------------ shapes
def test_layer_shapes_match_lecture_printout():
    """Golden: the Llama-3.2-1B layer dump on NJU lecture 5 fixes the projection shapes of the
    llama32_1b_prefill workload; the fused Q|K|V and gate|up weights must split into exactly those."""
    rows = {}
    with open(os.path.join(GOLDEN, "llama32_1b_layer_shapes.txt")) as fh:
        for line in fh:
            line = line.strip()
            if line and not line.startswith("#"):
                parts = line.split()
                rows[parts[0]] = tuple(float(p) for p in parts[1:])
    cfg = CONFIGS["llama32_1b_prefill"]
    assert cfg.eps == rows["rmsnorm_eps"][0]
    qkv = np.zeros((1, cfg.qkv_dim))
    q, k, v = ref.split_qkv(qkv, cfg.n_heads, cfg.n_kv_heads, cfg.head_dim)
    assert (cfg.hidden, q.shape[-2] * q.shape[-1]) == rows["q_proj"]
    assert (cfg.hidden, k.shape[-2] * k.shape[-1]) == rows["k_proj"]
    assert (cfg.hidden, v.shape[-2] * v.shape[-1]) == rows["v_proj"]
    assert (cfg.n_heads * cfg.head_dim, cfg.hidden) == rows["o_proj"]
    assert (cfg.hidden, cfg.intermediate) == rows["gate_proj"] == rows["up_proj"]
    assert (cfg.intermediate, cfg.hidden) == rows["down_proj"]
    act = ref.swiglu_act(np.zeros((1, cfg.hidden)), np.zeros((2 * cfg.intermediate, cfg.hidden)), cfg.intermediate)
    assert act.shape == (1, rows["down_proj"][0])


@pytest.mark.parametrize("name,want", [("tiny_f32", 46208), ("llama32_1b_prefill", 60821504),
                                       ("llama3_8b_prefill", 218112000), ("llama3_8b_decode", 218112000),
                                       ("llama3_8b_long_llama3rope", 218112000)])
def test_parameter_count_per_layer(name, want):
    """Parameter count per layer (the CSDN answer's test tooling sums p.numel()): hand-derived totals of
    W_qkv + W_o + W_gate_up + W_down + two gains."""
    cfg = CONFIGS[name]
    H, nh, nkv, d, I = cfg.hidden, cfg.n_heads, cfg.n_kv_heads, cfg.head_dim, cfg.intermediate
    shapes = [((nh + 2 * nkv) * d, H), (H, nh * d), (2 * I, H), (H, I), (H,), (H,)]
    assert sum(int(np.prod(s)) for s in shapes) == want
