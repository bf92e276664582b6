"""GPU parity of each C-ABI entry point against the fp64 oracle, on seeded inputs.

Sizes span several tiles plus a ragged tail. Bounds: normwise max relative error <= 2e-2 (bf16) or
1e-4 (fp32); integer-valued outcomes (untouched values, cache slots not written) are compared
bit for bit."""
import numpy as np
import pytest
import torch

import transformer_layer_forward_amd as L
from oracle import ref
from synth_inputs import RopeCfg, normal, to_f64 as bits_to_f64
from tests.gpu_util import DEV, require_gpu, tol, to_dev, to_f64

pytestmark = pytest.mark.gpu

TD = {"bf16": torch.bfloat16, "f32": torch.float32}


def _rope(rc: RopeCfg) -> L.Rope:
    return L.Rope(type=rc.type, theta=rc.theta, factor=rc.factor, low_freq_factor=rc.low_freq_factor,
                  high_freq_factor=rc.high_freq_factor, original_max_pos=rc.original_max_pos,
                  interleaved=rc.interleaved)


# ------------------------------------------------------------------ RMSNorm
@pytest.mark.parametrize("dtype,rows,H", [("bf16", 37, 4096), ("bf16", 5, 2048), ("bf16", 3, 8200), ("bf16", 4, 60),
                                          ("f32", 32, 64), ("f32", 7, 102), ("f32", 9, 4096)])
def test_rmsnorm(dtype, rows, H):
    require_gpu()
    x = normal(0, 100, (rows, H), dtype)
    g = normal(0, 101, (H,), dtype, std=0.1, mean=1.0)
    y = L.rmsnorm(to_dev(x, dtype), to_dev(g, dtype), 1e-5)
    torch.cuda.synchronize()
    want = ref.rmsnorm(bits_to_f64(x, dtype), bits_to_f64(g, dtype), 1e-5)
    assert ref.max_rel_err(to_f64(y), want) <= tol(dtype)


def test_rmsnorm_constant_rows_return_gain():
    """RMSNorm of a constant row c*1 is g*sign(c) up to eps (llama3 结构详解 §3.1)."""
    require_gpu()
    H = 4096
    x = torch.full((3, H), 2.5, device=DEV, dtype=torch.bfloat16)
    x[1] = -0.75
    g = to_dev(normal(0, 102, (H,), "bf16", std=0.1, mean=1.0), "bf16")
    y = to_f64(L.rmsnorm(x, g, 1e-5))
    gg = to_f64(g)
    np.testing.assert_allclose(y[0], gg, rtol=8e-3)
    np.testing.assert_allclose(y[1], -gg, rtol=8e-3)


# ------------------------------------------------------------------ RoPE apply
ROPES = [RopeCfg(theta=500000.0), RopeCfg(type="linear", theta=10000.0, factor=4.0),
         RopeCfg(type="dynamic_ntk", theta=10000.0, factor=2.0, original_max_pos=256),
         RopeCfg(type="llama3", theta=500000.0, factor=8.0, low_freq_factor=1.0, high_freq_factor=4.0,
                 original_max_pos=8192)]


@pytest.mark.parametrize("rc", ROPES, ids=lambda r: r.type)
@pytest.mark.parametrize("il", [False, True])
@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f32", 16)])
def test_rope_apply(rc, il, dtype, d):
    require_gpu()
    import dataclasses
    rc = dataclasses.replace(rc, interleaved=il)
    B, S, nh, nkv = 2, 37, 4, 2
    L_ = 20000
    qkv = normal(1, 110, (B, S, (nh + 2 * nkv) * d), dtype)
    pos = np.random.default_rng([1, 111]).integers(0, L_, (B, S)).astype(np.int64)
    t = to_dev(qkv, dtype)
    L.rope_apply(_rope(rc), t, torch.from_numpy(pos).to(DEV), nh, nkv, d, L_)
    got = to_f64(t)
    x = bits_to_f64(qkv, dtype)
    f = ref.rope_frequencies(d, rc, L_)
    q, k, v = ref.split_qkv(x, nh, nkv, d)
    gq, gk, gv = ref.split_qkv(got, nh, nkv, d)
    assert ref.max_rel_err(gq, ref.rope_rotate(q, pos[..., None], f, il)) <= tol(dtype)
    assert ref.max_rel_err(gk, ref.rope_rotate(k, pos[..., None], f, il)) <= tol(dtype)
    np.testing.assert_array_equal(gv, v)


# ------------------------------------------------------------------ projections (via the MLP entry point)
@pytest.mark.parametrize("dtype,M,H,I", [("bf16", 1, 256, 512), ("bf16", 37, 512, 1000), ("bf16", 64, 256, 384),
                                         ("bf16", 48, 1288, 2056), ("bf16", 65, 256, 384), ("bf16", 300, 1024, 2048),
                                         ("bf16", 515, 512, 1032), ("bf16", 20, 200, 1000), ("bf16", 33, 520, 240),
                                         ("bf16", 200, 512, 4096), ("bf16", 96, 256, 1984), ("bf16", 16, 2048, 256),
                                         ("bf16", 64, 384, 1152),
                                         # K walks of one to five 64-wide stages on the 256 x 256 / 256 x 128 kernels
                                         ("bf16", 300, 64, 128), ("bf16", 520, 192, 320),
                                         ("f32", 32, 64, 176), ("f32", 45, 96, 200)])
@pytest.mark.parametrize("with_residual", [False, True])
def test_swiglu_mlp(dtype, M, H, I, with_residual):
    require_gpu()
    x = normal(2, 120, (M, H), dtype)
    wgu = normal(2, 121, (2 * I, H), dtype, std=0.02)
    wd = normal(2, 122, (H, I), dtype, std=0.02)
    r = normal(2, 123, (M, H), dtype)
    res = to_dev(r, dtype) if with_residual else None
    out = L.swiglu_mlp(to_dev(x, dtype), to_dev(wgu, dtype), to_dev(wd, dtype), residual=res)
    want = ref.linear(ref.swiglu_act(bits_to_f64(x, dtype), bits_to_f64(wgu, dtype), I), bits_to_f64(wd, dtype))
    got = to_f64(out)
    if with_residual:
        rr = bits_to_f64(r, dtype)
        assert ref.max_rel_err(got, want + rr) <= tol(dtype)
        # the branch alone: out - residual inherits out's own rounding (half an ulp, 2^-9 |out| in bf16)
        bound = tol(dtype) * np.max(np.abs(want)) + (2.0 ** -8 if dtype == "bf16" else 1e-6) * np.max(np.abs(got))
        assert np.max(np.abs(got - rr - want)) <= bound
    else:
        assert ref.max_rel_err(got, want) <= tol(dtype)


@pytest.mark.parametrize("with_residual", [False, True])
def test_swiglu_mlp_wide_tiles_sampled_rows(with_residual):
    """M = 2048, hidden = intermediate = 4096: the down projection has 128 tiles of 256 x 256, so it runs
    unsplit on 256 x 128 tiles with its epilogue (residual or plain store) in the kernel. The oracle is
    evaluated on 16 sampled rows (first, last and 14 seeded)."""
    require_gpu()
    dtype, M, H, I = "bf16", 2048, 4096, 4096
    x = normal(5, 140, (M, H), dtype)
    wgu = normal(5, 141, (2 * I, H), dtype, std=0.02)
    wd = normal(5, 142, (H, I), dtype, std=0.02)
    r = normal(5, 143, (M, H), dtype)
    res = to_dev(r, dtype) if with_residual else None
    out = L.swiglu_mlp(to_dev(x, dtype), to_dev(wgu, dtype), to_dev(wd, dtype), residual=res)
    rows = sorted({0, M - 1, *np.random.default_rng([7, 140]).integers(0, M, 14).tolist()})
    want = ref.linear(ref.swiglu_act(bits_to_f64(x, dtype)[rows], bits_to_f64(wgu, dtype), I), bits_to_f64(wd, dtype))
    got = to_f64(out)[rows]
    if with_residual:
        rr = bits_to_f64(r, dtype)[rows]
        assert ref.max_rel_err(got, want + rr) <= tol(dtype)
        bound = tol(dtype) * np.max(np.abs(want)) + 2.0 ** -8 * np.max(np.abs(got))
        assert np.max(np.abs(got - rr - want)) <= bound
    else:
        assert ref.max_rel_err(got, want) <= tol(dtype)


@pytest.mark.parametrize("M,H,I", [(2300, 4096, 14208), (2560, 2048, 8192), (4096, 128, 4096), (4096, 192, 4096),
                                   (4096, 4096, 4096)])
def test_swiglu_mlp_many_tiles_sampled_rows(M, H, I):
    """Shapes with several 256 x 256 tiles per compute unit and a ragged last token tile.
    M = 2300, I = 14208: gate_up has 9 x 111 = 999 tiles (not a multiple of 8: the plain tile order instead of
    the per-XCD one); M = 2560, H = 2048, I = 8192: gate_up 10 x 64 = 640 tiles (per-XCD order; the persistent
    kernel, 2 or 3 tiles per workgroup), down 10 x 8 = 80 tiles (K split); M = 4096, H = 128 / 192: the
    persistent gate_up kernel on 512 tiles whose K walk is two / three stages; M = H = I = 4096: both
    projections on whole 256 x 256 tiles (gate_up 512 on the persistent kernel, down 256), so gate_up hands
    its output to down K-blocked. 24 sampled rows (first, last, the edges of the last token tile, seeded),
    with the residual."""
    require_gpu()
    dtype = "bf16"
    x = normal(6, 150, (M, H), dtype)
    wgu = normal(6, 151, (2 * I, H), dtype, std=0.02)
    wd = normal(6, 152, (H, I), dtype, std=0.02)
    r = normal(6, 153, (M, H), dtype)
    out = L.swiglu_mlp(to_dev(x, dtype), to_dev(wgu, dtype), to_dev(wd, dtype), residual=to_dev(r, dtype))
    last0 = (M - 1) // 256 * 256
    rows = sorted({0, 255, 256, last0, M - 1, *np.random.default_rng([8, M]).integers(0, M, 19).tolist()})
    want = ref.linear(ref.swiglu_act(bits_to_f64(x, dtype)[rows], bits_to_f64(wgu, dtype), I), bits_to_f64(wd, dtype))
    got = to_f64(out)[rows]
    rr = bits_to_f64(r, dtype)[rows]
    assert ref.max_rel_err(got, want + rr) <= tol(dtype)
    bound = tol(dtype) * np.max(np.abs(want)) + 2.0 ** -8 * np.max(np.abs(got))
    assert np.max(np.abs(got - rr - want)) <= bound


# ------------------------------------------------------------------ prefill attention
PREFILL = [
    # dtype, B, S, nh, nkv, d
    ("bf16", 2, 130, 8, 2, 128),
    ("bf16", 1, 200, 8, 8, 64),
    ("bf16", 2, 64, 4, 2, 64),
    ("bf16", 1, 100, 16, 2, 128),
    ("bf16", 3, 1, 4, 1, 128),
    ("bf16", 1, 257, 6, 2, 64),      # g = 3 (one head per block)
    ("bf16", 1, 150, 6, 2, 128),     # g = 3 at d = 128
    ("bf16", 1, 700, 8, 2, 128),     # 11 key tiles, ragged last tile
    ("bf16", 1, 50, 4, 2, 96),       # generic kernel
    ("f32", 1, 32, 4, 2, 16),
    ("f32", 2, 45, 6, 3, 32),
]


def _attn_inputs(dtype, B, S, nh, nkv, d, seed=3):
    qkv = normal(seed, 130, (B, S, (nh + 2 * nkv) * d), dtype)
    return qkv, bits_to_f64(qkv, dtype)


@pytest.mark.parametrize("case", PREFILL, ids=lambda c: "-".join(map(str, c)))
@pytest.mark.parametrize("mode", ["rotated", "rotated_cache", "rope", "rope_il_cache"])
def test_attn_prefill(case, mode):
    require_gpu()
    dtype, B, S, nh, nkv, d = case
    qkv, x = _attn_inputs(dtype, B, S, nh, nkv, d)
    pos = np.broadcast_to(np.arange(S, dtype=np.int64), (B, S)).copy()
    rc = None
    q, k, v = ref.split_qkv(x, nh, nkv, d)
    if mode.startswith("rope"):
        rc = RopeCfg(type="llama3", theta=500000.0, factor=8.0, low_freq_factor=1.0, high_freq_factor=4.0,
                     original_max_pos=64, interleaved=(mode == "rope_il_cache"))
        f = ref.rope_frequencies(d, rc, S)
        q = ref.rope_rotate(q, pos[..., None], f, rc.interleaved)
        k = ref.rope_rotate(k, pos[..., None], f, rc.interleaved)
    want = ref.attention_prefill(q, k, v)
    kc = vc = None
    ctx = S + 7
    if mode.endswith("_cache"):
        kc = torch.zeros((B, ctx, nkv, d), device=DEV, dtype=TD[dtype])
        vc = torch.zeros((B, ctx, nkv, d), device=DEV, dtype=TD[dtype])
    o = L.gqa_attn_prefill(to_dev(qkv, dtype), torch.from_numpy(pos).to(DEV), nh, nkv, d,
                           rope=_rope(rc) if rc else None, kv_seq_len=S, k_cache=kc, v_cache=vc)
    got = to_f64(o)
    assert got.shape == (B, S, nh * d)
    assert ref.max_rel_err(got, want) <= tol(dtype)
    if kc is not None:
        gk, gv = to_f64(kc), to_f64(vc)
        assert ref.max_rel_err(gk[:, :S], k) <= tol(dtype)
        np.testing.assert_array_equal(gv[:, :S], v)
        assert np.all(gk[:, S:] == 0) and np.all(gv[:, S:] == 0)


def test_attn_prefill_causality_bitwise():
    """Perturbing tokens after t leaves outputs of tokens <= t bit-identical (CSDN answer "#### 5." mask)."""
    require_gpu()
    B, S, nh, nkv, d = 1, 192, 8, 2, 128
    qkv, _ = _attn_inputs("bf16", B, S, nh, nkv, d, seed=4)
    a = to_dev(qkv, "bf16")
    o1 = L.gqa_attn_prefill(a, None, nh, nkv, d)
    b = a.clone()
    b[:, 100:] = torch.randn_like(b[:, 100:].float()).to(torch.bfloat16)
    o2 = L.gqa_attn_prefill(b, None, nh, nkv, d)
    torch.cuda.synchronize()
    assert torch.equal(o1[:, :100], o2[:, :100])
    assert not torch.equal(o1[:, 100:], o2[:, 100:])


def test_attn_prefill_mha_equals_repeated_gqa():
    """GQA with n_kv < n_h equals MHA on explicitly repeated K/V (llama3 结构详解 §3.2)."""
    require_gpu()
    B, S, nh, nkv, d = 1, 150, 8, 2, 64
    qkv, x = _attn_inputs("bf16", B, S, nh, nkv, d, seed=5)
    q, k, v = ref.split_qkv(qkv.reshape(B, S, -1).view(np.uint16), nh, nkv, d)
    k_rep = np.repeat(k, nh // nkv, axis=2)
    v_rep = np.repeat(v, nh // nkv, axis=2)
    mha = np.concatenate([q.reshape(B, S, -1), k_rep.reshape(B, S, -1), v_rep.reshape(B, S, -1)], axis=-1)
    o_gqa = L.gqa_attn_prefill(to_dev(qkv, "bf16"), None, nh, nkv, d)
    o_mha = L.gqa_attn_prefill(to_dev(np.ascontiguousarray(mha), "bf16"), None, nh, nh, d)
    torch.cuda.synchronize()
    assert ref.max_rel_err(to_f64(o_gqa), to_f64(o_mha)) <= 1e-2


# ------------------------------------------------------------------ decode attention
DECODE = [
    # dtype, B, ctx, nh, nkv, d
    ("bf16", 4, 1500, 8, 2, 128),
    ("bf16", 2, 700, 4, 4, 64),
    ("bf16", 3, 1100, 32, 8, 128),
    ("bf16", 12, 1300, 16, 2, 128),  # 8 query heads per kv head; positions at tile and chunk edges
    ("bf16", 12, 900, 4, 2, 64),
    ("bf16", 48, 2000, 32, 8, 128),  # few key splits per sequence, several 128-key blocks each
    ("bf16", 64, 1200, 32, 8, 64),
    ("bf16", 3, 700, 32, 16, 128),   # 16 kv heads: two head groups of 8 per sequence
    ("bf16", 5, 900, 8, 1, 128),     # one kv head: the 8 waves split its tiles by phase and merge
    ("bf16", 2, 300, 4, 2, 96),      # generic kernel
    ("f32", 2, 40, 4, 2, 16),
]


@pytest.mark.parametrize("case", DECODE, ids=lambda c: "-".join(map(str, c)))
@pytest.mark.parametrize("with_rope", [False, "half", "interleaved"])
def test_attn_decode(case, with_rope):
    require_gpu()
    dtype, B, ctx, nh, nkv, d = case
    qkv = normal(6, 140, (B, (nh + 2 * nkv) * d), dtype)
    kc = normal(6, 141, (B, ctx, nkv, d), dtype)
    vc = normal(6, 142, (B, ctx, nkv, d), dtype)
    pos = np.array(([0, ctx - 1, 511, 512, 1023, 1024, 31, 32, 33, 127, 128, 129][:B] + [ctx // 2] * B)[:B],
                   dtype=np.int64)
    pos = np.minimum(pos, ctx - 1)
    rc = RopeCfg(theta=500000.0, interleaved=with_rope == "interleaved") if with_rope else None
    x = bits_to_f64(qkv, dtype)
    q, k, v = ref.split_qkv(x, nh, nkv, d)
    if rc:
        f = ref.rope_frequencies(d, rc, ctx)
        q = ref.rope_rotate(q, pos[:, None], f, rc.interleaved)
        k = ref.rope_rotate(k, pos[:, None], f, rc.interleaved)
    tk, tv = to_dev(kc, dtype), to_dev(vc, dtype)
    o = L.gqa_attn_decode(to_dev(qkv, dtype), torch.from_numpy(pos).to(DEV), tk, tv, nh, nkv, d,
                          rope=_rope(rc) if rc else None, kv_seq_len=ctx)
    got = to_f64(o)
    K0, V0 = bits_to_f64(kc, dtype), bits_to_f64(vc, dtype)
    gk, gv = to_f64(tk), to_f64(tv)
    for b in range(B):
        p = int(pos[b])
        K = K0[b, :p + 1].copy()
        V = V0[b, :p + 1].copy()
        K[p], V[p] = k[b], v[b]
        want = ref.attention_one_query(q[b], K, V)
        assert ref.max_rel_err(got[b], want) <= tol(dtype), b
        assert ref.max_rel_err(gk[b, p], k[b]) <= tol(dtype)
        np.testing.assert_array_equal(gv[b, p], v[b])
        keep = np.ones(ctx, bool)
        keep[p] = False
        np.testing.assert_array_equal(gk[b, keep], K0[b, keep])
        np.testing.assert_array_equal(gv[b, keep], V0[b, keep])


# ------------------------------------------------------------------ chunked prefill on a cache prefix
CHUNK = [
    # dtype, B, S, nh, nkv, d, ctx, starts, order
    ("bf16", 2, 130, 8, 2, 128, 320, (0, 70), "up"),          # empty prefix and a prefix off a tile edge
    ("bf16", 1, 64, 8, 2, 64, 200, (100,), "up"),
    ("bf16", 2, 1, 8, 2, 128, 600, (500, 37), "up"),          # one-token chunks
    ("bf16", 1, 200, 16, 2, 128, 1300, (1000,), "up"),        # long prefix, g = 8
    ("bf16", 1, 257, 6, 2, 64, 400, (33,), "up"),             # g = 3 (one head per block)
    ("bf16", 1, 90, 6, 2, 128, 300, (120,), "up"),            # g = 3 at d = 128
    ("bf16", 1, 100, 8, 2, 128, 200, (60,), "down"),          # positions in reverse order
    ("bf16", 1, 64, 8, 2, 128, 2048, (500,), "up"),           # keys split over 16 workgroups, some of
    ("bf16", 1, 64, 8, 2, 128, 2048, (500,), "down"),         # them wholly masked for early queries
    ("bf16", 2, 40, 16, 2, 64, 1024, (700, 33), "up"),        # split keys at d = 64, g = 8
    ("bf16", 1, 50, 4, 2, 96, 120, (20,), "up"),              # generic kernel (d = 96)
    ("f32", 2, 20, 4, 2, 16, 48, (3, 11), "up"),
]


@pytest.mark.parametrize("case", CHUNK, ids=lambda c: "-".join(map(str, c)))
def test_attn_prefill_chunk(case):
    """gqa_attn_prefill_chunk against the oracle's attention_chunk: the chunk's K/V land at their slots
    (bit for bit), other slots stay as they were, and each query attends over slots 0 .. its position."""
    require_gpu()
    dtype, B, S, nh, nkv, d, ctx, starts, order = case
    qkv = normal(7, 150, (B, S, (nh + 2 * nkv) * d), dtype)
    kc = normal(7, 151, (B, ctx, nkv, d), dtype)
    vc = normal(7, 152, (B, ctx, nkv, d), dtype)
    pos = np.stack([np.arange(P, P + S) if order == "up" else np.arange(P + S - 1, P - 1, -1) for P in starts])
    pos = pos.astype(np.int64)
    x = bits_to_f64(qkv, dtype)
    q, k, v = ref.split_qkv(x, nh, nkv, d)
    K0, V0 = bits_to_f64(kc, dtype), bits_to_f64(vc, dtype)
    want, WK, WV = ref.attention_chunk(q, k, v, pos, K0, V0)
    tk, tv = to_dev(kc, dtype), to_dev(vc, dtype)
    o = L.gqa_attn_prefill_chunk(to_dev(qkv, dtype), torch.from_numpy(pos).to(DEV), tk, tv, nh, nkv, d)
    got = to_f64(o)
    assert got.shape == (B, S, nh * d)
    assert ref.max_rel_err(got, want) <= tol(dtype)
    np.testing.assert_array_equal(to_f64(tk), WK)
    np.testing.assert_array_equal(to_f64(tv), WV)


def test_attn_prefill_chunk_split_matches_unsplit():
    """A small chunk on a long prefix with its keys shared out over workgroups (partial records merged
    by the combine pass) agrees with one workgroup per query block, to bf16 rounding."""
    require_gpu()
    B, S, nh, nkv, d, ctx, P = 1, 96, 32, 8, 128, 4096, 3900
    lib = L._lib.load()
    assert lib.gqa_attn_prefill_chunk_workspace_bytes(B, S, nh, nkv, d, ctx, 1) > 0   # the split path is taken
    qkv = to_dev(normal(9, 154, (B, S, (nh + 2 * nkv) * d), "bf16"), "bf16")
    kc = to_dev(normal(9, 155, (B, ctx, nkv, d), "bf16"), "bf16")
    vc = to_dev(normal(9, 156, (B, ctx, nkv, d), "bf16"), "bf16")
    pos = torch.arange(P, P + S, device=DEV, dtype=torch.int64).expand(B, S).contiguous()
    k2, v2 = kc.clone(), vc.clone()
    o1 = L.gqa_attn_prefill_chunk(qkv, pos, kc, vc, nh, nkv, d, split_keys=True)
    o2 = L.gqa_attn_prefill_chunk(qkv, pos, k2, v2, nh, nkv, d, split_keys=False)
    torch.cuda.synchronize()
    assert torch.equal(kc, k2) and torch.equal(vc, v2)
    assert ref.max_rel_err(to_f64(o1), to_f64(o2)) <= 1e-2


def test_attn_prefill_chunk_empty_prefix_equals_prefill():
    """With positions 0..S-1 the chunked path computes the one-call prefill (same inputs, same cache
    writes); both are bf16 kernels, so they agree to bf16 rounding."""
    require_gpu()
    B, S, nh, nkv, d, ctx = 2, 190, 8, 2, 128, 256
    qkv = to_dev(normal(8, 153, (B, S, (nh + 2 * nkv) * d), "bf16"), "bf16")
    pos = torch.arange(S, device=DEV, dtype=torch.int64).expand(B, S).contiguous()
    k1 = torch.zeros((B, ctx, nkv, d), device=DEV, dtype=torch.bfloat16)
    v1, k2, v2 = k1.clone(), k1.clone(), k1.clone()
    o1 = L.gqa_attn_prefill(qkv, pos, nh, nkv, d, kv_seq_len=ctx, k_cache=k1, v_cache=v1)
    o2 = L.gqa_attn_prefill_chunk(qkv, pos, k2, v2, nh, nkv, d)
    torch.cuda.synchronize()
    assert torch.equal(k1, k2) and torch.equal(v1, v2)
    assert ref.max_rel_err(to_f64(o2), to_f64(o1)) <= 1e-2


# ------------------------------------------------------------------ varlen packed prefill
VARLEN = [
    # dtype, sequence lengths, nh, nkv, d
    ("bf16", (130, 1, 0, 64, 200), 8, 2, 128),    # one-token and empty sequences, exact and ragged tiles
    ("bf16", (70, 257), 6, 2, 64),                # g = 3
    ("bf16", (33, 100), 16, 2, 128),              # g = 8
    ("bf16", (10, 50), 4, 2, 96),                 # generic kernel
    ("f32", (5, 20, 1), 4, 2, 16),
]


@pytest.mark.parametrize("case", VARLEN, ids=lambda c: f"{c[0]}-{'_'.join(map(str, c[1]))}-{c[2]}-{c[3]}-{c[4]}")
def test_attn_prefill_varlen(case):
    """gqa_attn_prefill_varlen against the oracle's attention_varlen (causal within each packed sequence)."""
    require_gpu()
    dtype, lens, nh, nkv, d = case
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    qkv = normal(9, 170, (T, (nh + 2 * nkv) * d), dtype)
    q, k, v = ref.split_qkv(bits_to_f64(qkv, dtype), nh, nkv, d)
    want = ref.attention_varlen(q, k, v, cu)
    o = L.gqa_attn_prefill_varlen(to_dev(qkv, dtype), torch.from_numpy(cu).to(DEV), max(lens), nh, nkv, d)
    got = to_f64(o)
    assert got.shape == (T, nh * d)
    assert ref.max_rel_err(got, want) <= tol(dtype)
