"""Pins of the fp64 oracle against an independent library implementation of the same model (CPU only).

The pages build their layer on the Hugging Face Llama modules: verl "parallel_attention.py — LLaMA 并行注意力"
§1 names LlamaRotaryEmbedding and its linear, dynamic-NTK and Llama3 variants, and §2 calls repeat_kv and the
eager softmax; nanotron "模型层：从 Embedding 到 Loss 的实现" §9.3 calls repeat_kv. The transformers package is
that library. Its RoPE frequency initialisers and its LlamaDecoderLayer / LlamaForCausalLM (run here in float64
with scaled-dot-product attention) are a second implementation written by other people, so agreement with them
pins the oracle's readings of the pages' unprinted parts:
  * the dynamic-NTK base rescaling for kv_seq_len > original_max_pos,
  * the Llama3 piecewise scaling, including its interpolated middle band,
  * the repeat_kv head mapping (query head h reads kv head h // (n_heads / n_kv_heads)),
  * the composition of the layer and of the model stack (embedding, layers in order, final norm, lm head).

transformers' RMSNorm converts its input to float32 before the mean of squares, and its RoPE initialisers
return float32 frequencies, so the tolerances are set just above float32 rounding (1e-6 relative), far below
what any structural mistake moves.
"""
import dataclasses
import os
import warnings

import numpy as np
import pytest
import torch

from oracle import ref
from synth_inputs import (CONFIGS, RopeCfg, make_hidden, make_model_weights, make_prefill_positions, make_tokens,
                          make_weights, scaled, to_f64)

transformers = pytest.importorskip("transformers")
os.environ.setdefault("TRANSFORMERS_VERBOSITY", "error")
from transformers import LlamaConfig, LlamaForCausalLM  # noqa: E402
from transformers.modeling_rope_utils import ROPE_INIT_FUNCTIONS  # noqa: E402
from transformers.models.llama.modeling_llama import LlamaDecoderLayer, LlamaRotaryEmbedding  # noqa: E402

RTOL_F32 = 1e-6


def _rope_params(rc: RopeCfg) -> dict:
    if rc.type == "default":
        return {"rope_type": "default", "rope_theta": rc.theta}
    if rc.type == "linear":
        return {"rope_type": "linear", "rope_theta": rc.theta, "factor": rc.factor}
    if rc.type == "dynamic_ntk":
        return {"rope_type": "dynamic", "rope_theta": rc.theta, "factor": rc.factor}
    if rc.type == "llama3":
        return {"rope_type": "llama3", "rope_theta": rc.theta, "factor": rc.factor,
                "low_freq_factor": rc.low_freq_factor, "high_freq_factor": rc.high_freq_factor,
                "original_max_position_embeddings": rc.original_max_pos}
    raise ValueError(rc.type)


def _hf_config(cfg, max_pos: int, vocab: int = 32, n_layers: int = 1) -> "LlamaConfig":
    """A transformers LlamaConfig of the same shape. For dynamic-NTK, transformers takes original_max_pos from
    max_position_embeddings; for Llama3 it reads it from the RoPE parameters."""
    with warnings.catch_warnings():
        warnings.simplefilter("ignore")
        return LlamaConfig(hidden_size=cfg.hidden, intermediate_size=cfg.intermediate,
                           num_attention_heads=cfg.n_heads, num_key_value_heads=cfg.n_kv_heads,
                           head_dim=cfg.head_dim, rms_norm_eps=cfg.eps, max_position_embeddings=max_pos,
                           rope_parameters=_rope_params(cfg.rope), attention_bias=False, mlp_bias=False,
                           vocab_size=vocab, num_hidden_layers=n_layers, tie_word_embeddings=False,
                           attn_implementation="sdpa")


@dataclasses.dataclass
class _Shape:
    hidden: int
    intermediate: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    eps: float
    rope: RopeCfg


def _shape_for(d, rc=None):
    return _Shape(hidden=2 * d, intermediate=4 * d, n_heads=2, n_kv_heads=1, head_dim=d, eps=1e-5,
                  rope=rc or RopeCfg())


def _hf_freqs(d: int, rc: RopeCfg, seq_len=None, max_pos=None) -> np.ndarray:
    hc = _hf_config(_shape_for(d, rc), max_pos if max_pos is not None else rc.original_max_pos)
    kind = {"default": "default", "linear": "linear", "dynamic_ntk": "dynamic", "llama3": "llama3"}[rc.type]
    if kind == "default":
        return 1.0 / (rc.theta ** (np.arange(0, d, 2, dtype=np.float64) / d))
    kw = {"seq_len": seq_len} if seq_len is not None else {}
    inv, _ = ROPE_INIT_FUNCTIONS[kind](hc, device="cpu", **kw)
    return inv.double().numpy()


# ------------------------------------------------------------------ RoPE frequencies
LLAMA3_SETTINGS = [
    # the 32k workload's constants (factor 8, low 1, high 4, original 8192, theta 5e5), d = 128
    (128, RopeCfg(type="llama3", theta=5e5, factor=8.0, low_freq_factor=1.0, high_freq_factor=4.0,
                  original_max_pos=8192)),
    # a wider middle band and another factor
    (128, RopeCfg(type="llama3", theta=5e5, factor=32.0, low_freq_factor=0.5, high_freq_factor=16.0,
                  original_max_pos=8192)),
    # small theta, d = 64, a short original context
    (64, RopeCfg(type="llama3", theta=1e4, factor=4.0, low_freq_factor=1.0, high_freq_factor=8.0,
                 original_max_pos=2048)),
]


@pytest.mark.parametrize("d,rc", LLAMA3_SETTINGS, ids=["c5", "wide-band", "d64"])
def test_llama3_frequencies_match_transformers(d, rc):
    """verl §1 Llama3 variant: every scaled frequency, including the interpolated middle band, equals the
    library's llama3 initialiser (float32) to float32 rounding."""
    mine = ref.rope_frequencies(d, rc, 0)
    lib = _hf_freqs(d, rc)
    f0 = ref.rope_frequencies(d, RopeCfg(theta=rc.theta), 0)
    ratio = mine / f0
    mid = (ratio < 1.0) & (ratio > 1.0 / rc.factor)
    assert mid.sum() >= 3, "the setting must exercise the interpolated band"
    np.testing.assert_allclose(mine, lib, rtol=RTOL_F32, atol=0)


@pytest.mark.parametrize("d,theta,factor,orig,L", [
    (128, 5e5, 8.0, 8192, 8193), (128, 5e5, 8.0, 8192, 12000), (128, 1e4, 2.0, 4096, 20000),
    (64, 1e4, 4.0, 2048, 2049), (64, 1e4, 4.0, 2048, 65536),
])
def test_dynamic_ntk_frequencies_match_transformers(d, theta, factor, orig, L):
    """verl §1 dynamic-NTK ("dynamically adjust base"), with L = kv_seq_len > original_max_pos: the rescaled
    base theta * (factor*L/orig - (factor-1))^(d/(d-2)) equals the library's dynamic initialiser at
    seq_len = L."""
    rc = RopeCfg(type="dynamic_ntk", theta=theta, factor=factor, original_max_pos=orig)
    mine = ref.rope_frequencies(d, rc, L)
    lib = _hf_freqs(d, rc, seq_len=L, max_pos=orig)
    assert not np.allclose(mine, ref.rope_frequencies(d, RopeCfg(theta=theta), 0), rtol=1e-4)
    np.testing.assert_allclose(mine, lib, rtol=RTOL_F32, atol=0)


@pytest.mark.parametrize("factor", [2.0, 8.0])
def test_linear_frequencies_match_transformers(factor):
    """verl §1 linear variant: the library's linear initialiser divides every frequency by the factor."""
    rc = RopeCfg(type="linear", theta=5e5, factor=factor)
    np.testing.assert_allclose(ref.rope_frequencies(128, rc, 0), _hf_freqs(128, rc), rtol=RTOL_F32, atol=0)


# ------------------------------------------------------------------ the decoder layer
def _load_layer(layer, cfg, W):
    nh, nkv, d, I = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim, cfg.intermediate
    qd, kd = nh * d, nkv * d
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a))
    with torch.no_grad():
        layer.self_attn.q_proj.weight.copy_(T(W["w_qkv"][:qd]))
        layer.self_attn.k_proj.weight.copy_(T(W["w_qkv"][qd:qd + kd]))
        layer.self_attn.v_proj.weight.copy_(T(W["w_qkv"][qd + kd:]))
        layer.self_attn.o_proj.weight.copy_(T(W["w_o"]))
        layer.mlp.gate_proj.weight.copy_(T(W["w_gate_up"][:I]))
        layer.mlp.up_proj.weight.copy_(T(W["w_gate_up"][I:]))
        layer.mlp.down_proj.weight.copy_(T(W["w_down"]))
        layer.input_layernorm.weight.copy_(T(W["g_attn"]))
        layer.post_attention_layernorm.weight.copy_(T(W["g_mlp"]))


def _causal_mask(B, S):
    return torch.full((S, S), -torch.inf, dtype=torch.float64).triu(1)[None, None].expand(B, 1, S, S)


def _hf_layer_out(cfg, W, x, pos, max_pos):
    hc = _hf_config(cfg, max_pos)
    layer = LlamaDecoderLayer(hc, 0).to(torch.float64).eval()
    rot = LlamaRotaryEmbedding(hc).to(torch.float64)
    _load_layer(layer, cfg, W)
    with torch.no_grad():
        xt, pt = torch.from_numpy(x), torch.from_numpy(pos)
        cos, sin = rot(xt, pt)
        out = layer(xt, attention_mask=_causal_mask(x.shape[0], x.shape[1]), position_ids=pt,
                    position_embeddings=(cos.to(torch.float64), sin.to(torch.float64)))
    out = out[0] if isinstance(out, tuple) else out
    return out.numpy()


def _layer_cases():
    base = scaled(CONFIGS["tiny_f32"], B=2, S=24, hidden=64, n_heads=8, n_kv_heads=2, head_dim=16)
    return [
        # name, cfg, max_position_embeddings for the library, kv_seq_len for the oracle
        ("default-g4", base, 64, 24),
        ("mha", scaled(base, n_kv_heads=8), 64, 24),
        ("g2-theta5e5", scaled(base, n_kv_heads=4, rope=RopeCfg(theta=5e5)), 64, 24),
        ("linear", scaled(base, rope=RopeCfg(type="linear", theta=1e4, factor=3.0)), 64, 24),
        # the library recomputes dynamic-NTK frequencies at seq_len = max(position_ids) + 1 = S when S exceeds
        # max_position_embeddings; the oracle takes L = kv_seq_len = S
        ("dynamic-L>orig", scaled(base, rope=RopeCfg(type="dynamic_ntk", theta=1e4, factor=2.0,
                                                     original_max_pos=10)), 10, 24),
        # d = 16, theta 1e4: wavelengths 6.3, 19.9, 62.8, 199, 628, 1987, 6283, 19869; original 2048 with
        # low 1 / high 16 puts pairs 3, 4, 5 in the interpolated band
        ("llama3-midband", scaled(base, rope=RopeCfg(type="llama3", theta=1e4, factor=8.0, low_freq_factor=1.0,
                                                     high_freq_factor=16.0, original_max_pos=2048)), 4096, 24),
        ("d64-g4", scaled(base, hidden=128, n_heads=4, n_kv_heads=1, head_dim=64, intermediate=96), 64, 24),
    ]


@pytest.mark.parametrize("name,cfg,max_pos,L", _layer_cases(), ids=[c[0] for c in _layer_cases()])
def test_layer_matches_transformers_decoder_layer(name, cfg, max_pos, L):
    """nanotron §9.5 LlamaDecoderLayer: the whole layer (both norms, the Q/K/V split of the fused weight,
    RoPE with its scaling, repeat_kv grouping, causal softmax, o_proj and residual, gate/up/down and residual)
    equals the library's LlamaDecoderLayer in float64. Compared on the residual-free branch out - x so the
    N(0,1) residual stream cannot hide a branch error."""
    W = {k: to_f64(v, "f32") for k, v in make_weights(dataclasses.replace(cfg, dtype="f32")).items()}
    x = to_f64(make_hidden(dataclasses.replace(cfg, dtype="f32")), "f32")
    pos = make_prefill_positions(cfg)
    got = ref.layer_prefill(cfg, W, x, pos, L)["out"]
    want = _hf_layer_out(cfg, W, x, pos, max_pos)
    assert ref.max_rel_err(got - x, want - x) < RTOL_F32, name
    assert ref.max_rel_err(got, want) < RTOL_F32, name


def test_gqa_mapping_matches_repeat_kv():
    """nanotron §9.3 / verl §2 repeat_kv: with 8 query heads on 2 kv heads, query head h reads kv head h // 4.
    The library layer with kv heads 0 and 1 swapped in the weights must then disagree with the oracle, so the
    agreement above is not blind to the mapping."""
    name, cfg, max_pos, L = _layer_cases()[0]
    W = {k: to_f64(v, "f32") for k, v in make_weights(dataclasses.replace(cfg, dtype="f32")).items()}
    x = to_f64(make_hidden(dataclasses.replace(cfg, dtype="f32")), "f32")
    pos = make_prefill_positions(cfg)
    got = ref.layer_prefill(cfg, W, x, pos, L)["out"] - x
    nh, nkv, d = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
    Ws = dict(W)
    wq = W["w_qkv"].copy()
    k0 = nh * d
    for base in (k0, k0 + nkv * d):                  # swap kv heads 0 and 1 in both K and V rows
        a = wq[base:base + d].copy()
        wq[base:base + d] = wq[base + d:base + 2 * d]
        wq[base + d:base + 2 * d] = a
    Ws["w_qkv"] = wq
    swapped = _hf_layer_out(cfg, Ws, x, pos, max_pos) - x
    assert ref.max_rel_err(got, swapped) > 1e-2


# ------------------------------------------------------------------ the model stack
def _hf_model_logits(cfg, M, tokens, pos, vocab):
    hc = _hf_config(cfg, 64, vocab=vocab, n_layers=len(M["layers"]))
    model = LlamaForCausalLM(hc).to(torch.float64).eval()
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a))
    with torch.no_grad():
        model.model.embed_tokens.weight.copy_(T(M["tok_embeddings"]))
        for layer, W in zip(model.model.layers, M["layers"]):
            _load_layer(layer, cfg, W)
        model.model.norm.weight.copy_(T(M["g_final"]))
        model.lm_head.weight.copy_(T(M["lm_head"]))
        out = model(input_ids=T(tokens), position_ids=T(pos), use_cache=False)
    return out.logits.numpy()


@pytest.mark.parametrize("n_layers", [0, 1, 3])
def test_model_stack_matches_transformers_causal_lm(n_layers):
    """meta-qa #### 5 Transformer.forward (tok_embeddings, the layers in order, the final norm, the output
    projection): the oracle's model driver equals the library's LlamaForCausalLM in float64 with the same
    weights, for 0, 1 and 3 distinct layers (3 layers apply in list order: any other order differs)."""
    cfg = scaled(CONFIGS["tiny_f32"], B=2, S=11)
    vocab = 37
    raw = make_model_weights(cfg, n_layers, vocab)
    M = {"layers": [{k: to_f64(v, "f32") for k, v in W.items()} for W in raw["layers"]],
         "tok_embeddings": to_f64(raw["tok_embeddings"], "f32"), "g_final": to_f64(raw["g_final"], "f32"),
         "lm_head": to_f64(raw["lm_head"], "f32")}
    tok = make_tokens(cfg, vocab)
    pos = make_prefill_positions(cfg)
    got = ref.model_prefill(cfg, M, tok, pos, cfg.S)["logits"]
    want = _hf_model_logits(cfg, M, tok, pos, vocab)
    assert got.shape == want.shape == (2, 11, vocab)
    assert ref.max_rel_err(got, want) < RTOL_F32
    if n_layers == 3:
        M2 = dict(M, layers=[M["layers"][1], M["layers"][0], M["layers"][2]])
        assert ref.max_rel_err(ref.model_prefill(cfg, M2, tok, pos, cfg.S)["logits"], want) > 1e-4
