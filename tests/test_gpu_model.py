"""GPU parity of llama_model_forward (token embeddings -> decoder layers -> final RMSNorm -> output
projection; CSDN answer "#### 5." Transformer.forward at start_pos = 0) against the fp64 oracle's
model_prefill, on seeded synthetic weights."""
import numpy as np
import pytest
import torch

import transformer_layer_forward_amd as L
from oracle import ref
from synth_inputs import (CONFIGS, make_model_weights, make_prefill_positions, make_tokens, scaled,
                          to_f64 as bits_to_f64)
from tests.gpu_util import DEV, require_gpu, tol, to_dev, to_f64
from tests.test_gpu_layer import layer_cfg

pytestmark = pytest.mark.gpu

MODEL = [
    # config, layers, vocab
    (scaled(CONFIGS["tiny_f32"], B=2, S=17), 3, 97),
    (scaled(CONFIGS["llama32_1b_prefill"], B=1, S=100), 2, 1001),     # vocab not a multiple of 8
    (scaled(CONFIGS["llama3_8b_prefill"], B=2, S=70), 2, 512),
    (scaled(CONFIGS["llama32_1b_prefill"], B=2, S=24), 2, 1001),      # 48 tokens: decode-sized projections
]


def _dev_model(M, dtype):
    return {"layers": [{k: to_dev(v, dtype) for k, v in W.items()} for W in M["layers"]],
            "tok_embeddings": to_dev(M["tok_embeddings"], dtype), "g_final": to_dev(M["g_final"], dtype),
            "lm_head": to_dev(M["lm_head"], dtype)}


def _f64_model(M, dtype):
    return {"layers": [{k: bits_to_f64(v, dtype) for k, v in W.items()} for W in M["layers"]],
            "tok_embeddings": bits_to_f64(M["tok_embeddings"], dtype), "g_final": bits_to_f64(M["g_final"], dtype),
            "lm_head": bits_to_f64(M["lm_head"], dtype)}


@pytest.mark.parametrize("case", MODEL, ids=lambda c: f"{c[0].name}-B{c[0].B}xS{c[0].S}-L{c[1]}-V{c[2]}")
def test_model_prefill(case):
    require_gpu()
    cfg, n_layers, vocab = case
    M = make_model_weights(cfg, n_layers, vocab, seed=1)
    tok = make_tokens(cfg, vocab, seed=1)
    pos = make_prefill_positions(cfg)
    logits = L.llama_model_forward(layer_cfg(cfg), _dev_model(M, cfg.dtype), torch.from_numpy(tok).to(DEV),
                                   torch.from_numpy(pos).to(DEV), kv_seq_len=cfg.S)
    got = to_f64(logits)
    want = ref.model_prefill(cfg, _f64_model(M, cfg.dtype), tok, pos, cfg.S)["logits"]
    assert got.shape == (cfg.B, cfg.S, vocab)
    err = ref.max_rel_err(got, want)
    print(f"{cfg.name} layers {n_layers} vocab {vocab}: logits err {err:.3e}", flush=True)
    assert err <= tol(cfg.dtype)


def test_model_causality_bitwise():
    """Changing tokens after position i leaves the logits of positions <= i bit-identical."""
    require_gpu()
    cfg = scaled(CONFIGS["llama32_1b_prefill"], B=1, S=150)
    M = _dev_model(make_model_weights(cfg, 2, 512, seed=2), cfg.dtype)
    tok = torch.from_numpy(make_tokens(cfg, 512, seed=2)).to(DEV)
    pos = torch.from_numpy(make_prefill_positions(cfg)).to(DEV)
    lc = layer_cfg(cfg)
    a = L.llama_model_forward(lc, M, tok, pos)
    tok2 = tok.clone()
    tok2[:, 100:] = (tok2[:, 100:] + 7) % 512
    b = L.llama_model_forward(lc, M, tok2, pos)
    torch.cuda.synchronize()
    assert torch.equal(a[:, :100], b[:, :100])
    assert not torch.equal(a[:, 100:], b[:, 100:])
