"""llama_layer_forward_noalloc (the layer with its workspace and RoPE table in the library's static device
scratch) against llama_layer_forward, through the C ABI: two calls in a row, the second with a smaller input,
for decode against a KV cache and for prefill; each output also against the fp64 oracle."""
import numpy as np
import pytest
import torch

import transformer_layer_forward_amd as L
from oracle import ref
from synth_inputs import (CONFIGS, RopeCfg, make_cache, make_decode_positions, make_hidden, make_prefill_positions,
                          make_weights, scaled, to_f64 as bits_to_f64)
from tests.gpu_util import DEV, require_gpu, tol, to_dev, to_f64
from tests.test_gpu_layer import dev_weights, layer_cfg, w64

pytestmark = pytest.mark.gpu


def _compare(a, b, want, dtype, label):
    ga, gb = to_f64(a), to_f64(b)
    e_ab = ref.max_rel_err(ga, gb)
    e_ref = ref.max_rel_err(ga, want)
    print(f"{label}: noalloc vs workspace entry {e_ab:.3e} (bitwise {torch.equal(a, b)}), vs oracle {e_ref:.3e}",
          flush=True)
    assert e_ab <= tol(dtype), label
    assert e_ref <= tol(dtype), label


def test_noalloc_decode_twice_second_smaller():
    require_gpu()
    big = scaled(CONFIGS["llama3_8b_decode"], B=64, ctx=8192)
    small = scaled(CONFIGS["llama3_8b_decode"], B=5, ctx=1500)
    for step, cfg in enumerate((big, small)):
        print(f"case noalloc decode B={cfg.B} ctx={cfg.ctx}", flush=True)
        W = make_weights(cfg, seed=11)
        Wd = dev_weights(W, cfg.dtype)
        x = make_hidden(cfg, seed=11 + step)
        pos = make_decode_positions(cfg, seed=11 + step, lo=1 if cfg.ctx < 2048 else 1024)
        kc, vc = make_cache(cfg, "k", seed=11), make_cache(cfg, "v", seed=11)
        lc = layer_cfg(cfg)
        xd, pd = to_dev(x, cfg.dtype), torch.from_numpy(pos).to(DEV)
        k1, v1 = to_dev(kc, cfg.dtype), to_dev(vc, cfg.dtype)
        k2, v2 = k1.clone(), v1.clone()
        a = torch.empty_like(xd)
        L.llama_layer_forward_noalloc(lc, Wd, xd, pd, kv_seq_len=cfg.ctx, k_cache=k1, v_cache=v1, out=a)
        b = L.llama_layer_forward(lc, Wd, xd, pd, kv_seq_len=cfg.ctx, k_cache=k2, v_cache=v2)
        torch.cuda.synchronize()
        x64 = bits_to_f64(x, cfg.dtype)
        bs = list(range(cfg.B)) if cfg.B <= 8 else [0, 31, cfg.B - 1]
        want = ref.layer_decode(cfg, w64(W, cfg.dtype), x64, pos, cfg.ctx, lambda r: bits_to_f64(kc[r], cfg.dtype),
                                lambda r: bits_to_f64(vc[r], cfg.dtype), batch_rows=bs)
        _compare(a[bs, 0], b[bs, 0], want["out"], cfg.dtype, f"decode B={cfg.B}")
        idx = torch.from_numpy(pos).to(DEV)
        ar = torch.arange(cfg.B, device=DEV)
        assert ref.max_rel_err(to_f64(k1[ar, idx]), to_f64(k2[ar, idx])) <= tol(cfg.dtype)
        assert ref.max_rel_err(to_f64(v1[ar, idx]), to_f64(v2[ar, idx])) <= tol(cfg.dtype)
        del kc, vc, k1, v1, k2, v2


def test_noalloc_prefill_twice_second_smaller():
    require_gpu()
    cases = [scaled(CONFIGS["llama3_8b_prefill"], B=1, S=300,
                    rope=RopeCfg(type="llama3", theta=500000.0, factor=8.0, original_max_pos=128)),
             scaled(CONFIGS["llama3_8b_prefill"], B=1, S=70,
                    rope=RopeCfg(type="dynamic_ntk", theta=500000.0, factor=2.0, original_max_pos=32))]
    for step, cfg in enumerate(cases):
        print(f"case noalloc prefill S={cfg.S} rope={cfg.rope.type}", flush=True)
        W = make_weights(cfg, seed=12)
        Wd = dev_weights(W, cfg.dtype)
        x = make_hidden(cfg, seed=12 + step)
        pos = make_prefill_positions(cfg)
        lc = layer_cfg(cfg)
        xd, pd = to_dev(x, cfg.dtype), torch.from_numpy(pos).to(DEV)
        a = torch.empty_like(xd)
        L.llama_layer_forward_noalloc(lc, Wd, xd, pd, kv_seq_len=cfg.S, out=a)
        b = L.llama_layer_forward(lc, Wd, xd, pd, kv_seq_len=cfg.S)
        torch.cuda.synchronize()
        want = ref.layer_prefill(cfg, w64(W, cfg.dtype), bits_to_f64(x, cfg.dtype), pos, cfg.S)
        _compare(a, b, want["out"], cfg.dtype, f"prefill S={cfg.S}")


def test_noalloc_rejects_calls_beyond_its_scratch():
    """A prefill whose workspace exceeds the 64 MiB scratch is refused with LL_EINVAL and a message."""
    require_gpu()
    cfg = scaled(CONFIGS["llama3_8b_prefill"], B=1, S=4096)
    W = dev_weights(make_weights(cfg, seed=13), cfg.dtype)
    x = to_dev(make_hidden(cfg, seed=13), cfg.dtype)
    pos = torch.from_numpy(make_prefill_positions(cfg)).to(DEV)
    out = torch.empty_like(x)
    with pytest.raises(RuntimeError, match="static scratch"):
        L.llama_layer_forward_noalloc(layer_cfg(cfg), W, x, pos, out=out)
