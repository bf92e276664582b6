"""Benchmark: Llama-3-8B-shaped decoder-layer forward (bf16 prefill, B=2, S=4096) on one MI355X.

One step = one llama_layer_forward over the whole batch (RMSNorm, QKV, RoPE, causal GQA attention,
o_proj + residual, RMSNorm, gate_up + SwiGLU, down + residual), inputs resident in HBM.
Prints one JSON line: tokens/s, per-stage times from HIP events recorded by the library on the
launch stream during the timed steps, the roofline position of the dominant kernel (the fused
gate_up GEMM) and the fp64 CPU oracle timed on a bounded sample of the same workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MI355X_BF16_DENSE_TFLOPS = 2500.0   # published dense bf16 matrix peak
MI355X_HBM_GBS = 8000.0
WORKLOAD = "llama3_8b_prefill"
PMC_SUMMARY = os.path.join(ROOT, "profiles", "gate_up_silu_gemm_llama3_8b_prefill_pmc.json")
GEMM_SRC = os.path.join(ROOT, "transformer_layer_forward_amd", "csrc", "gemm.hip")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=1024)
    return ap.parse_args()


def gemm_source_hash() -> str:
    return hashlib.sha256(open(GEMM_SRC, "rb").read()).hexdigest()[:16]


def measured_traffic():
    """HBM bytes per gate_up launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE summary, if it
    was taken on the current kernel source; None otherwise."""
    try:
        rec = json.load(open(PMC_SUMMARY))
    except (OSError, ValueError):
        return None
    if rec.get("gemm_source_sha256_16") != gemm_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(cfg, W_bits, x_bits, tokens):
    """fp64 oracle on sequence 0, tokens 0..tokens-1 of the same workload (a bounded sample)."""
    import numpy as np

    from oracle import ref
    from synth_inputs import to_f64
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    except Exception:  # noqa: BLE001
        threads = os.cpu_count() or 1
    W = {k: to_f64(v, "bf16") for k, v in W_bits.items()}
    x = to_f64(x_bits[:1, :tokens], "bf16")
    pos = np.arange(tokens, dtype=np.int64)[None, :]
    from synth_inputs import scaled
    c = scaled(cfg, B=1, S=tokens)
    t0 = time.perf_counter()
    ref.layer_prefill(c, W, x, pos, tokens)
    dt = time.perf_counter() - t0
    return {"value": tokens / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{WORKLOAD} layer on sequence 0, tokens 0..{tokens - 1} ({tokens} of {cfg.B * cfg.S} tokens; "
                      f"causal attention over a {tokens}-token prefix instead of up to {cfg.S}), fp64 NumPy, "
                      f"{dt:.1f} s"}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (each MI355X runs the whole "
              "layer on its own sequences; see the sharding notes). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import transformer_layer_forward_amd as L
    from synth_inputs import CONFIGS, make_hidden, make_prefill_positions, make_weights

    cfg = CONFIGS[WORKLOAD]
    dev = "cuda:0"
    torch.cuda.set_device(0)
    W_bits = make_weights(cfg, seed=0)
    x_bits = make_hidden(cfg, seed=0)

    def to_dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    W = {k: to_dev(v) for k, v in W_bits.items()}
    x = to_dev(x_bits)
    pos = torch.from_numpy(make_prefill_positions(cfg)).to(dev)
    rc = cfg.rope
    lc = L.LayerConfig(cfg.hidden, cfg.n_heads, cfg.n_kv_heads, cfg.head_dim, cfg.intermediate, cfg.eps,
                       L.Rope(type=rc.type, theta=rc.theta), torch.bfloat16)
    ws = torch.empty(L.layer_workspace_bytes(lc, cfg.B, cfg.S), dtype=torch.uint8, device=dev)
    out = torch.empty_like(x)

    for _ in range(args.warmup):
        L.llama_layer_forward(lc, W, x, pos, kv_seq_len=cfg.S, out=out, workspace=ws)
    torch.cuda.synchronize()

    L.profile_begin(args.steps)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        L.llama_layer_forward(lc, W, x, pos, kv_seq_len=cfg.S, out=out, workspace=ws)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    stages = L.profile_end()
    assert torch.isfinite(out.float()).all().item()

    ms_per_step = wall * 1e3 / args.steps
    tokens = cfg.B * cfg.S
    value = tokens / (ms_per_step / 1e3)

    M, H, I, d = cfg.M, cfg.hidden, cfg.intermediate, cfg.head_dim
    gate_up_flops = 2.0 * M * (2 * I) * H
    gu_ms = stages["gate_up_silu"][0] / stages["gate_up_silu"][1]
    achieved = gate_up_flops / (gu_ms / 1e3) / 1e12
    attn_flops = 4.0 * cfg.B * cfg.n_heads * d * (cfg.S * (cfg.S + 1) / 2)   # QK^T and PV over visible pairs
    attn_ms = stages["attention"][0] / stages["attention"][1]
    gemm_flops = 2.0 * M * H * (cfg.qkv_dim + H + 2 * I) + 2.0 * M * I * H
    gemm_ms = sum(stages[k][0] / stages[k][1] for k in ("qkv_proj", "o_proj_residual", "gate_up_silu", "down_residual"))
    norm_bytes = 2 * (2 * M * H * 2 + H * 2)
    norm_ms = sum(stages[k][0] / stages[k][1] for k in ("rmsnorm_attn", "rmsnorm_mlp"))

    rec = {
        "metric": "decoder-layer tokens/s (Llama-3-8B shape, bf16) + attention MFMA util %",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) hidden, N(0,0.02) weights, 1+N(0,0.1) gains)",
        "config": {"workload": "Llama-3-8B-shaped decoder layer, bf16 prefill, causal", "B": cfg.B, "S": cfg.S,
                   "hidden": H, "n_heads": cfg.n_heads, "n_kv_heads": cfg.n_kv_heads, "head_dim": d,
                   "intermediate": I, "rope_theta": rc.theta, "tokens_per_step": tokens},
        "attention_mfma_util_pct": round(100.0 * attn_flops / (attn_ms / 1e3) / 1e12 / MI355X_BF16_DENSE_TFLOPS, 2),
        "gemm_mfma_util_pct": round(100.0 * gemm_flops / (gemm_ms / 1e3) / 1e12 / MI355X_BF16_DENSE_TFLOPS, 2),
        "rmsnorm_hbm_gbs": round(norm_bytes / (norm_ms / 1e3) / 1e9, 1),
        "stages_ms": {k: round(v[0] / v[1], 4) for k, v in stages.items()},
        "roofline": {
            "kernel": "gemm_bf16_big_kernel<EPI_SILU> (fused gate_up + silu*up)",
            "bound": "mfma",
            "achieved": round(achieved, 1),
            "peak": MI355X_BF16_DENSE_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / MI355X_BF16_DENSE_TFLOPS, 4),
            "traffic": measured_traffic(),
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(cfg, W_bits, x_bits, args.cpu_sample_tokens)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
