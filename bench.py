"""Benchmark: Llama-3-8B-shaped decoder-layer forward (bf16 prefill, B=2, S=4096) on one MI355X.

One step = one llama_layer_forward over the whole batch (RMSNorm, QKV, RoPE, causal GQA attention,
o_proj + residual, RMSNorm, gate_up + SwiGLU, down + residual), inputs resident in HBM.
Prints one JSON line: tokens/s, the roofline position of the dominant kernel (the fused gate_up GEMM,
timed by HIP events the library records on the launch stream around that kernel during the timed
steps), per-stage times from a second pass of the same calls with every stage's events on, and the
fp64 CPU oracle timed on a bounded sample of the same workload.

The headline run also times, cache-cold (a 512 MiB read before each call), the stand-alone RMSNorm on the
workload's hidden states ("rmsnorm_cold") and the 8B decode step (B=64 against 8192-slot KV caches,
"decode"), each with its HBM GB/s.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-decode] [--no-cpu-baseline]
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
COMMON_H = os.path.join(ROOT, "transformer_layer_forward_amd", "csrc", "common.h")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=WORKLOAD,
                    choices=[WORKLOAD, "llama32_1b_prefill", "llama3_8b_long_llama3rope", "llama3_8b_decode",
                             CHUNK_WORKLOAD, CHUNK_SMALL_WORKLOAD, VARLEN_WORKLOAD, MODEL_WORKLOAD],
                    help="the headline line is the 8B prefill; the others print the same record for that workload")
    ap.add_argument("--no-decode", action="store_true",
                    help="skip the cache-cold decode measurement that the headline run adds as \"decode\"")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=0,
                    help="time the oracle on the first N tokens of sequence 0 only (0: the whole workload)")
    ap.add_argument("--rocpd-summary", metavar="DB",
                    help="print per-kernel duration statistics from a rocprofv3 results database and exit")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DB", "WRITE_DB"),
                    help="combine rocprofv3 FETCH_SIZE and WRITE_SIZE databases (bench + copy calibration) "
                         "into the per-launch HBM traffic record of the gate_up kernel and exit")
    ap.add_argument("--counter-summary", nargs="+", metavar="DB",
                    help="per-kernel medians of the rocprofv3 --pmc counters in these databases (and derived MFMA "
                         "busy share, shader clock, HBM bytes) as a markdown table, then exit")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the bench, run a plain 1 GiB device-to-device copy 3 times (counter calibration)")
    return ap.parse_args()


COPY_BYTES = 1 << 30


def copy_calibration() -> None:
    import torch
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"copied {COPY_BYTES} bytes x3", flush=True)


def pmc_summary(fetch_db: str, write_db: str) -> None:
    """Per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of the gate_up GEMM, scaled by what the same counters read
    for the plain copy (which must move COPY_BYTES each way)."""
    import sqlite3

    def per_kernel(db, counter):
        con = sqlite3.connect(db)
        rows = con.execute("select name, dispatch_id, sum(counter_value) from pmc_events where counter_name = ? "
                           "group by dispatch_id", (counter,)).fetchall()
        out = {}
        for name, _, v in rows:
            out.setdefault(name, []).append(v)
        return out

    f = per_kernel(fetch_db, "FETCH_SIZE")
    w = per_kernel(write_db, "WRITE_SIZE")

    def pick(d, key):
        vals = [v for name, vs in d.items() if key in name for v in vs]
        return sorted(vals)[len(vals) // 2] if vals else None  # median dispatch

    def pick_copy(d):
        # the 1 GiB device copies are the largest copy-kernel dispatches of the run
        vals = sorted(v for name, vs in d.items() if "copyBuffer" in name for v in vs)
        return vals[-1] if vals else None

    gu_key = "gemm_bf16_mfma32_silu_persist_kernel"
    f_copy, w_copy = pick_copy(f), pick_copy(w)
    f_gu, w_gu = pick(f, gu_key), pick(w, gu_key)
    kib = COPY_BYTES / 1024.0
    f_scale = kib / f_copy if f_copy else None
    w_scale = kib / w_copy if w_copy else None
    rec = {"kernel_source_sha256_16": gemm_source_hash(), "fetch_kib_per_launch_raw": f_gu,
           "write_kib_per_launch_raw": w_gu, "copy_fetch_kib_raw": f_copy, "copy_write_kib_raw": w_copy,
           "copy_bytes": COPY_BYTES, "fetch_scale": f_scale, "write_scale": w_scale}
    if None not in (f_gu, w_gu, f_scale, w_scale):
        rec["hbm_bytes_per_launch"] = round((f_gu * f_scale + w_gu * w_scale) * 1024.0)
    print(json.dumps(rec, indent=1))


SIMDS = 1024   # 256 compute units x 4 SIMDs


def counter_summary(dbs) -> None:
    """Per kernel and grid size (the library's own kernels and the 1 GiB copy used for calibration): dispatches, median
    duration and the median per dispatch of every counter found in the databases. SQ counters are summed
    over the instances rocprofv3 reports, GRBM_GUI_ACTIVE takes their maximum. Derived:
    mfma_busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE x 1024 SIMDs), the matrix cores' busy share per
    shader clock; clock = GRBM_GUI_ACTIVE / duration; bf16_tflops = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 /
    duration; FETCH_SIZE and WRITE_SIZE are in KiB."""
    import sqlite3
    vals, durs = {}, {}
    for db in dbs:
        con = sqlite3.connect(db)
        rows = con.execute("select name, dispatch_id, counter_name, counter_value, duration from pmc_events").fetchall()
        grid = dict(con.execute("select dispatch_id, max(grid_size) from counters_collection group by dispatch_id"))
        per = {}
        for name, disp, cname, v, dur in rows:
            key = (db, disp)
            # one kernel serves several projections: the grid size tells them apart
            rec = per.setdefault(key, {"name": f"{name.split('(')[0]} grid {grid.get(disp)}", "dur": dur, "c": {}})
            acc = rec["c"].setdefault(cname, [])
            acc.append(v)
        # one kernel and grid size can still serve two projections of different K (o_proj and down at the
        # 8B prefill shape): dispatches of one key whose durations differ by more than 2x form two groups
        bykey = {}
        for (db_, disp), rec in per.items():
            bykey.setdefault(rec["name"], []).append(rec)
        for name, recs in bykey.items():
            ds = sorted(r["dur"] for r in recs if r["dur"])
            if len(ds) >= 2 and ds[-1] > 2.0 * ds[0]:
                cut = max(range(1, len(ds)), key=lambda i: ds[i] / ds[i - 1])
                thr = ds[cut]
                for r in recs:
                    r["name"] = f"{name} ({'long' if r['dur'] and r['dur'] >= thr else 'short'} dispatches)"
        for (db_, disp), rec in per.items():
            name = rec["name"]
            if not (name.startswith("void ll::") or name.startswith("ll::") or "copyBuffer" in name):
                continue
            short = name.replace("void ", "")
            d = durs.setdefault(short, [])
            if rec["dur"]:
                d.append(rec["dur"])
            for cname, vs in rec["c"].items():
                agg = max(vs) if cname.startswith("GRBM") else sum(vs)
                vals.setdefault(short, {}).setdefault(cname, []).append(agg)

    def med(xs):
        xs = sorted(xs)
        return xs[len(xs) // 2] if xs else None

    cols = sorted({c for v in vals.values() for c in v})
    print("| kernel | dispatches | median us | " + " | ".join(cols) + " | mfma_busy | clock GHz | bf16 TFLOP/s |")
    print("|---" * (len(cols) + 6) + "|")
    for k in sorted(vals, key=lambda k: -(med(durs.get(k, [])) or 0) * len(durs.get(k, []))):
        c = {n: med(v) for n, v in vals[k].items()}
        dur_ns = med(durs.get(k, []))
        busy = c.get("SQ_VALU_MFMA_BUSY_CYCLES")
        grbm = c.get("GRBM_GUI_ACTIVE")
        mops = c.get("SQ_INSTS_VALU_MFMA_MOPS_BF16")
        mb = f"{busy / (grbm * SIMDS):.3f}" if busy is not None and grbm else ""
        clk = f"{grbm / dur_ns:.2f}" if grbm and dur_ns else ""
        tf = f"{mops * 512 / (dur_ns * 1e-9) / 1e12:.0f}" if mops and dur_ns else ""
        cells = " | ".join(f"{c[n]:.4g}" if c.get(n) is not None else "" for n in cols)
        print(f"| `{k[:90]}` | {len(durs.get(k, []))} | {dur_ns / 1e3 if dur_ns else 0:.1f} | {cells} | {mb} | {clk} | {tf} |")


def rocpd_summary(db: str) -> None:
    """Per-kernel calls / average / min / max durations (microseconds) from a rocprofv3 SQLite database."""
    import sqlite3
    con = sqlite3.connect(db)
    rows = con.execute("select name, count(*), avg(duration), min(duration), max(duration), sum(duration) "
                       "from kernels group by name order by sum(duration) desc").fetchall()
    total = sum(r[5] for r in rows) or 1
    print("| kernel | calls | avg us | min us | max us | share |")
    print("|---|---|---|---|---|---|")
    for name, n, avg, lo, hi, tot in rows:
        print(f"| `{name[:110]}` | {n} | {avg / 1e3:.1f} | {lo / 1e3:.1f} | {hi / 1e3:.1f} | {100 * tot / total:.1f}% |")


# the fused gate_up kernel at each prefill workload's shape: the persistent kernel where the projection is made
# of whole tiles with at least two per compute unit, else the one-tile kernel or its K-split form
GATE_UP_KERNEL = {"llama3_8b_chunk_small": "gemm_bf16_mfma32_kernel<EPI_SILU> (few-tile plan)"}


def gemm_source_hash() -> str:
    """Hash of the code the gate_up kernel is built from: the 32x32 section of gemm.hip (both the one-tile and the
    persistent kernel), their launchers and the shared header, without comments. Other GEMM paths (decode, fp32) may
    change without invalidating the counters."""
    src = open(GEMM_SRC).read()
    dash = "// " + "-" * 66
    a = src.index(dash + " bf16, large M, 32x32 matrix ops")
    b = src.index(dash + " bf16, small M (decode)")
    la = src.index("static hipError_t mfma32_launch(")
    lb = src.index("\n}\n", la)
    pa = src.index("static bool mfp_usable(")
    pb = src.index("\n}\n", src.index("static hipError_t mfp_launch("))
    text = src[a:b] + src[la:lb] + src[pa:pb] + open(COMMON_H).read()
    # comments and blank lines do not change the machine code
    code = [ln.split("//", 1)[0].rstrip() for ln in text.splitlines()]
    return hashlib.sha256("\n".join(ln for ln in code if ln).encode()).hexdigest()[:16]


def measured_traffic():
    """HBM bytes per gate_up launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE summary, if it
    was taken on the current kernel source; None otherwise."""
    try:
        rec = json.load(open(PMC_SUMMARY))
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256_16") != gemm_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(cfg, W_bits, x_bits, tokens):
    """fp64 oracle timed on the host: the whole workload (tokens = 0) or, to bound the time on a slow host,
    sequence 0 truncated to its first `tokens` tokens."""
    import numpy as np

    from oracle import ref
    from synth_inputs import scaled, to_f64
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    except Exception:  # noqa: BLE001
        threads = os.cpu_count() or 1
    W = {k: to_f64(v, "bf16") for k, v in W_bits.items()}
    if tokens <= 0 or tokens >= cfg.S:
        c, x = cfg, to_f64(x_bits, "bf16")
        sample = f"the whole {WORKLOAD} workload (B={cfg.B}, S={cfg.S}, {cfg.B * cfg.S} tokens)"
    else:
        c, x = scaled(cfg, B=1, S=tokens), to_f64(x_bits[:1, :tokens], "bf16")
        sample = (f"{WORKLOAD} layer on sequence 0, tokens 0..{tokens - 1} ({tokens} of {cfg.B * cfg.S} tokens; "
                  f"causal attention over a {tokens}-token prefix instead of up to {cfg.S})")
    pos = np.broadcast_to(np.arange(c.S, dtype=np.int64), (c.B, c.S))
    t0 = time.perf_counter()
    ref.layer_prefill(c, W, x, pos, c.S)
    dt = time.perf_counter() - t0
    return {"value": c.B * c.S / dt, "unit": "tokens/s", "cores": int(threads), "cpu_model": cpu_model(),
            "kind": "oracle", "sample": f"{sample}, fp64 NumPy, {dt:.1f} s"}


def cpu_model() -> str:
    """The host CPU's model name (first /proc/cpuinfo entry) and its logical CPU count."""
    name = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    name = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return f"{name} ({os.cpu_count()} logical CPUs)"


FLUSH_BYTES = 512 << 20


def cache_flusher(torch, dev):
    """A 512 MiB buffer whose full read (outside any timed region) evicts L2 and the 256 MB Infinity Cache
    with clean lines, so the next kernel starts cache-cold without write-backs of dirty lines."""
    buf = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)

    def flush():
        buf.amax()
    return flush


def rmsnorm_cold(L, torch, np, cfg, W, steps=30):
    """The stand-alone RMSNorm on the workload's [B*S, H] hidden states, cache-cold: a 512 MiB read before
    each call, each call timed by HIP events on its stream; median, p10, p90 and HBM GB/s of its
    algorithmic bytes (read x and the gain, write y)."""
    from synth_inputs import make_hidden
    dev = "cuda:0"
    x = torch.from_numpy(np.ascontiguousarray(make_hidden(cfg, seed=0)).view(np.int16)).to(dev).view(torch.bfloat16)
    y = torch.empty_like(x)
    flush = cache_flusher(torch, dev)
    stream = torch.cuda.current_stream()
    for _ in range(3):
        L.rmsnorm(x, W["g_attn"], cfg.eps, out=y)
    times = []
    for _ in range(steps):
        flush()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        L.rmsnorm(x, W["g_attn"], cfg.eps, out=y)
        e1.record(stream)
        e1.synchronize()
        times.append(e0.elapsed_time(e1))
    times.sort()
    ms = times[len(times) // 2]
    nbytes = 2 * x.numel() * 2 + cfg.hidden * 2
    return {"kernel": "rmsnorm_vec_kernel", "rows": cfg.B * cfg.S, "hidden": cfg.hidden,
            "timing": "median of per-call HIP events, 512 MiB read before each call (cache-cold)",
            "ms": round(ms, 4), "p10_ms": round(times[len(times) // 10], 4),
            "p90_ms": round(times[(9 * len(times)) // 10], 4), "algorithmic_bytes": nbytes,
            "hbm_gbs": round(nbytes / (ms / 1e3) / 1e9, 1),
            "hbm_frac": round(nbytes / (ms / 1e3) / 1e9 / MI355X_HBM_GBS, 4)}


def lib_config(L, cfg, torch):
    rc = cfg.rope
    rope = L.Rope(type=rc.type, theta=rc.theta, factor=rc.factor, low_freq_factor=rc.low_freq_factor,
                  high_freq_factor=rc.high_freq_factor, original_max_pos=rc.original_max_pos,
                  interleaved=rc.interleaved)
    return L.LayerConfig(cfg.hidden, cfg.n_heads, cfg.n_kv_heads, cfg.head_dim, cfg.intermediate, cfg.eps, rope,
                         torch.bfloat16)


def stage_ms(stages, key):
    tot, n = stages[key]
    return tot / n


def gemm_flops_per_token(cfg):
    return 2.0 * cfg.hidden * (cfg.qkv_dim + cfg.hidden + 2 * cfg.intermediate) + 2.0 * cfg.intermediate * cfg.hidden


def weight_bytes(cfg):
    return 2 * (cfg.hidden * (cfg.qkv_dim + cfg.hidden + 2 * cfg.intermediate) + cfg.intermediate * cfg.hidden
                + 2 * cfg.hidden)


def run_prefill(L, torch, np, cfg, W, args):
    """K timed prefill layer calls back to back, with the library's HIP events around the gate_up stage only
    (the dominant kernel the roofline is priced on; each event between two kernels costs a few
    microseconds), then K more calls with every stage timed for the stage breakdown. Returns
    (ms_per_step, stages, gate_up (ms, calls) of the timed calls, x_bits)."""
    from synth_inputs import make_hidden, make_prefill_positions
    dev = "cuda:0"
    x_bits = make_hidden(cfg, seed=0)
    x = torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).to(dev).view(torch.bfloat16)
    pos = torch.from_numpy(make_prefill_positions(cfg)).to(dev)
    lc = lib_config(L, cfg, torch)
    ws = torch.empty(L.layer_workspace_bytes(lc, cfg.B, cfg.S), dtype=torch.uint8, device=dev)
    out = torch.empty_like(x)
    for _ in range(args.warmup):
        L.llama_layer_forward(lc, W, x, pos, kv_seq_len=cfg.S, out=out, workspace=ws)
    torch.cuda.synchronize()
    L.profile_begin(args.steps, stages=["gate_up_silu"])
    t0 = time.perf_counter()
    for _ in range(args.steps):
        L.llama_layer_forward(lc, W, x, pos, kv_seq_len=cfg.S, out=out, workspace=ws)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    timed = L.profile_end()["gate_up_silu"]
    L.profile_begin(args.steps)
    for _ in range(args.steps):
        L.llama_layer_forward(lc, W, x, pos, kv_seq_len=cfg.S, out=out, workspace=ws)
    torch.cuda.synchronize()
    stages = L.profile_end()
    assert torch.isfinite(out.float()).all().item()
    return wall * 1e3 / args.steps, stages, timed, x_bits


CHUNK_WORKLOAD = "llama3_8b_chunk"
CHUNK_SMALL_WORKLOAD = "llama3_8b_chunk_small"
CHUNK_CTX = 8192
# workload -> (sequences, new tokens per sequence, cached prefix length)
CHUNK_SHAPES = {CHUNK_WORKLOAD: (None, 2048, 6144), CHUNK_SMALL_WORKLOAD: (1, 256, 7936)}


def run_chunk(L, torch, np, cfg, W, args, start):
    """Chunked prefill on a cache prefix: each sequence's S new tokens sit at positions
    start .. start + S - 1 of CHUNK_CTX-slot caches whose earlier slots (the prefix) hold
    N(0,1) values from torch's seeded device generator. Every call rewrites the same slots with the same
    values, so calls are idempotent. The workspace is sized for the cache length, so attention may split
    a small chunk's keys over several workgroups. Returns (ms_per_step, stages)."""
    from synth_inputs import make_hidden
    dev = "cuda:0"
    x = torch.from_numpy(np.ascontiguousarray(make_hidden(cfg, seed=0)).view(np.int16)).to(dev).view(torch.bfloat16)
    pos = (torch.arange(cfg.S, device=dev, dtype=torch.int64) + start).expand(cfg.B, cfg.S).contiguous()
    g = torch.Generator(device=dev)
    shape = (cfg.B, CHUNK_CTX, cfg.n_kv_heads, cfg.head_dim)
    g.manual_seed(8)
    kc = torch.randn(shape, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    g.manual_seed(9)
    vc = torch.randn(shape, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    lc = lib_config(L, cfg, torch)
    ws = torch.empty(L.layer_workspace_bytes(lc, cfg.B, cfg.S, CHUNK_CTX), dtype=torch.uint8, device=dev)
    out = torch.empty_like(x)
    for _ in range(args.warmup):
        L.llama_layer_forward_chunk(lc, W, x, pos, kc, vc, out=out, workspace=ws)
    torch.cuda.synchronize()
    L.profile_begin(args.steps)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        L.llama_layer_forward_chunk(lc, W, x, pos, kc, vc, out=out, workspace=ws)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    stages = L.profile_end()
    assert torch.isfinite(out.float()).all().item()
    return wall * 1e3 / args.steps, stages


VARLEN_WORKLOAD = "llama3_8b_varlen"
VARLEN_TOKENS = 8192


def varlen_lengths(np):
    """Seeded ragged length mix for the packed workload: lengths integer-uniform on [64, 2048] drawn
    until VARLEN_TOKENS tokens are reached (the last one shortened to fit)."""
    rng = np.random.default_rng([0, 20])
    lens, tot = [], 0
    while tot < VARLEN_TOKENS:
        n = int(min(rng.integers(64, 2049), VARLEN_TOKENS - tot))
        lens.append(n)
        tot += n
    return lens


def run_varlen(L, torch, np, cfg, W, args, lens):
    """Packed prefill of the sequences `lens` (total VARLEN_TOKENS) through llama_layer_forward_varlen,
    RoPE at in-sequence positions. Returns (ms_per_step, stages)."""
    from synth_inputs import make_hidden
    dev = "cuda:0"
    x = torch.from_numpy(np.ascontiguousarray(make_hidden(cfg, seed=0)[0]).view(np.int16)).to(dev).view(torch.bfloat16)
    cu = torch.from_numpy(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)).to(dev)
    pos = torch.from_numpy(np.concatenate([np.arange(n) for n in lens]).astype(np.int64)).to(dev)
    lc = lib_config(L, cfg, torch)
    T = sum(lens)
    ws = torch.empty(L.layer_workspace_bytes(lc, 1, T), dtype=torch.uint8, device=dev)
    out = torch.empty_like(x)
    mx = max(lens)
    for _ in range(args.warmup):
        L.llama_layer_forward_varlen(lc, W, x, pos, cu, mx, out=out, workspace=ws)
    torch.cuda.synchronize()
    L.profile_begin(args.steps)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        L.llama_layer_forward_varlen(lc, W, x, pos, cu, mx, out=out, workspace=ws)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    stages = L.profile_end()
    assert torch.isfinite(out.float()).all().item()
    return wall * 1e3 / args.steps, stages


MODEL_WORKLOAD = "llama32_1b_model"
MODEL_LAYERS, MODEL_VOCAB = 16, 128256


def run_model(L, torch, np, cfg, args):
    """The Llama-3.2-1B-shaped stack (16 decoder layers, 128256-token vocabulary, the layer dump on the
    NJU lecture page) over B x S token ids. Weights come from torch's seeded device generator (N(0,0.02)
    projections, 1+N(0,0.1) gains, N(0,1) embeddings; their values do not change the work); token ids
    integer-uniform on the vocabulary. Returns (ms_per_step, stages)."""
    dev = "cuda:0"
    g = torch.Generator(device=dev)

    def draw(shape, std, mean, seed):
        g.manual_seed(seed)
        return (torch.randn(shape, generator=g, device=dev, dtype=torch.float32) * std + mean).to(torch.bfloat16)

    H, I = cfg.hidden, cfg.intermediate
    layers = []
    for l in range(MODEL_LAYERS):
        s = 1000 + 10 * l
        layers.append({"w_qkv": draw((cfg.qkv_dim, H), 0.02, 0.0, s), "w_o": draw((H, cfg.n_heads * cfg.head_dim), 0.02, 0.0, s + 1),
                       "w_gate_up": draw((2 * I, H), 0.02, 0.0, s + 2), "w_down": draw((H, I), 0.02, 0.0, s + 3),
                       "g_attn": draw((H,), 0.1, 1.0, s + 4), "g_mlp": draw((H,), 0.1, 1.0, s + 5)})
    model = {"layers": layers, "tok_embeddings": draw((MODEL_VOCAB, H), 1.0, 0.0, 1), "g_final": draw((H,), 0.1, 1.0, 2),
             "lm_head": draw((MODEL_VOCAB, H), 0.02, 0.0, 3)}
    g.manual_seed(4)
    tok = torch.randint(0, MODEL_VOCAB, (cfg.B, cfg.S), generator=g, device=dev, dtype=torch.int64)
    pos = torch.arange(cfg.S, device=dev, dtype=torch.int64).expand(cfg.B, cfg.S).contiguous()
    lc = lib_config(L, cfg, torch)
    logits = torch.empty((cfg.B, cfg.S, MODEL_VOCAB), device=dev, dtype=torch.bfloat16)
    import ctypes
    c = lc.to_c()
    ws = torch.empty(L.load().llama_model_workspace_bytes(ctypes.byref(c), MODEL_VOCAB, cfg.B, cfg.S),
                     dtype=torch.uint8, device=dev)
    for _ in range(args.warmup):
        L.llama_model_forward(lc, model, tok, pos, out=logits, workspace=ws)
    torch.cuda.synchronize()
    L.profile_begin(args.steps * MODEL_LAYERS)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        L.llama_model_forward(lc, model, tok, pos, out=logits, workspace=ws)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    stages = L.profile_end()
    assert torch.isfinite(logits[:, -1].float()).all().item()
    return wall * 1e3 / args.steps, stages


def run_model_record(args):
    import torch

    import transformer_layer_forward_amd as L
    from synth_inputs import CONFIGS
    torch.cuda.set_device(0)
    cfg = CONFIGS["llama32_1b_prefill"]
    ms, stages = run_model(L, torch, None, cfg, args)
    per_layer = {k: v[0] / v[1] for k, v in stages.items()}
    layers_ms = MODEL_LAYERS * sum(per_layer.values())
    M, H, I, d = cfg.M, cfg.hidden, cfg.intermediate, cfg.head_dim
    gate_up_ms = per_layer["gate_up_silu"]
    achieved = 2.0 * M * (2 * I) * H / (gate_up_ms / 1e3) / 1e12
    flops = (MODEL_LAYERS * (gemm_flops_per_token(cfg) * M + 4.0 * cfg.B * cfg.n_heads * d * cfg.S * (cfg.S + 1) / 2)
             + 2.0 * M * MODEL_VOCAB * H)
    rec = {
        "metric": f"model tokens/s (Llama-3.2-1B-shaped stack: embeddings, {MODEL_LAYERS} decoder layers, final "
                  f"RMSNorm, {H}->{MODEL_VOCAB} output projection; bf16 prefill)",
        "value": round(M / (ms / 1e3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "ms_per_step": round(ms, 4),
        "data": "synthetic (weights and token ids from torch's seeded device generator)",
        "config": {"workload": f"Llama-3.2-1B-shaped model stack, {MODEL_LAYERS} layers, vocab {MODEL_VOCAB}",
                   "B": cfg.B, "S": cfg.S, "hidden": H, "n_heads": cfg.n_heads, "n_kv_heads": cfg.n_kv_heads,
                   "head_dim": d, "intermediate": I, "layers": MODEL_LAYERS, "vocab": MODEL_VOCAB},
        "model_tflops": round(flops / (ms / 1e3) / 1e12, 1),
        "layers_ms": round(layers_ms, 4),
        "embedding_norm_head_ms": round(ms - layers_ms, 4),
        "per_layer_stages_ms": {k: round(v, 4) for k, v in per_layer.items()},
        "roofline": {"kernel": "gemm_bf16_mfma32_silu_persist_kernel (fused gate_up + silu*up), per layer",
                     "bound": "mfma", "achieved": round(achieved, 1), "peak": MI355X_BF16_DENSE_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / MI355X_BF16_DENSE_TFLOPS, 4), "traffic": None},
        "cpu_baseline": None,
    }
    print(json.dumps(rec), flush=True)


def decode_inputs(L, torch, np, cfg, W):
    """Decode step inputs on the device: hidden [B,1,H], positions [B] integer-uniform on [1024, ctx),
    and K/V caches [B, ctx, n_kv, d] of N(0,1) values drawn by torch's seeded device generator (the
    caches are 2 GiB; their values do not change the work)."""
    from synth_inputs import make_decode_positions, make_hidden
    dev = "cuda:0"
    x = torch.from_numpy(np.ascontiguousarray(make_hidden(cfg, seed=0)).view(np.int16)).to(dev).view(torch.bfloat16)
    pos_np = make_decode_positions(cfg, seed=0)
    pos = torch.from_numpy(pos_np).to(dev)
    g = torch.Generator(device=dev)
    g.manual_seed(8)
    shape = (cfg.B, cfg.ctx, cfg.n_kv_heads, cfg.head_dim)
    kc = torch.randn(shape, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    g.manual_seed(9)
    vc = torch.randn(shape, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    return x, pos, pos_np, kc, vc


def decode_bytes(cfg, pos_np):
    """Algorithmic HBM bytes of one decode layer call: every weight once, K and V of slots 0..pos_b of every
    sequence, the new K/V slot writes, hidden in and out."""
    kv_read = int(sum(int(p) + 1 for p in pos_np)) * cfg.n_kv_heads * cfg.head_dim * 2 * 2
    kv_write = cfg.B * cfg.n_kv_heads * cfg.head_dim * 2 * 2
    io = 2 * cfg.B * cfg.hidden * 2
    return weight_bytes(cfg), kv_read, kv_write + io


def run_decode(L, torch, np, cfg, W, steps, warmup, cold):
    """Decode layer calls. cold=True: before each call a 512 MiB buffer is read (outside the timed region)
    so that L2 and the Infinity Cache start cold, and each call is timed by HIP events on the launch
    stream; the median is reported. cold=False: `steps` calls back to back, wall clock. The timed calls
    record no stage events (each event the library records between two kernels of a 0.36 ms call adds a
    few microseconds); the stage times come from a second pass of `steps` calls, made the same way, with
    the library's stage events on."""
    dev = "cuda:0"
    x, pos, pos_np, kc, vc = decode_inputs(L, torch, np, cfg, W)
    lc = lib_config(L, cfg, torch)
    ws = torch.empty(L.layer_workspace_bytes(lc, cfg.B, 1, cfg.ctx), dtype=torch.uint8, device=dev)
    out = torch.empty_like(x)

    def call():
        L.llama_layer_forward(lc, W, x, pos, kv_seq_len=cfg.ctx, k_cache=kc, v_cache=vc, out=out, workspace=ws)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    flush = cache_flusher(torch, dev) if cold else None
    stream = torch.cuda.current_stream()

    def timed():
        if cold:
            times = []
            for _ in range(steps):
                flush()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                call()
                e1.record(stream)
                e1.synchronize()
                times.append(e0.elapsed_time(e1))
            times.sort()
            return times[len(times) // 2], times[len(times) // 10], times[(9 * len(times)) // 10]
        t0 = time.perf_counter()
        for _ in range(steps):
            call()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / steps, None, None

    ms, p10, p90 = timed()
    L.profile_begin(steps)
    timed()
    stages = L.profile_end()
    assert torch.isfinite(out.float()).all().item()
    return ms, p10, p90, stages, pos_np


def decode_summary(cfg, ms, p10, p90, stages, pos_np, cold):
    wb, kvb, other = decode_bytes(cfg, pos_np)
    tot = wb + kvb + other
    attn_ms = stage_ms(stages, "attention")
    gemm_ms = sum(stage_ms(stages, k) for k in ("qkv_proj", "o_proj_residual", "gate_up_silu", "down_residual"))
    rec = {"workload": f"Llama-3-8B-shaped decode step, B={cfg.B} against [{cfg.B}, {cfg.ctx}, {cfg.n_kv_heads}, "
                       f"{cfg.head_dim}] bf16 K/V caches, positions uniform on [1024, {cfg.ctx})",
           "timing": ("median of per-call HIP events, 512 MiB read before each call (cache-cold)" if cold
                      else "back-to-back calls, wall clock")
                     + "; stage times from a second pass with the library's stage events",
           "ms_per_step": round(ms, 4), "tokens_per_s": round(cfg.B / (ms / 1e3), 1),
           "algorithmic_bytes": tot, "hbm_gbs": round(tot / (ms / 1e3) / 1e9, 1),
           "hbm_frac": round(tot / (ms / 1e3) / 1e9 / MI355X_HBM_GBS, 4),
           "attention_kv_gbs": round(kvb / (attn_ms / 1e3) / 1e9, 1),
           "gemm_weight_gbs": round(wb / (gemm_ms / 1e3) / 1e9, 1),
           "stages_ms": {k: round(v[0] / v[1], 4) for k, v in stages.items()}}
    if p10 is not None:
        rec["p10_ms"], rec["p90_ms"] = round(p10, 4), round(p90, 4)
    return rec


def main():
    args = parse()
    if args.rocpd_summary:
        rocpd_summary(args.rocpd_summary)
        return
    if args.pmc_summary:
        pmc_summary(*args.pmc_summary)
        return
    if args.counter_summary:
        counter_summary(args.counter_summary)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (data parallel, each MI355X "
              "would run the whole layer on its own sequences). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import transformer_layer_forward_amd as L
    from synth_inputs import CONFIGS, make_weights

    if args.workload == MODEL_WORKLOAD:
        run_model_record(args)
        return
    chunk = args.workload in CHUNK_SHAPES
    varlen = args.workload == VARLEN_WORKLOAD
    lens = None
    if chunk:
        from synth_inputs import scaled
        nb, ns, chunk_start = CHUNK_SHAPES[args.workload]
        cfg = scaled(CONFIGS[WORKLOAD], name=args.workload, S=ns, **({"B": nb} if nb else {}))
    elif varlen:
        from synth_inputs import scaled
        lens = varlen_lengths(np)
        cfg = scaled(CONFIGS[WORKLOAD], name=VARLEN_WORKLOAD, B=1, S=sum(lens))
    else:
        cfg = CONFIGS[args.workload]
    dev = "cuda:0"
    torch.cuda.set_device(0)
    W_bits = make_weights(cfg, seed=0)

    def to_dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    W = {k: to_dev(v) for k, v in W_bits.items()}
    rc = cfg.rope
    H, I, d = cfg.hidden, cfg.intermediate, cfg.head_dim
    common = {"n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": True,
              "scaling": "weak", "vs_baseline": None, "dtype": "bf16"}
    shape = {"hidden": H, "n_heads": cfg.n_heads, "n_kv_heads": cfg.n_kv_heads, "head_dim": d, "intermediate": I,
             "rope": rc.type, "rope_theta": rc.theta}

    if cfg.decode:
        ms, p10, p90, stages, pos_np = run_decode(L, torch, np, cfg, W, args.steps, args.warmup, cold=False)
        summ = decode_summary(cfg, ms, p10, p90, stages, pos_np, cold=False)
        wb, kvb, other = decode_bytes(cfg, pos_np)
        attn_ms = stage_ms(stages, "attention")
        rec = {"metric": "decode-step tokens/s (Llama-3-8B shape, bf16, B=64, KV cache) + HBM GB/s",
               "value": summ["tokens_per_s"], "unit": "tokens/s", **common, "ms_per_step": round(ms, 4),
               "data": "synthetic (seeded N(0,1) hidden and caches, N(0,0.02) weights, 1+N(0,0.1) gains)",
               "config": {"workload": summ["workload"], "B": cfg.B, "ctx": cfg.ctx, **shape},
               "hbm_gbs": summ["hbm_gbs"], "stages_ms": summ["stages_ms"],
               "roofline": {"kernel": "attention stage (attn_decode_bal_kernel + combine; the cache append rides in the QKV reduce)",
                            "bound": "hbm", "achieved": round(kvb / (attn_ms / 1e3) / 1e9, 1),
                            "peak": MI355X_HBM_GBS, "unit": "GB/s",
                            "frac": round(kvb / (attn_ms / 1e3) / 1e9 / MI355X_HBM_GBS, 4), "traffic": None},
               "cold": decode_summary(cfg, *run_decode(L, torch, np, cfg, W, args.steps, 2, cold=True), cold=True),
               "cpu_baseline": None}
        print(json.dumps(rec), flush=True)
        if args.copy_calibration:
            copy_calibration()
        return

    if chunk:
        ms_per_step, stages = run_chunk(L, torch, np, cfg, W, args, chunk_start)
        timed_gate_up = None
        x_bits = None
    elif varlen:
        ms_per_step, stages = run_varlen(L, torch, np, cfg, W, args, lens)
        timed_gate_up = None
        x_bits = None
    else:
        ms_per_step, stages, timed_gate_up, x_bits = run_prefill(L, torch, np, cfg, W, args)
    tokens = cfg.B * cfg.S
    value = tokens / (ms_per_step / 1e3)
    M = cfg.M
    gate_up_flops = 2.0 * M * (2 * I) * H
    # the roofline's kernel time: HIP events around gate_up in the timed calls (headline prefill), else the
    # stage pass of the same calls
    gate_up_ms = (timed_gate_up[0] / timed_gate_up[1] if timed_gate_up is not None
                  else stage_ms(stages, "gate_up_silu"))
    achieved = gate_up_flops / (gate_up_ms / 1e3) / 1e12
    start = chunk_start if chunk else 0
    # QK^T and PV over the visible (query, key) pairs: query s sees keys 0 .. start + s
    if varlen:
        attn_flops = 4.0 * cfg.n_heads * d * sum(n * (n + 1) / 2 for n in lens)
    else:
        attn_flops = 4.0 * cfg.B * cfg.n_heads * d * (cfg.S * start + cfg.S * (cfg.S + 1) / 2)
    gemm_flops = gemm_flops_per_token(cfg) * M
    gemm_ms = sum(stage_ms(stages, k) for k in ("qkv_proj", "o_proj_residual", "gate_up_silu", "down_residual"))
    norm_bytes = 2 * (2 * M * H * 2 + H * 2)
    norm_ms = sum(stage_ms(stages, k) for k in ("rmsnorm_attn", "rmsnorm_mlp"))
    name = {"llama3_8b_prefill": "Llama-3-8B-shaped decoder layer, bf16 prefill, causal",
            "llama32_1b_prefill": "Llama-3.2-1B-shaped decoder layer, bf16 prefill, causal",
            "llama3_8b_long_llama3rope": "Llama-3-8B-shaped decoder layer, bf16 32k prefill, causal, "
                                         "Llama3 RoPE scaling",
            **{w: f"Llama-3-8B-shaped decoder layer, bf16 chunked prefill: {cfg.S} new tokens per "
                  f"sequence on a {start}-token cached prefix ({CHUNK_CTX}-slot KV cache)" for w in CHUNK_SHAPES},
            VARLEN_WORKLOAD: f"Llama-3-8B-shaped decoder layer, bf16 varlen packed prefill: {len(lens or [])} "
                             f"sequences of 64-2048 tokens packed into {cfg.S} tokens, causal within each"
            }[args.workload]
    metric = ("decoder-layer tokens/s (Llama-3-8B shape, bf16) + attention MFMA util %"
              if args.workload == WORKLOAD else f"decoder-layer tokens/s ({name})")
    rec = {
        "metric": metric,
        "value": round(value, 1),
        "unit": "tokens/s",
        **common,
        "ms_per_step": round(ms_per_step, 4),
        "data": ("synthetic (seeded N(0,1) hidden" + (" and cache prefix" if chunk else "")
                 + ", N(0,0.02) weights, 1+N(0,0.1) gains)"),
        "config": {"workload": name, "B": cfg.B, "S": cfg.S, **shape, "tokens_per_step": tokens,
                   **({"prefix": start, "ctx": CHUNK_CTX} if chunk else {}),
                   **({"seq_lens": lens} if varlen else {})},
        "attention_mfma_util_pct": round(100.0 * attn_flops / (stage_ms(stages, "attention") / 1e3) / 1e12
                                         / MI355X_BF16_DENSE_TFLOPS, 2),
        "gemm_mfma_util_pct": round(100.0 * gemm_flops / (gemm_ms / 1e3) / 1e12 / MI355X_BF16_DENSE_TFLOPS, 2),
        "rmsnorm_hbm_gbs": round(norm_bytes / (norm_ms / 1e3) / 1e9, 1),   # in-layer (warm) stages
        "stages_ms": {k: round(v[0] / v[1], 4) for k, v in stages.items()},
        "roofline": {
            "kernel": GATE_UP_KERNEL.get(args.workload, "gemm_bf16_mfma32_silu_persist_kernel")
                      + " (fused gate_up + silu*up)",
            "bound": "mfma",
            "achieved": round(achieved, 1),
            "peak": MI355X_BF16_DENSE_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / MI355X_BF16_DENSE_TFLOPS, 4),
            "traffic": measured_traffic() if args.workload == WORKLOAD else None,
        },
        "cpu_baseline": None,
    }
    if args.workload == WORKLOAD:
        rec["rmsnorm_cold"] = rmsnorm_cold(L, torch, np, cfg, W)
    if args.workload == WORKLOAD and not args.no_decode:
        dcfg = CONFIGS["llama3_8b_decode"]      # same 8B weights (same seed and shapes)
        rec["decode"] = decode_summary(dcfg, *run_decode(L, torch, np, dcfg, W, 30, 3, cold=True), cold=True)
    if args.workload == WORKLOAD and not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(cfg, W_bits, x_bits, args.cpu_sample_tokens)
    print(json.dumps(rec), flush=True)
    if args.copy_calibration:
        copy_calibration()


if __name__ == "__main__":
    main()
