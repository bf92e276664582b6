"""Mutation check of the oracle's pins (run by hand: ``python tests/oracle_mutations.py``).

Plants one plausible mistake at a time (a dropped term, a wrong sign or index, a
transposed operand, a moved threshold) in a temporary copy of oracle/ref.py and
runs tests/test_oracle_pins.py and tests/test_oracle_library_pins.py against that copy. Every mutant must make at
least one pin fail; the script exits non-zero if any survives. Takes ~15 minutes
on 8 cores, so it is not part of the collected suite.
"""
import os, shutil, subprocess, sys, tempfile
REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = open(f"{REPO}/oracle/ref.py").read()
MUTS = [
    ("rmsnorm eps outside sqrt", "x / np.sqrt(ms + eps)", "x / (np.sqrt(ms) + eps)"),
    ("rmsnorm mean->sum", "np.mean(x * x, axis=-1", "np.sum(x * x, axis=-1"),
    ("rmsnorm gain dropped", "/ np.sqrt(ms + eps) * np.asarray(g, dtype=F64)", "/ np.sqrt(ms + eps)"),
    ("theta exponent d-1", "f = theta ** (-(2.0 * i) / d)", "f = theta ** (-(2.0 * i) / (d - 1))"),
    ("theta exponent i not 2i", "f = theta ** (-(2.0 * i) / d)", "f = theta ** (-(1.0 * i) / d)"),
    ("linear multiplies", "return f / rope.factor\n    if t == \"llama3\"", "return f * rope.factor\n    if t == \"llama3\""),
    ("ntk exponent", "** (d / (d - 2.0))", "** (d / (d - 1.0))"),
    ("ntk ge", "if L > orig:", "if L >= orig - 1:"),
    ("ntk off by one", "if L > orig:", "if L > orig + 1:"),
    ("llama3 interp swapped", "(1.0 - s) * f[j] / rope.factor + s * f[j]", "s * f[j] / rope.factor + (1.0 - s) * f[j]"),
    ("llama3 band edges swapped", "if lam[j] < lam_hi:", "if lam[j] < lam_lo:"),
    ("llama3 interpolation linear in wavelength", "s = (orig / lam[j] - rope.low_freq_factor) / (rope.high_freq_factor - rope.low_freq_factor)", "s = (lam_lo - lam[j]) / (lam_lo - lam_hi)"),
    ("llama3 interpolation on theta not f", "out[j] = (1.0 - s) * f[j] / rope.factor + s * f[j]", "out[j] = f[j] / ((1.0 - s) * rope.factor + s)"),
    ("ntk base without the factor", "theta * (rope.factor * L / orig - (rope.factor - 1.0))", "theta * (L / orig)"),
    ("ntk exponent dropped", "** (d / (d - 2.0))", "** 1.0"),
    ("rope sign half", "out[..., :h] = a * c - b * s", "out[..., :h] = a * c + b * s"),
    ("rope sign half2", "out[..., h:] = b * c + a * s", "out[..., h:] = b * c - a * s"),
    ("rope sign interleaved", "out[..., 0::2] = a * c - b * s", "out[..., 0::2] = a * c + b * s"),
    ("interleaved uses half pairs", "a, b = x[..., 0::2], x[..., 1::2]", "a, b = x[..., :h], x[..., h:]"),
    ("scale 1/d", "scale = 1.0 / math.sqrt(d)", "scale = 1.0 / d"),
    ("mask off by one", "s = np.where(cols > rows, -np.inf, s)", "s = np.where(cols >= rows + 2, -np.inf, s)"),
    ("gqa mapping modulo", "            c = h // g\n            kk", "            c = h % nkv\n            kk"),
    ("one-query gqa modulo", "        c = h // g\n        s = (keys", "        c = h % nkv\n        s = (keys"),
    ("one-query scale", "s = (keys[:, c, :] @ q[h]) / math.sqrt(d)", "s = (keys[:, c, :] @ q[h])"),
    ("silu sign", "z / (1.0 + np.exp(-z))", "z / (1.0 + np.exp(z))"),
    ("silu on up", "silu(gu[..., :intermediate]) * gu[..., intermediate:]", "gu[..., :intermediate] * silu(gu[..., intermediate:])"),
    ("split k/v swapped", "    k = qkv[..., qd:qd + kd].reshape(*lead, n_kv_heads, head_dim)\n    v = qkv[..., qd + kd:]", "    v = qkv[..., qd:qd + kd].reshape(*lead, n_kv_heads, head_dim)\n    k = qkv[..., qd + kd:]"),
    ("linear transposed", "@ np.asarray(w, dtype=F64).T", "@ np.asarray(w, dtype=F64).T[::-1]"),
    ("attn residual dropped", "    h = x + attn_proj\n    hn", "    h = attn_proj\n    hn"),
    ("mlp residual dropped", "    out = h + mlp_out\n    return", "    out = mlp_out + x\n    return"),
    ("second norm uses g_attn", "hn = rmsnorm(h, W[\"g_mlp\"], cfg.eps)\n    act", "hn = rmsnorm(h, W[\"g_attn\"], cfg.eps)\n    act"),
    ("v rotated", "o = attention_prefill(qr, kr, v, causal=True)", "o = attention_prefill(qr, kr, rope_rotate(v, np.asarray(position_ids)[..., None], rope_frequencies(cfg.head_dim, cfg.rope, kv_seq_len)), causal=True)"),
    ("decode new key unrotated", "        K[p] = kr\n", "        K[p] = k\n"),
    ("decode attends p slots", "K = cache_row_k(b)[:p + 1].copy()\n        V = cache_row_v(b)[:p + 1].copy()", "K = cache_row_k(b)[:p + 2].copy()\n        V = cache_row_v(b)[:p + 2].copy()"),
    ("softmax sum over all rows", "return p / np.sum(p, axis=-1, keepdims=True)", "return p / np.sum(p)"),
    ("chunk attends one slot too many", "o[b, s] = attention_one_query(np.asarray(q[b, s], dtype=F64), K[b, :p + 1], V[b, :p + 1])", "o[b, s] = attention_one_query(np.asarray(q[b, s], dtype=F64), K[b, :p + 2], V[b, :p + 2])"),
    ("chunk v not written", "            V[b, int(positions[b, s])] = v_new[b, s]\n", "            pass\n"),
    ("chunk writes slot by index", "            K[b, int(positions[b, s])] = k_new[b, s]", "            K[b, s] = k_new[b, s]"),
    ("chunk layer unrotated k", "o, K, V = attention_chunk(qr, kr, v, np.asarray(position_ids), cache_k, cache_v)", "o, K, V = attention_chunk(qr, k, v, np.asarray(position_ids), cache_k, cache_v)"),
    ("chunk attn residual dropped", "    h = attn_proj + x\n", "    h = attn_proj\n"),
    ("chunk second norm uses g_attn", "hn = rmsnorm(h, W[\"g_mlp\"], eps=cfg.eps)", "hn = rmsnorm(h, W[\"g_attn\"], eps=cfg.eps)"),
    ("varlen ignores boundaries", "out[a:b] = attention_prefill(q[None, a:b], k[None, a:b], v[None, a:b])[0]", "out[a:b] = attention_prefill(q[None, :b], k[None, :b], v[None, :b])[0][a:b]"),
    ("varlen layer mlp residual", "\"out\": mlp_out + h}", "\"out\": mlp_out + x}"),
    ("varlen attn residual dropped", "h = np.add(x, attn_proj)", "h = np.add(0.0, attn_proj)"),
    ("varlen second norm uses g_attn", "hn = rmsnorm(h, g=W[\"g_mlp\"], eps=cfg.eps)", "hn = rmsnorm(h, g=W[\"g_attn\"], eps=cfg.eps)"),
    ("embedding row off by one", "return np.asarray(table, dtype=F64)[np.asarray(tokens)]", "return np.asarray(table, dtype=F64)[np.asarray(tokens) - 1]"),
    ("model final norm dropped", "hn = rmsnorm(h, M[\"g_final\"], cfg.eps)", "hn = h"),
    ("model layers reversed", "for W in M[\"layers\"]:", "for W in M[\"layers\"][::-1]:"),
    ("rows path second norm eps", "hn = rmsnorm(h, W[\"g_mlp\"], cfg.eps)\n            act", "hn = rmsnorm(h, W[\"g_mlp\"], 0.1)\n            act"),
]
results = []
for name, a, b in MUTS:
    n = SRC.count(a)
    if n != 1:
        results.append((name, f"PATTERN COUNT {n}"))
        continue
    d = tempfile.mkdtemp(prefix="oracle_mut_")
    for f in ("synth_inputs.py", "pytest.ini"):
        shutil.copy(f"{REPO}/{f}", d)
    shutil.copytree(f"{REPO}/oracle", f"{d}/oracle")
    shutil.copytree(f"{REPO}/tests", f"{d}/tests", ignore=shutil.ignore_patterns("__pycache__", "test_gpu*", "test_abi.py", "test_zz*"))
    open(f"{d}/oracle/ref.py", "w").write(SRC.replace(a, b))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu", "-p", "no:cacheprovider",
                        "tests/test_oracle_pins.py", "tests/test_oracle_library_pins.py"],
                       cwd=d, capture_output=True, text=True)
    caught = r.returncode != 0
    failing = [l for l in r.stdout.splitlines() if l.startswith("FAILED")]
    results.append((name, "caught " + (failing[0][7:90] if failing else r.stdout.splitlines()[-1][:80]) if caught else "MISSED"))
    shutil.rmtree(d)
for n, s in results:
    print(f"{n:40s} {s}")
survivors = [n for n, s in results if not s.startswith("caught")]
print(f"{len(results) - len(survivors)}/{len(results)} mutants caught")
sys.exit(1 if survivors else 0)
