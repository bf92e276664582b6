"""Scalar-loop twin of the oracle for tiny shapes.

TEST INFRASTRUCTURE ONLY (same import rule as oracle/ref.py). Written
independently of ref.py: plain Python floats and index loops, no NumPy
arithmetic, so that a vectorisation or indexing mistake in either one shows up
as a disagreement. Each function restates its passage (sources as in ref.py).
"""
from __future__ import annotations

import math


def rmsnorm_row(x, g, eps):
    """[llama3] §3.1 / [nju] "编码实现RMSNorm": x_i * rsqrt(mean(x^2) + eps) * g_i."""
    n = len(x)
    acc = 0.0
    for v in x:
        acc += v * v
    r = 1.0 / math.sqrt(acc / n + eps)
    return [x[i] * r * g[i] for i in range(n)]


def matvec(w, x):
    """y_n = sum_k W[n][k] x[k] (nn.Linear without bias; W rows are output features)."""
    return [sum(w[n][kk] * x[kk] for kk in range(len(x))) for n in range(len(w))]


def inv_freq(d, rope, L):
    """Frequencies per pair, restated from [verl] §1 and [meta-qa] think §3 (see ref.py)."""
    base = rope.theta
    if rope.type == "dynamic_ntk" and L > rope.original_max_pos:
        base = base * ((rope.factor * L / rope.original_max_pos) - (rope.factor - 1)) ** (d / (d - 2))
    out = []
    for i in range(d // 2):
        f = 1.0 / (base ** ((2 * i) / d))
        if rope.type == "linear":
            f = f / rope.factor
        elif rope.type == "llama3":
            wavelen = 2 * math.pi / f
            hi_wl = rope.original_max_pos / rope.high_freq_factor
            lo_wl = rope.original_max_pos / rope.low_freq_factor
            if wavelen < hi_wl:
                pass
            elif wavelen > lo_wl:
                f = f / rope.factor
            else:
                sm = (rope.original_max_pos / wavelen - rope.low_freq_factor) / (
                    rope.high_freq_factor - rope.low_freq_factor)
                f = (1 - sm) * (f / rope.factor) + sm * f
        out.append(f)
    return out


def rope_vec(x, pos, freqs, interleaved):
    """Rotate one head vector by position pos ([nju] rotate_half; [meta-qa] complex pairs)."""
    d = len(x)
    y = list(x)
    for j in range(d // 2):
        a_i, b_i = (2 * j, 2 * j + 1) if interleaved else (j, j + d // 2)
        ang = pos * freqs[j]
        c, s = math.cos(ang), math.sin(ang)
        y[a_i] = x[a_i] * c - x[b_i] * s
        y[b_i] = x[b_i] * c + x[a_i] * s
    return y


def attend(q, keys, vals):
    """One query against a list of keys/values: softmax(q.k/sqrt(d)) weighted sum."""
    d = len(q)
    sc = [sum(q[t] * k[t] for t in range(d)) / math.sqrt(d) for k in keys]
    m = max(sc)
    e = [math.exp(s - m) for s in sc]
    z = sum(e)
    return [sum(e[j] * vals[j][t] for j in range(len(keys))) / z for t in range(d)]


def layer_prefill(cfg, W, x, positions, L):
    """Decoder layer over x[b][s][hidden] (nested lists of floats); W values nested lists.

    Returns out[b][s][hidden] and o[b][s][n_h*d]."""
    nh, nkv, d, I = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim, cfg.intermediate
    grp = nh // nkv
    fr = inv_freq(d, cfg.rope, L)
    il = cfg.rope.interleaved
    out_all, o_all = [], []
    for b in range(len(x)):
        S = len(x[b])
        Q, K, V = [], [], []
        for s in range(S):
            xn = rmsnorm_row(x[b][s], W["g_attn"], cfg.eps)
            row = matvec(W["w_qkv"], xn)
            p = positions[b][s]
            Q.append([rope_vec(row[h * d:(h + 1) * d], p, fr, il) for h in range(nh)])
            K.append([rope_vec(row[nh * d + c * d: nh * d + (c + 1) * d], p, fr, il) for c in range(nkv)])
            V.append([row[(nh + nkv) * d + c * d: (nh + nkv) * d + (c + 1) * d] for c in range(nkv)])
        outs, os_ = [], []
        for i in range(S):
            o = []
            for h in range(nh):
                c = h // grp
                o += attend(Q[i][h], [K[j][c] for j in range(i + 1)], [V[j][c] for j in range(i + 1)])
            hres = [a + bb for a, bb in zip(x[b][i], matvec(W["w_o"], o))]
            hn = rmsnorm_row(hres, W["g_mlp"], cfg.eps)
            gu = matvec(W["w_gate_up"], hn)
            act = [gu[t] / (1 + math.exp(-gu[t])) * gu[I + t] for t in range(I)]
            dn = matvec(W["w_down"], act)
            outs.append([a + bb for a, bb in zip(hres, dn)])
            os_.append(o)
        out_all.append(outs)
        o_all.append(os_)
    return out_all, o_all
