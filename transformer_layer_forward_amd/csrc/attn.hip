// Grouped-query causal attention: prefill (flash-style, matrix cores) and KV-cache decode.
//
// Semantics (verl "parallel_attention.py" §2 eager attention; nanotron "模型层" §9.3
// flash_attn_func(causal=True); llama3 结构详解 §3.2 GQA and KV cache):
//   o[b,i,h] = sum_{j<=i} softmax_j(q'_{b,i,h} . k'_{b,j,c} / sqrt(d)) v_{b,j,c},  c = h / (n_h/n_kv).
// repeat_kv is never materialised: one workgroup serves every query head of a K/V head.
//
// Prefill kernels (bf16, d in {64, 128}): a workgroup owns (sequence b, kv head c, 64 queries) and
// runs 2 waves per query head of the group (32 queries each). Each 64-key K tile and V tile is
// staged once in LDS (double-buffered) and read by all waves of the group. Scores are formed
// transposed, S^T = K Q^T, with K as the MFMA A operand and Q (in registers) as B: the output
// fragment then holds, per lane, one query column and a few keys, which after the fp32 online
// softmax (exp2 with log2(e)/sqrt(d) folded into the scale) is exactly the B-operand layout of
// O^T += V^T P^T. Two variants: with q and k already rotated (the layer, varlen and chunked paths:
// attn_prefill_m32_kernel, on 32x32x16 matrix ops) K and V go global -> LDS by direct loads, V stays
// [key][d] and its V^T operand comes from transposing LDS reads; with RoPE applied on load (the
// standalone entry point: attn_prefill_mfma_kernel, 16x16x32) tiles pass through registers, are
// rotated there, and V is transposed into LDS as [d][key] while it is stored.
// Rows are XOR-swizzled so the lanes of an operand read hit distinct banks.
// Causality: query block qb only visits key tiles 0..qb; only the diagonal tile is masked.
// Blocks are issued heaviest-first (largest qb first); consecutive blocks of one qb level
// cycle over (b, c), so one (b, c) pair keeps landing on the same XCD and its K/V stays in
// that XCD's L2.
//
// Decode (bf16, d in {64, 128}, n_h/n_kv in {1, 2, 4, 8}): an append kernel writes the new key
// (rotated) and value to slot pos[b]; the split kernel cuts each sequence's visible slots into
// 128-key blocks shared out evenly over a fixed number of workgroups per (b, c), whose 4 waves step
// through 32-key tiles with the next tiles' K and V already loading into registers. Q K^T uses the
// matrix cores with K streamed from HBM straight into operand registers (every K element is used
// once); P V runs on the matrix cores too, P^T straight from the score accumulators and V^T read
// transposed from a wave-private LDS copy of the tile. Waves merge through LDS; each workgroup writes
// (max, sum, o) to workspace and a combine kernel merges the splits with the log-sum-exp rule.
//
// Generic kernels (fp32, or any even d <= 256): one wave per query, lanes over d, exact two-level
// online softmax; used for the fp32 configuration and for head sizes the matrix-core kernels
// do not cover.
#include "common.h"
#include "decode_partition.h"

namespace ll {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kSlack = 8.f;  // lazy-rescale threshold of the prefill kernel, in log2 units

// 2^x with the hardware v_exp_f32 (no denormal range fix-up): exp2(-inf) = 0, and results below
// 2^-126 (which only arise for weights negligible against the running sum) flush to 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ------------------------------------------------------------------ RoPE helpers (device)
// Rotate the 8 values f[] (dims d0 .. d0+7 of a head) given their partners g[] (dims d0 + d/2 ..),
// half-split pairing: x' = x c - y s, y' = y c + x s, with j = d0 + e.
__device__ __forceinline__ void rope8_half(float* f, float* g, const float2* __restrict__ cs_row, int j0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float2 t = cs_row[j0 + e];
        const float x = f[e], y = g[e];
        f[e] = x * t.x - y * t.y;
        g[e] = y * t.x + x * t.y;
    }
}

// Interleaved pairing inside one 8-value chunk starting at dim d0 (even): pairs (d0+2i, d0+2i+1).
__device__ __forceinline__ void rope8_inter(float* f, const float2* __restrict__ cs_row, int d0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float2 t = cs_row[(d0 >> 1) + i];
        const float x = f[2 * i], y = f[2 * i + 1];
        f[2 * i] = x * t.x - y * t.y;
        f[2 * i + 1] = y * t.x + x * t.y;
    }
}

// ------------------------------------------------------------------ prefill, matrix cores
template <int D>
struct PrefillCfg {
    static constexpr int BQ = 64, BKV = 64;
    static constexpr int KCH = D / 8;                 // 16-byte chunks per K row
    static constexpr int KC32 = D / 32;               // 32-wide k steps of Q K^T
    static constexpr int DF = D / 16;                 // output fragments along d
    static constexpr int K_ELEMS = BKV * D;
    static constexpr int V_ELEMS = D * BKV;
};

// physical chunk of K row r (D=128: 16 chunks per row; D=64: 8 chunks)
template <int D>
__device__ __forceinline__ int k_phys(int r, int ch) {
    if constexpr (D == 128) return ch ^ (r & 15);
    else return ch ^ ((r & 7) ^ ((r >> 3) & 1));
}
// V^T rows (one per head dimension, 64 keys = 128 B) hold 8 chunks of 16 B. Chunk 4t + g holds keys
// 32t + 4g .. +3 (low 8 B) and 32t + 16 + 4g .. +3 (high 8 B): exactly the 8 keys one lane of the
// P V operand needs, so a fragment is one 16-byte read. Chunks are XOR-swizzled by row so the 16
// lanes of a read (16 rows, same chunk) hit distinct banks.
__device__ __forceinline__ int vt_swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

template <int D, int HPB, bool ROPE, bool IL>
__global__ __launch_bounds__(128 * HPB) void attn_prefill_mfma_kernel(
    const bf16_t* __restrict__ qkv, const int64_t* __restrict__ pos, const float2* __restrict__ cs, int64_t rope_rows,
    bf16_t* __restrict__ out, bf16_t* __restrict__ kc, bf16_t* __restrict__ vc, int64_t ctx, int B, int S, int nh,
    int nkv, float scale_log2) {
    using C = PrefillCfg<D>;
    constexpr int NT = 128 * HPB;
    __shared__ __align__(16) bf16_t sK[2][C::K_ELEMS];
    __shared__ __align__(16) bf16_t sV[2][C::V_ELEMS];

    const int g = nh / nkv;
    const int hchunks = g / HPB;
    const int nqb = (S + C::BQ - 1) / C::BQ;
    const int per_qb = B * nkv * hchunks;
    const int qb = nqb - 1 - static_cast<int>(blockIdx.x) / per_qb;
    int rem = static_cast<int>(blockIdx.x) % per_qb;
    const int hc = rem % hchunks;
    rem /= hchunks;
    const int c = rem % nkv;
    const int b = rem / nkv;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lrow = lane & 15, lgrp = lane >> 4;
    const int h = c * g + hc * HPB + (wave >> 1);
    const int64_t rs = static_cast<int64_t>(nh + 2 * nkv) * D;  // packed row stride
    const bf16_t* qkv_b = qkv + static_cast<int64_t>(b) * S * rs;
    const int64_t* pos_b = pos ? pos + static_cast<int64_t>(b) * S : nullptr;
    const int q0 = qb * C::BQ + (wave & 1) * 32;
    const bool write_cache = (kc != nullptr) && hc == 0;

    // ---- Q fragments: lane holds query q0 + qf*16 + lrow, dims kc*32 + lgrp*8 .. +7
    bf16x8 qfr[2][C::KC32];
#pragma unroll
    for (int qf = 0; qf < 2; ++qf) {
        const int qi = q0 + qf * 16 + lrow;
        const int qs = qi < S ? qi : S - 1;
        const bf16_t* qp = qkv_b + static_cast<int64_t>(qs) * rs + static_cast<int64_t>(h) * D;
        float f[C::KC32][8];
#pragma unroll
        for (int k = 0; k < C::KC32; ++k) unpack8(*reinterpret_cast<const uint4*>(qp + k * 32 + lgrp * 8), f[k]);
        if constexpr (ROPE) {
            const float2* row = cs + clamp_pos(pos_b[qs], rope_rows) * (D / 2);
            if constexpr (IL) {
#pragma unroll
                for (int k = 0; k < C::KC32; ++k) rope8_inter(f[k], row, k * 32 + lgrp * 8);
            } else {
#pragma unroll
                for (int k = 0; k < C::KC32 / 2; ++k) rope8_half(f[k], f[k + C::KC32 / 2], row, k * 32 + lgrp * 8);
            }
        }
#pragma unroll
        for (int k = 0; k < C::KC32; ++k) {
            // fold log2(e)/sqrt(d) into q: the scores come out in log2 units, ready for exp2
#pragma unroll
            for (int e = 0; e < 8; ++e) f[k][e] *= scale_log2;
            uint4 u = pack8(f[k]);
            if (qi >= S) u = make_uint4(0, 0, 0, 0);
            qfr[qf][k] = __builtin_bit_cast(bf16x8, u);
        }
    }

    // ---- tile loader: K jobs (key r, chunk pair), V jobs (4 keys x 8 dims)
    constexpr int KJOBS = C::BKV * C::KCH / 2;
    constexpr int VJOBS = (C::BKV / 4) * C::KCH;
    constexpr int KJ = (KJOBS + NT - 1) / NT;
    constexpr int VJ = (VJOBS + NT - 1) / NT;
    uint4 kr[KJ][2], vr[VJ][4];
    const uint4 zero = make_uint4(0, 0, 0, 0);
    const bf16_t* kbase = qkv_b + static_cast<int64_t>(nh) * D + static_cast<int64_t>(c) * D;
    const bf16_t* vbase = qkv_b + static_cast<int64_t>(nh + nkv) * D + static_cast<int64_t>(c) * D;

    // per-thread source rows of the tile at key 0 (the tile at key0 adds key0 * rs)
    const bf16_t* ksrc[KJ];
    const bf16_t* vsrc[VJ];
#pragma unroll
    for (int i = 0; i < KJ; ++i) {
        const int job = tid + i * NT;
        const int r = job / (C::KCH / 2), ch = job % (C::KCH / 2);
        ksrc[i] = kbase + static_cast<int64_t>(r) * rs + (IL ? 2 * ch : ch) * 8;
    }
#pragma unroll
    for (int i = 0; i < VJ; ++i) {
        const int job = tid + i * NT;
        vsrc[i] = vbase + static_cast<int64_t>((job / C::KCH) * 4) * rs + (job % C::KCH) * 8;
    }

#define AP_LOAD(kt)                                                                                        \
    do {                                                                                                   \
        const int key0_ = (kt) * C::BKV;                                                                   \
        const int64_t toff_ = static_cast<int64_t>(key0_) * rs;                                            \
        /* keys past S (only in the last, masked tile) read the clamped row S-1: finite values, */      \
        /* masked out of the scores, multiplied by zero weights                                  */      \
        _Pragma("unroll") for (int i = 0; i < KJ; ++i) {                                                   \
            const int job = tid + i * NT;                                                                  \
            const int key = key0_ + job / (C::KCH / 2);                                                    \
            if (job < KJOBS) {                                                                             \
                const bf16_t* p = ksrc[i] + toff_ - (key < S ? 0 : static_cast<int64_t>(key - S + 1) * rs); \
                kr[i][0] = *reinterpret_cast<const uint4*>(p);                                             \
                kr[i][1] = *reinterpret_cast<const uint4*>(p + (IL ? 8 : 8 * (C::KCH / 2)));               \
            }                                                                                              \
        }                                                                                                  \
        _Pragma("unroll") for (int i = 0; i < VJ; ++i) {                                                   \
            const int job = tid + i * NT;                                                                  \
            const bf16_t* p = vsrc[i] + toff_;                                                             \
            _Pragma("unroll") for (int t = 0; t < 4; ++t) {                                                \
                const int key = key0_ + (job / C::KCH) * 4 + t;                                            \
                if (job < VJOBS)                                                                           \
                    vr[i][t] = *reinterpret_cast<const uint4*>(                                            \
                        p + static_cast<int64_t>(key < S ? t : S - 1 - (key0_ + (job / C::KCH) * 4)) * rs); \
            }                                                                                              \
        }                                                                                                  \
    } while (0)

#define AP_STORE(kt, st)                                                                                   \
    do {                                                                                                   \
        const int key0_ = (kt) * C::BKV;                                                                   \
        const bool diag_ = write_cache && (kt) == qb;                                                      \
        _Pragma("unroll") for (int i = 0; i < KJ; ++i) {                                                   \
            const int job = tid + i * NT;                                                                  \
            if (job < KJOBS) {                                                                             \
                const int r = job / (C::KCH / 2), ch = job % (C::KCH / 2);                                 \
                const int c0 = IL ? 2 * ch : ch, c1 = IL ? 2 * ch + 1 : ch + C::KCH / 2;                   \
                uint4 a0 = kr[i][0], a1 = kr[i][1];                                                        \
                const int key = key0_ + r;                                                                 \
                if (ROPE && key < S) {                                                                     \
                    float f0[8], f1[8];                                                                    \
                    unpack8(a0, f0);                                                                       \
                    unpack8(a1, f1);                                                                       \
                    const float2* row = cs + clamp_pos(pos_b[key], rope_rows) * (D / 2);                   \
                    if (IL) {                                                                              \
                        rope8_inter(f0, row, c0 * 8);                                                      \
                        rope8_inter(f1, row, c1 * 8);                                                      \
                    } else {                                                                               \
                        rope8_half(f0, f1, row, c0 * 8);                                                   \
                    }                                                                                      \
                    a0 = pack8(f0);                                                                        \
                    a1 = pack8(f1);                                                                        \
                }                                                                                          \
                *reinterpret_cast<uint4*>(&sK[st][r * D + k_phys<D>(r, c0) * 8]) = a0;                     \
                *reinterpret_cast<uint4*>(&sK[st][r * D + k_phys<D>(r, c1) * 8]) = a1;                     \
                if (diag_ && key < S) {                                                                    \
                    const int64_t slot = clamp_pos(pos_b[key], ctx);                                       \
                    bf16_t* dst = kc + ((static_cast<int64_t>(b) * ctx + slot) * nkv + c) * D;             \
                    *reinterpret_cast<uint4*>(dst + c0 * 8) = a0;                                          \
                    *reinterpret_cast<uint4*>(dst + c1 * 8) = a1;                                          \
                }                                                                                          \
            }                                                                                              \
        }                                                                                                  \
        _Pragma("unroll") for (int i = 0; i < VJ; ++i) {                                                   \
            const int job = tid + i * NT;                                                                  \
            if (job < VJOBS) {                                                                             \
                const int r4 = job / C::KCH, ch = job % C::KCH;                                            \
                const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&vr[i][0]);                         \
                const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&vr[i][1]);                         \
                const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&vr[i][2]);                         \
                const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&vr[i][3]);                         \
                const int vq_ = (r4 >> 3) * 4 + (r4 & 3), vh_ = ((r4 >> 2) & 1) * 4;                       \
                _Pragma("unroll") for (int e = 0; e < 8; ++e) {                                            \
                    const int sh = (e & 1) * 16;                                                           \
                    const uint32_t k0 = (w0[e >> 1] >> sh) & 0xffffu, k1 = (w1[e >> 1] >> sh) & 0xffffu;  \
                    const uint32_t k2 = (w2[e >> 1] >> sh) & 0xffffu, k3 = (w3[e >> 1] >> sh) & 0xffffu;  \
                    const int dr = ch * 8 + e;                                                             \
                    *reinterpret_cast<uint2*>(&sV[st][dr * C::BKV + ((vq_ ^ vt_swz(dr)) << 3) + vh_]) =    \
                        make_uint2(k0 | (k1 << 16), k2 | (k3 << 16));                                      \
                }                                                                                          \
                if (diag_) {                                                                               \
                    _Pragma("unroll") for (int t = 0; t < 4; ++t) {                                        \
                        const int key = key0_ + r4 * 4 + t;                                                \
                        if (key < S) {                                                                     \
                            const int64_t slot = clamp_pos(pos_b[key], ctx);                               \
                            bf16_t* dst = vc + ((static_cast<int64_t>(b) * ctx + slot) * nkv + c) * D;     \
                            *reinterpret_cast<uint4*>(dst + ch * 8) = vr[i][t];                            \
                        }                                                                                  \
                    }                                                                                      \
                }                                                                                          \
            }                                                                                              \
        }                                                                                                  \
    } while (0)

    float m_i[2] = {-1e30f, -1e30f}, l_i[2] = {0.f, 0.f};
    f32x4 oacc[C::DF][2];
#pragma unroll
    for (int a = 0; a < C::DF; ++a) oacc[a][0] = oacc[a][1] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nkt = qb + 1;
    AP_LOAD(0);
    AP_STORE(0, 0);
    __syncthreads();
    for (int kt = 0; kt < nkt; ++kt) {
        const int st = kt & 1;
        if (kt + 1 < nkt) AP_LOAD(kt + 1);
        // S^T = K Q^T
        f32x4 sacc[4][2];
#pragma unroll
        for (int kf = 0; kf < 4; ++kf) sacc[kf][0] = sacc[kf][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < C::KC32; ++k) {
#pragma unroll
            for (int kf = 0; kf < 4; ++kf) {
                const int r = kf * 16 + lrow;
                const bf16x8 kfr = *reinterpret_cast<const bf16x8*>(&sK[st][r * D + k_phys<D>(r, k * 4 + lgrp) * 8]);
                sacc[kf][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kfr, qfr[0][k], sacc[kf][0], 0, 0, 0);
                sacc[kf][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kfr, qfr[1][k], sacc[kf][1], 0, 0, 0);
            }
        }
        // scale, mask (diagonal / tail tile only), online softmax per query column
        const bool last = (kt == nkt - 1);
        bf16x8 pfr[2][2];
#pragma unroll
        for (int qf = 0; qf < 2; ++qf) {
            const int qi = q0 + qf * 16 + lrow;
            float s[4][4];
            float mx = -1e30f;
#pragma unroll
            for (int kf = 0; kf < 4; ++kf)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float v = sacc[kf][qf][r];
                    if (last) {
                        const int key = kt * C::BKV + kf * 16 + 4 * lgrp + r;
                        if (key > qi || key >= S) v = -INFINITY;
                    }
                    s[kf][r] = v;
                    mx = fmaxf(mx, v);
                }
            mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
            mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
            // the reference max moves only when the tile max exceeds it by more than kSlack (log2
            // units), so P stays <= 2^kSlack and the O rescale is skipped while no column moves
            const float mnew = (mx > m_i[qf] + kSlack) ? mx : m_i[qf];
            const bool moved = mnew != m_i[qf];
            float ls = 0.f;
            float p[4][4];
#pragma unroll
            for (int kf = 0; kf < 4; ++kf)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    p[kf][r] = fast_exp2(s[kf][r] - mnew);
                    ls += p[kf][r];
                }
            if (__any(moved)) {
                const float alpha = fast_exp2(m_i[qf] - mnew);
                l_i[qf] *= alpha;
#pragma unroll
                for (int a = 0; a < C::DF; ++a) oacc[a][qf] *= alpha;
            }
            m_i[qf] = mnew;
            l_i[qf] += ls;
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                uint4 u;
                u.x = pack_bf16x2(p[2 * t][0], p[2 * t][1]);
                u.y = pack_bf16x2(p[2 * t][2], p[2 * t][3]);
                u.z = pack_bf16x2(p[2 * t + 1][0], p[2 * t + 1][1]);
                u.w = pack_bf16x2(p[2 * t + 1][2], p[2 * t + 1][3]);
                pfr[qf][t] = __builtin_bit_cast(bf16x8, u);
            }
        }
        // O^T += V^T P^T ; V^T fragment rows = dims, k = keys {32t + 4 lgrp + 0..3, 32t + 16 + 4 lgrp + 0..3}
#pragma unroll
        for (int t = 0; t < 2; ++t) {
#pragma unroll
            for (int a = 0; a < C::DF; ++a) {
                const int dr = a * 16 + lrow;
                const bf16x8 vfr =
                    *reinterpret_cast<const bf16x8*>(&sV[st][dr * C::BKV + (((4 * t + lgrp) ^ vt_swz(dr)) << 3)]);
                oacc[a][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vfr, pfr[0][t], oacc[a][0], 0, 0, 0);
                oacc[a][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vfr, pfr[1][t], oacc[a][1], 0, 0, 0);
            }
        }
        if (kt + 1 < nkt) AP_STORE(kt + 1, st ^ 1);
        __syncthreads();
    }
#undef AP_LOAD
#undef AP_STORE

    // ---- normalise and store: lane holds dims a*16 + 4 lgrp + {0..3} of query q0 + qf*16 + lrow
#pragma unroll
    for (int qf = 0; qf < 2; ++qf) {
        float l = l_i[qf];
        l += __shfl_xor(l, 16, 64);
        l += __shfl_xor(l, 32, 64);
        const float inv = 1.f / l;
        const int qi = q0 + qf * 16 + lrow;
        if (qi >= S) continue;
        bf16_t* op = out + (static_cast<int64_t>(b) * S + qi) * nh * D + static_cast<int64_t>(h) * D;
#pragma unroll
        for (int a = 0; a < C::DF; ++a) {
            const f32x4 v = oacc[a][qf];
            *reinterpret_cast<uint2*>(op + a * 16 + 4 * lgrp) =
                make_uint2(pack_bf16x2(v[0] * inv, v[1] * inv), pack_bf16x2(v[2] * inv, v[3] * inv));
        }
    }
}

// ------------------------------------------------------------------ prefill, direct tile loads: helpers
// max / sum over lanes l, l^16, l^32, l^48 (the four 16-lane rows of a wave) with the gfx950 lane
// swaps: vector ALU only, so unlike an LDS-routed shuffle it does not wait behind pending LDS reads
__device__ __forceinline__ float rows_max(float x) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float rows_sum(float x) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

template <int D>
__device__ __forceinline__ int vt_phys(int r, int c) {
    if constexpr (D == 128) return c ^ (2 * (r & 3)) ^ (8 * ((r >> 2) & 1));
    else return c ^ (2 * ((r >> 1) & 1)) ^ (4 * ((r >> 2) & 1));
}

// ------------------------------------------------------------------ prefill, 32x32 matrix ops
// Causal prefill with q and k already rotated: the layer and varlen paths, and chunked prefill over a
// cache prefix (CACHED, with an optional key split, SPLIT). Workgroup = (sequence, kv head, 64 queries)
// with 2 waves per query head of the group (HPB heads), 32 queries per wave. On
// v_mfma_f32_32x32x16_bf16, which issues at full rate from one wave (the 16x16x32 form needs two
// waves per SIMD to keep the matrix core fed).
//  * K and V tiles (64 keys) go global -> LDS by buffer loads straight into LDS (no register staging),
//    both row-major [key][dim] with 16-byte chunks XOR-swizzled by row; double-buffered (in the
//    pipelined loop V runs one tile behind K); every wave of the group reads them.
//  * S^T = K Q^T per 32-key block: A = 32 keys x 16 dims of K (one 16-byte LDS read), B = the wave's
//    resident Q^T (16 dims x 32 queries). The accumulator gives lane l query l % 32 and keys
//    8i + 4(l/32) + r in register 4i + r, so a query's scores sit in two lanes (l, l ^ 32): its row
//    max and row sum take one lane swap (v_permlane32_swap, no LDS round trip).
//  * Registers 8s .. 8s + 7 of a block are exactly the B operand (16 keys x 32 queries) of
//    O^T += V^T P^T for keys 16s .. 16s + 15 of the block, in the key order {4h .. 4h+3, 8+4h .. 8+4h+3}
//    for h = l / 32. The V^T operand (32 dims x those keys) comes from two transposing LDS reads
//    (ds_read_b64_tr_b16: within each 16-lane group, lane i receives element i % 4 of the 8-byte words
//    addressed by lanes 4e + i/4, e = 0..3, so lanes addressing 4 consecutive key rows x 4 dim groups
//    hand every lane 4 consecutive keys of one dim).
//  * Online softmax in log2 units (q pre-scaled by log2(e)/sqrt(d)); score accumulators start at minus
//    the running reference max, which moves only when a tile max exceeds it by more than kSlack (rare:
//    corrected under a wave-uniform branch). Only tiles past the block's smallest visibility limit
//    (the diagonal, over the call's own tokens) are masked.
//  * OCC waves per SIMD (the register budget is 512 / OCC). With PIPE a wave overlaps tile j+1's scores
//    with tile j's softmax (two score sets); without, it runs scores, softmax and P V of one tile in turn
//    (one set, fewer registers), leaving the overlap to the other waves of its SIMD.
//  * CACHED: chunked prefill over a cache prefix (keys are cache slots, query i sees slots
//    0 .. position_ids[b, i], clamped to the cache); SPLIT: the block's key tiles shared out over nsplit
//    workgroups, each writing a (max, sum, unnormalised o) record per query for the combine kernel.
template <int D, int HPB, int OCC, bool PIPE, bool CACHED = false, bool SPLIT = false>
__global__ __launch_bounds__(128 * HPB, OCC) void attn_prefill_m32_kernel(
    const bf16_t* __restrict__ qkv, const int64_t* __restrict__ pos, bf16_t* __restrict__ out, bf16_t* __restrict__ kc,
    bf16_t* __restrict__ vc, int64_t ctx, int B, int S_max, int nh, int nkv, float scale_log2,
    const int* __restrict__ cu, int total, int nsplit, float* __restrict__ part) {
    constexpr int BQ = 64, BKV = 64;
    constexpr int NKF = BKV / 32;                    // 32-key blocks per tile
    constexpr int NKS = BKV / 16;                    // 16-key steps of P V per tile
    constexpr int HS = NKS / 2;
    constexpr int KS = D / 16;                       // 16-wide k steps of Q K^T
    constexpr int KH = KS / 2;
    constexpr int DB = D / 32;                       // 32-dim blocks of O^T
    constexpr int NT = 128 * HPB, NW = NT / 64;
    constexpr int CH = D / 8;                        // 16-byte chunks per row
    constexpr int RPI = 64 / CH;                     // rows per 1 KiB direct load
    constexpr int LOADS = BKV / RPI;                 // direct loads per K (or V) tile
    constexpr int LPW = (2 * LOADS) / NW;            // direct loads per wave per iteration (K and V)
    static_assert((2 * LOADS) % NW == 0, "loads split evenly over the waves");
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    __shared__ __align__(16) bf16_t sK[2][BKV * D];
    __shared__ __align__(16) bf16_t sV[2][BKV * D];

    const int g = nh / nkv;
    const int hchunks = g / HPB;
    const int nqb = (S_max + BQ - 1) / BQ;
    if constexpr (!SPLIT) nsplit = 1;
    const int per_qb = B * nkv * hchunks * nsplit;
    const int qb = nqb - 1 - static_cast<int>(blockIdx.x) / per_qb;   // heaviest blocks first
    int rem = static_cast<int>(blockIdx.x) % per_qb;
    const int split = rem % nsplit;
    rem /= nsplit;
    const int hc = rem % hchunks;
    rem /= hchunks;
    const int c = rem % nkv;
    const int b = rem / nkv;

    int seq0, S;
    if (cu != nullptr) {   // packed sequences: bounds clamped into range, so any cu contents stay in bounds
        const int a0 = min(max(cu[b], 0), total);
        const int a1 = min(max(cu[b + 1], a0), total);
        seq0 = a0;
        S = min(a1 - a0, S_max);
    } else {
        seq0 = b * S_max;
        S = S_max;
    }
    if (qb * BQ >= S) return;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, lh = lane >> 5;
    const int h = c * g + hc * HPB + (wave >> 1);
    const int64_t rs = static_cast<int64_t>(nh + 2 * nkv) * D;
    const bf16_t* qkv_b = qkv + static_cast<int64_t>(seq0) * rs;
    // visibility: query i sees keys 0 .. lim(i): lim(i) = i over the call's own tokens, position_ids[b, i]
    // (clamped to the cache) over a cache. The block's smallest and largest limits give the key tiles it
    // visits (0 .. hi / BKV) and the first one that needs the mask.
    const int64_t* pos_b = CACHED ? pos + seq0 : nullptr;
    auto lim_of = [&](int q) -> int {
        if constexpr (CACHED) return static_cast<int>(clamp_pos(pos_b[q], ctx));
        else return q;
    };
    int lo, hi;
    if constexpr (CACHED) {
        int l = lim_of(min(qb * BQ + lane, S - 1));
        int m = l;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            l = min(l, __shfl_xor(l, o, 64));
            m = max(m, __shfl_xor(m, o, 64));
        }
        lo = __builtin_amdgcn_readfirstlane(l);
        hi = __builtin_amdgcn_readfirstlane(m);
    } else {
        lo = qb * BQ;
        hi = min(qb * BQ + BQ - 1, S - 1);
    }
    const int nkt_all = hi / BKV + 1;
    const int j0 = SPLIT ? split * nkt_all / nsplit : 0;
    const int j1 = SPLIT ? (split + 1) * nkt_all / nsplit : nkt_all;
    const int qi = qb * BQ + (wave & 1) * 32 + l32;
    const int qrow = min(qi, S - 1);
    const int qlim = lim_of(qrow);
    auto record = [&](int q) {   // this split's record of query q: [0] max (log2 units), [1] sum, [4..) o
        return part + ((static_cast<int64_t>(seq0) + q) * nh + h) * nsplit * (D + 4) + static_cast<int64_t>(split) * (D + 4);
    };
    if (SPLIT && j0 >= j1) {   // no visible key tile here: an empty record (weight zero in the combine)
        if (qi < S) {
            float* rec = record(qi);
            if (lh == 0) {
                rec[0] = -INFINITY;
                rec[1] = 0.f;
            }
#pragma unroll
            for (int e = 0; e < D / 8; ++e)
                *reinterpret_cast<f32x4*>(rec + 4 + 8 * e + 4 * lh) = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        return;
    }

    // Q^T fragments: lane holds query qi, dims 16k + 8 lh .. + 7, pre-scaled by log2(e)/sqrt(d), bf16
    bf16x8 qfr[KS];
    {
        const bf16_t* qp = qkv_b + static_cast<int64_t>(qrow) * rs + static_cast<int64_t>(h) * D;
#pragma unroll
        for (int k = 0; k < KS; ++k) {
            float f[8];
            unpack8(*reinterpret_cast<const uint4*>(qp + 16 * k + 8 * lh), f);
#pragma unroll
            for (int e = 0; e < 8; ++e) f[e] *= scale_log2;
            uint4 u = pack8(f);
            if (qi >= S) u = make_uint4(0, 0, 0, 0);
            qfr[k] = __builtin_bit_cast(bf16x8, u);
        }
    }

    const int64_t cache_b = (static_cast<int64_t>(b) * ctx * nkv + c) * D;
    const bf16_t* kbase = CACHED ? kc + cache_b : qkv_b + static_cast<int64_t>(nh + c) * D;
    const bf16_t* vbase = CACHED ? vc + cache_b : qkv_b + static_cast<int64_t>(nh + nkv + c) * D;
    const uint32_t rs_bytes = static_cast<uint32_t>(CACHED ? static_cast<int64_t>(nkv) * D : rs) * 2u;
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(kbase), (short)0, -1, 0x00020000);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(vbase), (short)0, -1, 0x00020000);

    // cache append: the first head chunk of each query block copies the block's own keys and values
    if (!CACHED && kc != nullptr && hc == 0 && split == 0) {
        const int64_t* pos_b = pos + seq0;
        for (int job = tid; job < 2 * BQ * CH; job += NT) {
            const bool isv = job >= BQ * CH;
            const int jj = isv ? job - BQ * CH : job;
            const int r = jj / CH, ch = jj % CH;
            const int key = qb * BQ + r;
            if (key < S) {
                const int64_t slot = clamp_pos(pos_b[key], ctx);
                const uint4 v = *reinterpret_cast<const uint4*>((isv ? vbase : kbase) + static_cast<int64_t>(key) * rs + ch * 8);
                bf16_t* dst = (isv ? vc : kc) + ((static_cast<int64_t>(b) * ctx + slot) * nkv + c) * D + ch * 8;
                *reinterpret_cast<uint4*>(dst) = v;
            }
        }
    }
    // direct loads. Load q (0 .. 2 LOADS - 1; q < LOADS: K, else V) covers rows (q % LOADS) * RPI .. + RPI - 1
    // of the tile; lane l lands at physical chunk l % CH of row l / CH and fetches the logical chunk the
    // swizzle puts there. Keys past the block's last visible key read that key's row (masked, zero weight).
    // Buffer loads based at this kv head's first K and V element, with 32-bit byte offsets (the caller checks
    // that the rows fit).
    auto issue_tiles = [&](int ktile, int kbuf, int vtile, int vbuf) {
#pragma unroll
        for (int i = 0; i < LPW; ++i) {
            const int q = wave * LPW + i;
            const bool isv = q >= LOADS;
            const int r = (q % LOADS) * RPI + lane / CH, pc = lane % CH;
            const int key = min((isv ? vtile : ktile) * BKV + r, hi);
            const int lc = isv ? vt_phys<D>(r, pc) : k_phys<D>(r, pc);
            const uint32_t off = static_cast<uint32_t>(key) * rs_bytes + static_cast<uint32_t>(lc) * 16u;
            bf16_t* dst = isv ? &sV[vbuf][(q % LOADS) * RPI * D] : &sK[kbuf][(q % LOADS) * RPI * D];
            __builtin_amdgcn_raw_ptr_buffer_load_lds(isv ? rv : rk, (__attribute__((address_space(3))) void*)dst, 16,
                                                     off, 0, 0, 0);
        }
    };
    auto issue_k_only = [&](int ktile, int kbuf) {
#pragma unroll
        for (int i = 0; i < LPW; ++i) {
            const int q = wave * LPW + i;
            if (q < LOADS) {
                const int r = q * RPI + lane / CH, pc = lane % CH;
                const int key = min(ktile * BKV + r, hi);
                const uint32_t off = static_cast<uint32_t>(key) * rs_bytes + static_cast<uint32_t>(k_phys<D>(r, pc)) * 16u;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (__attribute__((address_space(3))) void*)&sK[kbuf][q * RPI * D],
                                                         16, off, 0, 0, 0);
            }
        }
    };

    // k steps [k0, k0 + KH) of the scores of the tile in K buffer kb, both 32-key blocks
#define PM_QK(SN, kb, k0)                                                                                  \
    _Pragma("unroll") for (int k = (k0); k < (k0) + KH; ++k) {                                             \
        _Pragma("unroll") for (int kf = 0; kf < NKF; ++kf) {                                               \
            const int r = kf * 32 + l32;                                                                   \
            const bf16x8 kfr = *reinterpret_cast<const bf16x8*>(&sK[kb][r * D + k_phys<D>(r, 2 * k + lh) * 8]); \
            SN[kf] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kfr, qfr[k], SN[kf], 0, 0, 0);                \
        }                                                                                                  \
    }
    // O^T += V^T P^T over keys 16 ks .. 16 ks + 15 of the tile (V buffer vb)
#define PM_PV_STEP(vb, ks)                                                                                 \
    _Pragma("unroll") for (int db = 0; db < DB; ++db) {                                                    \
        s16x4 h_[2];                                                                                       \
        _Pragma("unroll") for (int u = 0; u < 2; ++u) {                                                    \
            const int r = 16 * (ks) + 8 * u + 4 * lh + ((lane & 15) >> 2);                                 \
            const int cc = 4 * db + 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);                             \
            h_[u] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(      \
                &sV[vb][r * D + vt_phys<D>(r, cc) * 8 + (lane & 1) * 4]));                                 \
        }                                                                                                  \
        const bf16x8 vfr = __builtin_bit_cast(bf16x8, __builtin_shufflevector(h_[0], h_[1], 0, 1, 2, 3, 4, 5, 6, 7)); \
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vfr, pfr[ks], oacc[db], 0, 0, 0);               \
    }
    // P for keys 16 ks .. 16 ks + 15: registers 8 (ks % 2) .. + 7 of score block ks / 2
#define PM_EXP_STEP(SC, ks)                                                                                \
    {                                                                                                      \
        float p_[8];                                                                                       \
        _Pragma("unroll") for (int e = 0; e < 8; ++e) {                                                    \
            p_[e] = fast_exp2(SC[(ks) >> 1][8 * ((ks) & 1) + e]);                                          \
            ls += p_[e];                                                                                   \
        }                                                                                                  \
        pfr[ks] = __builtin_bit_cast(bf16x8, pack8(p_));                                                   \
    }

    float m_i = 0.f, l_i = 0.f;
    f32x16 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
    f32x16 sA[NKF];
    bf16x8 pfr[NKS];

    if constexpr (!PIPE) {
        // tile j's K and V load during tile j-1; both buffers of tile j-1 are free after its barrier
        if constexpr (SPLIT) m_i = -INFINITY;   // no reference yet (a split may start wholly masked)
        issue_tiles(j0, 0, j0, 0);
        __syncthreads();
        for (int j = j0; j < j1; ++j) {
            const int bf = (j - j0) & 1;
            issue_tiles(j + 1, bf ^ 1, j + 1, bf ^ 1);
            const bool fresh = SPLIT ? m_i == -INFINITY : j == j0;
            {
                const float ref = fresh ? 0.f : m_i;
                f32x16 z_;
#pragma unroll
                for (int e = 0; e < 16; ++e) z_[e] = -ref;
#pragma unroll
                for (int kf = 0; kf < NKF; ++kf) sA[kf] = z_;
            }
            PM_QK(sA, bf, 0)
            PM_QK(sA, bf, KH)
            if (__builtin_expect((j + 1) * BKV - 1 > lo, 0)) {
                __asm__ volatile("");
#pragma unroll
                for (int kf = 0; kf < NKF; ++kf)
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int key = j * BKV + kf * 32 + 8 * (e >> 2) + 4 * lh + (e & 3);
                        if (key > qlim) sA[kf][e] = -INFINITY;
                    }
            }
            float mx = -INFINITY;
#pragma unroll
            for (int kf = 0; kf < NKF; ++kf)
#pragma unroll
                for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sA[kf][e]);
            {
                const auto a_ = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
                mx = fmaxf(__uint_as_float(a_[0]), __uint_as_float(a_[1]));
            }
            // the scores are relative to the reference: set it on the first tile with a visible key, move it
            // when a tile max exceeds it by more than kSlack
            const bool upd = fresh ? mx > -INFINITY : mx > kSlack;
            const float shift_ = upd ? mx : 0.f;
            if (__builtin_expect(__any(upd), 0)) {
                __asm__ volatile("");
                const float alpha = fresh ? 1.f : fast_exp2(-shift_);
                if (upd) m_i = (fresh ? 0.f : m_i) + shift_;
                l_i *= alpha;
#pragma unroll
                for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
#pragma unroll
                for (int kf = 0; kf < NKF; ++kf) sA[kf] -= shift_;
            }
            float ls = 0.f;
#pragma unroll
            for (int ks = 0; ks < HS; ++ks) PM_EXP_STEP(sA, ks)
#pragma unroll
            for (int ks = 0; ks < HS; ++ks) PM_PV_STEP(bf, ks)
#pragma unroll
            for (int ks = HS; ks < NKS; ++ks) PM_EXP_STEP(sA, ks)
#pragma unroll
            for (int ks = HS; ks < NKS; ++ks) PM_PV_STEP(bf, ks)
            l_i += ls;
            __syncthreads();
        }
    } else {
    float mbA = 0.f, mbB = 0.f;
    f32x16 sB[NKF];
    if constexpr (SPLIT) m_i = -INFINITY;   // no reference yet (a split may start wholly masked)
    issue_tiles(j0, 0, j0, 0);
    issue_k_only(j0 + 1, 1);
    __syncthreads();
#pragma unroll
    for (int kf = 0; kf < NKF; ++kf) sA[kf] = f32x16{};
    PM_QK(sA, 0, 0)
    PM_QK(sA, 0, KH)
    __syncthreads();   // K buffer 0 is refilled by the first iteration

#define PM_ITER(SC, MBC, SN, MBN)                                                                          \
    {                                                                                                      \
        issue_tiles(j + 2, (j - j0) & 1, j + 1, (j - j0 + 1) & 1);                                         \
        if (__builtin_expect((j + 1) * BKV - 1 > lo, 0)) {                                                 \
            __asm__ volatile("");                                                                          \
            _Pragma("unroll") for (int kf = 0; kf < NKF; ++kf)                                             \
                _Pragma("unroll") for (int e = 0; e < 16; ++e) {                                           \
                    const int key = j * BKV + kf * 32 + 8 * (e >> 2) + 4 * lh + (e & 3);                   \
                    if (key > qlim) SC[kf][e] = -INFINITY;                                                 \
                }                                                                                          \
        }                                                                                                  \
        /* stage 1: first half of tile j+1's scores || row max of tile j */                               \
        MBN = (SPLIT ? m_i > -INFINITY : j != j0) ? m_i : 0.f;                                             \
        {                                                                                                  \
            f32x16 z_;                                                                                     \
            _Pragma("unroll") for (int e = 0; e < 16; ++e) z_[e] = -MBN;                                   \
            _Pragma("unroll") for (int kf = 0; kf < NKF; ++kf) SN[kf] = z_;                                \
        }                                                                                                  \
        PM_QK(SN, (j - j0 + 1) & 1, 0)                                                                     \
        float mx = -INFINITY;                                                                              \
        _Pragma("unroll") for (int kf = 0; kf < NKF; ++kf)                                                 \
            _Pragma("unroll") for (int e = 0; e < 16; ++e) mx = fmaxf(mx, SC[kf][e]);                      \
        {                                                                                                  \
            const auto a_ = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false); \
            mx = fmaxf(__uint_as_float(a_[0]), __uint_as_float(a_[1]));                                    \
        }                                                                                                  \
        const bool fresh_ = SPLIT ? m_i == -INFINITY : j == j0;                                            \
        const float delta_ = (SPLIT && fresh_) ? 0.f : m_i - MBC;                                          \
        const float rel_ = mx - delta_;                                                                    \
        const float shift_ = (SPLIT ? (fresh_ ? rel_ > -INFINITY : rel_ > kSlack)                          \
                                    : (fresh_ || rel_ > kSlack)) ? rel_ : 0.f;                             \
        const float sub_ = delta_ + shift_;                                                                \
        /* stage 2 (rare): re-reference tile j's scores, rescale O and l where the reference moved */     \
        if (__builtin_expect(__any(sub_ != 0.f), 0)) {                                                     \
            __asm__ volatile("");                                                                          \
            const float alpha = fresh_ ? 1.f : fast_exp2(-shift_);                                         \
            m_i = (SPLIT && fresh_ ? 0.f : m_i) + shift_;                                                  \
            l_i *= alpha;                                                                                  \
            _Pragma("unroll") for (int db = 0; db < DB; ++db) oacc[db] *= alpha;                           \
            _Pragma("unroll") for (int kf = 0; kf < NKF; ++kf) SC[kf] -= sub_;                             \
        }                                                                                                  \
        float ls = 0.f;                                                                                    \
        /* stage 3: second half of tile j+1's scores || exponentials of the first half of the keys */     \
        PM_QK(SN, (j - j0 + 1) & 1, KH)                                                                    \
        _Pragma("unroll") for (int ks = 0; ks < HS; ++ks) PM_EXP_STEP(SC, ks)                              \
        /* stage 4: P V of the first half || exponentials of the second half */                            \
        _Pragma("unroll") for (int ks = 0; ks < HS; ++ks) PM_PV_STEP((j - j0) & 1, ks)                     \
        _Pragma("unroll") for (int ks = HS; ks < NKS; ++ks) PM_EXP_STEP(SC, ks)                            \
        /* stage 5: P V of the second half */                                                              \
        _Pragma("unroll") for (int ks = HS; ks < NKS; ++ks) PM_PV_STEP((j - j0) & 1, ks)                   \
        l_i += ls;                                                                                         \
        __syncthreads();                                                                                   \
    }
    for (int j = j0; j < j1; j += 2) {
        PM_ITER(sA, mbA, sB, mbB)
        if (j + 1 >= j1) break;
        {
            const int j_ = j;
            {
                const int j = j_ + 1;
                PM_ITER(sB, mbB, sA, mbA)
            }
        }
    }
    }
#undef PM_ITER
#undef PM_QK
#undef PM_PV_STEP
#undef PM_EXP_STEP

    // lane holds dims 32 db + 8 i + 4 lh + {0..3} of query qi
    float lsum;
    {
        const auto a_ = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_i), __float_as_uint(l_i), false, false);
        lsum = __uint_as_float(a_[0]) + __uint_as_float(a_[1]);
    }
    if constexpr (SPLIT) {
        if (qi < S) {
            float* rec = record(qi);
            if (lh == 0) {
                rec[0] = m_i;
                rec[1] = lsum;
            }
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const f32x16& v = oacc[db];
                    *reinterpret_cast<f32x4*>(rec + 4 + 32 * db + 8 * i + 4 * lh) =
                        f32x4{v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]};
                }
        }
        return;
    }
    const float inv = 1.f / lsum;
    if (qi < S) {
        bf16_t* op = out + (static_cast<int64_t>(seq0) + qi) * nh * D + static_cast<int64_t>(h) * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const f32x16& v = oacc[db];
                *reinterpret_cast<uint2*>(op + 32 * db + 8 * i + 4 * lh) =
                    make_uint2(pack_bf16x2(v[4 * i] * inv, v[4 * i + 1] * inv),
                               pack_bf16x2(v[4 * i + 2] * inv, v[4 * i + 3] * inv));
            }
    }
}

// ------------------------------------------------------------------ generic (fp32 / any even d)
template <typename T> __device__ __forceinline__ float ldf(const T* p);
template <> __device__ __forceinline__ float ldf<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float ldf<bf16_t>(const bf16_t* p) { return bf2f(*p); }
template <typename T> __device__ __forceinline__ void stf(T* p, float v);
template <> __device__ __forceinline__ void stf<float>(float* p, float v) { *p = v; }
template <> __device__ __forceinline__ void stf<bf16_t>(bf16_t* p, float v) { *p = f2bf(v); }

constexpr int GEN_DPL = 4;  // dims per lane (d <= 256)

// Load one head vector (d dims, lanes over dims) and rotate it at position p if cs != null.
template <typename T>
__device__ __forceinline__ void gen_load_head(const T* __restrict__ v, int d, int lane, const float2* __restrict__ cs,
                                              int64_t rows, int64_t p, int il, float* out) {
    const int half = d >> 1;
#pragma unroll
    for (int i = 0; i < GEN_DPL; ++i) {
        const int dd = lane + 64 * i;
        float x = 0.f;
        if (dd < d) {
            x = ldf<T>(v + dd);
            if (cs) {
                const float2* row = cs + clamp_pos(p, rows) * half;
                int partner, j;
                float sign;
                if (il) {
                    partner = dd ^ 1;
                    j = dd >> 1;
                    sign = (dd & 1) ? 1.f : -1.f;
                } else {
                    partner = dd < half ? dd + half : dd - half;
                    j = dd < half ? dd : dd - half;
                    sign = dd < half ? -1.f : 1.f;
                }
                const float y = ldf<T>(v + partner);
                const float2 t = row[j];
                x = x * t.x + sign * y * t.y;
            }
        }
        out[i] = x;
    }
}

// one wave per (b, i, h); 4 waves per block
template <typename T>
__global__ __launch_bounds__(256) void attn_prefill_generic_kernel(const T* __restrict__ qkv,
                                                                   const int64_t* __restrict__ pos,
                                                                   const float2* __restrict__ cs, int64_t rope_rows,
                                                                   int il, T* __restrict__ out, int B, int S, int nh,
                                                                   int nkv, int d, float scale,
                                                                   const int* __restrict__ cu, int nseq) {
    const int lane = threadIdx.x & 63;
    const int64_t w = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (w >= static_cast<int64_t>(B) * S * nh) return;
    const int h = static_cast<int>(w % nh);
    const int64_t bi = w / nh;
    const int i = static_cast<int>(bi % S);
    const int b = static_cast<int>(bi / S);
    const int c = h / (nh / nkv);
    const int64_t rs = static_cast<int64_t>(nh + 2 * nkv) * d;
    const T* base = qkv + static_cast<int64_t>(b) * S * rs;
    const int64_t* pb = pos ? pos + static_cast<int64_t>(b) * S : nullptr;
    // packed sequences (cu given, B = 1, S = all tokens): token i attends from the first token of its
    // own sequence, the largest cu[k] <= i (binary search; cu entries clamped into [0, S])
    int start = 0;
    if (cu != nullptr) {
        auto cuc = [&](int k_) { return min(max(cu[k_], 0), S); };
        int lo_ = 0, hi_ = nseq;
        while (lo_ < hi_) {
            const int mid = (lo_ + hi_ + 1) >> 1;
            if (cuc(mid) <= i) lo_ = mid;
            else hi_ = mid - 1;
        }
        start = min(cuc(lo_), i);
    }
    float q[GEN_DPL], acc[GEN_DPL] = {0.f, 0.f, 0.f, 0.f};
    gen_load_head<T>(base + static_cast<int64_t>(i) * rs + static_cast<int64_t>(h) * d, d, lane, cs, rope_rows,
                     cs ? pb[i] : 0, il, q);
    float m = -INFINITY, l = 0.f;
    for (int j = start; j <= i; ++j) {
        float k[GEN_DPL];
        const T* kp = base + static_cast<int64_t>(j) * rs + static_cast<int64_t>(nh + c) * d;
        gen_load_head<T>(kp, d, lane, cs, rope_rows, cs ? pb[j] : 0, il, k);
        float dot = 0.f;
#pragma unroll
        for (int e = 0; e < GEN_DPL; ++e) dot += q[e] * k[e];
        const float s = wave_sum(dot) * scale;
        const float mn = fmaxf(m, s);
        const float alpha = expf(m - mn), p = expf(s - mn);
        l = l * alpha + p;
        const T* vp = base + static_cast<int64_t>(j) * rs + static_cast<int64_t>(nh + nkv + c) * d;
#pragma unroll
        for (int e = 0; e < GEN_DPL; ++e) {
            const int dd = lane + 64 * e;
            acc[e] = acc[e] * alpha + (dd < d ? p * ldf<T>(vp + dd) : 0.f);
        }
        m = mn;
    }
    T* op = out + (static_cast<int64_t>(b) * S + i) * nh * d + static_cast<int64_t>(h) * d;
#pragma unroll
    for (int e = 0; e < GEN_DPL; ++e) {
        const int dd = lane + 64 * e;
        if (dd < d) stf<T>(op + dd, acc[e] / l);
    }
}

// Store rotated K and V of each token at slot pos into the caches (generic prefill path and decode append).
// One wave per (token, kv head).
template <typename T>
__global__ __launch_bounds__(256) void kv_store_kernel(const T* __restrict__ qkv, const int64_t* __restrict__ pos,
                                                       const float2* __restrict__ cs, int64_t rope_rows, int il,
                                                       T* __restrict__ kc, T* __restrict__ vc, int64_t ctx, int B,
                                                       int S, int nh, int nkv, int d) {
    const int lane = threadIdx.x & 63;
    const int64_t w = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (w >= static_cast<int64_t>(B) * S * nkv) return;
    const int c = static_cast<int>(w % nkv);
    const int64_t t = w / nkv;  // token = b * S + s
    const int b = static_cast<int>(t / S);
    const int64_t rs = static_cast<int64_t>(nh + 2 * nkv) * d;
    const T* row = qkv + t * rs;
    const int64_t p = pos[t];
    float k[GEN_DPL];
    gen_load_head<T>(row + static_cast<int64_t>(nh + c) * d, d, lane, cs, rope_rows, p, il, k);
    const int64_t slot = clamp_pos(p, ctx);
    T* kd = kc + ((static_cast<int64_t>(b) * ctx + slot) * nkv + c) * d;
    T* vd = vc + ((static_cast<int64_t>(b) * ctx + slot) * nkv + c) * d;
    const T* vs = row + static_cast<int64_t>(nh + nkv + c) * d;
#pragma unroll
    for (int e = 0; e < GEN_DPL; ++e) {
        const int dd = lane + 64 * e;
        if (dd < d) {
            stf<T>(kd + dd, k[e]);
            vd[dd] = vs[dd];
        }
    }
}

// Generic decode: one wave per (b, h) over cache slots 0..pos[b] (slot pos[b] already appended).
template <typename T>
__global__ __launch_bounds__(256) void attn_decode_generic_kernel(const T* __restrict__ qkv,
                                                                  const int64_t* __restrict__ pos,
                                                                  const float2* __restrict__ cs, int64_t rope_rows,
                                                                  int il, const T* __restrict__ kc,
                                                                  const T* __restrict__ vc, int64_t ctx,
                                                                  T* __restrict__ out, int B, int S, int nh, int nkv,
                                                                  int d, float scale) {
    const int lane = threadIdx.x & 63;
    const int64_t w = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (w >= static_cast<int64_t>(B) * S * nh) return;
    const int h = static_cast<int>(w % nh);
    const int64_t t = w / nh;            // token b * S + s
    const int b = static_cast<int>(t / S);
    const int c = h / (nh / nkv);
    const int64_t rs = static_cast<int64_t>(nh + 2 * nkv) * d;
    const int64_t p = clamp_pos(pos[t], ctx);
    float q[GEN_DPL], acc[GEN_DPL] = {0.f, 0.f, 0.f, 0.f};
    gen_load_head<T>(qkv + t * rs + static_cast<int64_t>(h) * d, d, lane, cs, rope_rows, pos[t], il, q);
    float m = -INFINITY, l = 0.f;
    for (int64_t j = 0; j <= p; ++j) {
        const T* kp = kc + ((static_cast<int64_t>(b) * ctx + j) * nkv + c) * d;
        const T* vp = vc + ((static_cast<int64_t>(b) * ctx + j) * nkv + c) * d;
        float dot = 0.f;
#pragma unroll
        for (int e = 0; e < GEN_DPL; ++e) {
            const int dd = lane + 64 * e;
            if (dd < d) dot += q[e] * ldf<T>(kp + dd);
        }
        const float s = wave_sum(dot) * scale;
        const float mn = fmaxf(m, s);
        const float alpha = expf(m - mn), pr = expf(s - mn);
        l = l * alpha + pr;
#pragma unroll
        for (int e = 0; e < GEN_DPL; ++e) {
            const int dd = lane + 64 * e;
            acc[e] = acc[e] * alpha + (dd < d ? pr * ldf<T>(vp + dd) : 0.f);
        }
        m = mn;
    }
    T* op = out + t * nh * d + static_cast<int64_t>(h) * d;
#pragma unroll
    for (int e = 0; e < GEN_DPL; ++e) {
        const int dd = lane + 64 * e;
        if (dd < d) stf<T>(op + dd, acc[e] / l);
    }
}

// ------------------------------------------------------------------ decode, matrix cores
// Workgroup = (sequence b, kv head c, key split), 4 waves. The sequence's visible slots 0..pos[b] are
// cut into 128-key blocks and the blocks are shared out evenly among nsplit workgroups, so every
// workgroup has work in proportion to the sequence's own length (no workgroup scans empty slots).
// Within a block wave w takes the 32-key tile w. Each lane loads its K fragments (MFMA A operand: key
// row l%16, 8 dims) and its V row pieces (8 dims of one key) for the next two tiles while it computes
// the current one; loads use slot indices clamped to the workgroup's last slot. Both products run on
// the matrix cores: S = K q (columns = the group's query heads, the rest zero), online softmax per head
// in the log2 domain, then O^T += V^T P^T, where P^T is the lane's own probabilities (the B operand's
// key order is that of the score accumulator) and V^T comes from the tile's rows written to the wave's
// own LDS tile (XOR-swizzled) and read back with transposing reads. No workgroup barrier or fence sits
// inside the key loop: LDS instructions of one wave execute in order.
constexpr int DEC_TILE = 32;     // keys per wave step
constexpr int DEC_WAVES = 4;
constexpr int DEC_THREADS = 64 * DEC_WAVES;
constexpr int DEC_BLOCK = DEC_TILE * DEC_WAVES;   // keys per workgroup step (128)
constexpr int DEC_TARGET = 6144;                  // (workgroups x query heads) aimed for per call

template <int D>
struct DecTile {
    static constexpr int KC32 = D / 32;          // 32-dim k steps of Q K^T
    static constexpr int DL = D / 8;             // lanes per V row (8 dims each)
    static constexpr int KPI = 64 / DL;          // keys per V row load
    static constexpr int PV_IT = DEC_TILE / KPI;
    uint4 k[2][KC32];
    uint4 v[PV_IT];
};

template <int D>
__device__ __forceinline__ void dec_load(DecTile<D>& t, const bf16_t* __restrict__ kb, const bf16_t* __restrict__ vb,
                                         int64_t kstride, int64_t t0, int64_t last, int lrow, int lgrp, int dch,
                                         int ksub) {
#pragma unroll
    for (int kf = 0; kf < 2; ++kf) {
        const int64_t kk = t0 + kf * 16 + lrow, key = kk < last ? kk : last;
#pragma unroll
        for (int k = 0; k < DecTile<D>::KC32; ++k)
            t.k[kf][k] = *reinterpret_cast<const uint4*>(kb + key * kstride + k * 32 + lgrp * 8);
    }
#pragma unroll
    for (int it = 0; it < DecTile<D>::PV_IT; ++it) {
        const int64_t kk = t0 + it * DecTile<D>::KPI + ksub, key = kk < last ? kk : last;
        t.v[it] = *reinterpret_cast<const uint4*>(vb + key * kstride + dch * 8);
    }
}

// The same tile through buffer loads: one 32-bit byte offset per cache row (the dims' 64-byte steps
// ride in the instruction's offset field) instead of a 64-bit address per load. The resource covers the
// rows of one (sequence, kv head); offsets stay below 2^31 (checked by the launcher).
template <int D>
__device__ __forceinline__ void dec_load_buf(DecTile<D>& t, __amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv,
                                             int row_bytes, int t0, int last, int lrow, int lgrp, int dch,
                                             int ksub) {
#pragma unroll
    for (int kf = 0; kf < 2; ++kf) {
        const int kk = t0 + kf * 16 + lrow, key = kk < last ? kk : last;
        const int off = key * row_bytes + lgrp * 16;
#pragma unroll
        for (int k = 0; k < DecTile<D>::KC32; ++k)
            t.k[kf][k] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, off + k * 64, 0, 0));
    }
#pragma unroll
    for (int it = 0; it < DecTile<D>::PV_IT; ++it) {
        const int kk = t0 + it * DecTile<D>::KPI + ksub, key = kk < last ? kk : last;
        t.v[it] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rv, key * row_bytes + dch * 16, 0, 0));
    }
}

// number of key splits per (sequence, kv head) for a call: enough workgroups to fill the chip, at most
// one per 128-key block of the cache
static int dec_nsplit(int64_t B, int64_t nh, int64_t ctx) {
    const int64_t want = (DEC_TARGET + B * nh - 1) / (B * nh > 0 ? B * nh : 1);
    const int64_t cap = (ctx + DEC_BLOCK - 1) / DEC_BLOCK;
    return static_cast<int>(std::max<int64_t>(1, std::min(want, cap)));
}

// blocks [j0, j1) of split s among nsplit over nblk blocks; empty when j0 == j1
__device__ __forceinline__ int dec_split_begin(int s, int nblk, int nsplit) {
    return static_cast<int>(static_cast<int64_t>(s) * nblk / nsplit);
}

// partial record per (b, h, split): [0] = max (log2 domain), [1] = sum, [2..2+d) = unnormalised o
template <int D, int G, bool ROPE, bool IL>
__global__ __launch_bounds__(DEC_THREADS) void attn_decode_split_kernel(
    const bf16_t* __restrict__ qkv, const int64_t* __restrict__ pos, const float2* __restrict__ cs, int64_t rope_rows,
    const bf16_t* __restrict__ kc, const bf16_t* __restrict__ vc, int64_t ctx, float* __restrict__ part, int nsplit,
    int nh, int nkv, float scale_log2) {
    using TT = DecTile<D>;
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    constexpr int DF = D / 16;                     // 16-dim blocks of the output
    __shared__ __align__(16) bf16_t sV[DEC_WAVES][DEC_TILE * D];
    __shared__ float sM[DEC_WAVES][G], sL[DEC_WAVES][G];
    __shared__ float sO[DEC_WAVES][G][D];

    // the kv heads of one (b, split) are adjacent block ids: they read adjacent pieces of the same rows
    const int blk = blockIdx.x;
    const int c = blk % nkv;
    const int split = (blk / nkv) % nsplit;
    const int b = blk / (nkv * nsplit);
    const int64_t L = clamp_pos(pos[b], ctx) + 1;
    const int nblk = static_cast<int>((L + DEC_BLOCK - 1) / DEC_BLOCK);
    const int j0 = dec_split_begin(split, nblk, nsplit), j1 = dec_split_begin(split + 1, nblk, nsplit);
    if (j0 >= j1) return;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lrow = lane & 15, lgrp = lane >> 4;
    const int dch = lane % TT::DL, ksub = lane / TT::DL;
    const int64_t kstride = static_cast<int64_t>(nkv) * D;
    const bf16_t* kb = kc + (static_cast<int64_t>(b) * ctx * nkv + c) * D;
    const bf16_t* vb = vc + (static_cast<int64_t>(b) * ctx * nkv + c) * D;
    const int64_t lastw = std::min<int64_t>(L, static_cast<int64_t>(j1) * DEC_BLOCK) - 1;
    const int64_t base = static_cast<int64_t>(j0) * DEC_BLOCK + wave * DEC_TILE;

    // B operand of S = K q: column lrow = query head c*G + lrow (zero for lrow >= G), k = dims.
    bf16x8 qfr[TT::KC32];
    {
        const int64_t rs = static_cast<int64_t>(nh + 2 * nkv) * D;
        const bf16_t* qp = qkv + b * rs + static_cast<int64_t>(c * G + (lrow < G ? lrow : 0)) * D;
        const float2* row = ROPE ? cs + clamp_pos(pos[b], rope_rows) * (D / 2) : nullptr;
#pragma unroll
        for (int k = 0; k < TT::KC32; ++k) {
            const int d0 = k * 32 + lgrp * 8;
            float f[8];
            unpack8(*reinterpret_cast<const uint4*>(qp + d0), f);
            if (ROPE) {
                if (IL) {
                    rope8_inter(f, row, d0);
                } else {
                    float g8[8];
                    const int pd = d0 < D / 2 ? d0 + D / 2 : d0 - D / 2;
                    unpack8(*reinterpret_cast<const uint4*>(qp + pd), g8);
                    if (d0 < D / 2) rope8_half(f, g8, row, d0);
                    else rope8_half(g8, f, row, pd);
                }
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) f[e] = lrow < G ? f[e] : 0.f;
            qfr[k] = __builtin_bit_cast(bf16x8, pack8(f));
        }
    }

    float m_w = -INFINITY, l_w = 0.f;   // per lane: stats of head column lrow
    f32x4 oacc[DF];                     // O^T: dims 16a + 4*lgrp + r, head column lrow
#pragma unroll
    for (int a = 0; a < DF; ++a) oacc[a] = f32x4{0.f, 0.f, 0.f, 0.f};
    bf16_t* sVw = sV[wave];

    auto compute = [&](const DecTile<D>& t, int64_t t0) {
        // the tile's V rows into the wave's LDS tile; the previous tile's transposing reads were
        // consumed by its matrix ops, and one wave's LDS instructions execute in order
#pragma unroll
        for (int it = 0; it < TT::PV_IT; ++it) {
            const int r = it * TT::KPI + ksub;
            *reinterpret_cast<uint4*>(&sVw[r * D + vt_phys<D>(r, dch) * 8]) = t.v[it];
        }
        f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int k = 0; k < TT::KC32; ++k)
#pragma unroll
            for (int kf = 0; kf < 2; ++kf)
                sacc[kf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, t.k[kf][k]), qfr[k],
                                                                    sacc[kf], 0, 0, 0);
        // lane holds scores of keys t0 + 16 kf + 4 lgrp + r for head column lrow
        float s[2][4], mx = -INFINITY;
#pragma unroll
        for (int kf = 0; kf < 2; ++kf)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t key = t0 + kf * 16 + 4 * lgrp + r;
                const float v = key < L ? sacc[kf][r] * scale_log2 : -INFINITY;
                s[kf][r] = v;
                mx = fmaxf(mx, v);
            }
        mx = rows_max(mx);
        const float mnew = fmaxf(m_w, mx);
        const float alpha = fast_exp2(m_w - mnew);
        m_w = mnew;
        float p[2][4], ls = 0.f;
#pragma unroll
        for (int kf = 0; kf < 2; ++kf)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                p[kf][r] = fast_exp2(s[kf][r] - mnew);
                ls += p[kf][r];
            }
        l_w = l_w * alpha + ls;
        if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
            for (int a = 0; a < DF; ++a) oacc[a] *= alpha;
        }
        uint4 pu;
        pu.x = pack_bf16x2(p[0][0], p[0][1]);
        pu.y = pack_bf16x2(p[0][2], p[0][3]);
        pu.z = pack_bf16x2(p[1][0], p[1][1]);
        pu.w = pack_bf16x2(p[1][2], p[1][3]);
        const bf16x8 pfr = __builtin_bit_cast(bf16x8, pu);
        // A operand V^T (dims 16a + lrow, the lane group's 8 keys in the order of pfr) by two
        // transposing reads of 4 keys each
#pragma unroll
        for (int a = 0; a < DF; ++a) {
            s16x4 h[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int r = 16 * u + 4 * lgrp + (lrow >> 2);
                const int cc = 2 * a + ((lrow & 3) >> 1);
                h[u] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(
                    &sVw[r * D + vt_phys<D>(r, cc) * 8 + (lrow & 1) * 4]));
            }
            const bf16x8 vfr = __builtin_bit_cast(bf16x8, __builtin_shufflevector(h[0], h[1], 0, 1, 2, 3, 4, 5, 6, 7));
            oacc[a] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vfr, pfr, oacc[a], 0, 0, 0);
        }
    };

    // two tiles in flight; loads are unconditional (slots clamped to the workgroup's last one) so the
    // waits on them are exact, only the compute of a tile past the end is skipped
    DecTile<D> ta, tb;
    dec_load<D>(ta, kb, vb, kstride, base, lastw, lrow, lgrp, dch, ksub);
    dec_load<D>(tb, kb, vb, kstride, base + DEC_BLOCK, lastw, lrow, lgrp, dch, ksub);
    const int nt = j1 - j0;
    for (int i = 0; i < nt; i += 2) {
        const int64_t t0 = base + static_cast<int64_t>(i) * DEC_BLOCK, t1 = t0 + DEC_BLOCK;
        if (t0 < L) compute(ta, t0);
        dec_load<D>(ta, kb, vb, kstride, t0 + 2 * DEC_BLOCK, lastw, lrow, lgrp, dch, ksub);
        if (i + 1 < nt && t1 < L) compute(tb, t1);
        dec_load<D>(tb, kb, vb, kstride, t0 + 3 * DEC_BLOCK, lastw, lrow, lgrp, dch, ksub);
    }

    const float lt = rows_sum(l_w);
    if (lgrp == 0 && lrow < G) {
        sM[wave][lrow] = m_w;      // -inf for a wave that saw no key
        sL[wave][lrow] = lt;
    }
    if (lrow < G) {
#pragma unroll
        for (int a = 0; a < DF; ++a)
#pragma unroll
            for (int r = 0; r < 4; ++r) sO[wave][lrow][16 * a + 4 * lgrp + r] = oacc[a][r];
    }
    __syncthreads();
    // merge the waves (wave 0 always saw key 128*j0, so M is finite) and write the split's record
    for (int e = tid; e < G * (D + 2); e += DEC_THREADS) {
        const int h = e / (D + 2), k = e % (D + 2);
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < DEC_WAVES; ++w) M = fmaxf(M, sM[w][h]);
        float v = 0.f;
#pragma unroll
        for (int w = 0; w < DEC_WAVES; ++w) {
            const float sc = exp2f(sM[w][h] - M);
            if (k == 1) v += sL[w][h] * sc;
            else if (k >= 2) v += sO[w][h][k - 2] * sc;
        }
        if (k == 0) v = M;
        part[((static_cast<int64_t>(b) * nh + c * G + h) * nsplit + split) * (D + 2) + k] = v;
    }
}

// One wave per (b, h): log-sum-exp merge of the records of the splits that had keys.
template <typename T>
__global__ __launch_bounds__(64) void attn_decode_combine_kernel(const float* __restrict__ part,
                                                                 const int64_t* __restrict__ pos, int64_t ctx,
                                                                 T* __restrict__ out, int nh, int d, int nsplit) {
    const int bh = blockIdx.x, lane = threadIdx.x;
    const int b = bh / nh;
    const int64_t L = clamp_pos(pos[b], ctx) + 1;
    const int nblk = static_cast<int>((L + DEC_BLOCK - 1) / DEC_BLOCK);
    const int64_t rec = d + 2;
    const float* pr = part + static_cast<int64_t>(bh) * nsplit * rec;
    auto live = [&](int k) { return dec_split_begin(k, nblk, nsplit) < dec_split_begin(k + 1, nblk, nsplit); };
    float M = -INFINITY;
    for (int k = lane; k < nsplit; k += 64)
        if (live(k)) M = fmaxf(M, pr[k * rec]);
    M = wave_max(M);
    float den = 0.f;
    for (int k = lane; k < nsplit; k += 64)
        if (live(k)) den += pr[k * rec + 1] * exp2f(pr[k * rec] - M);
    den = wave_sum(den);
    const float inv = 1.f / den;
    // splits outer: one weight per split, the lane's dims lane, lane + 64, ... (d <= 256) in registers
    float num[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int k = 0; k < nsplit; ++k) {
        if (!live(k)) continue;   // uniform
        const float w = exp2f(pr[k * rec] - M);
        const float* po = pr + k * rec + 2;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (lane + 64 * i < d) num[i] += w * po[lane + 64 * i];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
        if (lane + 64 * i < d) stf<T>(out + static_cast<int64_t>(bh) * d + lane + 64 * i, num[i] * inv);
}

// ------------------------------------------------------------------ decode, balanced shares
// A persistent grid of NG workgroups (one per compute unit) splits the tiles of all sequences into equal
// contiguous shares (decode_partition.h), so the longest sequences no longer set the kernel's duration.
// A workgroup has 8 waves over the HW = min(n_kv, 8) kv heads of a head group: wave w serves head
// w % HW and, when HW < 8, every P-th tile of the share (phase w / HW, P = 8 / HW). With n_kv >= 8 the
// 8 waves read the 8 heads' slices of the same cache rows at the same time, i.e. whole contiguous
// rows. The key loop per wave is that of the split kernel above (32-key tiles, the next two tiles
// loading into registers, both products on the matrix cores). At the end of each piece (the part of the
// share inside one segment) the P waves of a head merge through LDS and the piece writes one
// (max, sum, o) record per query head at index g + s; the combine kernel merges a head's records.
constexpr int DV_WAVES = 8;
constexpr int DV_THREADS = 64 * DV_WAVES;
constexpr int DV_MAX_SEGS = 4096;   // (sequence, head group) pairs one call may have
constexpr int DV_MAX_WG = 512;
constexpr int DV_REC_PAD = 4;       // record = [max, sum, -, -, o[0 .. D)]: o starts 16-byte aligned

template <int D, int G, bool ROPE, bool IL>
__global__ __launch_bounds__(DV_THREADS) void attn_decode_bal_kernel(
    const bf16_t* __restrict__ qkv, const int64_t* __restrict__ pos, const float2* __restrict__ cs, int64_t rope_rows,
    const bf16_t* __restrict__ kc, const bf16_t* __restrict__ vc, int64_t ctx, float* __restrict__ part,
    int* __restrict__ seg_prefix, int nseg, int ngroups, int HW, int nh, int nkv, float scale_log2) {
    using TT = DecTile<D>;
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    constexpr int DF = D / 16;
    constexpr int REC = D + DV_REC_PAD;
    __shared__ int sPre[DV_MAX_SEGS + 1];
    __shared__ int sWave[DV_WAVES];
    __shared__ __align__(16) bf16_t sV[DV_WAVES][DEC_TILE * D];
    __shared__ float sM[DV_WAVES][G], sL[DV_WAVES][G];
    __shared__ float sO[DV_WAVES][G][D];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t NG = gridDim.x, g = blockIdx.x;
    const int P = DV_WAVES / HW;
    const int hw = wave % HW, ph = wave / HW;
    const int SEGH = HW * G;

    // 1. tiles per segment and their exclusive prefix: each thread sums a run of segments, a wave scan
    //    and the 8 wave totals give each run its start
    const int per = (nseg + DV_THREADS - 1) / DV_THREADS;
    const int s_a = min(nseg, tid * per), s_e = min(nseg, s_a + per);
    int run = 0;
    for (int sg = s_a; sg < s_e; ++sg) run += static_cast<int>(dv_tiles(pos[sg / ngroups], ctx));
    int inc = run;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(inc, o, 64);
        if (lane >= o) inc += t;
    }
    if (lane == 63) sWave[wave] = inc;
    __syncthreads();
    int acc = inc - run;
    int total = 0;
#pragma unroll
    for (int w = 0; w < DV_WAVES; ++w) {
        acc += w < wave ? sWave[w] : 0;
        total += sWave[w];
    }
    for (int sg = s_a; sg < s_e; ++sg) {
        sPre[sg] = acc;
        acc += static_cast<int>(dv_tiles(pos[sg / ngroups], ctx));
    }
    if (tid == 0) sPre[nseg] = total;
    __syncthreads();
    const int64_t T = total;
    if (g == 0)
        for (int sg = tid; sg <= nseg; sg += DV_THREADS) seg_prefix[sg] = sPre[sg];
    const int64_t t0 = dv_share_begin(g, T, NG), t1 = dv_share_begin(g + 1, T, NG);
    if (t0 >= t1) return;   // an empty share (T < NG): the whole workgroup leaves together

    // first segment of the share: the last one starting at or before t0
    int s0 = 0;
    {
        int hi = nseg - 1;
        while (s0 < hi) {
            const int mid = (s0 + hi + 1) >> 1;
            if (sPre[mid] <= t0) s0 = mid;
            else hi = mid - 1;
        }
    }

    const int lrow = lane & 15, lgrp = lane >> 4;
    const int dch = lane % TT::DL, ksub = lane / TT::DL;
    bf16_t* sVw = sV[wave];

    for (int sg = s0; sg < nseg && sPre[sg] < t1; ++sg) {
        int64_t ja, je;
        dv_piece(g, T, NG, sPre[sg], sPre[sg + 1] - sPre[sg], &ja, &je);
        const int b = sg / ngroups, hg = sg - b * ngroups;
        const int c = hg * HW + hw;
        const int L = static_cast<int>(clamp_pos(pos[b], ctx)) + 1;
        const int last = static_cast<int>(L < je * DEC_TILE ? L : je * DEC_TILE) - 1;
        const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<bf16_t*>(kc + (static_cast<int64_t>(b) * ctx * nkv + c) * D), (short)0, -1, 0x00020000);
        const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<bf16_t*>(vc + (static_cast<int64_t>(b) * ctx * nkv + c) * D), (short)0, -1, 0x00020000);
        const int row_bytes = nkv * D * 2;

        // B operand of S = K q: column lrow = query head c*G + lrow (zero for lrow >= G), k = dims
        bf16x8 qfr[TT::KC32];
        {
            const int64_t rs = static_cast<int64_t>(nh + 2 * nkv) * D;
            const bf16_t* qp = qkv + b * rs + static_cast<int64_t>(c * G + (lrow < G ? lrow : 0)) * D;
            const float2* row = ROPE ? cs + clamp_pos(pos[b], rope_rows) * (D / 2) : nullptr;
#pragma unroll
            for (int k = 0; k < TT::KC32; ++k) {
                const int d0 = k * 32 + lgrp * 8;
                float f[8];
                unpack8(*reinterpret_cast<const uint4*>(qp + d0), f);
                if (ROPE) {
                    if (IL) {
                        rope8_inter(f, row, d0);
                    } else {
                        float g8[8];
                        const int pd = d0 < D / 2 ? d0 + D / 2 : d0 - D / 2;
                        unpack8(*reinterpret_cast<const uint4*>(qp + pd), g8);
                        if (d0 < D / 2) rope8_half(f, g8, row, d0);
                        else rope8_half(g8, f, row, pd);
                    }
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) f[e] = lrow < G ? f[e] : 0.f;
                qfr[k] = __builtin_bit_cast(bf16x8, pack8(f));
            }
        }

        float m_w = -INFINITY, l_w = 0.f;
        f32x4 oacc[DF];
#pragma unroll
        for (int a = 0; a < DF; ++a) oacc[a] = f32x4{0.f, 0.f, 0.f, 0.f};

        auto compute = [&](const DecTile<D>& t, int k0) {
#pragma unroll
            for (int it = 0; it < TT::PV_IT; ++it) {
                const int r = it * TT::KPI + ksub;
                *reinterpret_cast<uint4*>(&sVw[r * D + vt_phys<D>(r, dch) * 8]) = t.v[it];
            }
            f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
            for (int k = 0; k < TT::KC32; ++k)
#pragma unroll
                for (int kf = 0; kf < 2; ++kf)
                    sacc[kf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, t.k[kf][k]), qfr[k],
                                                                        sacc[kf], 0, 0, 0);
            float sv[2][4], mx = -INFINITY;
#pragma unroll
            for (int kf = 0; kf < 2; ++kf)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int key = k0 + kf * 16 + 4 * lgrp + r;
                    const float v = key < L ? sacc[kf][r] * scale_log2 : -INFINITY;
                    sv[kf][r] = v;
                    mx = fmaxf(mx, v);
                }
            mx = rows_max(mx);
            const float mnew = fmaxf(m_w, mx);
            const float alpha = fast_exp2(m_w - mnew);
            m_w = mnew;
            float pr[2][4], ls = 0.f;
#pragma unroll
            for (int kf = 0; kf < 2; ++kf)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    pr[kf][r] = fast_exp2(sv[kf][r] - mnew);
                    ls += pr[kf][r];
                }
            l_w = l_w * alpha + ls;
            if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
                for (int a = 0; a < DF; ++a) oacc[a] *= alpha;
            }
            uint4 pu;
            pu.x = pack_bf16x2(pr[0][0], pr[0][1]);
            pu.y = pack_bf16x2(pr[0][2], pr[0][3]);
            pu.z = pack_bf16x2(pr[1][0], pr[1][1]);
            pu.w = pack_bf16x2(pr[1][2], pr[1][3]);
            const bf16x8 pfr = __builtin_bit_cast(bf16x8, pu);
#pragma unroll
            for (int a = 0; a < DF; ++a) {
                s16x4 hv[2];
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int r = 16 * u + 4 * lgrp + (lrow >> 2);
                    const int cc = 2 * a + ((lrow & 3) >> 1);
                    hv[u] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(
                        &sVw[r * D + vt_phys<D>(r, cc) * 8 + (lrow & 1) * 4]));
                }
                const bf16x8 vfr =
                    __builtin_bit_cast(bf16x8, __builtin_shufflevector(hv[0], hv[1], 0, 1, 2, 3, 4, 5, 6, 7));
                oacc[a] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vfr, pfr, oacc[a], 0, 0, 0);
            }
        };

        // this wave's tiles of the piece: ja + ph, ja + ph + P, ... < je; loads clamp their slots to the
        // piece's last one, so the two tiles loaded past the end stay in bounds
        const int first = static_cast<int>(ja) + ph;
        const int nt = first < je ? static_cast<int>((je - first + P - 1) / P) : 0;
        const int step = P * DEC_TILE;
        DecTile<D> ta, tb;
        dec_load_buf<D>(ta, rk, rv, row_bytes, first * DEC_TILE, last, lrow, lgrp, dch, ksub);
        dec_load_buf<D>(tb, rk, rv, row_bytes, first * DEC_TILE + step, last, lrow, lgrp, dch, ksub);
        for (int i = 0; i < nt; i += 2) {
            const int k0 = (first + i * P) * DEC_TILE;
            compute(ta, k0);
            dec_load_buf<D>(ta, rk, rv, row_bytes, k0 + 2 * step, last, lrow, lgrp, dch, ksub);
            if (i + 1 < nt) compute(tb, k0 + step);
            dec_load_buf<D>(tb, rk, rv, row_bytes, k0 + 3 * step, last, lrow, lgrp, dch, ksub);
        }

        const float lt = rows_sum(l_w);
        float* rec = part + (static_cast<int64_t>(g + sg) * SEGH) * REC;
        if (P == 1) {
            // one wave per head: its G records straight from registers
            if (lrow < G) {
                float* r = rec + static_cast<int64_t>(hw * G + lrow) * REC;
                if (lgrp == 0) {
                    r[0] = m_w;
                    r[1] = lt;
                }
#pragma unroll
                for (int a = 0; a < DF; ++a)
                    *reinterpret_cast<f32x4*>(r + DV_REC_PAD + 16 * a + 4 * lgrp) = oacc[a];
            }
        } else {
            // the P waves of each head merge through LDS (phase 0 always saw key 32 * ja: M is finite)
            if (lgrp == 0 && lrow < G) {
                sM[wave][lrow] = m_w;
                sL[wave][lrow] = lt;
            }
            if (lrow < G) {
#pragma unroll
                for (int a = 0; a < DF; ++a)
#pragma unroll
                    for (int r = 0; r < 4; ++r) sO[wave][lrow][16 * a + 4 * lgrp + r] = oacc[a][r];
            }
            __syncthreads();
            for (int e = tid; e < SEGH * (D + 2); e += DV_THREADS) {
                const int hh = e / (D + 2), k = e - hh * (D + 2);
                const int w0 = hh / G, gi = hh - w0 * G;
                float M = -INFINITY;
                for (int p2 = 0; p2 < P; ++p2) M = fmaxf(M, sM[w0 + HW * p2][gi]);
                float v = 0.f;
                for (int p2 = 0; p2 < P; ++p2) {
                    const int w = w0 + HW * p2;
                    const float sc = exp2f(sM[w][gi] - M);
                    if (k == 1) v += sL[w][gi] * sc;
                    else if (k >= 2) v += sO[w][gi][k - 2] * sc;
                }
                if (k == 0) v = M;
                rec[static_cast<int64_t>(hh) * REC + (k < 2 ? k : DV_REC_PAD + k - 2)] = v;
            }
            __syncthreads();   // sM, sL, sO are rewritten by the next piece
        }
    }
}

// One wave per (b, h), four per workgroup: log-sum-exp merge of the records of the pieces of h's segment. The pieces' weights
// exp2(m_p - M) are formed once (a lane per piece) and kept in LDS; the weighted sum then loads every
// piece's o with no branch between loads (pieces of workgroups whose share misses the segment have
// weight zero; their record slots are in bounds but unwritten, so their values are selected away).
template <int D>
__global__ __launch_bounds__(256) void attn_decode_bal_combine_kernel(const float* __restrict__ part,
                                                                     const int* __restrict__ seg_prefix, int nseg,
                                                                     int ngroups, int HW, int G, int NG, int nh,
                                                                     int nbh, bf16_t* __restrict__ out) {
    constexpr int REC = D + DV_REC_PAD;
    constexpr int DPL = D / 64;   // dims per lane
    __shared__ float sws[4][DV_MAX_WG];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int bh = blockIdx.x * 4 + wv;
    if (bh >= nbh) return;   // whole waves leave; the kernel has no workgroup barrier
    float* sw = sws[wv];
    const int b = bh / nh, h = bh - b * nh;
    const int c = h / G, hg = c / HW, hw = c - hg * HW;
    const int hh = hw * G + (h - c * G);
    const int sg = b * ngroups + hg;
    const int64_t T = seg_prefix[nseg];
    const int64_t ps = seg_prefix[sg], ns = seg_prefix[sg + 1] - ps;
    const int64_t g_lo = dv_owner(ps, T, NG), g_hi = dv_owner(ps + ns - 1, T, NG);
    const int np = static_cast<int>(g_hi - g_lo + 1);
    const int SEGH = HW * G;
    const float* rec0 = part + ((g_lo + sg) * SEGH + hh) * REC;   // piece p's record: rec0 + p * SEGH * REC
    const int64_t pstride = static_cast<int64_t>(SEGH) * REC;
    auto live = [&](int p) {
        int64_t lo, hi;
        dv_piece(g_lo + p, T, NG, ps, ns, &lo, &hi);
        return lo < hi;
    };
    float M = -INFINITY;
    for (int p = lane; p < np; p += 64)
        if (live(p)) M = fmaxf(M, rec0[p * pstride]);
    M = wave_max(M);
    float den = 0.f;
    for (int p = lane; p < np; p += 64) {
        float w = 0.f;
        if (live(p)) {
            w = exp2f(rec0[p * pstride] - M);
            den += w * rec0[p * pstride + 1];
        }
        sw[p] = w;
    }
    den = wave_sum(den);
    const float inv = 1.f / den;
    float num[DPL];
#pragma unroll
    for (int i = 0; i < DPL; ++i) num[i] = 0.f;
    // the wave's own LDS writes above are complete for its reads below (one wave, in order)
#pragma unroll 4
    for (int p = 0; p < np; ++p) {
        const float w = sw[p];
        const float* r = rec0 + p * pstride + DV_REC_PAD + lane;
#pragma unroll
        for (int i = 0; i < DPL; ++i) {
            const float o = r[64 * i];
            num[i] += w != 0.f ? w * o : 0.f;
        }
    }
#pragma unroll
    for (int i = 0; i < DPL; ++i) out[static_cast<int64_t>(bh) * D + lane + 64 * i] = f2bf(num[i] * inv);
}

// ------------------------------------------------------------------ dispatch
bool attn_mfma_supported(int dtype, int d, int nh, int nkv) {
    return dtype == LL_BF16 && (d == 64 || d == 128) && nkv > 0 && nh % nkv == 0 && (nh / nkv) <= 64;
}

template <int D, int HPB, bool ROPE, bool IL>
static hipError_t prefill_go(const void* qkv, const int64_t* pos, const RopeTab* tab, void* o, void* kc, void* vc,
                             int64_t ctx, int B, int S, int nh, int nkv, hipStream_t st) {
    const int g = nh / nkv;
    const int nqb = (S + 63) / 64;
    const unsigned blocks = static_cast<unsigned>(nqb) * B * nkv * (g / HPB);
    const float scale_log2 = kLog2e / sqrtf(static_cast<float>(D));
    hipLaunchKernelGGL((attn_prefill_mfma_kernel<D, HPB, ROPE, IL>), dim3(blocks), dim3(128 * HPB), 0, st,
                       static_cast<const bf16_t*>(qkv), pos, tab ? tab->cs : nullptr, tab ? tab->rows : 1,
                       static_cast<bf16_t*>(o), static_cast<bf16_t*>(kc), static_cast<bf16_t*>(vc), ctx, B, S, nh,
                       nkv, scale_log2);
    return hipGetLastError();
}

template <int D, int HPB>
static hipError_t prefill_rope_sel(const void* qkv, const int64_t* pos, const RopeTab* tab, int il, void* o, void* kc,
                                   void* vc, int64_t ctx, int B, int S, int nh, int nkv, hipStream_t st) {
    if (!tab) return prefill_go<D, HPB, false, false>(qkv, pos, tab, o, kc, vc, ctx, B, S, nh, nkv, st);
    if (il) return prefill_go<D, HPB, true, true>(qkv, pos, tab, o, kc, vc, ctx, B, S, nh, nkv, st);
    return prefill_go<D, HPB, true, false>(qkv, pos, tab, o, kc, vc, ctx, B, S, nh, nkv, st);
}

// the 32x32 prefill kernel's tile loop (pipelined at d = 128, plain at d = 64) and waves per SIMD
template <int D>
constexpr bool m32_pipe() { return D != 64; }
template <int D, int HPB>
constexpr int m32_occ() { return HPB == 1 ? 1 : (m32_pipe<D>() ? 2 : 4); }

// q and k already rotated: the 32x32 matrix-op kernel, HPB heads per workgroup
template <int D, int HPB>
static hipError_t m32_go(const void* qkv, const int64_t* pos, void* o, void* kc, void* vc, int64_t ctx, int B,
                         int S_max, int nh, int nkv, const int* cu, int total, hipStream_t st) {
    const int g = nh / nkv;
    const unsigned blocks = static_cast<unsigned>((S_max + 63) / 64) * B * nkv * (g / HPB);
    const float scale_log2 = kLog2e / sqrtf(static_cast<float>(D));
    // d = 128: the pipelined form at two waves per SIMD (~230 registers). d = 64: the plain form at four
    // waves per SIMD (117 registers): in the 1B layer 0.108 ms pipelined at two, 0.095 at three (150
    // registers), 0.090 plain at four. 32-key tiles measured slower: 4% at d = 128 (pipelined, two waves
    // per SIMD, or plain at three), 2% at d = 64.
    constexpr bool PIPE = m32_pipe<D>();
    constexpr int OCC = m32_occ<D, HPB>();
    hipLaunchKernelGGL((attn_prefill_m32_kernel<D, HPB, OCC, PIPE>), dim3(blocks), dim3(128 * HPB), 0, st,
                       static_cast<const bf16_t*>(qkv), pos, static_cast<bf16_t*>(o), static_cast<bf16_t*>(kc),
                       static_cast<bf16_t*>(vc), ctx, B, S_max, nh, nkv, scale_log2, cu, total, 1, nullptr);
    return hipGetLastError();
}

// two heads per workgroup and two workgroups per compute unit when the group size allows (see below)
template <int D>
static hipError_t m32_sel(const void* qkv, const int64_t* pos, void* o, void* kc, void* vc, int64_t ctx, int B,
                          int S_max, int nh, int nkv, const int* cu, int total, hipStream_t st) {
    if ((nh / nkv) % 2 == 0) return m32_go<D, 2>(qkv, pos, o, kc, vc, ctx, B, S_max, nh, nkv, cu, total, st);
    return m32_go<D, 1>(qkv, pos, o, kc, vc, ctx, B, S_max, nh, nkv, cu, total, st);
}

template <int D>
static hipError_t prefill_hpb_sel(const void* qkv, const int64_t* pos, const RopeTab* tab, int il, void* o, void* kc,
                                  void* vc, int64_t ctx, int B, int S, int nh, int nkv, hipStream_t st) {
    const int g = nh / nkv;
    // q and k already rotated (the layer path): the 32x32 matrix-op kernel (3.6% faster than the 16x16
    // direct-load kernel at d = 128 and 4.6% at d = 64 in the layer). Its byte offsets are 32-bit.
    if (!tab && static_cast<int64_t>(S) * (nh + 2 * nkv) * D * 2 < (int64_t(1) << 32))
        return m32_sel<D>(qkv, pos, o, kc, vc, ctx, B, S, nh, nkv, nullptr, 0, st);
    // RoPE on load (or offsets past 32 bits): two heads per workgroup and two workgroups per compute unit
    // (the kernel is built for two waves per SIMD), so the two waves on a SIMD belong to different
    // workgroups, whose tile barriers do not line them up.
    if (g % 2 == 0) return prefill_rope_sel<D, 2>(qkv, pos, tab, il, o, kc, vc, ctx, B, S, nh, nkv, st);
    return prefill_rope_sel<D, 1>(qkv, pos, tab, il, o, kc, vc, ctx, B, S, nh, nkv, st);
}

hipError_t launch_attn_prefill(int dtype, const void* qkv, const int64_t* pos, const RopeTab* tab, int il, void* o,
                               void* kc, void* vc, int64_t ctx, int B, int S, int nh, int nkv, int d,
                               hipStream_t st) {
    if (B == 0 || S == 0) return hipSuccess;
    if (attn_mfma_supported(dtype, d, nh, nkv)) {
        if (d == 128) return prefill_hpb_sel<128>(qkv, pos, tab, il, o, kc, vc, ctx, B, S, nh, nkv, st);
        return prefill_hpb_sel<64>(qkv, pos, tab, il, o, kc, vc, ctx, B, S, nh, nkv, st);
    }
    const int64_t waves = static_cast<int64_t>(B) * S * nh;
    const unsigned blocks = static_cast<unsigned>((waves + 3) / 4);
    const float scale = 1.f / sqrtf(static_cast<float>(d));
    const float2* cs = tab ? tab->cs : nullptr;
    const int64_t rows = tab ? tab->rows : 1;
    if (dtype == LL_BF16)
        hipLaunchKernelGGL(attn_prefill_generic_kernel<bf16_t>, dim3(blocks), dim3(256), 0, st,
                           static_cast<const bf16_t*>(qkv), pos, cs, rows, il, static_cast<bf16_t*>(o), B, S, nh, nkv,
                           d, scale, nullptr, 0);
    else
        hipLaunchKernelGGL(attn_prefill_generic_kernel<float>, dim3(blocks), dim3(256), 0, st,
                           static_cast<const float*>(qkv), pos, cs, rows, il, static_cast<float*>(o), B, S, nh, nkv, d,
                           scale, nullptr, 0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || kc == nullptr) return e;
    const int64_t kw = static_cast<int64_t>(B) * S * nkv;
    const unsigned kb = static_cast<unsigned>((kw + 3) / 4);
    if (dtype == LL_BF16)
        hipLaunchKernelGGL(kv_store_kernel<bf16_t>, dim3(kb), dim3(256), 0, st, static_cast<const bf16_t*>(qkv), pos,
                           cs, rows, il, static_cast<bf16_t*>(kc), static_cast<bf16_t*>(vc), ctx, B, S, nh, nkv, d);
    else
        hipLaunchKernelGGL(kv_store_kernel<float>, dim3(kb), dim3(256), 0, st, static_cast<const float*>(qkv), pos, cs,
                           rows, il, static_cast<float*>(kc), static_cast<float*>(vc), ctx, B, S, nh, nkv, d);
    return hipGetLastError();
}

// workgroups of the balanced decode kernel: one per compute unit (looked up once), at most DV_MAX_WG
static int dv_workgroups() {
    static const int n = [] {
        int dev = 0, cu = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cu <= 0)
            cu = 256;
        return cu < DV_MAX_WG ? cu : DV_MAX_WG;
    }();
    return n;
}

// head groups of the balanced kernel (HW = min(n_kv, 8) heads each), or 0 when it does not apply
static int dv_groups(int64_t B, int64_t nkv, int64_t ctx) {
    const bool shape = nkv <= 8 ? 8 % nkv == 0 : nkv % 8 == 0;
    if (!shape) return 0;
    const int64_t ng = nkv <= 8 ? 1 : nkv / 8;
    if (B * ng > DV_MAX_SEGS) return 0;
    if (B * ng * ((ctx + DEC_TILE - 1) / DEC_TILE) >= (int64_t(1) << 31)) return 0;
    // buffer offsets: one sequence's cache (ctx rows of n_kv heads of <= 128 bf16 dims) below 2^31 bytes
    if (ctx * nkv * 128 * 2 >= (int64_t(1) << 31)) return 0;
    return static_cast<int>(ng);
}

static size_t dv_workspace_bytes(int64_t B, int64_t nh, int64_t d, int64_t nseg) {
    const size_t rec = static_cast<size_t>((DV_MAX_WG + nseg) * nh * (d + DV_REC_PAD)) * sizeof(float);
    return ((rec + 255) & ~static_cast<size_t>(255)) + static_cast<size_t>(nseg + 1) * sizeof(int);
}

size_t attn_decode_workspace_bytes(int64_t B, int64_t nh, int64_t d, int64_t ctx) {
    const size_t split = static_cast<size_t>(B * nh * dec_nsplit(B, nh, ctx) * (d + 2)) * sizeof(float);
    // the balanced kernel: records of at most DV_MAX_WG + B * max(1, nh / 8) pieces of at most nh heads each
    const int64_t nseg = B * (nh >= 8 ? nh / 8 : 1);
    const size_t bal = dv_workspace_bytes(B, nh, d, nseg);
    return split > bal ? split : bal;
}

template <int D, int G, bool ROPE, bool IL>
static hipError_t decode_go(const void* qkv, const int64_t* pos, const RopeTab* tab, const void* kc, const void* vc,
                            int64_t ctx, void* o, int B, int nh, int nkv, void* ws, hipStream_t st) {
    const float scale_log2 = kLog2e / sqrtf(static_cast<float>(D));
    const int ngroups = dv_groups(B, nkv, ctx);
    if (ngroups > 0) {
        const int HW = nkv < 8 ? nkv : 8;
        const int nseg = B * ngroups;
        const int NG = dv_workgroups();
        const size_t rec = static_cast<size_t>((DV_MAX_WG + nseg) * static_cast<int64_t>(HW * G) * (D + DV_REC_PAD)) *
                           sizeof(float);
        float* part = static_cast<float*>(ws);
        int* prefix = reinterpret_cast<int*>(static_cast<char*>(ws) + ((rec + 255) & ~static_cast<size_t>(255)));
        hipLaunchKernelGGL((attn_decode_bal_kernel<D, G, ROPE, IL>), dim3(NG), dim3(DV_THREADS), 0, st,
                           static_cast<const bf16_t*>(qkv), pos, tab ? tab->cs : nullptr, tab ? tab->rows : 1,
                           static_cast<const bf16_t*>(kc), static_cast<const bf16_t*>(vc), ctx, part, prefix, nseg,
                           ngroups, HW, nh, nkv, scale_log2);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(attn_decode_bal_combine_kernel<D>, dim3((B * nh + 3) / 4), dim3(256), 0, st,
                           static_cast<const float*>(part), static_cast<const int*>(prefix), nseg, ngroups, HW, G, NG,
                           nh, B * nh, static_cast<bf16_t*>(o));
        return hipGetLastError();
    }
    const int nsplit = dec_nsplit(B, nh, ctx);
    const unsigned blocks = static_cast<unsigned>(static_cast<int64_t>(B) * nsplit * nkv);
    hipLaunchKernelGGL((attn_decode_split_kernel<D, G, ROPE, IL>), dim3(blocks), dim3(DEC_THREADS), 0, st,
                       static_cast<const bf16_t*>(qkv), pos, tab ? tab->cs : nullptr, tab ? tab->rows : 1,
                       static_cast<const bf16_t*>(kc), static_cast<const bf16_t*>(vc), ctx, static_cast<float*>(ws),
                       nsplit, nh, nkv, scale_log2);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(attn_decode_combine_kernel<bf16_t>, dim3(B * nh), dim3(64), 0, st,
                       static_cast<const float*>(ws), pos, ctx, static_cast<bf16_t*>(o), nh, D, nsplit);
    return hipGetLastError();
}

template <int D, int G>
static hipError_t decode_rope_sel(const void* qkv, const int64_t* pos, const RopeTab* tab, int il, const void* kc,
                                  const void* vc, int64_t ctx, void* o, int B, int nh, int nkv, void* ws,
                                  hipStream_t st) {
    if (!tab) return decode_go<D, G, false, false>(qkv, pos, tab, kc, vc, ctx, o, B, nh, nkv, ws, st);
    if (il) return decode_go<D, G, true, true>(qkv, pos, tab, kc, vc, ctx, o, B, nh, nkv, ws, st);
    return decode_go<D, G, true, false>(qkv, pos, tab, kc, vc, ctx, o, B, nh, nkv, ws, st);
}

template <int D>
static hipError_t decode_g_sel(const void* qkv, const int64_t* pos, const RopeTab* tab, int il, const void* kc,
                               const void* vc, int64_t ctx, void* o, int B, int nh, int nkv, void* ws,
                               hipStream_t st) {
    switch (nh / nkv) {
        case 1: return decode_rope_sel<D, 1>(qkv, pos, tab, il, kc, vc, ctx, o, B, nh, nkv, ws, st);
        case 2: return decode_rope_sel<D, 2>(qkv, pos, tab, il, kc, vc, ctx, o, B, nh, nkv, ws, st);
        case 4: return decode_rope_sel<D, 4>(qkv, pos, tab, il, kc, vc, ctx, o, B, nh, nkv, ws, st);
        default: return decode_rope_sel<D, 8>(qkv, pos, tab, il, kc, vc, ctx, o, B, nh, nkv, ws, st);
    }
}

hipError_t launch_attn_decode(int dtype, const void* qkv, const int64_t* pos, const RopeTab* tab, int il, void* kc,
                              void* vc, int64_t ctx, void* o, int B, int nh, int nkv, int d, void* ws,
                              size_t ws_bytes, hipStream_t st, bool appended) {
    if (B == 0) return hipSuccess;
    const float2* cs = tab ? tab->cs : nullptr;
    const int64_t rows = tab ? tab->rows : 1;
    // 1) append the new (rotated) key and value at slot pos[b], unless the QKV reduce already did
    if (!appended) {
        const unsigned kb = static_cast<unsigned>((static_cast<int64_t>(B) * nkv + 3) / 4);
        if (dtype == LL_BF16)
            hipLaunchKernelGGL(kv_store_kernel<bf16_t>, dim3(kb), dim3(256), 0, st, static_cast<const bf16_t*>(qkv),
                               pos, cs, rows, il, static_cast<bf16_t*>(kc), static_cast<bf16_t*>(vc), ctx, B, 1, nh,
                               nkv, d);
        else
            hipLaunchKernelGGL(kv_store_kernel<float>, dim3(kb), dim3(256), 0, st, static_cast<const float*>(qkv), pos,
                               cs, rows, il, static_cast<float*>(kc), static_cast<float*>(vc), ctx, B, 1, nh, nkv, d);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    // 2) attention over slots 0..pos[b]
    const int g = nkv > 0 ? nh / nkv : 0;
    if (attn_mfma_supported(dtype, d, nh, nkv) && (g == 1 || g == 2 || g == 4 || g == 8)) {
        if (ws_bytes < attn_decode_workspace_bytes(B, nh, d, ctx)) return hipErrorInvalidValue;
        if (d == 128) return decode_g_sel<128>(qkv, pos, tab, il, kc, vc, ctx, o, B, nh, nkv, ws, st);
        return decode_g_sel<64>(qkv, pos, tab, il, kc, vc, ctx, o, B, nh, nkv, ws, st);
    }
    const unsigned blocks = static_cast<unsigned>((static_cast<int64_t>(B) * nh + 3) / 4);
    const float scale = 1.f / sqrtf(static_cast<float>(d));
    if (dtype == LL_BF16)
        hipLaunchKernelGGL(attn_decode_generic_kernel<bf16_t>, dim3(blocks), dim3(256), 0, st,
                           static_cast<const bf16_t*>(qkv), pos, cs, rows, il, static_cast<const bf16_t*>(kc),
                           static_cast<const bf16_t*>(vc), ctx, static_cast<bf16_t*>(o), B, 1, nh, nkv, d, scale);
    else
        hipLaunchKernelGGL(attn_decode_generic_kernel<float>, dim3(blocks), dim3(256), 0, st,
                           static_cast<const float*>(qkv), pos, cs, rows, il, static_cast<const float*>(kc),
                           static_cast<const float*>(vc), ctx, static_cast<float*>(o), B, 1, nh, nkv, d, scale);
    return hipGetLastError();
}

// Chunked prefill on a cache prefix: store the chunk's (already rotated) keys and values at their
// slots, then every query attends over cache slots 0 .. its position. A small chunk gives few
// query-block workgroups; their key tiles are then shared out over nsplit workgroups each, which write
// (reference max, sum, unnormalised o) records that a combine kernel merges.
constexpr int CHUNK_SPLIT_TARGET = 256;   // workgroups aimed for when splitting keys
constexpr int CHUNK_SPLIT_MAX = 32;
static_assert(CHUNK_SPLIT_MAX <= 64, "the combine holds one split per lane");

static int chunk_hpb(int g) { return g % 4 == 0 ? 4 : (g % 2 == 0 ? 2 : 1); }

static int chunk_nsplit(int64_t B, int64_t S, int64_t nh, int64_t nkv, int64_t ctx) {
    const int64_t g = nh / nkv;
    const int64_t base = (S + 63) / 64 * B * nkv * (g / chunk_hpb(static_cast<int>(g)));
    if (base <= 0 || base >= CHUNK_SPLIT_TARGET) return 1;
    const int64_t tiles = (ctx + 63) / 64;
    const int64_t cap = std::min<int64_t>(CHUNK_SPLIT_MAX, std::max<int64_t>(1, tiles / 2));
    return static_cast<int>(std::max<int64_t>(1, std::min(cap, (CHUNK_SPLIT_TARGET + base - 1) / base)));
}

static bool chunk_mfma_path(int dtype, int64_t nh, int64_t nkv, int64_t d, int64_t ctx) {
    return attn_mfma_supported(dtype, static_cast<int>(d), static_cast<int>(nh), static_cast<int>(nkv)) &&
           ctx * nkv * d * 2 < (int64_t(1) << 32);
}

size_t attn_chunk_workspace_bytes(int dtype, int64_t B, int64_t S, int64_t nh, int64_t nkv, int64_t d, int64_t ctx) {
    if (B <= 0 || S <= 0 || nkv <= 0 || ctx <= 0 || !chunk_mfma_path(dtype, nh, nkv, d, ctx)) return 0;
    const int ns = chunk_nsplit(B, S, nh, nkv, ctx);
    return ns > 1 ? static_cast<size_t>(B * S * nh * ns * (d + 4)) * sizeof(float) : 0;
}

// One wave per (token, query head): log-sum-exp merge of its key-split records (layout [rows][nsplit][D + 4]).
template <int D>
__global__ __launch_bounds__(256) void attn_split_combine_kernel(const float* __restrict__ part,
                                                                 bf16_t* __restrict__ out, int64_t rows,
                                                                 int nsplit) {
    static_assert(D % 64 == 0 && D <= 256, "whole dims per lane");
    constexpr int DPL = D / 64;                 // output dims per lane
    const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;
    const int lane = threadIdx.x & 63;
    constexpr int REC = D + 4;
    const float* pr = part + row * nsplit * REC;
    // lane k holds split k's weight exp2(m_k - M) / sum_j l_j exp2(m_j - M) (nsplit <= 64)
    const float mk = lane < nsplit ? pr[lane * REC] : -INFINITY;
    const float lk = lane < nsplit ? pr[lane * REC + 1] : 0.f;
    const float M = wave_max(mk);     // finite: key 0 is visible to every query and lies in some split
    float wk = mk > -INFINITY ? exp2f(mk - M) : 0.f;
    wk *= 1.f / wave_sum(wk * lk);
    float acc[DPL];
#pragma unroll
    for (int i = 0; i < DPL; ++i) acc[i] = 0.f;
    const float* po = pr + 4 + lane * DPL;
#pragma unroll 4
    for (int k = 0; k < nsplit; ++k) {
        const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wk), k));
        if (w == 0.f) continue;   // a split that saw no key (uniform branch)
        if constexpr (DPL == 2) {
            const f32x2 v = *reinterpret_cast<const f32x2*>(po + k * REC);
            acc[0] += w * v[0];
            acc[1] += w * v[1];
        } else {
#pragma unroll
            for (int i = 0; i < DPL; ++i) acc[i] += w * po[k * REC + i];
        }
    }
#pragma unroll
    for (int i = 0; i < DPL; ++i) out[row * D + lane * DPL + i] = f2bf(acc[i]);
}

template <int D, int HPB>
static hipError_t chunk_go(const void* qkv, const int64_t* pos, void* o, void* kc, void* vc, int64_t ctx, int B,
                           int S, int nh, int nkv, int nsplit, float* part, hipStream_t st) {
    const int g = nh / nkv;
    const int nqb = (S + 63) / 64;
    const unsigned blocks = static_cast<unsigned>(nqb) * B * nkv * (g / HPB) * nsplit;
    const float scale_log2 = kLog2e / sqrtf(static_cast<float>(D));
    constexpr bool PIPE = m32_pipe<D>();
    constexpr int OCC = m32_occ<D, HPB>();
    if (nsplit > 1)
        hipLaunchKernelGGL((attn_prefill_m32_kernel<D, HPB, OCC, PIPE, true, true>), dim3(blocks), dim3(128 * HPB), 0,
                           st, static_cast<const bf16_t*>(qkv), pos, static_cast<bf16_t*>(o), static_cast<bf16_t*>(kc),
                           static_cast<bf16_t*>(vc), ctx, B, S, nh, nkv, scale_log2, nullptr, 0, nsplit, part);
    else
        hipLaunchKernelGGL((attn_prefill_m32_kernel<D, HPB, OCC, PIPE, true>), dim3(blocks), dim3(128 * HPB), 0, st,
                           static_cast<const bf16_t*>(qkv), pos, static_cast<bf16_t*>(o), static_cast<bf16_t*>(kc),
                           static_cast<bf16_t*>(vc), ctx, B, S, nh, nkv, scale_log2, nullptr, 0, 1, nullptr);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || nsplit == 1) return e;
    const int64_t rows = static_cast<int64_t>(B) * S * nh;
    hipLaunchKernelGGL(attn_split_combine_kernel<D>, dim3(static_cast<unsigned>((rows + 3) / 4)), dim3(256), 0, st,
                       static_cast<const float*>(part), static_cast<bf16_t*>(o), rows, nsplit);
    return hipGetLastError();
}

template <int D>
static hipError_t chunk_hpb_sel(const void* qkv, const int64_t* pos, void* o, void* kc, void* vc, int64_t ctx, int B,
                                int S, int nh, int nkv, int nsplit, float* part, hipStream_t st) {
    switch (chunk_hpb(nh / nkv)) {
        case 4: return chunk_go<D, 4>(qkv, pos, o, kc, vc, ctx, B, S, nh, nkv, nsplit, part, st);
        case 2: return chunk_go<D, 2>(qkv, pos, o, kc, vc, ctx, B, S, nh, nkv, nsplit, part, st);
        default: return chunk_go<D, 1>(qkv, pos, o, kc, vc, ctx, B, S, nh, nkv, nsplit, part, st);
    }
}

hipError_t launch_attn_prefill_chunk(int dtype, const void* qkv, const int64_t* pos, void* o, void* kc, void* vc,
                                     int64_t ctx, int B, int S, int nh, int nkv, int d, void* ws, size_t ws_bytes,
                                     hipStream_t st) {
    if (B == 0 || S == 0) return hipSuccess;
    // 1) append the chunk's keys and values at slots pos[b, s]
    const unsigned kb = static_cast<unsigned>((static_cast<int64_t>(B) * S * nkv + 3) / 4);
    if (dtype == LL_BF16)
        hipLaunchKernelGGL(kv_store_kernel<bf16_t>, dim3(kb), dim3(256), 0, st, static_cast<const bf16_t*>(qkv), pos,
                           nullptr, 1, 0, static_cast<bf16_t*>(kc), static_cast<bf16_t*>(vc), ctx, B, S, nh, nkv, d);
    else
        hipLaunchKernelGGL(kv_store_kernel<float>, dim3(kb), dim3(256), 0, st, static_cast<const float*>(qkv), pos,
                           nullptr, 1, 0, static_cast<float*>(kc), static_cast<float*>(vc), ctx, B, S, nh, nkv, d);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // 2) attention over slots 0 .. pos[b, s]
    if (chunk_mfma_path(dtype, nh, nkv, d, ctx)) {
        // key splits only with enough workspace for their records (none given: one workgroup per block)
        const size_t need = attn_chunk_workspace_bytes(dtype, B, S, nh, nkv, d, ctx);
        const int nsplit = (need > 0 && ws != nullptr && ws_bytes >= need) ? chunk_nsplit(B, S, nh, nkv, ctx) : 1;
        float* part = static_cast<float*>(ws);
        if (d == 128) return chunk_hpb_sel<128>(qkv, pos, o, kc, vc, ctx, B, S, nh, nkv, nsplit, part, st);
        return chunk_hpb_sel<64>(qkv, pos, o, kc, vc, ctx, B, S, nh, nkv, nsplit, part, st);
    }
    const unsigned blocks = static_cast<unsigned>((static_cast<int64_t>(B) * S * nh + 3) / 4);
    const float scale = 1.f / sqrtf(static_cast<float>(d));
    if (dtype == LL_BF16)
        hipLaunchKernelGGL(attn_decode_generic_kernel<bf16_t>, dim3(blocks), dim3(256), 0, st,
                           static_cast<const bf16_t*>(qkv), pos, nullptr, 1, 0, static_cast<const bf16_t*>(kc),
                           static_cast<const bf16_t*>(vc), ctx, static_cast<bf16_t*>(o), B, S, nh, nkv, d, scale);
    else
        hipLaunchKernelGGL(attn_decode_generic_kernel<float>, dim3(blocks), dim3(256), 0, st,
                           static_cast<const float*>(qkv), pos, nullptr, 1, 0, static_cast<const float*>(kc),
                           static_cast<const float*>(vc), ctx, static_cast<float*>(o), B, S, nh, nkv, d, scale);
    return hipGetLastError();
}

// Packed (varlen) prefill: sequence i is tokens cu[i] .. cu[i+1]-1 of `total`; causal attention within
// each sequence; q and k already rotated. The 32x32 matrix-op kernel with per-sequence bounds (two heads per
// workgroup, two workgroups per compute unit, as for prefill).
hipError_t launch_attn_prefill_varlen(int dtype, const void* qkv, const int* cu, int nseq, int max_seqlen, int total,
                                      void* o, int nh, int nkv, int d, hipStream_t st) {
    if (nseq == 0 || total == 0 || max_seqlen == 0) return hipSuccess;
    const bool offsets_ok = static_cast<int64_t>(max_seqlen) * (nh + 2 * nkv) * d * 2 < (int64_t(1) << 32);
    if (attn_mfma_supported(dtype, d, nh, nkv) && offsets_ok) {
        if (d == 128) return m32_sel<128>(qkv, nullptr, o, nullptr, nullptr, 1, nseq, max_seqlen, nh, nkv, cu, total, st);
        return m32_sel<64>(qkv, nullptr, o, nullptr, nullptr, 1, nseq, max_seqlen, nh, nkv, cu, total, st);
    }
    const unsigned blocks = static_cast<unsigned>((static_cast<int64_t>(total) * nh + 3) / 4);
    const float scale = 1.f / sqrtf(static_cast<float>(d));
    if (dtype == LL_BF16)
        hipLaunchKernelGGL(attn_prefill_generic_kernel<bf16_t>, dim3(blocks), dim3(256), 0, st,
                           static_cast<const bf16_t*>(qkv), nullptr, nullptr, 1, 0, static_cast<bf16_t*>(o), 1, total,
                           nh, nkv, d, scale, cu, nseq);
    else
        hipLaunchKernelGGL(attn_prefill_generic_kernel<float>, dim3(blocks), dim3(256), 0, st,
                           static_cast<const float*>(qkv), nullptr, nullptr, 1, 0, static_cast<float*>(o), 1, total,
                           nh, nkv, d, scale, cu, nseq);
    return hipGetLastError();
}

}  // namespace ll
