// Grouped-query causal attention: prefill (flash-style, matrix cores) and KV-cache decode.
//
// Semantics (verl "parallel_attention.py" §2 eager attention; nanotron "模型层" §9.3
// flash_attn_func(causal=True); llama3 结构详解 §3.2 GQA and KV cache):
//   o[b,i,h] = sum_{j<=i} softmax_j(q'_{b,i,h} . k'_{b,j,c} / sqrt(d)) v_{b,j,c},  c = h / (n_h/n_kv).
// repeat_kv is never materialised: one workgroup serves every query head of a K/V head.
//
// Prefill kernel (bf16, d in {64, 128}): a workgroup owns (sequence b, kv head c, 64 queries) and
// runs 2 waves per query head of the group (32 queries each). Each 64-key K tile and V tile is
// staged once in LDS (double-buffered) and read by all waves of the group. Scores are formed
// transposed, S^T = K Q^T, with K as the MFMA A operand and Q (in registers) as B: the
// 16x16 output fragment then holds, per lane, one query column and 4 keys, which after the
// fp32 online softmax (exp2 with log2(e)/sqrt(d) folded into the scale) is exactly the B-operand
// layout of O^T += V^T P^T. V is transposed into LDS as [d][key] when the tile is staged.
// K rows and V^T rows are XOR-swizzled so the 16 lanes of an operand read hit distinct banks.
// Causality: query block qb only visits key tiles 0..qb; only the diagonal tile is masked.
// Blocks are issued heaviest-first (largest qb first); consecutive blocks of one qb level
// cycle over (b, c), so one (b, c) pair keeps landing on the same XCD and its K/V stays in
// that XCD's L2.
//
// Decode (bf16, d in {64, 128}, n_h/n_kv in {1, 2, 4, 8}): an append kernel writes the new key
// (rotated) and value to slot pos[b]; the split kernel gives each workgroup (b, c, 512-key chunk)
// 4 waves that step through 32-key tiles with the next tile's K and V already loading. Q K^T uses
// the matrix cores with K streamed from HBM straight into operand registers (every K element is
// used once); P V runs on the vector ALUs on V rows as stored, so V is never transposed. Waves
// merge through LDS; each workgroup writes (max, sum, o) to workspace and a combine kernel merges
// the chunks with the log-sum-exp rule.
//
// Generic kernels (fp32, or any even d <= 256): one wave per query, lanes over d, exact two-level
// online softmax; used for the fp32 configuration and for head sizes the matrix-core kernels
// do not cover.
#include "common.h"

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
                                                                   int nkv, int d, float scale) {
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
    float q[GEN_DPL], acc[GEN_DPL] = {0.f, 0.f, 0.f, 0.f};
    gen_load_head<T>(base + static_cast<int64_t>(i) * rs + static_cast<int64_t>(h) * d, d, lane, cs, rope_rows,
                     cs ? pb[i] : 0, il, q);
    float m = -INFINITY, l = 0.f;
    for (int j = 0; j <= i; ++j) {
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
                                                                  T* __restrict__ out, int B, int nh, int nkv, int d,
                                                                  float scale) {
    const int lane = threadIdx.x & 63;
    const int64_t w = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (w >= static_cast<int64_t>(B) * nh) return;
    const int h = static_cast<int>(w % nh);
    const int b = static_cast<int>(w / nh);
    const int c = h / (nh / nkv);
    const int64_t rs = static_cast<int64_t>(nh + 2 * nkv) * d;
    const int64_t p = clamp_pos(pos[b], ctx);
    float q[GEN_DPL], acc[GEN_DPL] = {0.f, 0.f, 0.f, 0.f};
    gen_load_head<T>(qkv + b * rs + static_cast<int64_t>(h) * d, d, lane, cs, rope_rows, pos[b], il, q);
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
    T* op = out + static_cast<int64_t>(b) * nh * d + static_cast<int64_t>(h) * d;
#pragma unroll
    for (int e = 0; e < GEN_DPL; ++e) {
        const int dd = lane + 64 * e;
        if (dd < d) stf<T>(op + dd, acc[e] / l);
    }
}

// ------------------------------------------------------------------ decode, matrix cores
// Workgroup = (sequence b, kv head c, 512-key chunk), 4 waves. Wave w takes the 32-key tiles
// w, w+4, w+8, w+12 of the chunk, so in each step the 4 waves stream 128 consecutive cache slots.
// Every lane loads its K fragments (MFMA A operand: key row l%16, 8 dims) and its V rows (8 dims of
// one key) for the next tile before it computes the current one, so two tiles of K and V (32 KiB
// per wave) are in flight while the matrix and vector units work; loads use clamped slot indices
// and are masked afterwards. No workgroup barrier or memory fence sits inside the key loop.
constexpr int DEC_CHUNK = 512;   // keys per workgroup
constexpr int DEC_TILE = 32;     // keys per wave step
constexpr int DEC_WAVES = 4;
constexpr int DEC_THREADS = 64 * DEC_WAVES;
constexpr int DEC_TPW = DEC_CHUNK / (DEC_TILE * DEC_WAVES);   // tiles per wave

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

// One 32-key tile: S = K q (matrix cores; column = query head, only the first G are real),
// online softmax per head in the log2 domain, then o[h][8 dims] += p V on the vector ALUs.
// P goes through this wave's private LDS rows; LDS instructions of one wave execute in order, so
// the exchange needs only a compiler barrier.
template <int D, int G>
__device__ __forceinline__ void dec_compute(const DecTile<D>& t, const bf16x8* qfr, int64_t t0, int64_t L,
                                            float scale_log2, float& m_w, float& l_w, float (&o)[G][8],
                                            float (*sPw)[G], int lrow, int lgrp, int dch, int ksub) {
    using TT = DecTile<D>;
    f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int k = 0; k < TT::KC32; ++k)
#pragma unroll
        for (int kf = 0; kf < 2; ++kf)
            sacc[kf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, t.k[kf][k]), qfr[k],
                                                                sacc[kf], 0, 0, 0);
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
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float mnew = fmaxf(m_w, mx);
    const float alpha = fast_exp2(m_w - mnew);
    m_w = mnew;
    float ls = 0.f;
#pragma unroll
    for (int kf = 0; kf < 2; ++kf)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float pr = fast_exp2(s[kf][r] - mnew);
            ls += pr;
            if (lrow < G) sPw[kf * 16 + 4 * lgrp + r][lrow] = pr;
        }
    l_w = l_w * alpha + ls;
    // alpha of head h is the same in every lane of column h: move it to scalar registers
    float al[G];
    bool rescale = false;
#pragma unroll
    for (int h = 0; h < G; ++h) {
        al[h] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, alpha), h));
        rescale |= al[h] != 1.f;
    }
    if (rescale) {
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e) o[h][e] *= al[h];
    }
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
#pragma unroll
    for (int it = 0; it < TT::PV_IT; ++it) {
        const int kr = it * TT::KPI + ksub;
        float pv[G];
        if constexpr (G % 4 == 0) {
#pragma unroll
            for (int h = 0; h < G; h += 4) {
                const float4 q4 = *reinterpret_cast<const float4*>(&sPw[kr][h]);
                pv[h] = q4.x; pv[h + 1] = q4.y; pv[h + 2] = q4.z; pv[h + 3] = q4.w;
            }
        } else {
#pragma unroll
            for (int h = 0; h < G; ++h) pv[h] = sPw[kr][h];
        }
        float vf[8];
        unpack8(t.v[it], vf);
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e) o[h][e] += pv[h] * vf[e];
    }
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// partial record per (b, h, chunk): [0] = max (log2 domain), [1] = sum, [2..2+d) = unnormalised o
template <int D, int G, bool ROPE, bool IL>
__global__ __launch_bounds__(DEC_THREADS) void attn_decode_split_kernel(
    const bf16_t* __restrict__ qkv, const int64_t* __restrict__ pos, const float2* __restrict__ cs, int64_t rope_rows,
    const bf16_t* __restrict__ kc, const bf16_t* __restrict__ vc, int64_t ctx, float* __restrict__ part, int nchunks,
    int nh, int nkv, float scale_log2) {
    using TT = DecTile<D>;
    __shared__ __align__(16) float sP[DEC_WAVES][DEC_TILE][G];
    __shared__ float sM[DEC_WAVES][G], sL[DEC_WAVES][G];
    __shared__ float sO[DEC_WAVES][G][D];

    // the kv heads of one (b, chunk) are adjacent block ids: they read adjacent 256-byte pieces of
    // the same cache rows
    const int blk = blockIdx.x;
    const int c = blk % nkv;
    const int chunk = (blk / nkv) % nchunks;
    const int b = blk / (nkv * nchunks);
    const int64_t L = clamp_pos(pos[b], ctx) + 1;
    const int64_t k0 = static_cast<int64_t>(chunk) * DEC_CHUNK;
    if (k0 >= L) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lrow = lane & 15, lgrp = lane >> 4;
    const int dch = lane % TT::DL, ksub = lane / TT::DL;
    const int64_t kstride = static_cast<int64_t>(nkv) * D;
    const bf16_t* kb = kc + (static_cast<int64_t>(b) * ctx * nkv + c) * D;
    const bf16_t* vb = vc + (static_cast<int64_t>(b) * ctx * nkv + c) * D;
    const int64_t last = L - 1;
    const int64_t base = k0 + static_cast<int64_t>(wave) * DEC_TILE;
    constexpr int64_t STEP = static_cast<int64_t>(DEC_WAVES) * DEC_TILE;

    // B operand of S = K q: column lrow = query head c*G + lrow (zero for lrow >= G), k = dims.
    // Loaded before the first K/V tile and without branches, so no wait on it holds back the tiles.
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

    // two tiles in flight from the start; tile loads are unconditional (slot indices are clamped to
    // the last valid slot), only the compute of a tile past the end is skipped
    DecTile<D> ta, tb;
    dec_load<D>(ta, kb, vb, kstride, base, last, lrow, lgrp, dch, ksub);
    dec_load<D>(tb, kb, vb, kstride, base + STEP, last, lrow, lgrp, dch, ksub);

    float m_w = -INFINITY, l_w = 0.f;   // per lane: stats of head column lrow
    float o[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) o[h][e] = 0.f;

#pragma unroll
    for (int i = 0; i < DEC_TPW; i += 2) {
        const int64_t t0 = base + i * STEP, t1 = t0 + STEP;
        if (t0 < L) dec_compute<D, G>(ta, qfr, t0, L, scale_log2, m_w, l_w, o, sP[wave], lrow, lgrp, dch, ksub);
        if (i + 2 < DEC_TPW) dec_load<D>(ta, kb, vb, kstride, t0 + 2 * STEP, last, lrow, lgrp, dch, ksub);
        if (t1 < L) dec_compute<D, G>(tb, qfr, t1, L, scale_log2, m_w, l_w, o, sP[wave], lrow, lgrp, dch, ksub);
        if (i + 3 < DEC_TPW) dec_load<D>(tb, kb, vb, kstride, t0 + 3 * STEP, last, lrow, lgrp, dch, ksub);
    }

    // reduce o over the KPI key groups of the wave, l over the 4 row groups
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e)
#pragma unroll
            for (int off = TT::DL; off < 64; off <<= 1) o[h][e] += __shfl_xor(o[h][e], off, 64);
    float lt = l_w;
    lt += __shfl_xor(lt, 16, 64);
    lt += __shfl_xor(lt, 32, 64);
    if (lgrp == 0 && lrow < G) {
        sM[wave][lrow] = m_w;      // -inf for a wave that saw no key
        sL[wave][lrow] = lt;
    }
    if (lane < TT::DL) {
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e) sO[wave][h][lane * 8 + e] = o[h][e];
    }
    __syncthreads();
    // merge the waves (wave 0 always saw key k0, so M is finite) and write the chunk partial
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
        part[((static_cast<int64_t>(b) * nh + c * G + h) * nchunks + chunk) * (D + 2) + k] = v;
    }
}

// One wave per (b, h): log-sum-exp merge of the chunk partials. The chunk loop is unrolled so the
// partial rows of several chunks are loaded together.
template <typename T>
__global__ __launch_bounds__(64) void attn_decode_combine_kernel(const float* __restrict__ part,
                                                                 const int64_t* __restrict__ pos, int64_t ctx,
                                                                 T* __restrict__ out, int nh, int d, int nchunks) {
    const int bh = blockIdx.x, lane = threadIdx.x;
    const int b = bh / nh;
    const int64_t L = clamp_pos(pos[b], ctx) + 1;
    const int nc = static_cast<int>((L + DEC_CHUNK - 1) / DEC_CHUNK);
    const int64_t rec = d + 2;
    const float* pr = part + static_cast<int64_t>(bh) * nchunks * rec;
    float M = -INFINITY;
    for (int k = lane; k < nc; k += 64) M = fmaxf(M, pr[k * rec]);
    M = wave_max(M);
    float den = 0.f;
    for (int k = lane; k < nc; k += 64) den += pr[k * rec + 1] * exp2f(pr[k * rec] - M);
    den = wave_sum(den);
    const float inv = 1.f / den;
    for (int dd = lane; dd < d; dd += 64) {
        float num = 0.f;
#pragma unroll 8
        for (int k = 0; k < nc; ++k) num += pr[k * rec + 2 + dd] * exp2f(pr[k * rec] - M);
        stf<T>(out + static_cast<int64_t>(bh) * d + dd, num * inv);
    }
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
                       static_cast<bf16_t*>(o), static_cast<bf16_t*>(kc), static_cast<bf16_t*>(vc), ctx, B, S, nh, nkv,
                       scale_log2);
    return hipGetLastError();
}

template <int D, int HPB>
static hipError_t prefill_rope_sel(const void* qkv, const int64_t* pos, const RopeTab* tab, int il, void* o, void* kc,
                                   void* vc, int64_t ctx, int B, int S, int nh, int nkv, hipStream_t st) {
    if (!tab) return prefill_go<D, HPB, false, false>(qkv, pos, tab, o, kc, vc, ctx, B, S, nh, nkv, st);
    if (il) return prefill_go<D, HPB, true, true>(qkv, pos, tab, o, kc, vc, ctx, B, S, nh, nkv, st);
    return prefill_go<D, HPB, true, false>(qkv, pos, tab, o, kc, vc, ctx, B, S, nh, nkv, st);
}

template <int D>
static hipError_t prefill_hpb_sel(const void* qkv, const int64_t* pos, const RopeTab* tab, int il, void* o, void* kc,
                                  void* vc, int64_t ctx, int B, int S, int nh, int nkv, hipStream_t st) {
    const int g = nh / nkv;
    if (g % 4 == 0) return prefill_rope_sel<D, 4>(qkv, pos, tab, il, o, kc, vc, ctx, B, S, nh, nkv, st);
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
                           d, scale);
    else
        hipLaunchKernelGGL(attn_prefill_generic_kernel<float>, dim3(blocks), dim3(256), 0, st,
                           static_cast<const float*>(qkv), pos, cs, rows, il, static_cast<float*>(o), B, S, nh, nkv, d,
                           scale);
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

size_t attn_decode_workspace_bytes(int64_t B, int64_t nh, int64_t d, int64_t ctx) {
    const int64_t nchunks = (ctx + DEC_CHUNK - 1) / DEC_CHUNK;
    return static_cast<size_t>(B * nh * nchunks * (d + 2)) * sizeof(float);
}

template <int D, int G, bool ROPE, bool IL>
static hipError_t decode_go(const void* qkv, const int64_t* pos, const RopeTab* tab, const void* kc, const void* vc,
                            int64_t ctx, void* o, int B, int nh, int nkv, void* ws, hipStream_t st) {
    const int nchunks = static_cast<int>((ctx + DEC_CHUNK - 1) / DEC_CHUNK);
    const float scale_log2 = kLog2e / sqrtf(static_cast<float>(D));
    const unsigned blocks = static_cast<unsigned>(static_cast<int64_t>(B) * nchunks * nkv);
    hipLaunchKernelGGL((attn_decode_split_kernel<D, G, ROPE, IL>), dim3(blocks), dim3(DEC_THREADS), 0, st,
                       static_cast<const bf16_t*>(qkv), pos, tab ? tab->cs : nullptr, tab ? tab->rows : 1,
                       static_cast<const bf16_t*>(kc), static_cast<const bf16_t*>(vc), ctx, static_cast<float*>(ws),
                       nchunks, nh, nkv, scale_log2);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(attn_decode_combine_kernel<bf16_t>, dim3(B * nh), dim3(64), 0, st,
                       static_cast<const float*>(ws), pos, ctx, static_cast<bf16_t*>(o), nh, D, nchunks);
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
                              size_t ws_bytes, hipStream_t st) {
    if (B == 0) return hipSuccess;
    const float2* cs = tab ? tab->cs : nullptr;
    const int64_t rows = tab ? tab->rows : 1;
    // 1) append the new (rotated) key and value at slot pos[b]
    const unsigned kb = static_cast<unsigned>((static_cast<int64_t>(B) * nkv + 3) / 4);
    if (dtype == LL_BF16)
        hipLaunchKernelGGL(kv_store_kernel<bf16_t>, dim3(kb), dim3(256), 0, st, static_cast<const bf16_t*>(qkv), pos,
                           cs, rows, il, static_cast<bf16_t*>(kc), static_cast<bf16_t*>(vc), ctx, B, 1, nh, nkv, d);
    else
        hipLaunchKernelGGL(kv_store_kernel<float>, dim3(kb), dim3(256), 0, st, static_cast<const float*>(qkv), pos, cs,
                           rows, il, static_cast<float*>(kc), static_cast<float*>(vc), ctx, B, 1, nh, nkv, d);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
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
                           static_cast<const bf16_t*>(vc), ctx, static_cast<bf16_t*>(o), B, nh, nkv, d, scale);
    else
        hipLaunchKernelGGL(attn_decode_generic_kernel<float>, dim3(blocks), dim3(256), 0, st,
                           static_cast<const float*>(qkv), pos, cs, rows, il, static_cast<const float*>(kc),
                           static_cast<const float*>(vc), ctx, static_cast<float*>(o), B, nh, nkv, d, scale);
    return hipGetLastError();
}

}  // namespace ll
