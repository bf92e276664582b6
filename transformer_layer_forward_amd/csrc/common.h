// Shared device/host helpers of the gfx950 kernels (CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "llama_layer.h"

namespace ll {

typedef uint16_t bf16_t;  // bfloat16 bit pattern in memory
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf2f(bf16_t b) { return __uint_as_float(static_cast<uint32_t>(b) << 16); }

// Round-to-nearest-even fp32 -> bf16 (lowers to v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ bf16_t f2bf(float f) { return __builtin_bit_cast(bf16_t, static_cast<__bf16>(f)); }

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// two fp32 -> two bf16 (round to nearest even) in one v_cvt_pk_bf16_f32; lo in bits 0..15
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

// 8 bf16 held in a 16-byte word -> 8 floats
__device__ __forceinline__ void unpack8(const uint4& u, float* f) {
    f[0] = __uint_as_float(u.x << 16); f[1] = __uint_as_float(u.x & 0xffff0000u);
    f[2] = __uint_as_float(u.y << 16); f[3] = __uint_as_float(u.y & 0xffff0000u);
    f[4] = __uint_as_float(u.z << 16); f[5] = __uint_as_float(u.z & 0xffff0000u);
    f[6] = __uint_as_float(u.w << 16); f[7] = __uint_as_float(u.w & 0xffff0000u);
}

__device__ __forceinline__ uint4 pack8(const float* f) {
    uint4 u;
    u.x = pack_bf16x2(f[0], f[1]); u.y = pack_bf16x2(f[2], f[3]);
    u.z = pack_bf16x2(f[4], f[5]); u.w = pack_bf16x2(f[6], f[7]);
    return u;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

// Device RoPE table: cs[p * (d/2) + j] = (cos(p f'_j), sin(p f'_j)), fp32 values of fp64 angles.
struct RopeTab {
    const float2* cs;
    int64_t rows;   // positions covered; device code clamps into [0, rows)
};

// Pair frequencies f'_j (j < head_dim / 2 <= 128) handed to the table kernel by value.
struct RopeFreqs {
    double f[128];
};

__device__ __forceinline__ int64_t clamp_pos(int64_t p, int64_t rows) {
    return p < 0 ? 0 : (p >= rows ? rows - 1 : p);
}

enum Epi { EPI_STORE = 0, EPI_RESIDUAL = 1, EPI_SILU = 2, EPI_ROPE = 3 };

// RoPE applied in the QKV projection's epilogue: columns [0, rope_cols) are q and k heads of size d,
// rotated at position pos[row] (the packed row layout Q|K|V keeps every head inside rope_cols).
struct RopeEpi {
    const int64_t* pos;
    RopeTab tab;
    int rope_cols;
    int d;
    int interleaved;
    // optional: also store each token's rotated key and value columns at cache slot clamp(pos[row]) of
    // [rows, ctx, nkv, d] caches (one token per sequence: decode); only the partial-sum reduce does it
    void* kc = nullptr;
    void* vc = nullptr;
    int64_t ctx = 0;
    int nh = 0, nkv = 0;
};

// ---- launchers (host) ----
hipError_t launch_rmsnorm(int dtype, const void* x, const void* g, void* y, int64_t rows, int64_t H, float eps,
                          hipStream_t st);
// out[r, :] = table[clamp(tokens[r], 0, vocab-1), :] for r < rows
hipError_t launch_embedding(int dtype, const void* table, const int64_t* tokens, void* out, int64_t rows, int64_t H,
                            int64_t vocab, hipStream_t st);
// fill cs[0 .. rows * half) of a RoPE table from the pair frequencies (enqueued on st)
hipError_t launch_rope_table(float2* cs, int64_t rows, int half, const RopeFreqs& fr, hipStream_t st);
hipError_t launch_rope_apply(int dtype, void* qkv, const int64_t* pos, RopeTab tab, int64_t tokens, int nh, int nkv,
                             int d, int interleaved, hipStream_t st);
// C[M, ldc] (epi) = X[M, K] . W^T; W has N rows (EPI_SILU: 2*inter rows, N = inter output columns).
size_t gemm_workspace_bytes(int dtype, int64_t M, int64_t N, int64_t K, int epi);
// act_blocked: EPI_SILU writes C K-blocked ([N / 64][M][64]) and EPI_STORE / EPI_RESIDUAL read X K-blocked
// ([K / 64][M][64]); only where gemm_act_blocked(dtype, M, inter, hidden) holds for the gate_up/down pair.
hipError_t launch_gemm(int dtype, int epi, const void* X, const void* W, void* C, const void* R, int64_t M,
                       int64_t N, int64_t K, void* ws, size_t ws_bytes, hipStream_t st, const RopeEpi* re = nullptr,
                       bool act_blocked = false);
bool gemm_act_blocked(int dtype, int64_t M, int64_t inter, int64_t hidden);
// whether EPI_ROPE can be fused for this projection (else the caller rotates with launch_rope_apply)
bool gemm_rope_fusable(int dtype, int64_t M, int d);
// whether a fused-RoPE projection of this shape ends in the partial-sum reduce that can also append the
// rotated keys and values to the caches (RopeEpi::kc / vc)
bool gemm_rope_appends_cache(int dtype, int64_t M, int64_t N, int64_t K, int d, int rope_cols);
hipError_t launch_attn_prefill(int dtype, const void* qkv, const int64_t* pos, const RopeTab* tab, int interleaved,
                               void* o, void* kc, void* vc, int64_t ctx, int B, int S, int nh, int nkv, int d,
                               hipStream_t st);
// chunked prefill on a cache prefix: q and k already rotated; stores the chunk's K/V at slots pos[b, s],
// then query (b, s) attends over cache slots 0 .. pos[b, s]. With ws of at least
// attn_chunk_workspace_bytes bytes small chunks split their key range over several workgroups.
size_t attn_chunk_workspace_bytes(int dtype, int64_t B, int64_t S, int64_t nh, int64_t nkv, int64_t d, int64_t ctx);
hipError_t launch_attn_prefill_chunk(int dtype, const void* qkv, const int64_t* pos, void* o, void* kc, void* vc,
                                     int64_t ctx, int B, int S, int nh, int nkv, int d, void* ws, size_t ws_bytes,
                                     hipStream_t st);
// packed (varlen) prefill: q and k already rotated; sequence i is tokens cu[i] .. cu[i+1]-1 of `total`
hipError_t launch_attn_prefill_varlen(int dtype, const void* qkv, const int* cu, int nseq, int max_seqlen, int total,
                                      void* o, int nh, int nkv, int d, hipStream_t st);
size_t attn_decode_workspace_bytes(int64_t B, int64_t nh, int64_t d, int64_t ctx);
// appended: the new keys and values are already in the caches (the QKV reduce stored them)
hipError_t launch_attn_decode(int dtype, const void* qkv, const int64_t* pos, const RopeTab* tab, int interleaved,
                              void* kc, void* vc, int64_t ctx, void* o, int B, int nh, int nkv, int d, void* ws,
                              size_t ws_bytes, hipStream_t st, bool appended = false);
bool attn_mfma_supported(int dtype, int d, int nh, int nkv);

}  // namespace ll
