// RMSNorm and stand-alone RoPE kernels.
//
// RMSNorm (llama3 结构详解 §3.1; NJU LLM lecture 5 "编码实现RMSNorm"): one row per workgroup of
// 256 lanes; each lane loads 16-byte vectors, keeps them in registers, sums squares in fp32,
// reduces across the wave with shuffles and across the 4 waves through LDS, then writes
// x * rsqrt(mean + eps) * g rounded once. HBM-bound: 2 * H * sizeof(T) bytes per row plus the gain.
//
// Token embedding (CSDN answer "#### 5." tok_embeddings(tokens), nn.Embedding): one row per workgroup,
// copied from the table with 16-byte vectors; ids outside [0, vocab) are clamped (no out-of-bounds read).
//
// RoPE table: built on the device from the pair frequencies, fp64 angles and fp64 cos/sin rounded to fp32.
//
// RoPE apply (verl "parallel_attention.py" §1 rotary_emb/apply_rotary_pos_emb; NJU lecture 5
// "RoPE高效实现" rotate_half): one lane per (token, head, pair), in place on packed qkv, reading
// (cos, sin) from the fp32 table built from fp64 angles.
#include "common.h"

namespace ll {

template <typename T> struct VecIO;

template <> struct VecIO<bf16_t> {
    static constexpr int V = 8;
    __device__ static void load(const bf16_t* p, float* f) { unpack8(*reinterpret_cast<const uint4*>(p), f); }
    __device__ static void store(bf16_t* p, const float* f) { *reinterpret_cast<uint4*>(p) = pack8(f); }
    __device__ static float one(const bf16_t* p) { return bf2f(*p); }
    __device__ static void put(bf16_t* p, float f) { *p = f2bf(f); }
};

template <> struct VecIO<float> {
    static constexpr int V = 4;
    __device__ static void load(const float* p, float* f) {
        float4 v = *reinterpret_cast<const float4*>(p);
        f[0] = v.x; f[1] = v.y; f[2] = v.z; f[3] = v.w;
    }
    __device__ static void store(float* p, const float* f) {
        *reinterpret_cast<float4*>(p) = make_float4(f[0], f[1], f[2], f[3]);
    }
    __device__ static float one(const float* p) { return *p; }
    __device__ static void put(float* p, float f) { *p = f; }
};

constexpr int kNormThreads = 256;
constexpr int kNormCache = 4;  // vectors kept in registers per lane

// Vector path: H % V == 0. Rows longer than kNormThreads*V*kNormCache re-read the tail in pass 2.
template <typename T>
__global__ __launch_bounds__(kNormThreads) void rmsnorm_vec_kernel(const T* __restrict__ x, const T* __restrict__ g,
                                                                   T* __restrict__ y, int64_t H, float eps) {
    using IO = VecIO<T>;
    constexpr int V = IO::V;
    __shared__ float red[kNormThreads / kWave];
    const int64_t row = blockIdx.x;
    const T* xr = x + row * H;
    T* yr = y + row * H;
    const int nv = static_cast<int>(H / V);
    float cache[kNormCache][V];
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < kNormCache; ++c) {
        const int v = threadIdx.x + c * kNormThreads;
        if (v < nv) {
            IO::load(xr + static_cast<int64_t>(v) * V, cache[c]);
#pragma unroll
            for (int e = 0; e < V; ++e) ss += cache[c][e] * cache[c][e];
        }
    }
    for (int v = threadIdx.x + kNormCache * kNormThreads; v < nv; v += kNormThreads) {
        float f[V];
        IO::load(xr + static_cast<int64_t>(v) * V, f);
#pragma unroll
        for (int e = 0; e < V; ++e) ss += f[e] * f[e];
    }
    ss = wave_sum(ss);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < kNormThreads / kWave; ++w) tot += red[w];
    const float r = rsqrtf(tot / static_cast<float>(H) + eps);
#pragma unroll
    for (int c = 0; c < kNormCache; ++c) {
        const int v = threadIdx.x + c * kNormThreads;
        if (v < nv) {
            float gg[V], o[V];
            IO::load(g + static_cast<int64_t>(v) * V, gg);
#pragma unroll
            for (int e = 0; e < V; ++e) o[e] = cache[c][e] * r * gg[e];
            IO::store(yr + static_cast<int64_t>(v) * V, o);
        }
    }
    for (int v = threadIdx.x + kNormCache * kNormThreads; v < nv; v += kNormThreads) {
        float f[V], gg[V], o[V];
        IO::load(xr + static_cast<int64_t>(v) * V, f);
        IO::load(g + static_cast<int64_t>(v) * V, gg);
#pragma unroll
        for (int e = 0; e < V; ++e) o[e] = f[e] * r * gg[e];
        IO::store(yr + static_cast<int64_t>(v) * V, o);
    }
}

// Scalar path for any H.
template <typename T>
__global__ __launch_bounds__(kNormThreads) void rmsnorm_scalar_kernel(const T* __restrict__ x,
                                                                      const T* __restrict__ g, T* __restrict__ y,
                                                                      int64_t H, float eps) {
    using IO = VecIO<T>;
    __shared__ float red[kNormThreads / kWave];
    const int64_t row = blockIdx.x;
    const T* xr = x + row * H;
    T* yr = y + row * H;
    float ss = 0.f;
    for (int64_t i = threadIdx.x; i < H; i += kNormThreads) {
        float f = IO::one(xr + i);
        ss += f * f;
    }
    ss = wave_sum(ss);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < kNormThreads / kWave; ++w) tot += red[w];
    const float r = rsqrtf(tot / static_cast<float>(H) + eps);
    for (int64_t i = threadIdx.x; i < H; i += kNormThreads) IO::put(yr + i, IO::one(xr + i) * r * IO::one(g + i));
}

template <typename T>
static hipError_t rmsnorm_t(const void* x, const void* g, void* y, int64_t rows, int64_t H, float eps,
                            hipStream_t st) {
    if (rows == 0) return hipSuccess;
    const bool vec = (H % VecIO<T>::V) == 0;
    if (vec)
        hipLaunchKernelGGL(rmsnorm_vec_kernel<T>, dim3(static_cast<unsigned>(rows)), dim3(kNormThreads), 0, st,
                           static_cast<const T*>(x), static_cast<const T*>(g), static_cast<T*>(y), H, eps);
    else
        hipLaunchKernelGGL(rmsnorm_scalar_kernel<T>, dim3(static_cast<unsigned>(rows)), dim3(kNormThreads), 0, st,
                           static_cast<const T*>(x), static_cast<const T*>(g), static_cast<T*>(y), H, eps);
    return hipGetLastError();
}

hipError_t launch_rmsnorm(int dtype, const void* x, const void* g, void* y, int64_t rows, int64_t H, float eps,
                          hipStream_t st) {
    return dtype == LL_BF16 ? rmsnorm_t<bf16_t>(x, g, y, rows, H, eps, st) : rmsnorm_t<float>(x, g, y, rows, H, eps, st);
}

// ------------------------------------------------------------------ RoPE apply
template <typename T>
__global__ __launch_bounds__(256) void rope_apply_kernel(T* __restrict__ qkv, const int64_t* __restrict__ pos,
                                                         const float2* __restrict__ cs, int64_t rows, int64_t tokens,
                                                         int nh, int nkv, int d, int interleaved) {
    using IO = VecIO<T>;
    const int half = d >> 1;
    const int64_t per_tok = static_cast<int64_t>(nh + nkv) * half;
    const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (idx >= tokens * per_tok) return;
    const int64_t t = idx / per_tok;
    const int rem = static_cast<int>(idx - t * per_tok);
    const int head = rem / half;  // q heads then k heads: contiguous in the packed row
    const int j = rem - head * half;
    const int64_t p = clamp_pos(pos[t], rows);
    const float2 c = cs[p * half + j];
    T* base = qkv + t * static_cast<int64_t>(nh + 2 * nkv) * d + static_cast<int64_t>(head) * d;
    const int ia = interleaved ? 2 * j : j;
    const int ib = interleaved ? 2 * j + 1 : j + half;
    const float a = IO::one(base + ia), b = IO::one(base + ib);
    IO::put(base + ia, a * c.x - b * c.y);
    IO::put(base + ib, b * c.x + a * c.y);
}

hipError_t launch_rope_apply(int dtype, void* qkv, const int64_t* pos, RopeTab tab, int64_t tokens, int nh, int nkv,
                             int d, int interleaved, hipStream_t st) {
    const int64_t n = tokens * static_cast<int64_t>(nh + nkv) * (d / 2);
    if (n == 0) return hipSuccess;
    const unsigned blocks = static_cast<unsigned>((n + 255) / 256);
    if (dtype == LL_BF16)
        hipLaunchKernelGGL(rope_apply_kernel<bf16_t>, dim3(blocks), dim3(256), 0, st, static_cast<bf16_t*>(qkv), pos,
                           tab.cs, tab.rows, tokens, nh, nkv, d, interleaved);
    else
        hipLaunchKernelGGL(rope_apply_kernel<float>, dim3(blocks), dim3(256), 0, st, static_cast<float*>(qkv), pos,
                           tab.cs, tab.rows, tokens, nh, nkv, d, interleaved);
    return hipGetLastError();
}

// ------------------------------------------------------------------ RoPE table
// cs[p * half + j] = (cos(p f_j), sin(p f_j)) for p < rows: the angle is formed and its cosine and sine
// evaluated in double precision (the device math library), then rounded to fp32 once. One lane per entry.
__global__ __launch_bounds__(256) void rope_table_kernel(float2* __restrict__ cs, int64_t rows, int half,
                                                         RopeFreqs fr) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (i >= rows * half) return;
    const int64_t p = i / half;
    const int j = static_cast<int>(i - p * half);
    const double a = static_cast<double>(p) * fr.f[j];
    double sn, cn;
    sincos(a, &sn, &cn);
    cs[i] = make_float2(static_cast<float>(cn), static_cast<float>(sn));
}

hipError_t launch_rope_table(float2* cs, int64_t rows, int half, const RopeFreqs& fr, hipStream_t st) {
    const int64_t n = rows * half;
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(rope_table_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, st, cs, rows,
                       half, fr);
    return hipGetLastError();
}

// ------------------------------------------------------------------ token embedding
__global__ __launch_bounds__(256) void embedding_vec_kernel(const uint4* __restrict__ table,
                                                            const int64_t* __restrict__ tokens,
                                                            uint4* __restrict__ out, int64_t vecs_per_row,
                                                            int64_t vocab) {
    const int64_t row = blockIdx.x;
    int64_t id = tokens[row];
    id = id < 0 ? 0 : (id >= vocab ? vocab - 1 : id);
    const uint4* src = table + id * vecs_per_row;
    uint4* dst = out + row * vecs_per_row;
    for (int64_t i = threadIdx.x; i < vecs_per_row; i += 256) dst[i] = src[i];
}

template <typename T>
__global__ __launch_bounds__(256) void embedding_scalar_kernel(const T* __restrict__ table,
                                                               const int64_t* __restrict__ tokens,
                                                               T* __restrict__ out, int64_t H, int64_t vocab) {
    const int64_t row = blockIdx.x;
    int64_t id = tokens[row];
    id = id < 0 ? 0 : (id >= vocab ? vocab - 1 : id);
    for (int64_t i = threadIdx.x; i < H; i += 256) out[row * H + i] = table[id * H + i];
}

hipError_t launch_embedding(int dtype, const void* table, const int64_t* tokens, void* out, int64_t rows, int64_t H,
                            int64_t vocab, hipStream_t st) {
    if (rows == 0) return hipSuccess;
    const int64_t row_bytes = H * (dtype == LL_BF16 ? 2 : 4);
    const bool vec = row_bytes % 16 == 0 && (reinterpret_cast<uintptr_t>(table) & 15) == 0 &&
                     (reinterpret_cast<uintptr_t>(out) & 15) == 0;
    if (vec)
        hipLaunchKernelGGL(embedding_vec_kernel, dim3(static_cast<unsigned>(rows)), dim3(256), 0, st,
                           static_cast<const uint4*>(table), tokens, static_cast<uint4*>(out), row_bytes / 16, vocab);
    else if (dtype == LL_BF16)
        hipLaunchKernelGGL(embedding_scalar_kernel<bf16_t>, dim3(static_cast<unsigned>(rows)), dim3(256), 0, st,
                           static_cast<const bf16_t*>(table), tokens, static_cast<bf16_t*>(out), H, vocab);
    else
        hipLaunchKernelGGL(embedding_scalar_kernel<float>, dim3(static_cast<unsigned>(rows)), dim3(256), 0, st,
                           static_cast<const float*>(table), tokens, static_cast<float*>(out), H, vocab);
    return hipGetLastError();
}

}  // namespace ll
