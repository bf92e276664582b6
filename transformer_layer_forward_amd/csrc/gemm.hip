// Dense projections of the layer: C = X W^T (nn.Linear without bias, W stored [out, in]).
//
// Used for the fused QKV projection (nanotron "模型层" §9.3 qkv_proj), o_proj + residual (§9.5),
// the fused gate_up projection with the silu(gate)*up epilogue (§9.4) and down + residual.
//
// bf16 path, prefill-sized M: one workgroup of 8 waves computes a 256 (tokens) x 256 (weight rows)
// tile over K in steps of 64. Both operands are K-contiguous, so global->LDS copies are 16-byte
// row chunks; LDS rows are XOR-swizzled per 16-byte chunk so that the 16 lanes of a
// matrix-core operand read (16 rows, same chunk) hit distinct banks. Two LDS stages: the next
// K-step is copied global -> LDS with global_load_lds_dwordx4 (no register staging; when K is not a
// multiple of 64 a register-staged copy with zero-filled K tails is used instead) while the
// current one feeds v_mfma_f32_16x16x32_bf16, operand reads interleaved with the matrix ops.
// The weight tile is the MFMA A operand and the token tile the B operand, so each lane ends with
// 4 consecutive output columns of one token row (8-byte stores).
// Tiles are numbered so that each XCD (blocks are dealt round-robin to the 8 XCDs) works on a
// contiguous range of tiles, grouped 8 token-tiles deep, for L2 reuse of both operands.
//
// gate_up: the weight tile interleaves 16-row blocks of W_gate and W_up for the same output
// columns, so the gate and up accumulators of one output sit in the same lane and
// silu(g)*u is formed in registers; the [M, 2I] product is never stored.
//
// bf16 path, small M (decode): workgroups stream W straight from HBM into matrix-core operands over
// K ranges sized to fill the chip; with one range the epilogue runs in the kernel, otherwise fp32
// partial sums go to workspace and a second kernel reduces them and applies the epilogue.
//
// fp32 path: a simple LDS-tiled FMA kernel (no bf16 or reduced-precision step anywhere).
#include "common.h"
#include <type_traits>

namespace ll {

// ------------------------------------------------------------------ bf16, large M
constexpr int GB_M = 256, GB_N = 256, GB_K = 64;
constexpr int GB_WAVES_N = 2, GB_WAVES_M = 4;
constexpr int GB_NWAVES = GB_WAVES_N * GB_WAVES_M;
constexpr int GB_THREADS = 64 * GB_NWAVES;               // 512
constexpr int GB_WTN = GB_N / GB_WAVES_N;                 // 128 weight rows per wave
constexpr int GB_WTM = GB_M / GB_WAVES_M;                 // 64 tokens per wave
constexpr int GB_FN = GB_WTN / 16, GB_FM = GB_WTM / 16;   // 8 x 4 fragments
constexpr int GB_STAGE = (GB_M + GB_N) * GB_K;            // elements per LDS stage
constexpr int GB_LDS_BYTES = 2 * GB_STAGE * 2;            // 128 KiB
constexpr int GB_LOADS = (GB_M * GB_K / 8) / GB_THREADS;  // 16-byte chunks per lane per operand (4)

// physical 16-byte chunk of logical chunk c in LDS row r (rows are 8 chunks = 128 bytes)
__device__ __forceinline__ int swz8(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// RD: head size of the fused RoPE epilogue (EPI_ROPE only; 32, 64 or 128 so that every wave's
// 128 output columns hold whole heads and a fragment's rotation partner sits in the same lane).
template <int EPI, bool DIRECT, int RD = 0>
__global__ __launch_bounds__(GB_THREADS, 1) void gemm_bf16_big_kernel(
    const bf16_t* __restrict__ X, const bf16_t* __restrict__ W, bf16_t* __restrict__ C, const bf16_t* __restrict__ R,
    int M, int N, int K, int tiles_m, int tiles_n, const int64_t* __restrict__ rpos, const float2* __restrict__ rcs,
    int64_t rrows, int rope_cols, int ril) {
    extern __shared__ __align__(16) bf16_t smem[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wn = wave % GB_WAVES_N, wm = wave / GB_WAVES_N;

    // ---- tile order: contiguous range per XCD, then groups of 8 token tiles
    const int T = tiles_m * tiles_n;
    int lin = blockIdx.x;
    if ((T & 7) == 0) lin = (lin & 7) * (T >> 3) + (lin >> 3);
    constexpr int GROUP = 8;
    const int group = lin / (GROUP * tiles_n);
    const int first_m = group * GROUP;
    const int gsz = min(tiles_m - first_m, GROUP);
    const int in_g = lin - group * GROUP * tiles_n;
    const int tm = first_m + in_g % gsz;
    const int tn = in_g / gsz;
    const int m0 = tm * GB_M;
    const int ncols = (EPI == EPI_SILU) ? GB_N / 2 : GB_N;  // output columns per tile
    const int n0 = tn * ncols;

    // ---- loader bookkeeping: lane handles chunk c = tid & 7 of rows (tid >> 3) + 64 i
    const int cch = tid & 7;
    const bf16_t* xsrc[GB_LOADS];
    const bf16_t* wsrc[GB_LOADS];
    bool xok[GB_LOADS], wok[GB_LOADS];
    int xdst[GB_LOADS], wdst[GB_LOADS];
#pragma unroll
    for (int i = 0; i < GB_LOADS; ++i) {
        const int r = (tid >> 3) + i * (GB_THREADS / 8);
        const int gm = m0 + r;
        xok[i] = gm < M;
        xsrc[i] = X + static_cast<int64_t>(xok[i] ? gm : 0) * K + cch * 8;
        xdst[i] = r * GB_K + ((cch ^ swz8(r)) << 3);
        int grow;
        if (EPI == EPI_SILU) {
            const int blk = r >> 4, col = n0 + (blk >> 1) * 16 + (r & 15);
            wok[i] = col < N;
            grow = (blk & 1) ? N + col : col;
        } else {
            grow = n0 + r;
            wok[i] = grow < N;
        }
        wsrc[i] = W + static_cast<int64_t>(wok[i] ? grow : 0) * K + cch * 8;
        wdst[i] = (GB_M + r) * GB_K + ((cch ^ swz8(r)) << 3);
    }
    // direct path (K % 64 == 0): each wave copies 1 KiB blocks (8 rows x 128 B) global -> LDS with
    // global_load_lds_dwordx4; lane l lands at block + 16 l, so lane l fetches the logical chunk that the
    // swizzle puts at physical chunk l % 8 of row l / 8. Rows past M or N read a clamped valid row;
    // their results are never stored.
    constexpr int GB_DJ = 64 / GB_NWAVES;
    const bf16_t* dsrc[GB_DJ];
    if constexpr (DIRECT) {
#pragma unroll
        for (int j = 0; j < GB_DJ; ++j) {
            const int row = (j * GB_NWAVES + wave) * 8 + (lane >> 3);  // 0..511: X rows then W rows
            const int r = row & 255;
            const int c = (lane & 7) ^ swz8(r);
            if (row < 256) {
                dsrc[j] = X + static_cast<int64_t>(min(m0 + r, M - 1)) * K + c * 8;
            } else {
                int grow;
                if (EPI == EPI_SILU) {
                    const int blk = r >> 4, col = min(n0 + (blk >> 1) * 16 + (r & 15), N - 1);
                    grow = (blk & 1) ? N + col : col;
                } else {
                    grow = min(n0 + r, N - 1);
                }
                dsrc[j] = W + static_cast<int64_t>(grow) * K + c * 8;
            }
        }
    }
#define GB_DISSUE(k0, stage)                                                                                  \
    _Pragma("unroll") for (int jj_ = 0; jj_ < GB_DJ; ++jj_) {                                                 \
        __builtin_amdgcn_global_load_lds(                                                                     \
            (const __attribute__((address_space(1))) void*)(dsrc[jj_] + (k0)),                                \
            (__attribute__((address_space(3))) void*)(smem + (stage) * GB_STAGE + (jj_ * GB_NWAVES + wave) * 8 * GB_K), \
            16, 0, 0);                                                                                        \
    }
    uint4 xr[DIRECT ? 1 : GB_LOADS], wr[DIRECT ? 1 : GB_LOADS];
#define GB_GLOAD(k0)                                                                              \
    do {                                                                                          \
        const bool kok_ = ((k0) + cch * 8) < K;                                                   \
        _Pragma("unroll") for (int i = 0; i < GB_LOADS; ++i) {                                    \
            xr[i] = make_uint4(0, 0, 0, 0);                                                       \
            wr[i] = make_uint4(0, 0, 0, 0);                                                       \
            if (xok[i] && kok_) xr[i] = *reinterpret_cast<const uint4*>(xsrc[i] + (k0)); \
            if (wok[i] && kok_) wr[i] = *reinterpret_cast<const uint4*>(wsrc[i] + (k0)); \
        }                                                                                         \
    } while (0)
#define GB_SSTORE(stage)                                                                          \
    do {                                                                                          \
        bf16_t* s_ = smem + (stage) * GB_STAGE;                                                   \
        _Pragma("unroll") for (int i = 0; i < GB_LOADS; ++i) {                                    \
            *reinterpret_cast<uint4*>(s_ + xdst[i]) = xr[i];                                      \
            *reinterpret_cast<uint4*>(s_ + wdst[i]) = wr[i];                                      \
        }                                                                                         \
    } while (0)

    f32x4 acc[GB_FN][GB_FM];
#pragma unroll
    for (int a = 0; a < GB_FN; ++a)
#pragma unroll
        for (int b = 0; b < GB_FM; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

    // operand read offsets (elements) within a stage, per fragment, for the two 32-wide k halves
    const int lrow = lane & 15, lgrp = lane >> 4;
    int aoff[2][GB_FN], boff[2][GB_FM];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        const int ch = s * 4 + lgrp;
#pragma unroll
        for (int f = 0; f < GB_FN; ++f) {
            const int r = wn * GB_WTN + f * 16 + lrow;
            aoff[s][f] = (GB_M + r) * GB_K + ((ch ^ swz8(r)) << 3);
        }
#pragma unroll
        for (int f = 0; f < GB_FM; ++f) {
            const int r = wm * GB_WTM + f * 16 + lrow;
            boff[s][f] = r * GB_K + ((ch ^ swz8(r)) << 3);
        }
    }

    const int nk = (K + GB_K - 1) / GB_K;
    if constexpr (DIRECT) {
        GB_DISSUE(0, 0);
        __builtin_amdgcn_s_waitcnt(0);
    } else {
        GB_GLOAD(0);
        GB_SSTORE(0);
    }
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) {
            if constexpr (DIRECT) {
                GB_DISSUE((kt + 1) * GB_K, cur ^ 1);
            } else {
                GB_GLOAD((kt + 1) * GB_K);
            }
        }
        const bf16_t* s = smem + cur * GB_STAGE;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            bf16x8 av[GB_FN], bv[GB_FM];
#pragma unroll
            for (int f = 0; f < GB_FM; ++f) bv[f] = *reinterpret_cast<const bf16x8*>(s + boff[h][f]);
#pragma unroll
            for (int f = 0; f < GB_FN; ++f) av[f] = *reinterpret_cast<const bf16x8*>(s + aoff[h][f]);
#pragma unroll
            for (int a = 0; a < GB_FN; ++a)
#pragma unroll
                for (int b = 0; b < GB_FM; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[a], bv[b], acc[a][b], 0, 0, 0);
            // schedule: all token-operand reads plus the first weight read, then each further weight read
            // interleaved with the matrix ops of the fragment before it
            __builtin_amdgcn_sched_group_barrier(0x100, GB_FM + 1, 0);
#pragma unroll
            for (int a = 0; a < GB_FN - 1; ++a) {
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, GB_FM, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, GB_FM, 0);
        }
        if (kt + 1 < nk) {
            if constexpr (DIRECT) {
                __builtin_amdgcn_s_waitcnt(0);
            } else {
                GB_SSTORE(cur ^ 1);
            }
        }
        __syncthreads();
    }

#undef GB_GLOAD
#undef GB_SSTORE
#undef GB_DISSUE

    // ---- epilogue: lane holds rows n = base + 4*lgrp + {0..3} of token m = ... + lrow
    const int ldc = N;
    const bool vec_ok = (N & 3) == 0;  // 8-byte aligned output rows
#pragma unroll
    for (int b = 0; b < GB_FM; ++b) {
        const int m = m0 + wm * GB_WTM + b * 16 + lrow;
        if (m >= M) continue;
        bf16_t* crow = C + static_cast<int64_t>(m) * ldc;
        if constexpr (EPI == EPI_ROPE) {
            // rotate q/k columns in registers: fragment a starts at head offset (a*16) % RD
            const float2* cs_row = rcs + clamp_pos(rpos[m], rrows) * (RD / 2);
#pragma unroll
            for (int a = 0; a < GB_FN; ++a) {
                if (n0 + wn * GB_WTN + a * 16 >= rope_cols) continue;  // value columns
                constexpr int PO = RD / 32;                            // partner fragment (half-split)
                const int jh = (a * 16) % RD;
                if (!ril) {
                    if (jh < RD / 2) {
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const float2 t = cs_row[jh + 4 * lgrp + r];
                            const float x = acc[a][b][r], y = acc[(a + PO) % GB_FN][b][r];
                            acc[a][b][r] = x * t.x - y * t.y;
                            acc[(a + PO) % GB_FN][b][r] = y * t.x + x * t.y;
                        }
                    }
                } else {
#pragma unroll
                    for (int r = 0; r < 4; r += 2) {
                        const float2 t = cs_row[(jh + 4 * lgrp + r) >> 1];
                        const float x = acc[a][b][r], y = acc[a][b][r + 1];
                        acc[a][b][r] = x * t.x - y * t.y;
                        acc[a][b][r + 1] = y * t.x + x * t.y;
                    }
                }
            }
        }
        if (EPI == EPI_SILU) {
#pragma unroll
            for (int a = 0; a < GB_FN; a += 2) {
                const int n = n0 + (wn * GB_WTN) / 2 + (a >> 1) * 16 + 4 * lgrp;
                float o[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float g = acc[a][b][r], u = acc[a + 1][b][r];
                    o[r] = g * __builtin_amdgcn_rcpf(1.f + __expf(-g)) * u;
                }
                if (vec_ok && n + 3 < N) {
                    *reinterpret_cast<uint2*>(crow + n) = make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (n + r < N) crow[n + r] = f2bf(o[r]);
                }
            }
        } else {
#pragma unroll
            for (int a = 0; a < GB_FN; ++a) {
                const int n = n0 + wn * GB_WTN + a * 16 + 4 * lgrp;
                float o[4] = {acc[a][b][0], acc[a][b][1], acc[a][b][2], acc[a][b][3]};
                if (vec_ok && n + 3 < N) {
                    if (EPI == EPI_RESIDUAL) {
                        const uint2 rv = *reinterpret_cast<const uint2*>(R + static_cast<int64_t>(m) * ldc + n);
                        o[0] += __uint_as_float(rv.x << 16); o[1] += __uint_as_float(rv.x & 0xffff0000u);
                        o[2] += __uint_as_float(rv.y << 16); o[3] += __uint_as_float(rv.y & 0xffff0000u);
                    }
                    *reinterpret_cast<uint2*>(crow + n) = make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        if (n + r < N) {
                            float v = o[r];
                            if (EPI == EPI_RESIDUAL) v += bf2f(R[static_cast<int64_t>(m) * ldc + n + r]);
                            crow[n + r] = f2bf(v);
                        }
                    }
                }
            }
        }
    }
}

// ------------------------------------------------------------------ bf16, large M, 32x32 matrix ops
// One workgroup of 4 waves (one per SIMD) computes a 256 (tokens) x 256 (weight rows) tile; each wave
// owns a 128 x 128 block as 4 x 4 v_mfma_f32_32x32x16_bf16 accumulators (256 accumulation
// registers). Larger per-wave blocks than the 8-wave kernel above read a third less operand data
// from LDS per matrix op. K runs in 64-wide stages through two LDS slots filled by direct
// global->LDS loads (full 128-byte row segments); operand fragments are double-buffered in
// registers across the four k16 quarters of a stage, each stage's barrier precedes its last
// quarter, and the loads of the stage after next are spread over that quarter and the next
// stage's first. The epilogue stages each wave's results through LDS and writes whole
// output rows (RoPE rotated in fp32 first, for head sizes 64 and 128). Used when K % 64 == 0 and
// N % 8 == 0 and the operands fit 32-bit byte offsets; shapes with few tiles use the split / 128-wide
// forms below.
constexpr int MF_M = 256, MF_N = 256, MF_K = 64;
constexpr int MF_THREADS = 256;                         // 4 waves, one per SIMD, 128 x 128 each
constexpr int MF_NSLOT = 2;

// physical 16-byte chunk of logical chunk c in an LDS row of 8 chunks (128 bytes)
__device__ __forceinline__ int mf_swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

#define MF_WAITVM0() __builtin_amdgcn_s_waitcnt(0x0F70)   // vmcnt(0) only

// SPLIT: the workgroup computes one K range (kw columns; blockIdx = tile * splits + range) and writes
// its fp32 sums to P[range][M][Nw] (gate_up: gate sums at column n, up sums at N + n) for
// gemm_splitk_reduce_kernel, which applies the epilogue. Few-tile shapes use it to fill the chip.
// TN = 128: the same kernel on a 256 x 128 tile (each wave 128 x 64: 4 x 2 accumulators, 12 loads per
// wave per stage, 96 KiB of LDS) for shapes with few 256 x 256 tiles; no fused RoPE (a wave's 64
// columns hold half a head), so RoPE goes through the split partials and the reduce.
template <int EPI, int RD = 0, bool SPLIT = false, int TN = MF_N, bool XBLK = false>
__global__ __launch_bounds__(MF_THREADS, 1) void gemm_bf16_mfma32_kernel(
    const bf16_t* __restrict__ X, const bf16_t* __restrict__ W, bf16_t* __restrict__ C, const bf16_t* __restrict__ R,
    int M, int N, int K, int tiles_m, int tiles_n, const int64_t* __restrict__ rpos, const float2* __restrict__ rcs,
    int64_t rrows, int rope_cols, int ril, float* __restrict__ P = nullptr, int kw = 0, int splits = 1) {
    static_assert(EPI != EPI_ROPE || RD == 64 || RD == 128, "fused RoPE for head sizes 64 and 128");
    static_assert(!SPLIT || EPI == EPI_STORE || EPI == EPI_SILU, "split partials: plain or gate/up layout");
    static_assert((TN == 256 || TN == 128) && (TN == 256 || EPI != EPI_ROPE), "tile widths 256 and 128");
    static_assert(!XBLK || (!SPLIT && TN == MF_N && (EPI == EPI_STORE || EPI == EPI_RESIDUAL)),
                  "K-blocked X: whole-K 256-wide tiles with a plain or residual epilogue");
    constexpr int FA = TN / 64;                  // 32-row weight fragments per wave
    constexpr int STAGE = (MF_M + TN) * MF_K;    // elements per LDS stage
    constexpr int LPW = 8 + TN / 32;             // direct loads per wave per stage
    constexpr int PST = 2 * FA;                  // matrix-op pairs per k16 quarter
    extern __shared__ __align__(16) bf16_t smem[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: LDS bases stay scalar
    const int wn = wave & 1, wm = wave >> 1;
    const int l32 = lane & 31, lh = lane >> 5;

    // ---- tile order: a contiguous range per XCD, then groups of 8 token tiles
    const int T = tiles_m * tiles_n;
    int lin = blockIdx.x;
    int range = 0, kb = 0;   // K range of this workgroup: columns [kb, min(K, kb + kw))
    if constexpr (SPLIT) {
        range = lin % splits;
        lin /= splits;
        kb = range * kw;
    }
    if ((T & 7) == 0) lin = (lin & 7) * (T >> 3) + (lin >> 3);
    constexpr int GROUP = 8;
    const int group = lin / (GROUP * tiles_n);
    const int first_m = group * GROUP;
    const int gsz = min(tiles_m - first_m, GROUP);
    const int in_g = lin - group * GROUP * tiles_n;
    const int tm = first_m + in_g % gsz, tn = in_g / gsz;
    const int m0 = tm * MF_M;
    constexpr int OUT_T = EPI == EPI_SILU ? TN / 2 : TN;         // output columns per tile
    const int n0 = tn * OUT_T;

    // ---- direct loads: instruction j (0..15) of this wave fills the 128-byte segments of stage rows
    // 32(j % 8) + 8*wave + lane/8 of the X (j < 8) or W (j >= 8) half; lane l lands at physical chunk
    // l % 8, so it fetches the logical chunk cj that the row swizzle puts there (the same for every j).
    // Rows past M or N read a clamped valid row; their results are never stored. The loads are buffer
    // loads (MUBUF) into LDS: descriptors based at the tile's first token row and first weight row,
    // per-lane byte offsets fixed per instruction, the stage's k offset in the scalar offset. (The
    // global_load_lds form is a flat-segment op, after which the compiler can only wait for all LDS
    // reads at once, lgkmcnt(0), where the buffer form lets it wait for just the oldest ones.)
    const int rsub = 8 * wave + (lane >> 3);
    const int cj = (lane & 7) ^ mf_swz(rsub);
    // X row-major [M][K], or (XBLK) K-blocked [K / 64][M][64]: a stage's X slice is then 256 rows of 128
    // contiguous bytes, where row-major rows lie K * 2 bytes apart
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<bf16_t*>(X + static_cast<int64_t>(m0) * (XBLK ? MF_K : K)), (short)0, -1, 0x00020000);
    const __amdgpu_buffer_rsrc_t rw =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(W + static_cast<int64_t>(n0) * K), (short)0, -1, 0x00020000);
    // sized for the widest tile: a lambda capturing an array whose size depends on a template
    // parameter leaves the kernel without its host-side launch stub
    uint32_t voff[8 + MF_N / 32];
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
        const int r = 32 * (j < 8 ? j : j - 8) + rsub;
        int row;
        if (j < 8) {
            row = min(m0 + r, M - 1) - m0;
        } else if (EPI == EPI_SILU) {   // 16-row blocks alternate W_gate and W_up rows of the same columns
            const int blk = r >> 4, col = min(n0 + (blk >> 1) * 16 + (r & 15), N - 1);
            row = ((blk & 1) ? N + col : col) - n0;
        } else {
            row = min(n0 + r, N - 1) - n0;
        }
        const int ld = XBLK && j < 8 ? MF_K : K;
        voff[j] = static_cast<uint32_t>(row) * static_cast<uint32_t>(ld) * 2u + static_cast<uint32_t>(cj) * 16u;
    }
    auto issue1 = [&](int slot, int k0, int j) {
        const uint32_t kofs = XBLK && j < 8 ? static_cast<uint32_t>(k0 / MF_K) * static_cast<uint32_t>(M) * (MF_K * 2u)
                                            : static_cast<uint32_t>(k0) * 2u;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            j < 8 ? rx : rw, (__attribute__((address_space(3))) void*)(smem + slot * STAGE + (4 * j + wave) * 8 * MF_K),
            16, voff[j], kofs, 0, 0);
    };
    // operand fragment offsets within a stage (A: weight rows, B: tokens), one per 32-row block; k16
    // quarter q of a fragment sits at chunk (2q + lh) ^ swizzle = chunk(0) ^ 2q, i.e. offset(0) ^ 16q
    int aoff[FA], boff[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) {
        const int ra = wn * (TN / 2) + 32 * f + l32, rb = wm * 128 + 32 * f + l32;
        if (f < FA) aoff[f] = (MF_M + ra) * MF_K + ((lh ^ mf_swz(ra)) << 3);
        boff[f] = rb * MF_K + ((lh ^ mf_swz(rb)) << 3);
    }
    f32x16 acc[FA][4];
#pragma unroll
    for (int a = 0; a < FA; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.f;

    // ---- main loop. Two 64-wide K stages; the prologue issues the loads of stages 0 and 1. The barrier
    // of iteration t sits before its last k16 quarter: each wave first waits for its own loads of stage
    // t+1 and for its reads of quarter 3 of stage t (already in registers), so after the barrier stage
    // t+1 is complete in LDS and no wave reads stage t's slot again. Quarter 3's matrix ops then hide
    // the reads of stage t+1's first fragments, and the first half of stage t+2's loads go into stage
    // t's slot, one per matrix-op pair; the other half follows in quarter 0 of iteration t+1. Past the
    // last stage the loads re-read it into a slot nobody reads, which keeps the loop free of branches.
    const int nk = SPLIT ? (min(K, kb + kw) - kb) / MF_K : K / MF_K;
#pragma unroll
    for (int j = 0; j < LPW; ++j) issue1(0, kb, j);
    if (nk > 1) {
#pragma unroll
        for (int j = 0; j < LPW; ++j) issue1(1, kb + MF_K, j);
    }
    bf16x8 fa[2][FA], fb[2][4];
#define MF_MMA2(FA, FB, p)                                                                                   \
    {                                                                                                      \
        const int a_ = (p) >> 1, b_ = ((p) & 1) * 2;                                                       \
        acc[a_][b_] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(FA[a_], FB[b_], acc[a_][b_], 0, 0, 0);       \
        acc[a_][b_ + 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(FA[a_], FB[b_ + 1], acc[a_][b_ + 1], 0, 0, 0); \
    }
    constexpr int LH = LPW / 2;   // loads of a stage issued in the quarter after the barrier
    // one stage's matrix work; the first issues no loads in quarter 0 (the prologue issued stage 1)
    auto stage = [&](int t, auto first) {
        const int slot = t & 1;
        const bf16_t* st = smem + slot * STAGE;
        const bf16_t* stn = smem + (slot ^ 1) * STAGE;
        const int k1 = kb + min(t + 1, nk - 1) * MF_K, k2 = kb + min(t + 2, nk - 1) * MF_K;
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            if (h == 3) {
                __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0)
                __builtin_amdgcn_s_barrier();
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int p = 0; p < PST; ++p) {
                MF_MMA2(fa[h & 1], fb[h & 1], p)
                if (p < 4) {
                    if (h < 3) {
                        if (p < FA) fa[(h + 1) & 1][p] = *reinterpret_cast<const bf16x8*>(st + (aoff[p] ^ (16 * (h + 1))));
                        fb[(h + 1) & 1][p] = *reinterpret_cast<const bf16x8*>(st + (boff[p] ^ (16 * (h + 1))));
                    } else {   // stage t+1, quarter 0
                        if (p < FA) fa[0][p] = *reinterpret_cast<const bf16x8*>(stn + aoff[p]);
                        fb[0][p] = *reinterpret_cast<const bf16x8*>(stn + boff[p]);
                    }
                }
                // loads j of a quarter: [p * LH / PST, (p + 1) * LH / PST)
#pragma unroll
                for (int j = p * LH / PST; j < (p + 1) * LH / PST; ++j) {
                    if (h == 3) issue1(slot, k2, j);   // first half of stage t+2
                    if constexpr (!decltype(first)::value)
                        if (h == 0) issue1(slot ^ 1, k1, LH + j);   // second half of stage t+1
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };
    // no scalar load may be outstanding at the loop head: the compiler then waits for just the first
    // fragments of each stage instead of all of them (LDS returns in order, scalar loads do not)
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    // stage 0: its LPW loads are the oldest; the LPW of stage 1 may still be in flight
    constexpr int W_LPW = 0x0F70 | (LPW & 15) | ((LPW >> 4) << 14);
    static_assert(LPW < 64 && LPW % 2 == 0, "vmcnt holds 6 bits; loads in two halves");
    if (nk > 1) __builtin_amdgcn_s_waitcnt(W_LPW);
    else MF_WAITVM0();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int f = 0; f < 4; ++f) {
        if (f < FA) fa[0][f] = *reinterpret_cast<const bf16x8*>(smem + aoff[f]);
        fb[0][f] = *reinterpret_cast<const bf16x8*>(smem + boff[f]);
    }
    stage(0, std::true_type{});
    for (int t = 1; t < nk; ++t) stage(t, std::false_type{});
#undef MF_MMA2
    // ---- epilogue. Lane holds, for 32x32 block (a, b): token m = 32b + l32 of the wave's 128 and
    // weight rows 8*(r/4) + 4*lh + r%4 of block a (r = 0..15). Results are rounded once to bf16,
    // written to this wave's 32 KiB of LDS as [token][column] rows (16-byte chunks XOR-swizzled by
    // row), and then stored with full-row 16-byte-per-lane writes.
    MF_WAITVM0();                        // tail loads have landed: the ring may be overwritten
    if constexpr (SPLIT) {
        // fp32 sums straight from the accumulators: per row, the four 16-byte stores of a block's
        // register groups fill whole 128-byte lines (gate_up: 64 bytes of gate and of up sums)
        const int Nw = EPI == EPI_SILU ? 2 * N : N;
        float* pr = P + static_cast<int64_t>(range) * M * Nw;
        constexpr int OCS = EPI == EPI_SILU ? TN / 4 : TN / 2;
        const int nws = n0 + wn * OCS;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int m = m0 + wm * 128 + 32 * b + l32;
            if (m >= M) continue;
            float* prow = pr + static_cast<int64_t>(m) * Nw;
#pragma unroll
            for (int a = 0; a < FA; ++a) {
                if constexpr (EPI == EPI_SILU) {
#pragma unroll
                    for (int g = 0; g < 2; ++g) {
                        const int c = nws + 16 * a + 8 * g + 4 * lh;
                        if (c >= N) continue;
                        const f32x4 gt = {acc[a][b][4 * g], acc[a][b][4 * g + 1], acc[a][b][4 * g + 2],
                                          acc[a][b][4 * g + 3]};
                        const f32x4 up = {acc[a][b][4 * g + 8], acc[a][b][4 * g + 9], acc[a][b][4 * g + 10],
                                          acc[a][b][4 * g + 11]};
                        *reinterpret_cast<f32x4*>(prow + c) = gt;
                        *reinterpret_cast<f32x4*>(prow + N + c) = up;
                    }
                } else {
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const int c = nws + 32 * a + 8 * g + 4 * lh;
                        if (c >= N) continue;
                        const f32x4 v = {acc[a][b][4 * g], acc[a][b][4 * g + 1], acc[a][b][4 * g + 2],
                                         acc[a][b][4 * g + 3]};
                        *reinterpret_cast<f32x4*>(prow + c) = v;
                    }
                }
            }
        }
        return;
    }
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    constexpr int OC = EPI == EPI_SILU ? TN / 4 : TN / 2;    // output columns of this wave
    constexpr int GPR = OC / 8;                               // 16-byte chunks per LDS row
    bf16_t* reg = smem + wave * (128 * OC);                   // 128 token rows of the wave
    const int mw = m0 + wm * 128;                             // first token of the wave
    const int nw = n0 + wn * OC;                              // first output column of the wave
    auto lds_at = [&](int m, int c) { return reg + m * OC + (((c >> 3) ^ (m & (GPR - 1))) << 3) + (c & 7); };

    if constexpr (EPI == EPI_RESIDUAL) {
        // residual rows of the wave into LDS, to be added in fp32 below: buffer loads straight into LDS,
        // all in flight at once (loaded through registers a few at a time, the residual cost o_proj 12%
        // of its time). Load i fills rows RPI*i .. of the region; lane l lands at physical chunk l % GPR
        // of its row and fetches the logical chunk the row swizzle puts there. Rows past M read row M - 1
        // and columns past N column N - 8; neither is stored.
        constexpr int RPI = 64 / GPR;
        const int mwc = min(mw, M - 1);
        const __amdgpu_buffer_rsrc_t rr = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<bf16_t*>(R + static_cast<int64_t>(mwc) * N), (short)0, -1, 0x00020000);
#pragma unroll
        for (int i = 0; i < 128 / RPI; ++i) {
            const int m = RPI * i + lane / GPR, g = (lane % GPR) ^ (m & (GPR - 1));
            const int gm = min(mw + m, M - 1) - mwc, gn = min(nw + 8 * g, N - 8);
            const uint32_t off = (static_cast<uint32_t>(gm) * static_cast<uint32_t>(N) + static_cast<uint32_t>(gn)) * 2u;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rr, (__attribute__((address_space(3))) void*)(reg + RPI * i * OC), 16,
                                                     off, 0, 0, 0);
        }
        MF_WAITVM0();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (EPI == EPI_ROPE) {
        // Rotate q/k columns in fp32 before the single rounding. The cos/sin factors of the tile's 256 token
        // rows (RD/2 pairs a row, 16-byte chunks XOR-swizzled by row) first go into LDS with buffer loads,
        // all in flight at once: fetched from global memory a pair or two at a time, a memory round trip
        // each, they cost ~7 us per tile. Load i of wave w fills rows 64w + RPL*i ..; lane l lands at
        // physical chunk l % CPR of row RPL*i + l / CPR and takes that row's position from the lane that
        // loaded it (lane h*CPR + i holds the position of row 64w + RPL*i + h).
        constexpr int CPR = RD / 4, RPL = 64 / CPR, NLD = 64 / RPL;
        {
            const int h = lane / CPR, k = lane % CPR;
            const int mine = static_cast<int>(clamp_pos(rpos[min(m0 + 64 * wave + RPL * k + h, M - 1)], rrows));
            const __amdgpu_buffer_rsrc_t rt =
                __builtin_amdgcn_make_buffer_rsrc(const_cast<float2*>(rcs), (short)0, -1, 0x00020000);
#pragma unroll
            for (int i = 0; i < NLD; ++i) {
                const int pos = __shfl(mine, h * CPR + i, 64);
                const int row = 64 * wave + RPL * i + h;
                const int c = k ^ (row & (CPR - 1));
                const uint32_t off = static_cast<uint32_t>(pos) * (RD / 2 * 8) + static_cast<uint32_t>(c) * 16u;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rt, (__attribute__((address_space(3))) void*)(smem + (64 * wave + RPL * i) * (CPR * 8)), 16, off, 0, 0, 0);
            }
        }
        MF_WAITVM0();
        __builtin_amdgcn_s_barrier();   // every wave's factors have landed
        __builtin_amdgcn_sched_barrier(0);
        // The wave's 128 columns start on a head boundary, so block a covers head dims (32a) % RD ..; a
        // lane's register i of block a is dim 8(i/4) + 4*lh + i%4 of it. Half-split: its partner (dim + RD/2)
        // is the same register of block a + RD/64; interleaved: the neighbouring register.
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int row = wm * 128 + 32 * b + l32;   // token row within the tile
            const bf16_t* frow = smem + row * (CPR * 8);
            auto chunk = [&](int c) {   // factors 2c and 2c + 1 of this row
                return *reinterpret_cast<const float4*>(frow + ((c ^ (row & (CPR - 1))) << 3));
            };
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                if (nw + 32 * a >= rope_cols) continue;   // value columns
                const int jb = (32 * a) % RD;
                if (!ril) {
                    constexpr int PA = RD / 64;
                    if (jb < RD / 2) {
#pragma unroll
                        for (int g4 = 0; g4 < 4; ++g4) {
                            const int d0 = jb + 8 * g4 + 4 * lh;
                            const float4 u = chunk(d0 / 2), v = chunk(d0 / 2 + 1);
                            const float2 t[4] = {{u.x, u.y}, {u.z, u.w}, {v.x, v.y}, {v.z, v.w}};
#pragma unroll
                            for (int q = 0; q < 4; ++q) {
                                const int i = 4 * g4 + q;
                                const float x = acc[a][b][i], y = acc[a + PA][b][i];
                                acc[a][b][i] = x * t[q].x - y * t[q].y;
                                acc[a + PA][b][i] = y * t[q].x + x * t[q].y;
                            }
                        }
                    }
                } else {
#pragma unroll
                    for (int g4 = 0; g4 < 4; ++g4) {
                        const float4 u = chunk((jb + 8 * g4 + 4 * lh) / 4);   // pairs (d0, d0+1), (d0+2, d0+3)
                        const float2 t[2] = {{u.x, u.y}, {u.z, u.w}};
#pragma unroll
                        for (int q = 0; q < 2; ++q) {
                            const int i = 4 * g4 + 2 * q;
                            const float x = acc[a][b][i], y = acc[a][b][i + 1];
                            acc[a][b][i] = x * t[q].x - y * t[q].y;
                            acc[a][b][i + 1] = y * t[q].x + x * t[q].y;
                        }
                    }
                }
            }
        }
        __builtin_amdgcn_s_barrier();   // every wave is done with the factors before the staging below
        __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const int m = 32 * b + l32;
#pragma unroll
        for (int a = 0; a < FA; ++a) {
            if constexpr (EPI == EPI_SILU) {
                // rows 0..15 of block a are gate columns 16a.., rows 16..31 the up columns of the same outputs
#pragma unroll
                for (int g = 0; g < 2; ++g) {
                    float o[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const float gt = acc[a][b][4 * g + q], up = acc[a][b][4 * g + q + 8];
                        o[q] = gt * __builtin_amdgcn_rcpf(1.f + __expf(-gt)) * up;
                    }
                    const int c = 16 * a + 8 * g + 4 * lh;
                    *reinterpret_cast<uint2*>(lds_at(m, c)) = make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
                }
            } else {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int c = 32 * a + 8 * g + 4 * lh;
                    float o[4] = {acc[a][b][4 * g], acc[a][b][4 * g + 1], acc[a][b][4 * g + 2], acc[a][b][4 * g + 3]};
                    uint2* p = reinterpret_cast<uint2*>(lds_at(m, c));
                    if constexpr (EPI == EPI_RESIDUAL) {
                        const uint2 rv = *p;
                        o[0] += __uint_as_float(rv.x << 16); o[1] += __uint_as_float(rv.x & 0xffff0000u);
                        o[2] += __uint_as_float(rv.y << 16); o[3] += __uint_as_float(rv.y & 0xffff0000u);
                    }
                    *p = make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
                }
            }
        }
    }
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_sched_barrier(0);
    // LDS instructions of one wave execute in order: the rows are complete for this wave's reads
#pragma unroll 4
    for (int i = 0; i < 128 * GPR / 64; ++i) {
        const int e = i * 64 + lane, m = e / GPR, g = e % GPR;
        const int gm = mw + m, gn = nw + 8 * g;
        const uint4 v = *reinterpret_cast<const uint4*>(lds_at(m, 8 * g));
        if (gm < M && gn < N) *reinterpret_cast<uint4*>(C + static_cast<int64_t>(gm) * N + gn) = v;
    }
}
#undef MF_WAITVM0

// Persistent form of the gate_up kernel for shapes made of whole tiles (M % 256 == 0, N % 128 == 0, a
// tile count divisible by 8, K >= 128): one workgroup per compute unit. Workgroup b walks the tiles its
// XCD owns in the order the one-tile kernel's dispatch would run them (slot b / 8, then every nper-th
// slot), and its two-slot stage pipeline runs on across tile boundaries: the next tile's first two
// stages load during the last two stages of the current one, and no workgroup is dispatched and
// started per tile. The epilogue stages its rows through 32 KiB of LDS beyond the two slots, 8 KiB
// per wave in two passes of 64 rows, so it needs no barrier and leaves both slots to the loads in flight.
constexpr int MFP_EXTRA = 4 * 64 * (MF_N / 4) * 2;   // per wave: 64 rows x 64 output columns, bf16
constexpr int mfp_lds_bytes() { return MF_NSLOT * (MF_M + MF_N) * MF_K * 2 + MFP_EXTRA; }   // 160 KiB

template <bool CBLK>
__global__ __launch_bounds__(MF_THREADS, 1) void gemm_bf16_mfma32_silu_persist_kernel(
    const bf16_t* __restrict__ X, const bf16_t* __restrict__ W, bf16_t* __restrict__ C, int N, int K, int tiles_m,
    int tiles_n) {
    constexpr int TN = MF_N, FA = TN / 64, STAGE = (MF_M + TN) * MF_K, LPW = 8 + TN / 32, PST = 2 * FA, LH = LPW / 2;
    constexpr int OUT_T = TN / 2, OC = TN / 4, GPR = OC / 8;
    static_assert(LH == PST, "one load per matrix-op pair in the quarters that carry loads");
    extern __shared__ __align__(16) bf16_t smem[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wn = wave & 1, wm = wave >> 1;
    const int l32 = lane & 31, lh = lane >> 5;
    const int T = tiles_m * tiles_n;
    const int per_x = T >> 3, nper = static_cast<int>(gridDim.x >> 3);
    const int xcd = static_cast<int>(blockIdx.x & 7u), li = static_cast<int>(blockIdx.x >> 3);
    if (li >= per_x) return;   // the whole workgroup leaves together
    const int ntile = (per_x - li + nper - 1) / nper;
    const int nk = K / MF_K;
    // first token row and first output column of this workgroup's tile i (the one-tile kernel's order)
    auto tile_at = [&](int i, int& m0, int& n0) {
        const int lin = xcd * per_x + li + i * nper;
        const int group = lin / (8 * tiles_n);
        const int first_m = group * 8;
        const int gsz = min(tiles_m - first_m, 8);
        const int in_g = lin - group * 8 * tiles_n;
        m0 = (first_m + in_g % gsz) * MF_M;
        n0 = (in_g / gsz) * OUT_T;
    };
    // direct loads as in the one-tile kernel; whole tiles, so the row offsets do not depend on the tile
    const int rsub = 8 * wave + (lane >> 3);
    const int cj = (lane & 7) ^ mf_swz(rsub);
    uint32_t voff[LPW];
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
        const int r = 32 * (j < 8 ? j : j - 8) + rsub;
        const int row = j < 8 ? r : (((r >> 4) & 1) ? N : 0) + (r >> 5) * 16 + (r & 15);
        voff[j] = static_cast<uint32_t>(row) * static_cast<uint32_t>(K) * 2u + static_cast<uint32_t>(cj) * 16u;
    }
    int m0, n0, m0n = 0, n0n = 0;
    tile_at(0, m0, n0);
    bool has_next = ntile > 1;
    if (has_next) tile_at(1, m0n, n0n);
    auto rsrc = [&](const bf16_t* base) {
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(base), (short)0, -1, 0x00020000);
    };
    auto issue1 = [&](int slot, __amdgpu_buffer_rsrc_t rs, int kst, int j) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rs, (__attribute__((address_space(3))) void*)(smem + slot * STAGE + (4 * j + wave) * 8 * MF_K), 16, voff[j],
            kst * MF_K * 2, 0, 0);
    };
    int aoff[FA], boff[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) {
        const int ra = wn * (TN / 2) + 32 * f + l32, rb = wm * 128 + 32 * f + l32;
        if (f < FA) aoff[f] = (MF_M + ra) * MF_K + ((lh ^ mf_swz(ra)) << 3);
        boff[f] = rb * MF_K + ((lh ^ mf_swz(rb)) << 3);
    }
    f32x16 acc[FA][4];
#pragma unroll
    for (int a = 0; a < FA; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.f;
    bf16x8 fa[2][FA], fb[2][4];
#define MF_MMA2(FA, FB, p)                                                                                   \
    {                                                                                                      \
        const int a_ = (p) >> 1, b_ = ((p) & 1) * 2;                                                       \
        acc[a_][b_] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(FA[a_], FB[b_], acc[a_][b_], 0, 0, 0);       \
        acc[a_][b_ + 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(FA[a_], FB[b_ + 1], acc[a_][b_ + 1], 0, 0, 0); \
    }
    // global stage g = local stage t of the current tile; its quarter 0 issues the W half of stage g+1
    // (except the very first stage: the prologue issued stages 0 and 1 whole), its quarter 3 the X half of
    // stage g+2. A stage past the current tile is the next tile's; with no next tile it re-reads the
    // current tile's last stage into a slot nobody reads.
    auto stage = [&](int g, int t, auto first, auto last) {
        const int slot = g & 1;
        const bf16_t* st = smem + slot * STAGE;
        const bf16_t* stn = smem + (slot ^ 1) * STAGE;
        const bool n1 = t + 1 >= nk, n2 = t + 2 >= nk;
        const int k1 = n1 ? (has_next ? t + 1 - nk : nk - 1) : t + 1;
        const int k2 = n2 ? (has_next ? t + 2 - nk : nk - 1) : t + 2;
        const __amdgpu_buffer_rsrc_t rw1 = rsrc(W + static_cast<int64_t>(n1 && has_next ? n0n : n0) * K);
        const __amdgpu_buffer_rsrc_t rx2 = rsrc(X + static_cast<int64_t>(n2 && has_next ? m0n : m0) * K);
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            if (h == 3) {
                __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0)
                __builtin_amdgcn_s_barrier();
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int p = 0; p < PST; ++p) {
                MF_MMA2(fa[h & 1], fb[h & 1], p)
                if (p < 4) {
                    if (h < 3) {
                        if (p < FA) fa[(h + 1) & 1][p] = *reinterpret_cast<const bf16x8*>(st + (aoff[p] ^ (16 * (h + 1))));
                        fb[(h + 1) & 1][p] = *reinterpret_cast<const bf16x8*>(st + (boff[p] ^ (16 * (h + 1))));
                    } else if constexpr (!decltype(last)::value) {   // stage g+1, quarter 0
                        if (p < FA) fa[0][p] = *reinterpret_cast<const bf16x8*>(stn + aoff[p]);
                        fb[0][p] = *reinterpret_cast<const bf16x8*>(stn + boff[p]);
                    }
                }
                if (h == 3) issue1(slot, rx2, k2, p);
                if constexpr (!decltype(first)::value)
                    if (h == 0) issue1(slot ^ 1, rw1, k1, LH + p);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };
    {
        const __amdgpu_buffer_rsrc_t rx = rsrc(X + static_cast<int64_t>(m0) * K);
        const __amdgpu_buffer_rsrc_t rw = rsrc(W + static_cast<int64_t>(n0) * K);
#pragma unroll
        for (int j = 0; j < LPW; ++j) issue1(0, j < 8 ? rx : rw, 0, j);
#pragma unroll
        for (int j = 0; j < LPW; ++j) issue1(1, j < 8 ? rx : rw, 1, j);
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): no scalar load outstanding at the loop head
    constexpr int W_LPW = 0x0F70 | (LPW & 15) | ((LPW >> 4) << 14);
    __builtin_amdgcn_s_waitcnt(W_LPW);    // stage 0 landed; stage 1 may be in flight
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int f = 0; f < 4; ++f) {
        if (f < FA) fa[0][f] = *reinterpret_cast<const bf16x8*>(smem + aoff[f]);
        fb[0][f] = *reinterpret_cast<const bf16x8*>(smem + boff[f]);
    }
    bf16_t* reg = smem + 2 * STAGE + wave * (64 * OC);   // this wave's 8 KiB epilogue region
    auto lds_at = [&](int m, int c) { return reg + m * OC + (((c >> 3) ^ (m & (GPR - 1))) << 3) + (c & 7); };
    int g = 0;
    for (int i = 0; i < ntile; ++i) {
        // (the last stage of a tile leaves the next tile's first fragments in LDS: read after the epilogue,
        // they would stay live through it)
        if (i == 0) stage(g++, 0, std::true_type{}, std::false_type{});
        for (int t = i == 0 ? 1 : 0; t < nk - 1; ++t) stage(g++, t, std::false_type{}, std::false_type{});
        stage(g++, nk - 1, std::false_type{}, std::true_type{});
        // epilogue of tile i: silu(gate) * up rounded once, 64 token rows per pass
        const int mw = m0 + wm * 128, nw = n0 + wn * OC;
#pragma unroll
        for (int ps = 0; ps < 2; ++ps) {
#pragma unroll
            for (int bb = 0; bb < 2; ++bb) {
                const int b = 2 * ps + bb, m = 32 * bb + l32;
#pragma unroll
                for (int a = 0; a < FA; ++a)
#pragma unroll
                    for (int gg = 0; gg < 2; ++gg) {
                        float o[4];
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const float gt = acc[a][b][4 * gg + q], up = acc[a][b][4 * gg + q + 8];
                            o[q] = gt * __builtin_amdgcn_rcpf(1.f + __expf(-gt)) * up;
                        }
                        *reinterpret_cast<uint2*>(lds_at(m, 16 * a + 8 * gg + 4 * lh)) =
                            make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
                    }
            }
            // the wave's LDS instructions run in order: its rows are complete for the reads below, and
            // these reads finish before the next pass overwrites the region
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int e8 = 0; e8 < 64 * GPR / 64; ++e8) {
                const int e = e8 * 64 + lane, m = e / GPR, gq = e % GPR;
                const uint4 v = *reinterpret_cast<const uint4*>(lds_at(m, 8 * gq));
                const int row = mw + 64 * ps + m, col = nw + 8 * gq;
                // row-major [M][N], or (CBLK) K-blocked for the next projection: [N / 64][M][64]
                const int64_t at = CBLK ? (static_cast<int64_t>(col >> 6) * (tiles_m * MF_M) + row) * 64 + (col & 63)
                                        : static_cast<int64_t>(row) * N + col;
                *reinterpret_cast<uint4*>(C + at) = v;
            }
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int a = 0; a < FA; ++a)
#pragma unroll
            for (int b = 0; b < 4; ++b)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.f;
        m0 = m0n;
        n0 = n0n;
        has_next = i + 2 < ntile;
        if (has_next) tile_at(i + 2, m0n, n0n);
        if (i + 1 < ntile) {   // the next tile's first stage is complete in its slot since the last barrier
            const bf16_t* st = smem + (g & 1) * STAGE;
#pragma unroll
            for (int f = 0; f < 4; ++f) {
                if (f < FA) fa[0][f] = *reinterpret_cast<const bf16x8*>(st + aoff[f]);
                fb[0][f] = *reinterpret_cast<const bf16x8*>(st + boff[f]);
            }
        }
    }
    // the last stages' re-reads must land before the workgroup's LDS is handed to another
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
#undef MF_MMA2
}

// ------------------------------------------------------------------ bf16, small M (decode)
// With M <= 64 tokens a projection is bound by streaming W from HBM once. A workgroup of 8 waves
// owns 128 weight rows (16 per wave; gate_up: 64 gate rows and the 64 matching up rows) over one K
// range; its waves walk that range together in 256-wide sub-chunks. The 64 x 256 activation
// sub-chunk sits in LDS (rows >= M and columns past the range are zero; 16-byte chunks XOR-swizzled
// by row so the 16 rows of a B fragment read distinct banks), double-buffered and staged through
// registers one sub-chunk ahead; each wave streams its 16 weight rows through a ring of SK_U 32-wide
// k steps of loads in flight, straight into matrix-core A operands. The K ranges are sized so the
// grid is about one workgroup per compute unit. With a single range the epilogue runs in the kernel
// (gate_up: the up waves hand their sums to the gate waves through LDS); otherwise fp32 range
// partials go to workspace and a reduce kernel sums them and applies the epilogue.
constexpr int SK_MAXM = 64, SK_SC = 256, SK_WAVES = 8, SK_THREADS = 64 * SK_WAVES, SK_U = 4;
constexpr int SK_CPR = SK_SC / 8;                  // 16-byte chunks per staged activation row (32)
constexpr int SK_XPT = 64 * SK_CPR / SK_THREADS;   // chunks of one sub-chunk staged per lane (4)
constexpr int SK_STEPS = SK_SC / 32;               // k steps per sub-chunk (8)
constexpr int SK_WG_TARGET = 256;                  // workgroups aimed for (one per compute unit)
static_assert(SK_XPT * SK_THREADS == 64 * SK_CPR && SK_STEPS % SK_U == 0, "skinny tiling");

// N = output columns (the weight has 2N rows for gate_up); P = partials [splits][M][Nw] (Nw = 2N
// for gate_up) when direct == 0.
template <int EPI>
__global__ __launch_bounds__(SK_THREADS) void gemm_bf16_skinny_kernel(
    const bf16_t* __restrict__ X, const bf16_t* __restrict__ W, bf16_t* __restrict__ C, const bf16_t* __restrict__ R,
    float* __restrict__ P, int M, int N, int K, int nrb, int kw, int direct) {
    __shared__ uint4 sX[2][64 * SK_CPR];           // 2 x 32 KiB
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lrow = lane & 15, lgrp = lane >> 4;
    const int rb = blockIdx.x % nrb, kc = blockIdx.x / nrb;
    const int kbeg = kc * kw, kend = min(K, kbeg + kw);
    const int nsc = (kend - kbeg + SK_SC - 1) / SK_SC;
    // first output column of this wave's 16-row block, and the weight row of that block's first row
    int col0, wrow0;
    if (EPI == EPI_SILU) {
        col0 = rb * 64 + 16 * (wave & 3);
        wrow0 = wave < 4 ? 0 : N;                 // gate rows [0, N), up rows [N, 2N)
    } else {
        col0 = rb * 128 + 16 * wave;
        wrow0 = 0;
    }
    const bf16_t* wrow = W + static_cast<int64_t>(wrow0 + min(col0 + lrow, N - 1)) * K;
    const int kmax = K - 8;
    // k of this lane's 8 weights in global step g; steps past the range (the last sub-chunk of the last
    // range) re-read columns K-8.. of the row, which meet zero activations
    auto wk = [&](int g) { return min(kbeg + 32 * g + 8 * lgrp, kmax); };
    auto xload = [&](int sc, uint4 (&r)[SK_XPT]) {
#pragma unroll
        for (int i = 0; i < SK_XPT; ++i) {
            const int e = tid + i * SK_THREADS, m = e / SK_CPR, c = e % SK_CPR;
            const int k = kbeg + sc * SK_SC + c * 8;
            r[i] = (m < M && k < kend) ? *reinterpret_cast<const uint4*>(X + static_cast<int64_t>(m) * K + k)
                                       : make_uint4(0, 0, 0, 0);
        }
    };
    auto xstore = [&](int buf, const uint4 (&r)[SK_XPT]) {
#pragma unroll
        for (int i = 0; i < SK_XPT; ++i) {
            const int e = tid + i * SK_THREADS, m = e / SK_CPR, c = e % SK_CPR;
            sX[buf][m * SK_CPR + (c ^ (m & 15))] = r[i];
        }
    };
    const int gsteps = nsc * SK_STEPS;
    uint4 wr[SK_U];
#pragma unroll
    for (int u = 0; u < SK_U; ++u) wr[u] = *reinterpret_cast<const uint4*>(wrow + wk(u));
    uint4 xr[SK_XPT];
    xload(0, xr);
    xstore(0, xr);
    if (nsc > 1) xload(1, xr);
    __syncthreads();
    f32x4 acc[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int sc = 0; sc < nsc; ++sc) {
        const uint4* sb = sX[sc & 1];
#pragma unroll
        for (int st = 0; st < SK_STEPS; ++st) {
            const int g = sc * SK_STEPS + st;
            bf16x8 xb[4];
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const int m = 16 * b + lrow, c = 4 * st + lgrp;
                xb[b] = __builtin_bit_cast(bf16x8, sb[m * SK_CPR + (c ^ (m & 15))]);
            }
            const bf16x8 cur = __builtin_bit_cast(bf16x8, wr[st % SK_U]);
            if (g + SK_U < gsteps) wr[st % SK_U] = *reinterpret_cast<const uint4*>(wrow + wk(g + SK_U));
#pragma unroll
            for (int b = 0; b < 4; ++b) acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur, xb[b], acc[b], 0, 0, 0);
        }
        // the buffer refilled here was last read in sub-chunk sc - 1, which the barrier below it closed
        if (sc + 1 < nsc) {
            xstore((sc + 1) & 1, xr);
            if (sc + 2 < nsc) xload(sc + 2, xr);
        }
        __syncthreads();
    }
    // lane holds acc[b][r] = sum for token 16b + lrow and output column col0 + 4*lgrp + r
    const int n = col0 + 4 * lgrp;
    if (!direct) {
        const int64_t Nw = EPI == EPI_SILU ? 2 * static_cast<int64_t>(N) : N;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int m = 16 * b + lrow;
            if (m >= M) continue;
            float* prow = P + (static_cast<int64_t>(kc) * M + m) * Nw + wrow0;
            if (n + 4 <= N) {
                *reinterpret_cast<f32x4*>(prow + n) = acc[b];
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (n + r < N) prow[n + r] = acc[b][r];
            }
        }
        return;
    }
    if (EPI == EPI_SILU) {
        // the LDS buffers are free after the loop's last barrier: the up waves pass their sums over
        f32x4* sU = reinterpret_cast<f32x4*>(&sX[0][0]);
        if (wave >= 4) {
#pragma unroll
            for (int b = 0; b < 4; ++b) sU[((wave - 4) * 4 + b) * 64 + lane] = acc[b];
        }
        __syncthreads();
        if (wave >= 4) return;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const f32x4 u = sU[(wave * 4 + b) * 64 + lane];
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[b][r] = acc[b][r] / (1.f + __expf(-acc[b][r])) * u[r];
        }
    }
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const int m = 16 * b + lrow;
        if (m >= M) continue;
        const int64_t o = static_cast<int64_t>(m) * N + n;
        float v[4] = {acc[b][0], acc[b][1], acc[b][2], acc[b][3]};
        if (n + 4 <= N) {
            if (EPI == EPI_RESIDUAL) {
                const uint2 rr = *reinterpret_cast<const uint2*>(R + o);
                v[0] += __uint_as_float(rr.x << 16); v[1] += __uint_as_float(rr.x & 0xffff0000u);
                v[2] += __uint_as_float(rr.y << 16); v[3] += __uint_as_float(rr.y & 0xffff0000u);
            }
            *reinterpret_cast<uint2*>(C + o) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (n + r < N) C[o + r] = f2bf(EPI == EPI_RESIDUAL ? v[r] + bf2f(R[o + r]) : v[r]);
        }
    }
}

// ------------------------------------------------------------------ bf16, small M, LDS ring (K % 128 == 0)
// The decode projections again (M <= 64), with the weight tile streamed through a ring of three LDS
// stages by buffer loads straight into LDS: a stage is 128 weight rows x 128 columns (256 bytes of
// each row) plus the matching 64 x 128 activation block, 48 KiB; two stages are in flight while the
// third is consumed, and no registers hold data in flight. Each workgroup walks its K range starting
// at a stage rotated by its row block, so at any moment the workgroups read different column
// offsets of their rows: with all of them at the same offset, rows a power-of-two stride apart crowd
// the same memory channels (one range over K = 4096: 4.6 -> 5.1-5.4 TB/s). Wave w owns weight rows
// 16w..16w+15 (gate_up: waves 0-3 gate rows, 4-7 the up rows of the same 64 columns) and multiplies
// them by the 64 tokens with v_mfma_f32_16x16x32_bf16. Single range: epilogue in the kernel (gate_up:
// the up waves hand their sums to the gate waves through LDS); several ranges: fp32 partials for
// gemm_splitk_reduce_kernel.
// NW = 4 is the same with 64 weight rows per workgroup (4 waves; each loads 4 KiB of weights and 4 KiB
// of activations per stage): twice the row blocks for the smaller projections, so they fill the chip
// with fewer, longer K ranges.
constexpr int SR_KS = 128, SR_NST = 3, SR_XST = 64 * SR_KS;
template <int NW>
constexpr int sr_lds_bytes() { return SR_NST * (16 * NW * SR_KS + SR_XST) * 2; }   // 144 / 96 KiB
#define SR_WAIT_VM0() __builtin_amdgcn_s_waitcnt(0x0F70)

template <int EPI, int NW>
__global__ __launch_bounds__(64 * NW, 1) void gemm_bf16_skinny_ring_kernel(
    const bf16_t* __restrict__ X, const bf16_t* __restrict__ W, bf16_t* __restrict__ C, const bf16_t* __restrict__ R,
    float* __restrict__ P, int M, int N, int K, int nrb, int kw, int direct) {
    static_assert(NW == 8 || NW == 4, "8 or 4 waves");
    constexpr int SR_R = 16 * NW;                        // weight rows per workgroup
    constexpr int SR_WST = SR_R * SR_KS, SR_STAGE = SR_WST + SR_XST;
    constexpr int XL = 16 / NW;                          // activation loads per wave per stage
    constexpr int HALF = SR_R / 2;                       // gate_up: gate rows, then their up rows
    extern __shared__ __align__(16) bf16_t smem[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lrow = lane & 15, lgrp = lane >> 4;
    const int rb = blockIdx.x % nrb, kc = blockIdx.x / nrb;
    const int kbeg = kc * kw, kend = min(K, kbeg + kw);
    const int nst = (kend - kbeg) / SR_KS;
    // weight row of tile row r (clamped to a valid row; results of clamped rows are never stored)
    const int wbase = EPI == EPI_SILU ? rb * HALF : rb * SR_R;
    auto wrow_of = [&](int r) {
        if (EPI == EPI_SILU) return r < HALF ? min(wbase + r, N - 1) : N + min(wbase + r - HALF, N - 1);
        return min(wbase + r, N - 1);
    };
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<bf16_t*>(W + static_cast<int64_t>(wbase) * K), (short)0, -1, 0x00020000);
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(X), (short)0, -1, 0x00020000);
    // W load j (0..3) of this wave fills KiB 4*wave + j of a stage's weight block, X load j (0..1) KiB
    // 2*wave + j of its activation block; lane l lands in row 4*KiB + l/16 at physical 16-byte chunk
    // l%16 and fetches the logical chunk that the row's XOR swizzle (chunk ^ row%16) puts there
    uint32_t wo[4], xo[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int r = (4 * wave + j) * 4 + (lane >> 4);
        const int c = (lane & 15) ^ (r & 15);
        wo[j] = static_cast<uint32_t>(wrow_of(r) - wbase) * static_cast<uint32_t>(K) * 2u + c * 16u;
    }
#pragma unroll
    for (int j = 0; j < XL; ++j) {
        const int m = (XL * wave + j) * 4 + (lane >> 4);
        const int c = (lane & 15) ^ (m & 15);
        xo[j] = static_cast<uint32_t>(min(m, M - 1)) * static_cast<uint32_t>(K) * 2u + c * 16u;
    }
    // first stage of this workgroup's walk: 5 stages further per row block (a step of 1 put the gate
    // and up halves of gate_up's blocks in lockstep on the same channels: 67 us against 45 at M = 64)
    const int off = (rb * 5) % nst;
    auto issue = [&](int s, int slot) {
        const int sp = s + off < nst ? s + off : s + off - nst;
        const int k0 = (kbeg + sp * SR_KS) * 2;
        bf16_t* base = smem + slot * SR_STAGE;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rw, (__attribute__((address_space(3))) void*)(base + (4 * wave + j) * 512), 16, wo[j], k0, 0, 0);
#pragma unroll
        for (int j = 0; j < XL; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rx, (__attribute__((address_space(3))) void*)(base + SR_WST + (XL * wave + j) * 512), 16, xo[j], k0, 0, 0);
    };
    f32x4 acc[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
    issue(0, 0);
    if (nst > 1) issue(1, 1);
    const int ra = 16 * wave + lrow;
    for (int t = 0; t < nst; ++t) {
        // this wave's loads of stage t have landed; after the barrier every wave's have, and every wave
        // is done with stage t - 1, whose slot receives stage t + 2
        if (t + 1 < nst) {
            if constexpr (NW == 8) __builtin_amdgcn_s_waitcnt(0x0F76);   // vmcnt(6): next stage's 6 loads out
            else __builtin_amdgcn_s_waitcnt(0x0F78);                      // vmcnt(8)
        } else {
            SR_WAIT_VM0();
        }
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        if (t + 2 < nst) issue(t + 2, (t + 2) % SR_NST);
        const bf16_t* sw = smem + (t % SR_NST) * SR_STAGE;
        const bf16_t* sx = sw + SR_WST;
#pragma unroll
        for (int s = 0; s < SR_KS / 32; ++s) {
            const int c = 4 * s + lgrp;
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(sw + ra * SR_KS + ((c ^ (ra & 15)) << 3));
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const int m = 16 * b + lrow;
                const bf16x8 x = *reinterpret_cast<const bf16x8*>(sx + m * SR_KS + ((c ^ (m & 15)) << 3));
                acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, x, acc[b], 0, 0, 0);
            }
        }
    }
    // lane holds acc[b][r] = sum for token 16b + lrow and output column col0 + 4*lgrp + r
    const int col0 = EPI == EPI_SILU ? wbase + 16 * (wave % (NW / 2)) : wbase + 16 * wave;
    const int n = col0 + 4 * lgrp;
    if (!direct) {
        const int64_t Nw = EPI == EPI_SILU ? 2 * static_cast<int64_t>(N) : N;
        const int wrow0 = EPI == EPI_SILU && wave >= NW / 2 ? N : 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int m = 16 * b + lrow;
            if (m >= M || n >= N) continue;
            *reinterpret_cast<f32x4*>(P + (static_cast<int64_t>(kc) * M + m) * Nw + wrow0 + n) = acc[b];
        }
        return;
    }
    if (EPI == EPI_SILU) {
        __syncthreads();   // every wave is past its last LDS read
        f32x4* sU = reinterpret_cast<f32x4*>(smem);
        if (wave >= NW / 2) {
#pragma unroll
            for (int b = 0; b < 4; ++b) sU[((wave - NW / 2) * 4 + b) * 64 + lane] = acc[b];
        }
        __syncthreads();
        if (wave >= NW / 2) return;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const f32x4 u = sU[(wave * 4 + b) * 64 + lane];
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[b][r] = acc[b][r] / (1.f + __expf(-acc[b][r])) * u[r];
        }
    }
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const int m = 16 * b + lrow;
        if (m >= M || n >= N) continue;
        const int64_t o = static_cast<int64_t>(m) * N + n;
        float v[4] = {acc[b][0], acc[b][1], acc[b][2], acc[b][3]};
        if (EPI == EPI_RESIDUAL) {
            const uint2 rr = *reinterpret_cast<const uint2*>(R + o);
            v[0] += __uint_as_float(rr.x << 16); v[1] += __uint_as_float(rr.x & 0xffff0000u);
            v[2] += __uint_as_float(rr.y << 16); v[3] += __uint_as_float(rr.y & 0xffff0000u);
        }
        *reinterpret_cast<uint2*>(C + o) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
    }
}
#undef SR_WAIT_VM0

// Sum split partials P[splits][M][Nw] and apply the epilogue; N = output columns.
template <int EPI>
__global__ __launch_bounds__(256) void gemm_splitk_reduce_kernel(const float* __restrict__ P, bf16_t* __restrict__ C,
                                                                 const bf16_t* __restrict__ R, int M, int N, int Nw,
                                                                 int splits, const int64_t* __restrict__ rpos,
                                                                 const float2* __restrict__ rcs, int64_t rrows,
                                                                 int rope_cols, int rd, int ril) {
    const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (idx >= static_cast<int64_t>(M) * N) return;
    const int m = static_cast<int>(idx / N), n = static_cast<int>(idx - static_cast<int64_t>(m) * N);
    float s = 0.f, u = 0.f;
    for (int k = 0; k < splits; ++k) {
        const float* prow = P + (static_cast<int64_t>(k) * M + m) * Nw;
        s += prow[n];
        if (EPI == EPI_SILU) u += prow[N + n];
    }
    if (EPI == EPI_ROPE && n < rope_cols) {
        // rotation partner of column n within its head (half-split pairs (j, j+d/2) or pairs (2j, 2j+1))
        const int j = n % rd;
        int partner, t;
        float sign;
        if (ril) {
            partner = n ^ 1;
            t = j >> 1;
            sign = (j & 1) ? 1.f : -1.f;
        } else {
            partner = j < rd / 2 ? n + rd / 2 : n - rd / 2;
            t = j < rd / 2 ? j : j - rd / 2;
            sign = j < rd / 2 ? -1.f : 1.f;
        }
        float y = 0.f;
        for (int k = 0; k < splits; ++k) y += P[(static_cast<int64_t>(k) * M + m) * Nw + partner];
        const float2 c = rcs[clamp_pos(rpos[m], rrows) * (rd / 2) + t];
        s = s * c.x + sign * y * c.y;
    }
    if (EPI == EPI_SILU) s = s / (1.f + __expf(-s)) * u;
    if (EPI == EPI_RESIDUAL) s += bf2f(R[idx]);
    C[idx] = f2bf(s);
}

// The same reduce four columns per thread (N % 4 == 0): 16-byte partial loads. A RoPE partner quad is
// the quad d/2 columns away (half-split; d % 8 == 0 keeps a quad inside one half) or the quad itself
// (interleaved pairs (2j, 2j+1)).
template <int EPI>
__global__ __launch_bounds__(256) void gemm_splitk_reduce4_kernel(const float* __restrict__ P, bf16_t* __restrict__ C,
                                                                  const bf16_t* __restrict__ R, int M, int N, int Nw,
                                                                  int splits, const int64_t* __restrict__ rpos,
                                                                  const float2* __restrict__ rcs, int64_t rrows,
                                                                  int rope_cols, int rd, int ril,
                                                                  bf16_t* __restrict__ kc = nullptr,
                                                                  bf16_t* __restrict__ vc = nullptr, int64_t ctx = 0,
                                                                  int nh = 0, int nkv = 0) {
    const int64_t nq = N / 4;
    const int64_t q = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (q >= static_cast<int64_t>(M) * nq) return;
    const int m = static_cast<int>(q / nq), n = static_cast<int>(q - static_cast<int64_t>(m) * nq) * 4;
    const bool rot = EPI == EPI_ROPE && n < rope_cols;
    const int j = n % rd;
    const int pn = ril ? n : (j < rd / 2 ? n + rd / 2 : n - rd / 2);
    f32x4 s = {0.f, 0.f, 0.f, 0.f}, u = {0.f, 0.f, 0.f, 0.f}, y = {0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k < splits; ++k) {
        const float* prow = P + (static_cast<int64_t>(k) * M + m) * Nw;
        s += *reinterpret_cast<const f32x4*>(prow + n);
        if (EPI == EPI_SILU) u += *reinterpret_cast<const f32x4*>(prow + N + n);
        if (EPI == EPI_ROPE && rot && !ril) y += *reinterpret_cast<const f32x4*>(prow + pn);
    }
    float v[4] = {s[0], s[1], s[2], s[3]};
    if (EPI == EPI_ROPE && rot) {
        const float2* cs = rcs + clamp_pos(rpos[m], rrows) * (rd / 2);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int ji = j + i;
            if (ril) {
                const float2 c = cs[ji >> 1];
                v[i] = s[i] * c.x + ((ji & 1) ? 1.f : -1.f) * s[i ^ 1] * c.y;
            } else {
                const float2 c = cs[ji < rd / 2 ? ji : ji - rd / 2];
                v[i] = s[i] * c.x + (ji < rd / 2 ? -1.f : 1.f) * y[i] * c.y;
            }
        }
    }
    if (EPI == EPI_SILU) {
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = v[i] / (1.f + __expf(-v[i])) * u[i];
    }
    const int64_t o = static_cast<int64_t>(m) * N + n;
    if (EPI == EPI_RESIDUAL) {
        const uint2 rr = *reinterpret_cast<const uint2*>(R + o);
        v[0] += __uint_as_float(rr.x << 16); v[1] += __uint_as_float(rr.x & 0xffff0000u);
        v[2] += __uint_as_float(rr.y << 16); v[3] += __uint_as_float(rr.y & 0xffff0000u);
    }
    const uint2 packed = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
    *reinterpret_cast<uint2*>(C + o) = packed;
    if (EPI == EPI_ROPE && kc != nullptr && n >= nh * rd) {
        // row m is sequence m's one new token: its rotated key / value quad also goes to the cache slot
        const int col = n - nh * rd;
        const bool is_k = col < nkv * rd;
        const int cc = is_k ? col : col - nkv * rd;
        bf16_t* cache = is_k ? kc : vc;
        const int64_t slot = clamp_pos(rpos[m], ctx);
        *reinterpret_cast<uint2*>(cache + ((static_cast<int64_t>(m) * ctx + slot) * nkv + cc / rd) * rd + cc % rd) =
            packed;
    }
}

// sum the ranges and apply the epilogue: the quad kernel when N % 4 == 0 (and, for RoPE, d % 8 == 0)
template <int EPI>
static hipError_t splitk_reduce_launch(const float* P, void* C, const void* R, int64_t M, int64_t N, int64_t Nw,
                                       int splits, const RopeEpi* re, hipStream_t st) {
    const bool quad = N % 4 == 0 && (EPI != EPI_ROPE || (re && re->d % 8 == 0 && re->rope_cols % 4 == 0));
    if (quad) {
        const int64_t total = M * (N / 4);
        hipLaunchKernelGGL(gemm_splitk_reduce4_kernel<EPI>, dim3(static_cast<unsigned>((total + 255) / 256)), dim3(256),
                           0, st, P, static_cast<bf16_t*>(C), static_cast<const bf16_t*>(R), static_cast<int>(M),
                           static_cast<int>(N), static_cast<int>(Nw), splits, re ? re->pos : nullptr,
                           re ? re->tab.cs : nullptr, re ? re->tab.rows : 1, re ? re->rope_cols : 0,
                           re ? re->d : 2, re ? re->interleaved : 0, re ? static_cast<bf16_t*>(re->kc) : nullptr,
                           re ? static_cast<bf16_t*>(re->vc) : nullptr, re ? re->ctx : 0, re ? re->nh : 0,
                           re ? re->nkv : 0);
    } else {
        const int64_t total = M * N;
        hipLaunchKernelGGL(gemm_splitk_reduce_kernel<EPI>, dim3(static_cast<unsigned>((total + 255) / 256)), dim3(256),
                           0, st, P, static_cast<bf16_t*>(C), static_cast<const bf16_t*>(R), static_cast<int>(M),
                           static_cast<int>(N), static_cast<int>(Nw), splits, re ? re->pos : nullptr,
                           re ? re->tab.cs : nullptr, re ? re->tab.rows : 1, re ? re->rope_cols : 0,
                           re ? re->d : 2, re ? re->interleaved : 0);
    }
    return hipGetLastError();
}

// ------------------------------------------------------------------ fp32
constexpr int GF_T = 32, GF_K = 16;

template <int EPI>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ X, const float* __restrict__ W,
                                                       float* __restrict__ C, const float* __restrict__ R, int M,
                                                       int N, int K) {
    __shared__ float xs[GF_T][GF_K + 1];
    __shared__ float ws[2][GF_T][GF_K + 1];
    const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 32 x 8
    const int m0 = blockIdx.y * GF_T, n0 = blockIdx.x * GF_T;
    float acc[4] = {0.f, 0.f, 0.f, 0.f}, accu[4] = {0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < K; k0 += GF_K) {
        for (int e = threadIdx.x; e < GF_T * GF_K; e += 256) {
            const int r = e / GF_K, c = e % GF_K;
            const int gm = m0 + r, gk = k0 + c, gn = n0 + r;
            xs[r][c] = (gm < M && gk < K) ? X[static_cast<int64_t>(gm) * K + gk] : 0.f;
            ws[0][r][c] = (gn < N && gk < K) ? W[static_cast<int64_t>(gn) * K + gk] : 0.f;
            if (EPI == EPI_SILU) ws[1][r][c] = (gn < N && gk < K) ? W[static_cast<int64_t>(N + gn) * K + gk] : 0.f;
        }
        __syncthreads();
#pragma unroll
        for (int c = 0; c < GF_K; ++c) {
            const float w0 = ws[0][tx][c];
            const float w1 = (EPI == EPI_SILU) ? ws[1][tx][c] : 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float xv = xs[ty + 8 * i][c];
                acc[i] = fmaf(xv, w0, acc[i]);
                if (EPI == EPI_SILU) accu[i] = fmaf(xv, w1, accu[i]);
            }
        }
        __syncthreads();
    }
    const int n = n0 + tx;
    if (n >= N) return;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int m = m0 + ty + 8 * i;
        if (m >= M) continue;
        float v = acc[i];
        if (EPI == EPI_SILU) v = v / (1.f + expf(-v)) * accu[i];
        if (EPI == EPI_RESIDUAL) v += R[static_cast<int64_t>(m) * N + n];
        C[static_cast<int64_t>(m) * N + n] = v;
    }
}

// ------------------------------------------------------------------ dispatch
static bool use_skinny(int64_t M) { return M <= SK_MAXM; }

// Decode plan. The LDS-ring kernel takes K % 128 == 0 and N % 8 == 0 (every Llama projection):
// workgroups over 128 weight rows (gate_up: 64 gate rows + their 64 up rows), times up to 8 K ranges
// of whole 128-column stages, as many as fill the chip (256 workgroups) while each range keeps at
// least 8 stages (a lab sweep at M = 64 put the best counts at gate_up 1, QKV 4, o_proj 4, down 8).
// Other shapes take the register-ring kernel: workgroups over 128 output columns (gate_up: 64) times
// K ranges of a multiple of SK_SC columns, as many as keep the grid near SK_WG_TARGET workgroups. A
// single range applies the epilogue in the kernel, except RoPE, whose rotation partner lives in
// another wave.
struct SkinnyPlan {
    int nrb, splits, kw, nw;
    bool direct, ring;
};

static SkinnyPlan skinny_plan(int epi, int64_t N, int64_t K) {
    SkinnyPlan p;
    const int64_t wspan = epi == EPI_SILU ? 2 * N : 128;   // weight rows one descriptor spans
    p.ring = K % SR_KS == 0 && N % 8 == 0 && wspan * K * 2 < (int64_t(1) << 32) && 64 * K * 2 < (int64_t(1) << 32);
    p.nrb = static_cast<int>(epi == EPI_SILU ? (N + 63) / 64 : (N + 127) / 128);
    p.nw = 8;
    if (p.ring && epi != EPI_SILU && p.nrb < 128) {   // 64-row workgroups for the smaller projections
        p.nw = 4;
        p.nrb = static_cast<int>((N + 63) / 64);
    }
    if (p.ring) {
        const int64_t nks = K / SR_KS;
        const int64_t s = std::max<int64_t>(1, std::min<int64_t>({8, SK_WG_TARGET / p.nrb, nks / 8}));
        const int64_t per = (nks + s - 1) / s;
        p.splits = static_cast<int>((nks + per - 1) / per);
        p.kw = static_cast<int>(per * SR_KS);
    } else {
        const int64_t want = std::max<int64_t>(1, SK_WG_TARGET / p.nrb);
        p.kw = static_cast<int>(((K + want - 1) / want + SK_SC - 1) / SK_SC * SK_SC);
        p.splits = static_cast<int>((K + p.kw - 1) / p.kw);
    }
    p.direct = p.splits == 1 && epi != EPI_ROPE;
    return p;
}

// Plan for the MFMA kernel: tile width (256, or 128 weight rows) and K ranges. A shape with at least as
// many 256 x 256 tiles as the chip has compute units (256) runs unsplit on 256-wide tiles. Otherwise the
// plan minimises a cost model over both widths and 1..32 ranges: the waves of workgroups times one
// range's matrix time (MF_STAGE_US per 64-wide stage of a 256-wide tile, measured on the unsplit
// kernel; MF_STAGE128_US for the 128-wide tile) plus, with fp32 partials, their bytes written and read
// back (MF_PART_BPUS bytes per microsecond) and the reduce launch (MF_REDUCE_US). The 128-wide tile
// writes partials even unsplit when the epilogue is RoPE, which it cannot apply itself.
struct MfPlan {
    int tn, splits, kw;
    bool partial;   // fp32 partials + reduce kernel
};
constexpr int MF_CUS = 256, MF_MAX_SPLITS = 32;
constexpr double MF_STAGE_US = 1.43, MF_STAGE128_US = 1.10, MF_PART_BPUS = 4.0e6, MF_REDUCE_US = 4.0;

static bool mf_usable(int epi, int64_t N, int64_t K, const RopeEpi* re) {
    const int64_t wspan = epi == EPI_SILU ? 2 * N : MF_N;
    const bool offsets_ok = 2 * wspan * K < (int64_t(1) << 32) && 2 * int64_t(MF_M) * K < (int64_t(1) << 32);
    const bool rope_ok = epi != EPI_ROPE || (re && (re->d == 64 || re->d == 128));
    return K % MF_K == 0 && N % 8 == 0 && offsets_ok && rope_ok;
}

static MfPlan mf_plan(int epi, int64_t M, int64_t N, int64_t K) {
    const int64_t nk = K / MF_K, Nw = epi == EPI_SILU ? 2 * N : N, tm = (M + MF_M - 1) / MF_M;
    auto tiles = [&](int tn) { const int64_t nc = epi == EPI_SILU ? tn / 2 : tn; return tm * ((N + nc - 1) / nc); };
    MfPlan best{MF_N, 1, static_cast<int>(K), false};
    if (tiles(MF_N) >= MF_CUS) return best;
    double best_t = static_cast<double>((tiles(MF_N) + MF_CUS - 1) / MF_CUS) * nk * MF_STAGE_US;
    for (int tn : {MF_N, 128}) {
        const int64_t T = tiles(tn);
        const double stage = tn == MF_N ? MF_STAGE_US : MF_STAGE128_US;
        for (int64_t s = 1; s <= MF_MAX_SPLITS && s <= nk; ++s) {
            const int64_t per = (nk + s - 1) / s, se = (nk + per - 1) / per;   // stages per range, ranges
            if (se != s) continue;
            const bool partial = s > 1 || (tn != MF_N && epi == EPI_ROPE);
            const double t = static_cast<double>((T * s + MF_CUS - 1) / MF_CUS) * per * stage +
                             (partial ? static_cast<double>(s * M * Nw * 8) / MF_PART_BPUS + MF_REDUCE_US : 0.0);
            if (t < best_t) {
                best_t = t;
                best = MfPlan{tn, static_cast<int>(s), static_cast<int>(per * MF_K), partial};
            }
        }
    }
    return best;
}

size_t gemm_workspace_bytes(int dtype, int64_t M, int64_t N, int64_t K, int epi) {
    if (dtype != LL_BF16 || M == 0 || N == 0) return 0;
    const int64_t Nw = epi == EPI_SILU ? 2 * N : N;
    if (use_skinny(M)) {
        const SkinnyPlan p = skinny_plan(epi, N, K);
        if (p.direct) return 0;
        return static_cast<size_t>(p.splits) * M * Nw * sizeof(float);
    }
    // the RoPE head size does not change the plan; a shape the 256 x 256 kernel cannot take needs none
    RopeEpi probe{};
    probe.d = 128;
    if (!mf_usable(epi, N, K, &probe)) return 0;
    const MfPlan p = mf_plan(epi, M, N, K);
    return p.partial ? static_cast<size_t>(p.splits) * M * Nw * sizeof(float) : 0;
}

template <int EPI, bool DIRECT, int RD>
static hipError_t big_launch_t(const void* X, const void* W, void* C, const void* R, int64_t M, int64_t N, int64_t K,
                               hipStream_t st, const RopeEpi* re) {
    static bool attr = [] {
        return hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_bf16_big_kernel<EPI, DIRECT, RD>),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, GB_LDS_BYTES) == hipSuccess;
    }();
    if (!attr) return hipErrorInvalidConfiguration;
    const int ncols = EPI == EPI_SILU ? GB_N / 2 : GB_N;
    const int tm = static_cast<int>((M + GB_M - 1) / GB_M), tn = static_cast<int>((N + ncols - 1) / ncols);
    hipLaunchKernelGGL((gemm_bf16_big_kernel<EPI, DIRECT, RD>), dim3(tm * tn), dim3(GB_THREADS), GB_LDS_BYTES, st,
                       static_cast<const bf16_t*>(X), static_cast<const bf16_t*>(W), static_cast<bf16_t*>(C),
                       static_cast<const bf16_t*>(R), static_cast<int>(M), static_cast<int>(N), static_cast<int>(K), tm,
                       tn, re ? re->pos : nullptr, re ? re->tab.cs : nullptr, re ? re->tab.rows : 1,
                       re ? re->rope_cols : 0, re ? re->interleaved : 0);
    return hipGetLastError();
}

template <int EPI, int RD = 0>
static hipError_t big_launch(const void* X, const void* W, void* C, const void* R, int64_t M, int64_t N, int64_t K,
                             hipStream_t st, const RopeEpi* re = nullptr) {
    if (K % GB_K == 0) return big_launch_t<EPI, true, RD>(X, W, C, R, M, N, K, st, re);
    return big_launch_t<EPI, false, RD>(X, W, C, R, M, N, K, st, re);
}

template <int TN>
constexpr int mf_lds_bytes() { return MF_NSLOT * (MF_M + TN) * MF_K * 2; }

// raise a kernel's dynamic LDS limit (once per instantiation, through a function-scope static)
template <typename Fn>
static bool allow_lds(Fn* kernel, int bytes) {
    return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                               bytes) == hipSuccess;
}

template <int EPI, int RD = 0, int TN = MF_N, bool XBLK = false>
static hipError_t mfma32_launch(const void* X, const void* W, void* C, const void* R, int64_t M, int64_t N,
                                int64_t K, hipStream_t st, const RopeEpi* re = nullptr) {
    static const bool attr = allow_lds(&gemm_bf16_mfma32_kernel<EPI, RD, false, TN, XBLK>, mf_lds_bytes<TN>());
    if (!attr) return hipErrorInvalidConfiguration;
    const int ncols = EPI == EPI_SILU ? TN / 2 : TN;
    const int tm = static_cast<int>((M + MF_M - 1) / MF_M), tn = static_cast<int>((N + ncols - 1) / ncols);
    hipLaunchKernelGGL((gemm_bf16_mfma32_kernel<EPI, RD, false, TN, XBLK>), dim3(tm * tn), dim3(MF_THREADS),
                       mf_lds_bytes<TN>(), st, static_cast<const bf16_t*>(X), static_cast<const bf16_t*>(W),
                       static_cast<bf16_t*>(C), static_cast<const bf16_t*>(R), static_cast<int>(M), static_cast<int>(N),
                       static_cast<int>(K), tm, tn, re ? re->pos : nullptr, re ? re->tab.cs : nullptr,
                       re ? re->tab.rows : 1, re ? re->rope_cols : 0, re ? re->interleaved : 0);
    return hipGetLastError();
}

// workgroups of the persistent gate_up kernel: one per compute unit, a multiple of 8 (the XCDs take
// workgroups in turn, so each XCD gets the same number of slots)
static int mfp_workgroups() {
    static const int n = [] {
        int dev = 0, cu = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cu < 8)
            cu = 256;
        return cu / 8 * 8;
    }();
    return n;
}

// whole 256 x 128-output tiles, a tile count divisible by 8 and at least two tiles per workgroup
static bool mfp_usable(int64_t M, int64_t N, int64_t K) {
    if (M % MF_M != 0 || N % (MF_N / 2) != 0 || K % MF_K != 0 || K < 2 * MF_K) return false;
    const int64_t T = (M / MF_M) * (N / (MF_N / 2));
    return T % 8 == 0 && T >= 2 * static_cast<int64_t>(mfp_workgroups());
}

template <bool CBLK>
static hipError_t mfp_launch(const void* X, const void* W, void* C, int64_t M, int64_t N, int64_t K, hipStream_t st) {
    static const bool attr = allow_lds(&gemm_bf16_mfma32_silu_persist_kernel<CBLK>, mfp_lds_bytes());
    if (!attr) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(gemm_bf16_mfma32_silu_persist_kernel<CBLK>, dim3(static_cast<unsigned>(mfp_workgroups())),
                       dim3(MF_THREADS), mfp_lds_bytes(), st, static_cast<const bf16_t*>(X),
                       static_cast<const bf16_t*>(W), static_cast<bf16_t*>(C), static_cast<int>(N),
                       static_cast<int>(K), static_cast<int>(M / MF_M), static_cast<int>(N / (MF_N / 2)));
    return hipGetLastError();
}

// K ranges of the MFMA kernel into fp32 partials (PE: plain layout, or gate/up apart for silu·up)
template <int PE, int TN>
static hipError_t mfma32_partials_launch(const void* X, const void* W, int64_t M, int64_t N, int64_t K,
                                         const MfPlan& p, void* ws, hipStream_t st) {
    static const bool attr = allow_lds(&gemm_bf16_mfma32_kernel<PE, 0, true, TN>, mf_lds_bytes<TN>());
    if (!attr) return hipErrorInvalidConfiguration;
    const int ncols = PE == EPI_SILU ? TN / 2 : TN;
    const int tm = static_cast<int>((M + MF_M - 1) / MF_M), tn = static_cast<int>((N + ncols - 1) / ncols);
    hipLaunchKernelGGL((gemm_bf16_mfma32_kernel<PE, 0, true, TN>), dim3(tm * tn * p.splits), dim3(MF_THREADS),
                       mf_lds_bytes<TN>(), st, static_cast<const bf16_t*>(X), static_cast<const bf16_t*>(W), nullptr,
                       nullptr, static_cast<int>(M), static_cast<int>(N), static_cast<int>(K), tm, tn, nullptr,
                       nullptr, int64_t(1), 0, 0, static_cast<float*>(ws), p.kw, p.splits);
    return hipGetLastError();
}

// partials, then the reduce sums the ranges and applies the epilogue
template <int EPI, int TN>
static hipError_t mfma32_split_launch_t(const void* X, const void* W, void* C, const void* R, int64_t M, int64_t N,
                                        int64_t K, const MfPlan& p, void* ws, hipStream_t st, const RopeEpi* re) {
    constexpr int PE = EPI == EPI_SILU ? EPI_SILU : EPI_STORE;
    hipError_t e = mfma32_partials_launch<PE, TN>(X, W, M, N, K, p, ws, st);
    if (e != hipSuccess) return e;
    const int64_t Nw = EPI == EPI_SILU ? 2 * N : N;
    return splitk_reduce_launch<EPI>(static_cast<const float*>(ws), C, R, M, N, Nw, p.splits, re, st);
}

template <int EPI>
static hipError_t mfma32_split_launch(const void* X, const void* W, void* C, const void* R, int64_t M, int64_t N,
                                      int64_t K, const MfPlan& p, void* ws, hipStream_t st,
                                      const RopeEpi* re = nullptr) {
    if (p.tn == MF_N) return mfma32_split_launch_t<EPI, MF_N>(X, W, C, R, M, N, K, p, ws, st, re);
    return mfma32_split_launch_t<EPI, 128>(X, W, C, R, M, N, K, p, ws, st, re);
}

template <int EPI, int NW>
static hipError_t skinny_ring_launch(const void* X, const void* W, void* C, const void* R, int64_t M, int64_t N,
                                     int64_t K, const SkinnyPlan& p, void* ws, hipStream_t st) {
    static const bool attr = allow_lds(&gemm_bf16_skinny_ring_kernel<EPI, NW>, sr_lds_bytes<NW>());
    if (!attr) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((gemm_bf16_skinny_ring_kernel<EPI, NW>), dim3(static_cast<unsigned>(p.nrb) * p.splits),
                       dim3(64 * NW), sr_lds_bytes<NW>(), st, static_cast<const bf16_t*>(X),
                       static_cast<const bf16_t*>(W), static_cast<bf16_t*>(C), static_cast<const bf16_t*>(R),
                       static_cast<float*>(ws), static_cast<int>(M), static_cast<int>(N), static_cast<int>(K), p.nrb,
                       p.kw, p.direct ? 1 : 0);
    return hipGetLastError();
}

template <int EPI>
static hipError_t skinny_launch(const void* X, const void* W, void* C, const void* R, int64_t M, int64_t N, int64_t K,
                                void* ws, hipStream_t st, const RopeEpi* re = nullptr) {
    const SkinnyPlan p = skinny_plan(EPI, N, K);
    const int64_t Nw = EPI == EPI_SILU ? 2 * N : N;
    if (p.ring) {
        hipError_t el = p.nw == 8 ? skinny_ring_launch<EPI, 8>(X, W, C, R, M, N, K, p, ws, st)
                                  : skinny_ring_launch<EPI, 4>(X, W, C, R, M, N, K, p, ws, st);
        if (el != hipSuccess) return el;
    } else {
        hipLaunchKernelGGL(gemm_bf16_skinny_kernel<EPI>, dim3(static_cast<unsigned>(p.nrb) * p.splits),
                           dim3(SK_THREADS), 0, st, static_cast<const bf16_t*>(X), static_cast<const bf16_t*>(W),
                           static_cast<bf16_t*>(C), static_cast<const bf16_t*>(R), static_cast<float*>(ws),
                           static_cast<int>(M), static_cast<int>(N), static_cast<int>(K), p.nrb, p.kw,
                           p.direct ? 1 : 0);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.direct) return e;
    return splitk_reduce_launch<EPI>(static_cast<const float*>(ws), C, R, M, N, Nw, p.splits, re, st);
}

template <int EPI>
static hipError_t f32_launch(const void* X, const void* W, void* C, const void* R, int64_t M, int64_t N, int64_t K,
                             hipStream_t st) {
    dim3 grid(static_cast<unsigned>((N + GF_T - 1) / GF_T), static_cast<unsigned>((M + GF_T - 1) / GF_T));
    hipLaunchKernelGGL(gemm_f32_kernel<EPI>, grid, dim3(256), 0, st, static_cast<const float*>(X),
                       static_cast<const float*>(W), static_cast<float*>(C), static_cast<const float*>(R),
                       static_cast<int>(M), static_cast<int>(N), static_cast<int>(K));
    return hipGetLastError();
}

bool gemm_rope_appends_cache(int dtype, int64_t M, int64_t N, int64_t K, int d, int rope_cols) {
    if (dtype != LL_BF16 || N % 4 || d % 8 || rope_cols % 4) return false;
    if (use_skinny(M)) return true;   // the decode kernels never rotate: always partials + the reduce
    RopeEpi probe{};
    probe.d = d;
    return mf_usable(EPI_ROPE, N, K, &probe) && mf_plan(EPI_ROPE, M, N, K).partial;
}

bool gemm_rope_fusable(int dtype, int64_t M, int d) {
    if (dtype != LL_BF16) return false;
    if (use_skinny(M)) return d >= 2 && d % 2 == 0;
    return d == 32 || d == 64 || d == 128;
}

// whether the gate_up output can be handed to the down projection K-blocked ([inter / 64][M][64]): both
// projections run whole 256 x 256 tiles over all of K (gate_up the persistent kernel), and the blocked
// offsets fit the down kernel's 32-bit byte offsets
bool gemm_act_blocked(int dtype, int64_t M, int64_t inter, int64_t hidden) {
    if (dtype != LL_BF16 || M == 0 || use_skinny(M) || inter % MF_K != 0) return false;
    if (!mf_usable(EPI_SILU, inter, hidden, nullptr) || !mfp_usable(M, inter, hidden)) return false;
    const MfPlan pu = mf_plan(EPI_SILU, M, inter, hidden);
    if (pu.partial || pu.tn != MF_N) return false;
    if (!mf_usable(EPI_RESIDUAL, hidden, inter, nullptr)) return false;
    const MfPlan pd = mf_plan(EPI_RESIDUAL, M, hidden, inter);
    return !pd.partial && pd.tn == MF_N && M * inter * 2 < (int64_t(1) << 32);
}

hipError_t launch_gemm(int dtype, int epi, const void* X, const void* W, void* C, const void* R, int64_t M, int64_t N,
                       int64_t K, void* ws, size_t ws_bytes, hipStream_t st, const RopeEpi* re, bool act_blocked) {
    if (M == 0 || N == 0) return hipSuccess;
    if (act_blocked) {   // the caller checked gemm_act_blocked for this pair of projections
        if (epi == EPI_SILU) return mfp_launch<true>(X, W, C, M, N, K, st);
        if (epi == EPI_RESIDUAL) return mfma32_launch<EPI_RESIDUAL, 0, MF_N, true>(X, W, C, R, M, N, K, st);
        if (epi == EPI_STORE) return mfma32_launch<EPI_STORE, 0, MF_N, true>(X, W, C, R, M, N, K, st);
        return hipErrorInvalidValue;
    }
    if (epi == EPI_ROPE && (!re || !gemm_rope_fusable(dtype, M, re->d))) return hipErrorInvalidValue;
    if (dtype == LL_F32) {
        switch (epi) {
            case EPI_STORE: return f32_launch<EPI_STORE>(X, W, C, R, M, N, K, st);
            case EPI_RESIDUAL: return f32_launch<EPI_RESIDUAL>(X, W, C, R, M, N, K, st);
            default: return f32_launch<EPI_SILU>(X, W, C, R, M, N, K, st);
        }
    }
    if (use_skinny(M)) {
        if (ws_bytes < gemm_workspace_bytes(dtype, M, N, K, epi)) return hipErrorInvalidValue;
        switch (epi) {
            case EPI_STORE: return skinny_launch<EPI_STORE>(X, W, C, R, M, N, K, ws, st);
            case EPI_RESIDUAL: return skinny_launch<EPI_RESIDUAL>(X, W, C, R, M, N, K, ws, st);
            case EPI_ROPE: return skinny_launch<EPI_ROPE>(X, W, C, R, M, N, K, ws, st, re);
            default: return skinny_launch<EPI_SILU>(X, W, C, R, M, N, K, ws, st);
        }
    }
    // the 4-wave kernel addresses operands by 32-bit byte offsets from its tile's first rows: 256 token
    // rows, and 256 weight rows (gate_up: up to row 2N - 1)
    if (mf_usable(epi, N, K, re)) {
        const MfPlan p = mf_plan(epi, M, N, K);
        const size_t need = static_cast<size_t>(p.splits) * M * (epi == EPI_SILU ? 2 * N : N) * sizeof(float);
        if (p.partial) {
            if (ws_bytes < need || !ws) return hipErrorInvalidValue;
            switch (epi) {
                case EPI_STORE: return mfma32_split_launch<EPI_STORE>(X, W, C, R, M, N, K, p, ws, st);
                case EPI_RESIDUAL: return mfma32_split_launch<EPI_RESIDUAL>(X, W, C, R, M, N, K, p, ws, st);
                case EPI_ROPE: return mfma32_split_launch<EPI_ROPE>(X, W, C, R, M, N, K, p, ws, st, re);
                default: return mfma32_split_launch<EPI_SILU>(X, W, C, R, M, N, K, p, ws, st);
            }
        }
        if (p.tn != MF_N) {   // 128-wide tiles, whole K, epilogue in the kernel (never RoPE: see the plan)
            switch (epi) {
                case EPI_STORE: return mfma32_launch<EPI_STORE, 0, 128>(X, W, C, R, M, N, K, st);
                case EPI_RESIDUAL: return mfma32_launch<EPI_RESIDUAL, 0, 128>(X, W, C, R, M, N, K, st);
                case EPI_SILU: return mfma32_launch<EPI_SILU, 0, 128>(X, W, C, R, M, N, K, st);
                default: return hipErrorInvalidValue;
            }
        }
        switch (epi) {
            case EPI_STORE: return mfma32_launch<EPI_STORE>(X, W, C, R, M, N, K, st);
            case EPI_RESIDUAL: return mfma32_launch<EPI_RESIDUAL>(X, W, C, R, M, N, K, st);
            case EPI_ROPE:
                if (re->d == 128) return mfma32_launch<EPI_ROPE, 128>(X, W, C, R, M, N, K, st, re);
                return mfma32_launch<EPI_ROPE, 64>(X, W, C, R, M, N, K, st, re);
            default:
                if (mfp_usable(M, N, K)) return mfp_launch<false>(X, W, C, M, N, K, st);
                return mfma32_launch<EPI_SILU>(X, W, C, R, M, N, K, st);
        }
    }
    switch (epi) {
        case EPI_STORE: return big_launch<EPI_STORE>(X, W, C, R, M, N, K, st);
        case EPI_RESIDUAL: return big_launch<EPI_RESIDUAL>(X, W, C, R, M, N, K, st);
        case EPI_ROPE:
            if (re->d == 128) return big_launch<EPI_ROPE, 128>(X, W, C, R, M, N, K, st, re);
            if (re->d == 64) return big_launch<EPI_ROPE, 64>(X, W, C, R, M, N, K, st, re);
            return big_launch<EPI_ROPE, 32>(X, W, C, R, M, N, K, st, re);
        default: return big_launch<EPI_SILU>(X, W, C, R, M, N, K, st);
    }
}

}  // namespace ll
