// Work partition of the balanced decode attention kernel (device and host; also compiled by a plain C++
// compiler for the CPU checks of this arithmetic, with __host__ / __device__ defined empty).
//
// The visible cache slots 0 .. pos[b] of every sequence are cut into 32-key tiles. A segment is one
// (sequence b, kv-head group hg) pair: kv heads hg*HW .. hg*HW + HW - 1 of sequence b, where a group holds
// HW = min(n_kv, 8) heads, so a tile of a segment is up to 8 heads' slices of 32 consecutive cache rows.
// Segment s = b * n_groups + hg has n_s = ceil((pos[b] + 1) / 32) tiles and starts at tile prefix[s] of the
// concatenation of all segments (prefix[n_seg] = T tiles in all). The NG workgroups of a call take equal
// contiguous shares of that concatenation: workgroup g takes tiles [floor(g T / NG), floor((g+1) T / NG)),
// so every workgroup moves the same number of bytes (to one tile) whatever the mix of sequence lengths.
// The part of a share that falls in one segment is a piece; piece (g, s) writes its partial softmax
// records at index g + s, which is unique: walking the pieces in order, each next piece has a larger g, a
// larger s, or both, so g + s strictly increases. There are at most NG + n_seg indices.
#pragma once

#include <stdint.h>

namespace ll {

constexpr int kDecTileKeys = 32;

__host__ __device__ inline int64_t dv_share_begin(int64_t g, int64_t T, int64_t NG) { return g * T / NG; }

// the workgroup whose (non-empty) share holds tile t, 0 <= t < T
__host__ __device__ inline int64_t dv_owner(int64_t t, int64_t T, int64_t NG) { return ((t + 1) * NG + T - 1) / T - 1; }

__host__ __device__ inline int64_t dv_tiles(int64_t pos, int64_t ctx) {
    const int64_t p = pos < 0 ? 0 : (pos >= ctx ? ctx - 1 : pos);
    return (p + 1 + kDecTileKeys - 1) / kDecTileKeys;
}

// tiles [lo, hi) of segment s (starting at tile prefix_s, n_s tiles) that workgroup g owns; empty if lo >= hi
__host__ __device__ inline void dv_piece(int64_t g, int64_t T, int64_t NG, int64_t prefix_s, int64_t n_s, int64_t* lo,
                                         int64_t* hi) {
    const int64_t a = dv_share_begin(g, T, NG), e = dv_share_begin(g + 1, T, NG);
    const int64_t l = a > prefix_s ? a : prefix_s;
    const int64_t h = e < prefix_s + n_s ? e : prefix_s + n_s;
    *lo = l - prefix_s;
    *hi = h - prefix_s;
}

}  // namespace ll
