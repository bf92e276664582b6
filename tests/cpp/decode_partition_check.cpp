// CPU check of the balanced decode partition (transformer_layer_forward_amd/csrc/decode_partition.h):
// replays the kernel's walk (prefix scan, equal shares, first segment by binary search, pieces) and the
// combine's walk (owner workgroups of a segment's first and last tile) for many random batches, and checks
// that every tile of every segment is processed exactly once, that record indices g + s never collide, and
// that the combine finds exactly the pieces the kernel wrote for each segment.
#define __host__
#define __device__
#include "decode_partition.h"

#include <cstdio>
#include <map>
#include <random>
#include <set>
#include <vector>

using namespace ll;

int main() {
    std::mt19937_64 rng(1234);
    int fails = 0;
    for (int trial = 0; trial < 3000; ++trial) {
        const int B = 1 + static_cast<int>(rng() % 70);
        const int ngroups = (trial % 3 == 0) ? 1 + static_cast<int>(rng() % 4) : 1;
        const int64_t ctx = 1 + static_cast<int64_t>(rng() % (trial % 5 == 0 ? 40 : 9000));
        const int64_t NG = 1 + static_cast<int64_t>(rng() % 520);
        std::vector<int64_t> pos(B);
        for (auto& p : pos) p = static_cast<int64_t>(rng() % (ctx + 3)) - 1;   // includes out-of-range ids (clamped)
        const int nseg = B * ngroups;
        std::vector<int64_t> pre(nseg + 1, 0);
        for (int s = 0; s < nseg; ++s) pre[s + 1] = pre[s] + dv_tiles(pos[s / ngroups], ctx);
        const int64_t T = pre[nseg];
        std::map<std::pair<int, int64_t>, int> seen;      // (segment, tile) -> times processed
        std::map<int64_t, std::pair<int64_t, int>> rec;   // record index -> (g, s)
        std::vector<std::set<int64_t>> written(nseg);
        for (int64_t g = 0; g < NG; ++g) {
            const int64_t t0 = dv_share_begin(g, T, NG), t1 = dv_share_begin(g + 1, T, NG);
            if (t0 >= t1) continue;
            int s0 = 0, hi = nseg - 1;
            while (s0 < hi) {
                const int mid = (s0 + hi + 1) >> 1;
                if (pre[mid] <= t0) s0 = mid;
                else hi = mid - 1;
            }
            for (int s = s0; s < nseg && pre[s] < t1; ++s) {
                int64_t lo, h;
                dv_piece(g, T, NG, pre[s], pre[s + 1] - pre[s], &lo, &h);
                if (lo >= h) { std::printf("empty piece g=%lld s=%d\n", (long long)g, s); ++fails; continue; }
                for (int64_t j = lo; j < h; ++j) seen[{s, j}]++;
                auto r = rec.emplace(g + s, std::make_pair(g, s));
                if (!r.second) { std::printf("record index %lld reused\n", (long long)(g + s)); ++fails; }
                if (g + s >= NG + nseg) { std::printf("record index beyond bound\n"); ++fails; }
                written[s].insert(g);
            }
        }
        for (int s = 0; s < nseg; ++s) {
            const int64_t n = pre[s + 1] - pre[s];
            for (int64_t j = 0; j < n; ++j)
                if (seen[{s, j}] != 1) { std::printf("tile (%d, %lld) seen %d times\n", s, (long long)j, seen[{s, j}]); ++fails; }
            // the combine: owners of the first and last tile, and every live piece between them
            std::set<int64_t> found;
            const int64_t glo = dv_owner(pre[s], T, NG), ghi = dv_owner(pre[s] + n - 1, T, NG);
            for (int64_t g = glo; g <= ghi; ++g) {
                int64_t lo, h;
                dv_piece(g, T, NG, pre[s], n, &lo, &h);
                if (lo < h) found.insert(g);
            }
            if (found != written[s]) { std::printf("combine of segment %d misses pieces\n", s); ++fails; }
        }
        if (fails > 20) break;
    }
    if (fails) return 1;
    std::printf("decode partition: all checks passed\n");
    return 0;
}
