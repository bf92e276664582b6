// CPU check of the RoPE table bookkeeping (transformer_layer_forward_amd/csrc/rope_cache.h) with a
// counting backend in place of device memory and the table kernel. Exits non-zero on the first
// failed check and prints what failed.
#include <cstdio>
#include <cstdlib>
#include <set>

#include "rope_cache.h"

using namespace ll;

namespace {

int g_fail = 0;
#define CHECK(c)                                                        \
    do {                                                                \
        if (!(c)) {                                                     \
            std::printf("FAILED line %d: %s\n", __LINE__, #c);          \
            ++g_fail;                                                   \
        }                                                               \
    } while (0)

struct FakeBackend {
    int allocs = 0, frees = 0, gens = 0;
    long long gen_rows_total = 0;
    long long last_gen_rows = -1, last_lkey = -1;
    std::set<void*> live;
    bool fail_alloc = false;
    void* alloc(int, size_t bytes) {
        if (fail_alloc) return nullptr;
        ++allocs;
        void* p = std::malloc(bytes);
        live.insert(p);
        return p;
    }
    void release(int, void* p) {
        ++frees;
        live.erase(p);
        std::free(p);
    }
    bool generate(const RopeFamily&, void*, int64_t rows, int64_t lkey) {
        ++gens;
        gen_rows_total += rows;
        last_gen_rows = rows;
        last_lkey = lkey;
        return true;
    }
};

RopeFamily fam(int type, const void* stream, int64_t omp = 8192) {
    RopeFamily f;
    f.type = type;
    f.d = 128;
    f.theta = 5e5;
    f.factor = type == 0 ? 1.0 : 8.0;
    f.omp = omp;
    f.stream = stream;
    return f;
}

}  // namespace

int main() {
    RopeTableCache<FakeBackend> c{FakeBackend{}};
    bool af = false;
    const void* s0 = reinterpret_cast<const void*>(0x1000);
    const void* s1 = reinterpret_cast<const void*>(0x2000);

    // default family: first use allocates max(need, 4096) rows and fills all of them
    const RopeSlot* t = c.get(fam(0, s0), 100, 0, false, &af);
    CHECK(t && t->cap == 4096 && t->valid == 4096 && c.backend().allocs == 1 && c.backend().gens == 1);
    // a shorter or equal length reuses it: no allocation, no kernel
    for (int64_t L : {1, 100, 4096}) c.get(fam(0, s0), L, 0, false, &af);
    CHECK(c.backend().allocs == 1 && c.backend().gens == 1);
    // growing one position at a time past the capacity doubles: O(log L) allocations
    for (int64_t L = 4097; L <= 40000; ++L) c.get(fam(0, s0), L, 0, false, &af);
    CHECK(c.backend().allocs == 5);               // 4096 -> 8192 -> 16384 -> 32768 -> 65536
    CHECK(c.slots() == 1 && c.retired() == 4);

    // dynamic-NTK with L > original_max_pos, growing by one per decode step (50 steps): one slot for the
    // family on this stream, regenerated in place each step (its rows only), allocating only when the
    // capacity is exceeded
    RopeTableCache<FakeBackend> d{FakeBackend{}};
    const int64_t L0 = 8193;
    for (int step = 0; step < 50; ++step) {
        const int64_t L = L0 + step;
        const RopeSlot* s = d.get(fam(2, s0), L, L, true, &af);
        CHECK(s && s->valid == L && s->lkey == L);
        CHECK(d.backend().last_gen_rows == L && d.backend().last_lkey == L);
    }
    CHECK(d.slots() == 1);
    CHECK(d.backend().allocs == 1 && d.retired() == 0);   // 16384 rows from the first call
    CHECK(d.get(fam(2, s0), L0 + 49, L0 + 49, true, &af)->cap == 16384);
    CHECK(d.backend().gens == 50);
    // the same length again: reused; a shorter length: regenerated (the frequencies depend on L)
    d.get(fam(2, s0), L0 + 49, L0 + 49, true, &af);
    CHECK(d.backend().gens == 50);
    d.get(fam(2, s0), L0, L0, true, &af);
    CHECK(d.backend().gens == 51 && d.backend().allocs == 1);
    // dynamic-NTK at or below original_max_pos uses the length-independent contents (key 0)
    d.get(fam(2, s0), 100, 0, false, &af);
    CHECK(d.backend().gens == 52 && d.backend().last_gen_rows == d.get(fam(2, s0), 100, 0, false, &af)->cap);
    CHECK(d.backend().gens == 52);

    // another stream gets its own slot (no stream ever reads a table another stream regenerates)
    d.get(fam(2, s1), L0, L0, true, &af);
    CHECK(d.slots() == 2);
    // at most one slot per (family, stream) whatever the sequence of lengths
    for (int i = 0; i < 200; ++i) {
        const int64_t L = 1 + (i * 7919) % 30000;
        const bool dyn = L > 8192;
        d.get(fam(2, (i & 1) ? s1 : s0), L, dyn ? L : 0, dyn, &af);
        d.get(fam(3, (i & 1) ? s1 : s0), L, 0, false, &af);
    }
    CHECK(d.slots() == 4);

    // allocation failure leaves no half-made slot and reports it
    RopeTableCache<FakeBackend> e{FakeBackend{}};
    e.backend().fail_alloc = true;
    CHECK(e.get(fam(0, s0), 10, 0, false, &af) == nullptr && af && e.slots() == 0);

    // release frees every buffer, current and retired
    c.release_all();
    d.release_all();
    CHECK(c.backend().live.empty() && d.backend().live.empty());
    CHECK(c.backend().frees == c.backend().allocs && d.backend().frees == d.backend().allocs);

    if (g_fail) return 1;
    std::printf("rope_cache: all checks passed\n");
    return 0;
}
