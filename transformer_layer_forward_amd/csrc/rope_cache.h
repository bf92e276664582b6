// Bookkeeping of the library-owned RoPE tables (host only; no HIP types, so it also builds with a
// plain C++ compiler for the CPU checks of this logic).
//
// A table holds cs[p * (d/2) + j] = (cos(p f'_j), sin(p f'_j)) for positions p < rows. Its contents
// depend on the RoPE parameters and the head size, and for dynamic-NTK scaling also on the call's
// length L = kv_seq_len once L exceeds original_max_pos (verl "parallel_attention.py — LLaMA 并行注意力"
// §1: the base is recomputed from the sequence length). So:
//   * there is exactly one slot per (RoPE parameters, head size, device, stream);
//   * a slot grows geometrically (its capacity is a power of two that at least doubles), so a growing
//     length causes O(log L) allocations; the buffer a slot outgrows is retired, not freed, because kernels already queued
//     on the stream may still read it (all retired buffers are freed by release);
//   * when a dynamic-NTK length changes, the slot's own buffer is regenerated in place on the slot's
//     stream: work queued earlier on that stream has finished reading it by then (stream order), and
//     no other stream ever reads this slot.
// Every regeneration is a device kernel enqueued on the stream: nothing here blocks or copies from
// the host.
#pragma once

#include <stdint.h>

#include <algorithm>
#include <map>
#include <tuple>
#include <utility>
#include <vector>

namespace ll {

struct RopeFamily {
    int type = 0, d = 0, dev = 0;
    double theta = 0, factor = 0, lff = 0, hff = 0;
    int64_t omp = 0;
    const void* stream = nullptr;
    bool operator<(const RopeFamily& o) const {
        return std::tie(type, d, dev, theta, factor, lff, hff, omp, stream) <
               std::tie(o.type, o.d, o.dev, o.theta, o.factor, o.lff, o.hff, o.omp, o.stream);
    }
};

struct RopeSlot {
    void* ptr = nullptr;
    int64_t cap = 0;     // rows allocated
    int64_t valid = 0;   // rows [0, valid) hold the table for length key `lkey`
    int64_t lkey = -1;   // dynamic-NTK length the contents were made for (0: length-independent)
};

// What one call must do before it can read the table.
struct RopePlan {
    bool reuse = false;     // the slot already holds what the call needs
    bool grow = false;      // allocate a buffer of new_cap rows first (retire the old one)
    int64_t new_cap = 0;
    int64_t gen_rows = 0;   // rows [0, gen_rows) to (re)generate
};

constexpr int64_t kRopeMinRows = 4096;

// need: rows the call reads (kv_seq_len); lkey: the call's length key (0 unless dynamic-NTK is active);
// length_dependent: the contents depend on lkey (then only the rows needed are generated, since the next
// length will replace them anyway).
inline RopePlan rope_plan(const RopeSlot& s, int64_t need, int64_t lkey, bool length_dependent) {
    RopePlan p;
    if (s.ptr && s.lkey == lkey && s.valid >= need) {
        p.reuse = true;
        return p;
    }
    int64_t cap = s.cap;
    if (!s.ptr || s.cap < need) {
        p.grow = true;
        cap = kRopeMinRows;
        while (cap < need) cap *= 2;   // a power of two: a length growing by one reallocates rarely
        cap = std::max<int64_t>(cap, 2 * s.cap);
        p.new_cap = cap;
    }
    p.gen_rows = length_dependent ? need : cap;
    return p;
}

// Backend: void* alloc(int dev, size_t bytes)  (nullptr on failure)
//          void  release(int dev, void* p)
//          bool  generate(const RopeFamily&, void* p, int64_t rows, int64_t lkey)   (enqueue; false on failure)
template <class Backend>
class RopeTableCache {
  public:
    explicit RopeTableCache(Backend b) : be_(std::move(b)) {}

    // Returns the slot for the family with at least `need` valid rows for length key lkey, or nullptr
    // (allocation or launch failure; *alloc_failed tells which).
    const RopeSlot* get(const RopeFamily& fam, int64_t need, int64_t lkey, bool length_dependent,
                        bool* alloc_failed) {
        *alloc_failed = false;
        RopeSlot& s = slots_[fam];
        const RopePlan p = rope_plan(s, need, lkey, length_dependent);
        if (p.reuse) return &s;
        if (p.grow) {
            void* np = be_.alloc(fam.dev, static_cast<size_t>(p.new_cap) * static_cast<size_t>(fam.d / 2) * 8u);
            if (!np) {
                *alloc_failed = true;
                if (!s.ptr) slots_.erase(fam);
                return nullptr;
            }
            if (s.ptr) retired_.emplace_back(fam.dev, s.ptr);
            s.ptr = np;
            s.cap = p.new_cap;
            s.valid = 0;
            s.lkey = -1;
        }
        if (!be_.generate(fam, s.ptr, p.gen_rows, lkey)) {
            s.valid = 0;
            s.lkey = -1;
            return nullptr;
        }
        s.valid = p.gen_rows;
        s.lkey = lkey;
        return &s;
    }

    void release_all() {
        for (auto& kv : slots_)
            if (kv.second.ptr) be_.release(kv.first.dev, kv.second.ptr);
        for (auto& r : retired_) be_.release(r.first, r.second);
        slots_.clear();
        retired_.clear();
    }

    size_t slots() const { return slots_.size(); }
    size_t retired() const { return retired_.size(); }
    Backend& backend() { return be_; }

  private:
    Backend be_;
    std::map<RopeFamily, RopeSlot> slots_;
    std::vector<std::pair<int, void*>> retired_;
};

}  // namespace ll
