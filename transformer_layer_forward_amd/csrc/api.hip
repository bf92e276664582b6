// Host side of the C ABI: argument validation, RoPE tables, workspace carving, the layer
// composition and per-stage timing. No kernels here.
//
// Layer (nanotron "模型层：从 Embedding 到 Loss 的实现", §9.5; llama3 结构详解 §3):
//   xn = rmsnorm(x; g_attn)              (§3.1)
//   qkv = xn W_qkv^T                      (§9.3 fused qkv_proj)
//   o = GQA causal attention with RoPE    (§9.3; verl "parallel_attention.py" §1-§2)
//   h = x + o W_o^T                        (§9.5 residual)
//   hn = rmsnorm(h; g_mlp)
//   act = silu(hn W_gate^T) * (hn W_up^T)  (§9.4)
//   out = h + act W_down^T
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <tuple>
#include <vector>

#include "common.h"
#include "rope_cache.h"

using namespace ll;

namespace {

thread_local std::string g_err;

ll_status fail(ll_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
ll_status fail(ll_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return st;
}

ll_status hip_fail(hipError_t e, const char* what) {
    return fail(LL_EHIP, "%s: %s", what, hipGetErrorString(e));
}

#define LL_CHECK_HIP(expr, what)                  \
    do {                                          \
        hipError_t e_ = (expr);                   \
        if (e_ != hipSuccess) return hip_fail(e_, what); \
    } while (0)

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int64_t kIntMax = 0x7fffffff;

size_t elem_size(int dtype) { return dtype == LL_BF16 ? 2 : 4; }

size_t round_up(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// ------------------------------------------------------------------ RoPE parameters / table
ll_status check_rope(const ll_rope* r) {
    if (!r) return LL_OK;
    if (r->type < LL_ROPE_DEFAULT || r->type > LL_ROPE_LLAMA3) return fail(LL_EINVAL, "rope.type %d unknown", r->type);
    if (r->interleaved != 0 && r->interleaved != 1) return fail(LL_EINVAL, "rope.interleaved must be 0 or 1");
    if (!(r->theta > 0.0) || !std::isfinite(r->theta)) return fail(LL_EINVAL, "rope.theta must be > 0");
    if (r->type != LL_ROPE_DEFAULT && (!(r->factor > 0.0) || !std::isfinite(r->factor)))
        return fail(LL_EINVAL, "rope.factor must be > 0");
    if ((r->type == LL_ROPE_DYNAMIC_NTK || r->type == LL_ROPE_LLAMA3) && r->original_max_pos <= 0)
        return fail(LL_EINVAL, "rope.original_max_pos must be > 0");
    if (r->type == LL_ROPE_LLAMA3 && (!(r->low_freq_factor > 0.0) || !(r->high_freq_factor > r->low_freq_factor)))
        return fail(LL_EINVAL, "llama3 rope needs 0 < low_freq_factor < high_freq_factor");
    return LL_OK;
}

// Angular frequency of pair i (verl "parallel_attention.py" §1 and its scaled variants; CSDN
// answer on Meta's model.py, apply_scaling). Computed in double on the host.
void rope_freqs(const ll_rope& r, int d, int64_t L, std::vector<double>& f) {
    const int half = d / 2;
    f.resize(half);
    double theta = r.theta;
    if (r.type == LL_ROPE_DYNAMIC_NTK && L > r.original_max_pos) {
        const double ratio = r.factor * static_cast<double>(L) / static_cast<double>(r.original_max_pos) - (r.factor - 1.0);
        theta = theta * std::pow(ratio, static_cast<double>(d) / (d - 2.0));
    }
    const double two_pi = 6.283185307179586476925286766559;
    for (int i = 0; i < half; ++i) {
        const double base = std::pow(theta, -2.0 * i / d);
        double v = base;
        if (r.type == LL_ROPE_LINEAR) {
            v = base / r.factor;
        } else if (r.type == LL_ROPE_LLAMA3) {
            const double orig = static_cast<double>(r.original_max_pos);
            const double wl = two_pi / base;
            if (wl < orig / r.high_freq_factor) {
                v = base;
            } else if (wl > orig / r.low_freq_factor) {
                v = base / r.factor;
            } else {
                const double s = (orig / wl - r.low_freq_factor) / (r.high_freq_factor - r.low_freq_factor);
                v = (1.0 - s) * base / r.factor + s * base;
            }
        }
        f[i] = v;
    }
}

// Library-owned tables: one slot per (RoPE parameters, head size, device, stream), generated on the
// device in stream order (rope_cache.h states the policy).
struct HipRopeBackend {
    const ll_rope* rope = nullptr;   // parameters of the call being served
    int64_t L = 0;                   // its kv_seq_len
    hipError_t last = hipSuccess;
    void* alloc(int, size_t bytes) {
        void* p = nullptr;
        last = hipMalloc(&p, bytes);
        return last == hipSuccess ? p : nullptr;
    }
    void release(int dev, void* p) {
        int cur = 0;
        (void)hipGetDevice(&cur);
        (void)hipSetDevice(dev);
        (void)hipFree(p);
        (void)hipSetDevice(cur);
    }
    bool generate(const RopeFamily& fam, void* p, int64_t rows, int64_t) {
        std::vector<double> f;
        rope_freqs(*rope, fam.d, L, f);
        RopeFreqs fr{};
        for (size_t i = 0; i < f.size(); ++i) fr.f[i] = f[i];
        last = launch_rope_table(static_cast<float2*>(p), rows, fam.d / 2, fr,
                                 static_cast<hipStream_t>(const_cast<void*>(fam.stream)));
        return last == hipSuccess;
    }
};

std::mutex g_tab_mu;
RopeTableCache<HipRopeBackend> g_tabs{HipRopeBackend{}};

RopeFamily rope_family(const ll_rope& r, int d, int dev, const void* stream) {
    RopeFamily k;
    k.type = r.type;
    k.d = d;
    k.dev = dev;
    k.theta = r.theta;
    k.factor = r.type == LL_ROPE_DEFAULT ? 1.0 : r.factor;
    k.lff = r.type == LL_ROPE_LLAMA3 ? r.low_freq_factor : 0.0;
    k.hff = r.type == LL_ROPE_LLAMA3 ? r.high_freq_factor : 0.0;
    k.omp = (r.type == LL_ROPE_LLAMA3 || r.type == LL_ROPE_DYNAMIC_NTK) ? r.original_max_pos : 0;
    k.stream = stream;
    return k;
}

// The table of (r, d) for positions < kv_seq_len, valid for work enqueued on `stream` after this call.
ll_status rope_table_get(const ll_rope& r, int d, int64_t kv_seq_len, hipStream_t stream, RopeTab* out) {
    int dev = 0;
    LL_CHECK_HIP(hipGetDevice(&dev), "hipGetDevice");
    const bool dyn = r.type == LL_ROPE_DYNAMIC_NTK && kv_seq_len > r.original_max_pos;
    std::lock_guard<std::mutex> lock(g_tab_mu);
    HipRopeBackend& be = g_tabs.backend();
    be.rope = &r;
    be.L = kv_seq_len;
    bool alloc_failed = false;
    const RopeSlot* slot = g_tabs.get(rope_family(r, d, dev, stream), kv_seq_len, dyn ? kv_seq_len : 0, dyn,
                                      &alloc_failed);
    if (!slot) {
        if (alloc_failed) return fail(LL_ENOMEM, "RoPE table allocation: %s", hipGetErrorString(be.last));
        return hip_fail(be.last, "RoPE table launch");
    }
    out->cs = static_cast<const float2*>(slot->ptr);
    out->rows = slot->valid;
    return LL_OK;
}

// ------------------------------------------------------------------ static scratch
// Device memory of llama_layer_forward_noalloc: the layer workspace and the call's RoPE table live in
// this file-scope array, so that entry point needs no allocation at all. Each device that runs it holds
// its own copy until the process ends. In host code `scratch` names a host-side stand-in, never the
// device address: host code uses only the per-device address from hipGetSymbolAddress below.
constexpr size_t kScratchBytes = size_t(64) << 20;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
std::map<int, void*> g_scratch_ptr;   // device -> device address of its scratch

// The current device's scratch address, looked up once per device (with that device current).
ll_status scratch_address(void** out) {
    int dev = 0;
    LL_CHECK_HIP(hipGetDevice(&dev), "hipGetDevice");
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    auto it = g_scratch_ptr.find(dev);
    if (it == g_scratch_ptr.end()) {
        void* p = nullptr;
        LL_CHECK_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
        if (!p) return fail(LL_EHIP, "hipGetSymbolAddress(scratch) returned NULL");
        it = g_scratch_ptr.emplace(dev, p).first;
    }
    *out = it->second;
    return LL_OK;
}

size_t rope_table_bytes(int64_t rows, int64_t d) { return static_cast<size_t>(rows) * static_cast<size_t>(d / 2) * 8u; }

// ------------------------------------------------------------------ profiling
constexpr int kMaxStages = 8;
const char* kStageNames[kMaxStages] = {"rmsnorm_attn", "qkv_proj",    "attention",   "o_proj_residual",
                                       "rmsnorm_mlp",  "gate_up_silu", "down_residual", "spare"};
constexpr int kLayerStages = 7;

struct ProfState {
    bool on = false;
    uint32_t mask = 0;   // stages timed: bit s = stage s
    // an event at stage boundary b (the start of stage b, the end of stage b-1) is recorded only when
    // a timed stage needs it
    bool boundary(int b) const { return ((mask >> b) & 1u) || (b > 0 && ((mask >> (b - 1)) & 1u)); }
    std::vector<hipEvent_t> pool;
    size_t used = 0;
    struct Call { size_t first; };
    std::vector<Call> calls;
    double ms[kMaxStages] = {};
    int64_t n[kMaxStages] = {};
};
thread_local ProfState g_prof;

hipEvent_t prof_event() {
    if (g_prof.used == g_prof.pool.size()) {
        hipEvent_t e;
        if (hipEventCreate(&e) != hipSuccess) return nullptr;
        g_prof.pool.push_back(e);
    }
    return g_prof.pool[g_prof.used++];
}

// ------------------------------------------------------------------ layer shapes
struct Shapes {
    int64_t M, H, nh, nkv, d, I, qkvd, od;
    int es;
};

Shapes shapes_of(const ll_layer_cfg* c, int64_t B, int64_t S) {
    Shapes s;
    s.M = B * S;
    s.H = c->hidden;
    s.nh = c->n_heads;
    s.nkv = c->n_kv_heads;
    s.d = c->head_dim;
    s.I = c->intermediate;
    s.qkvd = (s.nh + 2 * s.nkv) * s.d;
    s.od = s.nh * s.d;
    s.es = static_cast<int>(elem_size(c->dtype));
    return s;
}

struct LayerWs {
    size_t xn, qkv, o, h, act, gemm, dec, total;
};

LayerWs layer_ws(const ll_layer_cfg* c, int64_t B, int64_t S, int64_t ctx_for_decode) {
    Shapes s = shapes_of(c, B, S);
    LayerWs w;
    size_t off = 0;
    w.xn = off; off += round_up(static_cast<size_t>(s.M * s.H) * s.es);
    w.qkv = off; off += round_up(static_cast<size_t>(s.M * s.qkvd) * s.es);
    w.o = off; off += round_up(static_cast<size_t>(s.M * s.od) * s.es);
    w.h = off; off += round_up(static_cast<size_t>(s.M * s.H) * s.es);
    w.act = off; off += round_up(static_cast<size_t>(s.M * s.I) * s.es);
    size_t g = 0;
    g = std::max(g, gemm_workspace_bytes(c->dtype, s.M, s.qkvd, s.H, EPI_ROPE));
    g = std::max(g, gemm_workspace_bytes(c->dtype, s.M, s.H, s.od, EPI_RESIDUAL));
    g = std::max(g, gemm_workspace_bytes(c->dtype, s.M, s.I, s.H, EPI_SILU));
    g = std::max(g, gemm_workspace_bytes(c->dtype, s.M, s.H, s.I, EPI_RESIDUAL));
    w.gemm = off; off += round_up(g);
    w.dec = off;
    if (ctx_for_decode > 0) off += round_up(attn_decode_workspace_bytes(B, s.nh, s.d, ctx_for_decode));
    w.total = off;
    return w;
}

ll_status check_cfg(const ll_layer_cfg* c) {
    if (!c) return fail(LL_EINVAL, "cfg is NULL");
    if (c->dtype != LL_F32 && c->dtype != LL_BF16) return fail(LL_EINVAL, "dtype %d unknown", c->dtype);
    if (c->reserved != 0) return fail(LL_EINVAL, "cfg.reserved must be 0");
    if (c->hidden <= 0 || c->n_heads <= 0 || c->n_kv_heads <= 0 || c->head_dim <= 0 || c->intermediate <= 0)
        return fail(LL_EINVAL, "cfg dimensions must be positive");
    if (c->n_heads % c->n_kv_heads != 0) return fail(LL_EINVAL, "n_heads %% n_kv_heads != 0");
    if (c->head_dim % 2 != 0) return fail(LL_EINVAL, "head_dim must be even");
    if (c->head_dim > 256) return fail(LL_EUNSUPPORTED, "head_dim > 256 not supported");
    if (!(c->eps >= 0.0) || !std::isfinite(c->eps)) return fail(LL_EINVAL, "eps must be finite and >= 0");
    if (c->hidden > kIntMax || c->intermediate > kIntMax || (c->n_heads + 2 * c->n_kv_heads) * c->head_dim > kIntMax)
        return fail(LL_EUNSUPPORTED, "dimension exceeds 2^31-1");
    if (c->dtype == LL_BF16 &&
        (c->hidden % 8 != 0 || c->intermediate % 8 != 0 || (c->n_heads * c->head_dim) % 8 != 0 || c->head_dim % 8 != 0))
        return fail(LL_EUNSUPPORTED, "bf16 path needs hidden, intermediate and head_dim multiples of 8");
    return check_rope(&c->rope);
}

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

}  // namespace

// ====================================================================== C ABI
extern "C" {

const char* ll_last_error(void) { return g_err.c_str(); }

const char* ll_version(void) { return "llama_layer gfx950 1.0"; }

void ll_release_caches(void) {
    std::lock_guard<std::mutex> lock(g_tab_mu);
    g_tabs.release_all();
}

ll_status ll_profile_begin(int32_t reserve_calls) { return ll_profile_begin_stages(reserve_calls, 0x7Fu); }

ll_status ll_profile_begin_stages(int32_t reserve_calls, uint32_t stage_mask) {
    if (reserve_calls < 0) return fail(LL_EINVAL, "reserve_calls must be >= 0");
    if (stage_mask == 0 || (stage_mask >> kLayerStages) != 0)
        return fail(LL_EINVAL, "stage_mask must select stages 0 .. %d", kLayerStages - 1);
    g_prof.mask = stage_mask;
    const size_t want = static_cast<size_t>(reserve_calls) * (kLayerStages + 1);
    while (g_prof.pool.size() < want) {
        hipEvent_t e;
        LL_CHECK_HIP(hipEventCreate(&e), "hipEventCreate");
        g_prof.pool.push_back(e);
    }
    g_prof.on = true;
    g_prof.used = 0;
    g_prof.calls.clear();
    for (int i = 0; i < kMaxStages; ++i) {
        g_prof.ms[i] = 0.0;
        g_prof.n[i] = 0;
    }
    return LL_OK;
}

int32_t ll_profile_end(double* stage_ms, int64_t* stage_calls, int32_t max_stages) {
    g_prof.on = false;
    for (const auto& call : g_prof.calls) {
        int lastb = kLayerStages;
        while (!g_prof.boundary(lastb)) --lastb;   // the mask is non-empty: some boundary is recorded
        hipEvent_t last = g_prof.pool[call.first + lastb];
        if (hipEventSynchronize(last) != hipSuccess) {
            fail(LL_EHIP, "profile event synchronize failed");
            return -1;
        }
        for (int s = 0; s < kLayerStages; ++s) {
            if (!((g_prof.mask >> s) & 1u)) continue;
            float ms = 0.f;
            if (hipEventElapsedTime(&ms, g_prof.pool[call.first + s], g_prof.pool[call.first + s + 1]) != hipSuccess) {
                fail(LL_EHIP, "profile elapsed time failed");
                return -1;
            }
            g_prof.ms[s] += ms;
            g_prof.n[s] += 1;
        }
    }
    const int n = std::max<int32_t>(0, std::min<int32_t>(max_stages, kLayerStages));
    for (int i = 0; i < n; ++i) {
        if (stage_ms) stage_ms[i] = g_prof.ms[i];
        if (stage_calls) stage_calls[i] = g_prof.n[i];
    }
    g_prof.calls.clear();
    g_prof.used = 0;
    return n;
}

const char* ll_profile_stage_name(int32_t stage) {
    if (stage < 0 || stage >= kLayerStages) return "";
    return kStageNames[stage];
}

ll_status rmsnorm(const void* x, const void* gain, void* y, int64_t rows, int64_t hidden, double eps, int32_t dtype,
                  void* stream) {
    if (dtype != LL_F32 && dtype != LL_BF16) return fail(LL_EINVAL, "dtype %d unknown", dtype);
    if (rows < 0 || hidden <= 0) return fail(LL_EINVAL, "rows must be >= 0 and hidden > 0");
    if (rows > kIntMax) return fail(LL_EUNSUPPORTED, "rows exceeds 2^31-1");
    if (!(eps >= 0.0) || !std::isfinite(eps)) return fail(LL_EINVAL, "eps must be finite and >= 0");
    if (rows == 0) return LL_OK;
    if (!x || !gain || !y) return fail(LL_EINVAL, "NULL tensor pointer");
    if (!aligned16(x) || !aligned16(gain) || !aligned16(y)) return fail(LL_EINVAL, "pointers must be 16-byte aligned");
    hipError_t e = launch_rmsnorm(dtype, x, gain, y, rows, hidden, static_cast<float>(eps), as_stream(stream));
    if (e != hipSuccess) return hip_fail(e, "rmsnorm launch");
    return LL_OK;
}

ll_status rope_apply(const ll_rope* rope, void* qkv, const int64_t* position_ids, int64_t B, int64_t S,
                     int64_t n_heads, int64_t n_kv_heads, int64_t head_dim, int64_t kv_seq_len, int32_t dtype,
                     void* stream) {
    if (!rope) return fail(LL_EINVAL, "rope is NULL");
    ll_status st = check_rope(rope);
    if (st != LL_OK) return st;
    if (dtype != LL_F32 && dtype != LL_BF16) return fail(LL_EINVAL, "dtype %d unknown", dtype);
    if (B < 0 || S < 0 || n_heads <= 0 || n_kv_heads <= 0 || head_dim <= 0 || head_dim % 2)
        return fail(LL_EINVAL, "bad shape");
    if (n_heads % n_kv_heads) return fail(LL_EINVAL, "n_heads %% n_kv_heads != 0");
    if (head_dim > 256) return fail(LL_EUNSUPPORTED, "head_dim > 256 not supported");
    if (kv_seq_len <= 0) return fail(LL_EINVAL, "kv_seq_len must be > 0");
    if (B * S == 0) return LL_OK;
    if (!qkv || !position_ids) return fail(LL_EINVAL, "NULL tensor pointer");
    RopeTab tab;
    st = rope_table_get(*rope, static_cast<int>(head_dim), kv_seq_len, as_stream(stream), &tab);
    if (st != LL_OK) return st;
    hipError_t e = launch_rope_apply(dtype, qkv, position_ids, tab, B * S, static_cast<int>(n_heads),
                                     static_cast<int>(n_kv_heads), static_cast<int>(head_dim), rope->interleaved,
                                     as_stream(stream));
    if (e != hipSuccess) return hip_fail(e, "rope_apply launch");
    return LL_OK;
}

static ll_status check_attn_common(const void* qkv, const ll_rope* rope, const int64_t* pos, int64_t kv_seq_len,
                                   void* o, void* kc, void* vc, int64_t ctx, int64_t B, int64_t S, int64_t nh,
                                   int64_t nkv, int64_t d, int32_t dtype) {
    if (dtype != LL_F32 && dtype != LL_BF16) return fail(LL_EINVAL, "dtype %d unknown", dtype);
    if (B < 0 || S < 0 || nh <= 0 || nkv <= 0 || d <= 0) return fail(LL_EINVAL, "bad shape");
    if (nh % nkv) return fail(LL_EINVAL, "n_heads %% n_kv_heads != 0");
    if (d % 2) return fail(LL_EINVAL, "head_dim must be even");
    if (d > 256) return fail(LL_EUNSUPPORTED, "head_dim > 256 not supported");
    if (dtype == LL_BF16 && d % 8) return fail(LL_EUNSUPPORTED, "bf16 attention needs head_dim %% 8 == 0");
    if (B > kIntMax || S > kIntMax || B * S * nh > kIntMax * 4LL) return fail(LL_EUNSUPPORTED, "size too large");
    ll_status st = check_rope(rope);
    if (st != LL_OK) return st;
    if (rope && kv_seq_len <= 0) return fail(LL_EINVAL, "kv_seq_len must be > 0 when rope is given");
    if ((kc == nullptr) != (vc == nullptr)) return fail(LL_EINVAL, "k_cache and v_cache must both be given or both NULL");
    if (kc && ctx <= 0) return fail(LL_EINVAL, "ctx must be > 0 with caches");
    if (B * S == 0) return LL_OK;
    if (!qkv || !o) return fail(LL_EINVAL, "NULL tensor pointer");
    if ((rope || kc) && !pos) return fail(LL_EINVAL, "position ids required with rope or caches");
    if (!aligned16(qkv) || !aligned16(o) || (kc && (!aligned16(kc) || !aligned16(vc))))
        return fail(LL_EINVAL, "pointers must be 16-byte aligned");
    return LL_OK;
}

ll_status gqa_attn_prefill(const void* qkv, const ll_rope* rope, const int64_t* position_ids, int64_t kv_seq_len,
                           void* o, void* k_cache, void* v_cache, int64_t ctx, int64_t B, int64_t S, int64_t n_heads,
                           int64_t n_kv_heads, int64_t head_dim, int32_t dtype, void* stream) {
    ll_status st = check_attn_common(qkv, rope, position_ids, kv_seq_len, o, k_cache, v_cache, ctx, B, S, n_heads,
                                     n_kv_heads, head_dim, dtype);
    if (st != LL_OK || B * S == 0) return st;
    RopeTab tab;
    if (rope) {
        st = rope_table_get(*rope, static_cast<int>(head_dim), kv_seq_len, as_stream(stream), &tab);
        if (st != LL_OK) return st;
    }
    hipError_t e = launch_attn_prefill(dtype, qkv, position_ids, rope ? &tab : nullptr, rope ? rope->interleaved : 0, o,
                                       k_cache, v_cache, ctx, static_cast<int>(B), static_cast<int>(S),
                                       static_cast<int>(n_heads), static_cast<int>(n_kv_heads),
                                       static_cast<int>(head_dim), as_stream(stream));
    if (e != hipSuccess) return hip_fail(e, "gqa_attn_prefill launch");
    return LL_OK;
}

size_t gqa_attn_prefill_chunk_workspace_bytes(int64_t B, int64_t S, int64_t n_heads, int64_t n_kv_heads,
                                              int64_t head_dim, int64_t ctx, int32_t dtype) {
    if (B <= 0 || S <= 0 || n_heads <= 0 || n_kv_heads <= 0 || head_dim <= 0 || ctx <= 0) return 0;
    if (n_heads % n_kv_heads != 0) return 0;
    return attn_chunk_workspace_bytes(dtype, B, S, n_heads, n_kv_heads, head_dim, ctx);
}

ll_status gqa_attn_prefill_chunk(const void* qkv, const int64_t* position_ids, void* o, void* k_cache, void* v_cache,
                                 int64_t ctx, int64_t B, int64_t S, int64_t n_heads, int64_t n_kv_heads,
                                 int64_t head_dim, int32_t dtype, void* workspace, size_t workspace_bytes,
                                 void* stream) {
    if (!k_cache || !v_cache) return fail(LL_EINVAL, "chunked prefill needs k_cache and v_cache");
    ll_status st = check_attn_common(qkv, nullptr, position_ids, 0, o, k_cache, v_cache, ctx, B, S, n_heads,
                                     n_kv_heads, head_dim, dtype);
    if (st != LL_OK || B * S == 0) return st;
    if (ctx > kIntMax) return fail(LL_EUNSUPPORTED, "ctx exceeds 2^31-1");
    if (workspace && !aligned16(workspace)) return fail(LL_EINVAL, "workspace must be 16-byte aligned");
    hipError_t e = launch_attn_prefill_chunk(dtype, qkv, position_ids, o, k_cache, v_cache, ctx, static_cast<int>(B),
                                             static_cast<int>(S), static_cast<int>(n_heads),
                                             static_cast<int>(n_kv_heads), static_cast<int>(head_dim), workspace,
                                             workspace ? workspace_bytes : 0, as_stream(stream));
    if (e != hipSuccess) return hip_fail(e, "gqa_attn_prefill_chunk launch");
    return LL_OK;
}

ll_status gqa_attn_prefill_varlen(const void* qkv, const int32_t* cu_seqlens, int64_t n_seqs, int64_t max_seqlen,
                                  int64_t total_tokens, void* o, int64_t n_heads, int64_t n_kv_heads,
                                  int64_t head_dim, int32_t dtype, void* stream) {
    ll_status st = check_attn_common(qkv, nullptr, nullptr, 0, o, nullptr, nullptr, 0, 1, total_tokens, n_heads,
                                     n_kv_heads, head_dim, dtype);
    if (st != LL_OK) return st;
    if (n_seqs < 0 || max_seqlen < 0) return fail(LL_EINVAL, "n_seqs and max_seqlen must be >= 0");
    if (n_seqs > kIntMax || max_seqlen > kIntMax) return fail(LL_EUNSUPPORTED, "n_seqs or max_seqlen exceeds 2^31-1");
    if (max_seqlen > total_tokens) return fail(LL_EINVAL, "max_seqlen > total_tokens");
    if (total_tokens == 0 || n_seqs == 0) return LL_OK;
    if (!cu_seqlens) return fail(LL_EINVAL, "cu_seqlens is NULL");
    hipError_t e = launch_attn_prefill_varlen(dtype, qkv, cu_seqlens, static_cast<int>(n_seqs),
                                              static_cast<int>(max_seqlen), static_cast<int>(total_tokens), o,
                                              static_cast<int>(n_heads), static_cast<int>(n_kv_heads),
                                              static_cast<int>(head_dim), as_stream(stream));
    if (e != hipSuccess) return hip_fail(e, "gqa_attn_prefill_varlen launch");
    return LL_OK;
}

size_t gqa_attn_decode_workspace_bytes(int64_t B, int64_t n_heads, int64_t head_dim, int64_t ctx) {
    if (B < 0 || n_heads <= 0 || head_dim <= 0 || ctx <= 0) return 0;
    return attn_decode_workspace_bytes(B, n_heads, head_dim, ctx);
}

ll_status gqa_attn_decode(const void* qkv, const ll_rope* rope, const int64_t* pos, int64_t kv_seq_len, void* k_cache,
                          void* v_cache, int64_t ctx, void* o, int64_t B, int64_t n_heads, int64_t n_kv_heads,
                          int64_t head_dim, int32_t dtype, void* workspace, size_t workspace_bytes, void* stream) {
    if (!k_cache || !v_cache) return fail(LL_EINVAL, "decode needs k_cache and v_cache");
    ll_status st = check_attn_common(qkv, rope, pos, kv_seq_len, o, k_cache, v_cache, ctx, B, 1, n_heads, n_kv_heads,
                                     head_dim, dtype);
    if (st != LL_OK || B == 0) return st;
    if (!pos) return fail(LL_EINVAL, "pos is NULL");
    const size_t need = attn_decode_workspace_bytes(B, n_heads, head_dim, ctx);
    if (workspace_bytes < need) return fail(LL_EINVAL, "workspace too small: %zu < %zu", workspace_bytes, need);
    if (need && !workspace) return fail(LL_EINVAL, "workspace is NULL");
    RopeTab tab;
    if (rope) {
        st = rope_table_get(*rope, static_cast<int>(head_dim), kv_seq_len, as_stream(stream), &tab);
        if (st != LL_OK) return st;
    }
    hipError_t e = launch_attn_decode(dtype, qkv, pos, rope ? &tab : nullptr, rope ? rope->interleaved : 0, k_cache,
                                      v_cache, ctx, o, static_cast<int>(B), static_cast<int>(n_heads),
                                      static_cast<int>(n_kv_heads), static_cast<int>(head_dim), workspace,
                                      workspace_bytes, as_stream(stream));
    if (e != hipSuccess) return hip_fail(e, "gqa_attn_decode launch");
    return LL_OK;
}

size_t swiglu_mlp_workspace_bytes(int64_t M, int64_t hidden, int64_t intermediate, int32_t dtype) {
    if (M < 0 || hidden <= 0 || intermediate <= 0 || (dtype != LL_F32 && dtype != LL_BF16)) return 0;
    const size_t act = round_up(static_cast<size_t>(M * intermediate) * elem_size(dtype));
    const size_t g = std::max(gemm_workspace_bytes(dtype, M, intermediate, hidden, EPI_SILU),
                              gemm_workspace_bytes(dtype, M, hidden, intermediate, EPI_RESIDUAL));
    return act + round_up(g);
}

ll_status swiglu_mlp(const void* x, const void* w_gate_up, const void* w_down, const void* residual, void* out,
                     int64_t M, int64_t hidden, int64_t intermediate, int32_t dtype, void* workspace,
                     size_t workspace_bytes, void* stream) {
    if (dtype != LL_F32 && dtype != LL_BF16) return fail(LL_EINVAL, "dtype %d unknown", dtype);
    if (M < 0 || hidden <= 0 || intermediate <= 0) return fail(LL_EINVAL, "bad shape");
    if (M > kIntMax || hidden > kIntMax || intermediate > kIntMax) return fail(LL_EUNSUPPORTED, "size too large");
    if (dtype == LL_BF16 && (hidden % 8 || intermediate % 8))
        return fail(LL_EUNSUPPORTED, "bf16 path needs hidden and intermediate multiples of 8");
    if (M == 0) return LL_OK;
    if (!x || !w_gate_up || !w_down || !out) return fail(LL_EINVAL, "NULL tensor pointer");
    if (out == x) return fail(LL_EINVAL, "out must not alias x");
    if (!aligned16(x) || !aligned16(w_gate_up) || !aligned16(w_down) || !aligned16(out) ||
        (residual && !aligned16(residual)))
        return fail(LL_EINVAL, "pointers must be 16-byte aligned");
    const size_t need = swiglu_mlp_workspace_bytes(M, hidden, intermediate, dtype);
    if (workspace_bytes < need || !workspace) return fail(LL_EINVAL, "workspace too small: %zu < %zu", workspace_bytes, need);
    if (!aligned16(workspace)) return fail(LL_EINVAL, "workspace must be 16-byte aligned");
    char* ws = static_cast<char*>(workspace);
    void* act = ws;
    void* gws = ws + round_up(static_cast<size_t>(M * intermediate) * elem_size(dtype));
    const size_t gbytes = workspace_bytes - round_up(static_cast<size_t>(M * intermediate) * elem_size(dtype));
    hipStream_t st = as_stream(stream);
    const bool blk = gemm_act_blocked(dtype, M, intermediate, hidden);
    hipError_t e = launch_gemm(dtype, EPI_SILU, x, w_gate_up, act, nullptr, M, intermediate, hidden, gws, gbytes, st,
                               nullptr, blk);
    if (e != hipSuccess) return hip_fail(e, "gate_up launch");
    e = launch_gemm(dtype, residual ? EPI_RESIDUAL : EPI_STORE, act, w_down, out, residual, M, hidden, intermediate,
                    gws, gbytes, st, nullptr, blk);
    if (e != hipSuccess) return hip_fail(e, "down launch");
    return LL_OK;
}

size_t llama_layer_workspace_bytes(const ll_layer_cfg* cfg, int64_t B, int64_t S, int64_t ctx) {
    if (!cfg || B < 0 || S < 0 || ctx < 0) return 0;
    if (check_cfg(cfg) != LL_OK) return 0;
    if (S == 1 && ctx > 0) return layer_ws(cfg, B, S, ctx).total;
    // a chunk on a cache prefix may split its attention keys: room for the partial records
    const size_t split = ctx > 0 ? attn_chunk_workspace_bytes(cfg->dtype, B, S, cfg->n_heads, cfg->n_kv_heads,
                                                             cfg->head_dim, ctx)
                                 : 0;
    return layer_ws(cfg, B, S, 0).total + round_up(split);
}

struct Varlen {
    const int32_t* cu;
    int64_t nseq, max_seqlen;
};

static ll_status layer_forward_impl(const ll_layer_cfg* cfg, const ll_layer_weights* w, const void* hidden,
                                    const int64_t* position_ids, int64_t B, int64_t S, int64_t kv_seq_len,
                                    void* k_cache, void* v_cache, int64_t ctx, void* out, void* workspace,
                                    size_t workspace_bytes, void* stream, bool chunk,
                                    const Varlen* vl = nullptr, bool use_scratch = false) {
    ll_status st = check_cfg(cfg);
    if (st != LL_OK) return st;
    if (!w) return fail(LL_EINVAL, "weights is NULL");
    if (B < 0 || S < 0) return fail(LL_EINVAL, "B and S must be >= 0");
    if (B > kIntMax || S > kIntMax || B * S > kIntMax) return fail(LL_EUNSUPPORTED, "B*S exceeds 2^31-1");
    if (kv_seq_len <= 0) return fail(LL_EINVAL, "kv_seq_len must be > 0");
    if ((k_cache == nullptr) != (v_cache == nullptr)) return fail(LL_EINVAL, "k_cache and v_cache must both be given or both NULL");
    if (k_cache && ctx <= 0) return fail(LL_EINVAL, "ctx must be > 0 with caches");
    if (k_cache && ctx > kIntMax) return fail(LL_EUNSUPPORTED, "ctx exceeds 2^31-1");
    if (B * S == 0) return LL_OK;
    if (!hidden || !out || !position_ids) return fail(LL_EINVAL, "NULL tensor pointer");
    if (!w->w_qkv || !w->w_o || !w->w_gate_up || !w->w_down || !w->g_attn || !w->g_mlp)
        return fail(LL_EINVAL, "NULL weight pointer");
    const void* ptrs[] = {hidden, out, w->w_qkv, w->w_o, w->w_gate_up, w->w_down, w->g_attn, w->g_mlp, workspace};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return fail(LL_EINVAL, "pointers must be 16-byte aligned");
    if (k_cache && (!aligned16(k_cache) || !aligned16(v_cache))) return fail(LL_EINVAL, "pointers must be 16-byte aligned");
    if (chunk && !k_cache) return fail(LL_EINVAL, "chunked prefill needs k_cache and v_cache");
    const bool decode = !chunk && (S == 1 && k_cache != nullptr);
    const LayerWs lw = layer_ws(cfg, B, S, decode ? ctx : 0);
    const Shapes s = shapes_of(cfg, B, S);
    if (use_scratch) {
        // workspace, then this call's RoPE table, both in the static scratch
        const size_t need = round_up(lw.total) + rope_table_bytes(kv_seq_len, s.d);
        if (need > kScratchBytes)
            return fail(LL_EINVAL, "llama_layer_forward_noalloc needs %zu bytes of scratch; its static scratch holds %zu",
                        need, kScratchBytes);
    } else if (!workspace || workspace_bytes < lw.total) {
        return fail(LL_EINVAL, "workspace too small: %zu < %zu", workspace_bytes, lw.total);
    }

    RopeTab tab;
    if (use_scratch) {
        void* base = nullptr;
        st = scratch_address(&base);
        if (st != LL_OK) return st;
        workspace = base;
        workspace_bytes = round_up(lw.total);
        float2* cs = reinterpret_cast<float2*>(static_cast<char*>(base) + round_up(lw.total));
        std::vector<double> f;
        rope_freqs(cfg->rope, static_cast<int>(s.d), kv_seq_len, f);
        RopeFreqs fr{};
        for (size_t i = 0; i < f.size(); ++i) fr.f[i] = f[i];
        LL_CHECK_HIP(launch_rope_table(cs, kv_seq_len, static_cast<int>(s.d / 2), fr, as_stream(stream)),
                     "RoPE table launch");
        tab.cs = cs;
        tab.rows = kv_seq_len;
    } else {
        st = rope_table_get(cfg->rope, static_cast<int>(s.d), kv_seq_len, as_stream(stream), &tab);
        if (st != LL_OK) return st;
    }

    char* ws = static_cast<char*>(workspace);
    void* xn = ws + lw.xn;
    void* qkv = ws + lw.qkv;
    void* o = ws + lw.o;
    void* h = ws + lw.h;
    void* act = ws + lw.act;
    void* gws = ws + lw.gemm;
    const size_t gbytes = lw.dec - lw.gemm;
    void* dws = ws + lw.dec;
    const size_t dbytes = lw.total - lw.dec;
    const int dt = cfg->dtype;
    const float eps = static_cast<float>(cfg->eps);
    hipStream_t stream_h = as_stream(stream);

    const bool prof = g_prof.on && !use_scratch;   // the no-allocation entry point records no events
    size_t ev0 = 0;
    if (prof) {
        ev0 = g_prof.used;
        for (int i = 0; i <= kLayerStages; ++i)
            if (!prof_event()) return fail(LL_EHIP, "hipEventCreate failed");
        g_prof.calls.push_back({ev0});
        if (g_prof.boundary(0)) LL_CHECK_HIP(hipEventRecord(g_prof.pool[ev0], stream_h), "hipEventRecord");
    }
    int stage = 0;
    auto mark = [&]() -> hipError_t {
        ++stage;
        return prof && g_prof.boundary(stage) ? hipEventRecord(g_prof.pool[ev0 + stage], stream_h) : hipSuccess;
    };

    hipError_t e;
    // 1. input RMSNorm
    e = launch_rmsnorm(dt, hidden, w->g_attn, xn, s.M, s.H, eps, stream_h);
    if (e != hipSuccess) return hip_fail(e, "rmsnorm launch");
    LL_CHECK_HIP(mark(), "hipEventRecord");
    // 2. fused QKV projection; q and k are rotated in its epilogue (or by a rotation pass when the
    //    head layout does not allow the fused form), so attention reads rotated q and k
    RopeEpi re;
    re.pos = position_ids;
    re.tab = tab;
    re.rope_cols = static_cast<int>((s.nh + s.nkv) * s.d);
    re.d = static_cast<int>(s.d);
    re.interleaved = cfg->rope.interleaved;
    // decode: the QKV reduce also appends the new keys and values (no separate store pass)
    const bool appended = decode && gemm_rope_fusable(dt, s.M, re.d) &&
                          gemm_rope_appends_cache(dt, s.M, s.qkvd, s.H, re.d, re.rope_cols);
    if (appended) {
        re.kc = k_cache;
        re.vc = v_cache;
        re.ctx = ctx;
        re.nh = static_cast<int>(s.nh);
        re.nkv = static_cast<int>(s.nkv);
    }
    if (gemm_rope_fusable(dt, s.M, re.d)) {
        e = launch_gemm(dt, EPI_ROPE, xn, w->w_qkv, qkv, nullptr, s.M, s.qkvd, s.H, gws, gbytes, stream_h, &re);
        if (e != hipSuccess) return hip_fail(e, "qkv projection launch");
    } else {
        e = launch_gemm(dt, EPI_STORE, xn, w->w_qkv, qkv, nullptr, s.M, s.qkvd, s.H, gws, gbytes, stream_h);
        if (e != hipSuccess) return hip_fail(e, "qkv projection launch");
        e = launch_rope_apply(dt, qkv, position_ids, tab, s.M, static_cast<int>(s.nh), static_cast<int>(s.nkv),
                              re.d, re.interleaved, stream_h);
        if (e != hipSuccess) return hip_fail(e, "rope launch");
    }
    LL_CHECK_HIP(mark(), "hipEventRecord");
    // 3. attention on rotated q and k
    if (vl) {
        e = launch_attn_prefill_varlen(dt, qkv, vl->cu, static_cast<int>(vl->nseq), static_cast<int>(vl->max_seqlen),
                                       static_cast<int>(S), o, static_cast<int>(s.nh), static_cast<int>(s.nkv),
                                       static_cast<int>(s.d), stream_h);
    } else if (chunk) {
        // workspace past the layer's own part holds key-split records when the caller sized it for them
        e = launch_attn_prefill_chunk(dt, qkv, position_ids, o, k_cache, v_cache, ctx, static_cast<int>(B),
                                      static_cast<int>(S), static_cast<int>(s.nh), static_cast<int>(s.nkv),
                                      static_cast<int>(s.d), ws + lw.total, workspace_bytes - lw.total, stream_h);
    } else if (decode) {
        e = launch_attn_decode(dt, qkv, position_ids, nullptr, 0, k_cache, v_cache, ctx, o, static_cast<int>(B),
                               static_cast<int>(s.nh), static_cast<int>(s.nkv), static_cast<int>(s.d), dws, dbytes,
                               stream_h, appended);
    } else {
        e = launch_attn_prefill(dt, qkv, position_ids, nullptr, 0, o, k_cache, v_cache, ctx, static_cast<int>(B),
                                static_cast<int>(S), static_cast<int>(s.nh), static_cast<int>(s.nkv),
                                static_cast<int>(s.d), stream_h);
    }
    if (e != hipSuccess) return hip_fail(e, "attention launch");
    LL_CHECK_HIP(mark(), "hipEventRecord");
    // 4. o_proj + residual
    e = launch_gemm(dt, EPI_RESIDUAL, o, w->w_o, h, hidden, s.M, s.H, s.od, gws, gbytes, stream_h);
    if (e != hipSuccess) return hip_fail(e, "o_proj launch");
    LL_CHECK_HIP(mark(), "hipEventRecord");
    // 5. post-attention RMSNorm
    e = launch_rmsnorm(dt, h, w->g_mlp, xn, s.M, s.H, eps, stream_h);
    if (e != hipSuccess) return hip_fail(e, "rmsnorm launch");
    LL_CHECK_HIP(mark(), "hipEventRecord");
    // 6. gate_up + silu * up (written K-blocked for the down projection where both take whole tiles)
    const bool blk = gemm_act_blocked(dt, s.M, s.I, s.H);
    e = launch_gemm(dt, EPI_SILU, xn, w->w_gate_up, act, nullptr, s.M, s.I, s.H, gws, gbytes, stream_h, nullptr, blk);
    if (e != hipSuccess) return hip_fail(e, "gate_up launch");
    LL_CHECK_HIP(mark(), "hipEventRecord");
    // 7. down + residual
    e = launch_gemm(dt, EPI_RESIDUAL, act, w->w_down, out, h, s.M, s.H, s.I, gws, gbytes, stream_h, nullptr, blk);
    if (e != hipSuccess) return hip_fail(e, "down launch");
    LL_CHECK_HIP(mark(), "hipEventRecord");
    return LL_OK;
}

ll_status llama_layer_forward(const ll_layer_cfg* cfg, const ll_layer_weights* w, const void* hidden,
                              const int64_t* position_ids, int64_t B, int64_t S, int64_t kv_seq_len, void* k_cache,
                              void* v_cache, int64_t ctx, void* out, void* workspace, size_t workspace_bytes,
                              void* stream) {
    return layer_forward_impl(cfg, w, hidden, position_ids, B, S, kv_seq_len, k_cache, v_cache, ctx, out, workspace,
                              workspace_bytes, stream, false);
}

ll_status llama_layer_forward_noalloc(const ll_layer_cfg* cfg, const ll_layer_weights* w, const void* hidden,
                                      const int64_t* position_ids, int64_t B, int64_t S, int64_t kv_seq_len,
                                      void* k_cache, void* v_cache, int64_t ctx, void* out, void* stream) {
    return layer_forward_impl(cfg, w, hidden, position_ids, B, S, kv_seq_len, k_cache, v_cache, ctx, out, nullptr, 0,
                              stream, false, nullptr, true);
}

size_t llama_model_workspace_bytes(const ll_layer_cfg* cfg, int64_t vocab, int64_t B, int64_t S) {
    if (!cfg || vocab <= 0 || B < 0 || S < 0) return 0;
    if (check_cfg(cfg) != LL_OK) return 0;
    const Shapes s = shapes_of(cfg, B, S);
    const size_t act = round_up(static_cast<size_t>(s.M * s.H) * s.es);
    return 2 * act + round_up(gemm_workspace_bytes(cfg->dtype, s.M, vocab, s.H, EPI_STORE)) +
           layer_ws(cfg, B, S, 0).total;
}

ll_status llama_model_forward(const ll_layer_cfg* cfg, int64_t n_layers, const ll_layer_weights* layers,
                              const void* tok_embeddings, const void* final_norm_gain, const void* lm_head,
                              int64_t vocab, const int64_t* tokens, const int64_t* position_ids, int64_t B,
                              int64_t S, int64_t kv_seq_len, void* logits, void* workspace, size_t workspace_bytes,
                              void* stream) {
    ll_status st = check_cfg(cfg);
    if (st != LL_OK) return st;
    if (n_layers < 0) return fail(LL_EINVAL, "n_layers must be >= 0");
    if (n_layers > 0 && !layers) return fail(LL_EINVAL, "layers is NULL");
    if (vocab <= 0) return fail(LL_EINVAL, "vocab must be > 0");
    if (vocab > kIntMax) return fail(LL_EUNSUPPORTED, "vocab exceeds 2^31-1");
    if (B < 0 || S < 0) return fail(LL_EINVAL, "B and S must be >= 0");
    if (B > kIntMax || S > kIntMax || B * S > kIntMax) return fail(LL_EUNSUPPORTED, "B*S exceeds 2^31-1");
    if (kv_seq_len <= 0) return fail(LL_EINVAL, "kv_seq_len must be > 0");
    if (B * S == 0) return LL_OK;
    if (!tok_embeddings || !final_norm_gain || !lm_head || !tokens || !position_ids || !logits)
        return fail(LL_EINVAL, "NULL tensor pointer");
    const void* ptrs[] = {tok_embeddings, final_norm_gain, lm_head, logits, workspace};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return fail(LL_EINVAL, "pointers must be 16-byte aligned");
    const Shapes s = shapes_of(cfg, B, S);
    const size_t act = round_up(static_cast<size_t>(s.M * s.H) * s.es);
    const size_t gws = round_up(gemm_workspace_bytes(cfg->dtype, s.M, vocab, s.H, EPI_STORE));
    const size_t lws = layer_ws(cfg, B, S, 0).total;
    const size_t need = 2 * act + gws + lws;
    if (!workspace || workspace_bytes < need)
        return fail(LL_EINVAL, "workspace too small: %zu < %zu", workspace_bytes, need);
    char* ws = static_cast<char*>(workspace);
    void* h = ws;
    void* hn = ws + act;
    void* g = ws + 2 * act;
    void* lw = ws + 2 * act + gws;
    hipStream_t stream_h = as_stream(stream);
    // h = tok_embeddings(tokens); every layer runs in place on h
    hipError_t e = launch_embedding(cfg->dtype, tok_embeddings, tokens, h, s.M, s.H, vocab, stream_h);
    if (e != hipSuccess) return hip_fail(e, "embedding launch");
    for (int64_t l = 0; l < n_layers; ++l) {
        st = layer_forward_impl(cfg, &layers[l], h, position_ids, B, S, kv_seq_len, nullptr, nullptr, 0, h, lw, lws,
                                stream, false);
        if (st != LL_OK) return st;
    }
    // logits = output(norm(h))
    e = launch_rmsnorm(cfg->dtype, h, final_norm_gain, hn, s.M, s.H, static_cast<float>(cfg->eps), stream_h);
    if (e != hipSuccess) return hip_fail(e, "final rmsnorm launch");
    e = launch_gemm(cfg->dtype, EPI_STORE, hn, lm_head, logits, nullptr, s.M, vocab, s.H, g, gws, stream_h);
    if (e != hipSuccess) return hip_fail(e, "lm_head launch");
    return LL_OK;
}

ll_status llama_layer_forward_varlen(const ll_layer_cfg* cfg, const ll_layer_weights* w, const void* hidden,
                                     const int64_t* position_ids, const int32_t* cu_seqlens, int64_t n_seqs,
                                     int64_t max_seqlen, int64_t total_tokens, int64_t kv_seq_len, void* out,
                                     void* workspace, size_t workspace_bytes, void* stream) {
    if (n_seqs < 0 || max_seqlen < 0 || total_tokens < 0) return fail(LL_EINVAL, "n_seqs, max_seqlen, total_tokens must be >= 0");
    if (n_seqs > kIntMax || max_seqlen > kIntMax) return fail(LL_EUNSUPPORTED, "n_seqs or max_seqlen exceeds 2^31-1");
    if (max_seqlen > total_tokens) return fail(LL_EINVAL, "max_seqlen > total_tokens");
    if (total_tokens > 0 && n_seqs > 0 && !cu_seqlens) return fail(LL_EINVAL, "cu_seqlens is NULL");
    const Varlen vl{cu_seqlens, n_seqs, max_seqlen};
    return layer_forward_impl(cfg, w, hidden, position_ids, 1, total_tokens, kv_seq_len, nullptr, nullptr, 0, out,
                              workspace, workspace_bytes, stream, false, &vl);
}

ll_status llama_layer_forward_chunk(const ll_layer_cfg* cfg, const ll_layer_weights* w, const void* hidden,
                                    const int64_t* position_ids, int64_t B, int64_t S, int64_t kv_seq_len,
                                    void* k_cache, void* v_cache, int64_t ctx, void* out, void* workspace,
                                    size_t workspace_bytes, void* stream) {
    return layer_forward_impl(cfg, w, hidden, position_ids, B, S, kv_seq_len, k_cache, v_cache, ctx, out, workspace,
                              workspace_bytes, stream, true);
}

}  // extern "C"
