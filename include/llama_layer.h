/*
 * llama_layer.h — C ABI of a Llama decoder-layer forward for AMD Instinct MI355X (gfx950).
 *
 * The layer (nanotron tutorial "模型层：从 Embedding 到 Loss 的实现", §9.5 LlamaDecoderLayer):
 *     h   = x + o_proj( attention( rope( qkv_proj( rmsnorm(x; g_attn) ) ) ) )
 *     out = h + down( silu(gate(hn)) * up(hn) ),   hn = rmsnorm(h; g_mlp)
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers, owned by the caller, row-major and contiguous.
 *     Every tensor of one call has the same element type (ll_dtype); position ids are int64.
 *     Pointers must be 16-byte aligned.
 *   - Linear weights are stored [out_features, in_features] and applied as y = x W^T, without bias
 *     (NJU LLM lecture 5, "LlamaDecoderLayer内部结构"). Fused weights stack their row blocks:
 *     w_qkv = [W_q; W_k; W_v] (verl "parallel_attention.py", §2 split([q,k,v])), and
 *     w_gate_up = [W_gate; W_up] (nanotron §9.4 gate_up_proj + chunk(2)).
 *   - `stream` is a hipStream_t (NULL = the null stream). Calls only enqueue work on it: they never
 *     synchronise the device or the host. The one library-owned state is the RoPE cos/sin table: one
 *     per (rope parameters, head_dim, device, stream), generated on the device by a kernel enqueued on
 *     that stream (fp64 angles and fp64 cos/sin, stored fp32). A call allocates device memory only when
 *     it needs more table rows than the stream's table holds (the table then at least doubles, so a
 *     growing kv_seq_len allocates O(log kv_seq_len) times); outgrown tables are kept until
 *     ll_release_caches(). A dynamic-NTK call whose kv_seq_len differs from the table's regenerates the
 *     rows it needs in place, in stream order, without allocating.
 *   - Errors: every host-checkable precondition is validated before any HIP call; a failed check
 *     returns LL_EINVAL (bad argument) or LL_EUNSUPPORTED (valid but not implemented) and enqueues
 *     nothing. A failed launch returns LL_EHIP. ll_last_error() gives the text of the last failure
 *     on the calling thread. No call aborts the process.
 *   - Device-side values are not validated: a position id outside [0, kv_seq_len) or a decode
 *     position outside [0, ctx) is clamped into range (the result is then meaningless, but no
 *     access leaves its buffer).
 *   - Calls on one stream are ordered; calls that share output buffers on different streams race.
 */
#ifndef LLAMA_LAYER_H
#define LLAMA_LAYER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { LL_OK = 0, LL_EINVAL = 1, LL_EUNSUPPORTED = 2, LL_EHIP = 3, LL_ENOMEM = 4 } ll_status;

/* Element type of every tensor of a call. LL_BF16: bfloat16 storage, fp32 accumulation, one
 * rounding per stored tensor. LL_F32: fp32 storage and fp32 arithmetic throughout. */
typedef enum { LL_F32 = 0, LL_BF16 = 1 } ll_dtype;

/* RoPE frequency scaling (verl "parallel_attention.py", §1: LlamaRotaryEmbedding and its linear,
 * dynamic-NTK and Llama3 variants; CSDN answer on Meta's model.py, "#### 2." apply_scaling).
 *   f_i = theta^(-2i/d), i < d/2
 *   LINEAR:      f_i / factor
 *   DYNAMIC_NTK: if kv_seq_len > original_max_pos, theta is replaced by
 *                theta * (factor*kv_seq_len/original_max_pos - (factor-1))^(d/(d-2))
 *   LLAMA3:      wavelength w = 2*pi/f_i; w < original_max_pos/high_freq_factor keeps f_i;
 *                w > original_max_pos/low_freq_factor gives f_i/factor; in between
 *                (1-s) f_i/factor + s f_i with s = (original_max_pos/w - low)/(high - low).
 * Pairs: interleaved = 0 rotates (j, j+d/2) (rotate_half, NJU lecture 5 "RoPE高效实现");
 *        interleaved = 1 rotates (2j, 2j+1) (complex multiply, CSDN answer "#### 2."). */
typedef enum { LL_ROPE_DEFAULT = 0, LL_ROPE_LINEAR = 1, LL_ROPE_DYNAMIC_NTK = 2, LL_ROPE_LLAMA3 = 3 } ll_rope_type;

typedef struct {
    int32_t type;              /* ll_rope_type */
    int32_t interleaved;       /* 0 or 1 */
    double  theta;             /* > 0 */
    double  factor;            /* > 0 (LINEAR, DYNAMIC_NTK, LLAMA3) */
    double  low_freq_factor;   /* LLAMA3, > 0 */
    double  high_freq_factor;  /* LLAMA3, > low_freq_factor */
    int64_t original_max_pos;  /* DYNAMIC_NTK, LLAMA3, > 0 */
} ll_rope;

typedef struct {
    int64_t hidden;            /* H */
    int64_t n_heads;           /* query heads */
    int64_t n_kv_heads;        /* key/value heads; n_heads % n_kv_heads == 0 */
    int64_t head_dim;          /* d: even; bf16 prefill/decode attention use the matrix-core path for 64 and 128 */
    int64_t intermediate;      /* I */
    double  eps;               /* RMSNorm eps, added to mean(x^2) inside the square root */
    ll_rope rope;
    int32_t dtype;             /* ll_dtype */
    int32_t reserved;          /* must be 0 */
} ll_layer_cfg;

typedef struct {
    const void* w_qkv;         /* [(n_heads + 2 n_kv_heads) d, H], rows Q|K|V */
    const void* w_o;           /* [H, n_heads d] */
    const void* w_gate_up;     /* [2 I, H], rows gate|up */
    const void* w_down;        /* [H, I] */
    const void* g_attn;        /* [H] gain of the first RMSNorm */
    const void* g_mlp;         /* [H] gain of the second RMSNorm */
} ll_layer_weights;

/* Bytes of device workspace llama_layer_forward (and _chunk, _varlen) needs for B sequences of S tokens;
 * ctx is the cache length that will be passed (0 without caches). It matters for decode (S == 1: the
 * per-split attention records) and for chunked prefill (room for a small chunk's key-split records).
 * Returns 0 for invalid arguments. */
size_t llama_layer_workspace_bytes(const ll_layer_cfg* cfg, int64_t B, int64_t S, int64_t ctx);

/* One decoder-layer forward (nanotron §9.5; llama3 结构详解 §3 Transformer Block).
 *   hidden       [B, S, H] input x; out [B, S, H] (out may equal hidden).
 *   position_ids [B, S] int64 RoPE positions, each in [0, kv_seq_len).
 *   kv_seq_len   host value > every position id: the RoPE table length and, for DYNAMIC_NTK, L.
 *   k_cache, v_cache: NULL, or both [B, ctx, n_kv_heads, d] holding rotated keys and values
 *                (llama3 结构详解 §3.2, cache_k / cache_v; CSDN answer "#### 3.").
 * Modes:
 *   - S > 1 (prefill): attention is causal by token index over the S tokens of the call. If caches
 *     are given, the rotated K and V of token (b, s) are also stored at slot position_ids[b, s].
 *   - S == 1 with caches (decode): the new rotated key/value overwrite slot position_ids[b] and the
 *     query attends over slots 0 .. position_ids[b] (slots before it are used as stored).
 *   - S == 1 without caches: a one-token prefill.
 * workspace: device buffer of at least llama_layer_workspace_bytes(cfg, B, S, ctx) bytes, owned by
 * the caller; its contents are scratch. */
ll_status llama_layer_forward(const ll_layer_cfg* cfg, const ll_layer_weights* w,
                              const void* hidden, const int64_t* position_ids,
                              int64_t B, int64_t S, int64_t kv_seq_len,
                              void* k_cache, void* v_cache, int64_t ctx,
                              void* out, void* workspace, size_t workspace_bytes, void* stream);

/* llama_layer_forward for callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc. Same arguments, layout, modes and results as
 * llama_layer_forward, without the workspace: the workspace and the call's RoPE table (generated on the
 * device for kv_seq_len rows) live in a static 64 MiB device array of the library, one per GPU, held until
 * the process ends. The call performs no hipMalloc, hipFree or other allocation (the library-owned RoPE
 * tables are not used) and records no profiling events.
 * Limit: llama_layer_workspace_bytes(cfg, B, S, ctx) rounded up to 256, plus kv_seq_len * head_dim * 4
 * bytes of table, must not exceed 64 MiB (e.g. Llama-3-8B-shaped decode at B = 64 with kv_seq_len 8192);
 * larger calls return LL_EINVAL and enqueue nothing.
 * Every call on one GPU uses that GPU's one array, which keeps the last call's contents: calls that overlap
 * on one GPU (different streams, or host threads without ordering) race and must not be issued. */
ll_status llama_layer_forward_noalloc(const ll_layer_cfg* cfg, const ll_layer_weights* w,
                                      const void* hidden, const int64_t* position_ids,
                                      int64_t B, int64_t S, int64_t kv_seq_len,
                                      void* k_cache, void* v_cache, int64_t ctx,
                                      void* out, void* stream);

/* Chunked prefill on a cache prefix (llama3 结构详解 §3.2: the new keys/values go to cache slots
 * start_pos .. start_pos + seqlen - 1 and attention reads slots 0 .. start_pos + seqlen - 1; CSDN answer
 * "#### 5.": for start_pos > 0 the causal mask gains start_pos leading zero columns).
 * Same arguments and layout as llama_layer_forward; k_cache and v_cache are required. The rotated K
 * and V of token (b, s) are stored at slot position_ids[b, s]; then query (b, s) attends over cache
 * slots 0 .. position_ids[b, s] (slots not written by this call are used as stored, i.e. the prefix
 * written by earlier calls). With position_ids[b, s] = s it equals llama_layer_forward with caches.
 * Positions of one sequence must be distinct and in [0, ctx). Workspace: at least
 * llama_layer_workspace_bytes(cfg, B, S, 0); sized with the call's ctx instead, it also holds the
 * records that let a small chunk share each query block's keys out over several workgroups (same
 * results up to rounding, much faster for short chunks on long prefixes). */
ll_status llama_layer_forward_chunk(const ll_layer_cfg* cfg, const ll_layer_weights* w,
                                    const void* hidden, const int64_t* position_ids,
                                    int64_t B, int64_t S, int64_t kv_seq_len,
                                    void* k_cache, void* v_cache, int64_t ctx,
                                    void* out, void* workspace, size_t workspace_bytes, void* stream);

/* Decoder layer over packed (padding-free) sequences (parallel_attention.py §3 ParallelLlamaAttentionRmPad:
 * tokens of all sequences back to back, boundaries cu_seqlens, causal attention within each sequence).
 *   hidden, out   [total_tokens, H] (out may equal hidden);
 *   position_ids  [total_tokens] int64 RoPE positions (§4 apply_rotary_pos_emb_rmpad_flash rotates each
 *                 token by its index within its sequence: pass t - cu_seqlens[i] for that convention);
 *   cu_seqlens    [n_seqs + 1] int32 on the device: 0 = cu[0] <= cu[1] <= ... <= cu[n_seqs] = total_tokens;
 *   max_seqlen    host value >= every cu[i+1] - cu[i] (sizes the launch; longer sequences are cut there).
 * Entries out of order or out of range are clamped (no out-of-bounds access) but then give unspecified
 * results. No KV cache. Workspace as llama_layer_workspace_bytes(cfg, 1, total_tokens, 0). */
ll_status llama_layer_forward_varlen(const ll_layer_cfg* cfg, const ll_layer_weights* w,
                                     const void* hidden, const int64_t* position_ids,
                                     const int32_t* cu_seqlens, int64_t n_seqs, int64_t max_seqlen,
                                     int64_t total_tokens, int64_t kv_seq_len,
                                     void* out, void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace llama_model_forward needs for B sequences of S tokens. 0 for invalid input. */
size_t llama_model_workspace_bytes(const ll_layer_cfg* cfg, int64_t vocab, int64_t B, int64_t S);

/* The model stack at prefill (CSDN answer "#### 5." Transformer.forward with start_pos = 0: h =
 * tok_embeddings(tokens); for layer in layers: h = layer(h); return output(norm(h))):
 *   layers          host array of n_layers weight sets (device pointers), applied in order;
 *   tok_embeddings  [vocab, H]; final_norm_gain [H] (the final RMSNorm, eps = cfg->eps);
 *   lm_head         [vocab, H] output projection, logits = norm(h) lm_head^T (no bias);
 *   tokens          [B, S] int64 ids (ids outside [0, vocab) are clamped); position_ids [B, S] as in
 *                   llama_layer_forward; logits [B, S, vocab] in cfg->dtype.
 * No KV cache (prefill only). workspace: at least llama_model_workspace_bytes bytes, scratch. */
ll_status llama_model_forward(const ll_layer_cfg* cfg, int64_t n_layers, const ll_layer_weights* layers,
                              const void* tok_embeddings, const void* final_norm_gain, const void* lm_head,
                              int64_t vocab, const int64_t* tokens, const int64_t* position_ids,
                              int64_t B, int64_t S, int64_t kv_seq_len, void* logits,
                              void* workspace, size_t workspace_bytes, void* stream);

/* RMSNorm over rows (llama3 结构详解 §3.1; NJU lecture 5 "编码实现RMSNorm"):
 *   y[r, i] = x[r, i] / sqrt(mean_i x[r, i]^2 + eps) * gain[i], fp32 accumulation.
 * x, y [rows, hidden] (y may equal x); gain [hidden]. */
ll_status rmsnorm(const void* x, const void* gain, void* y, int64_t rows, int64_t hidden,
                  double eps, int32_t dtype, void* stream);

/* Rotate the q and k heads of a packed qkv buffer in place (verl §1 rotary_emb + apply_rotary_pos_emb;
 * NJU lecture 5 "RoPE高效实现"). qkv [B, S, (n_heads + 2 n_kv_heads) d]; v is left untouched.
 * position_ids [B, S] in [0, kv_seq_len). */
ll_status rope_apply(const ll_rope* rope, void* qkv, const int64_t* position_ids,
                     int64_t B, int64_t S, int64_t n_heads, int64_t n_kv_heads, int64_t head_dim,
                     int64_t kv_seq_len, int32_t dtype, void* stream);

/* Grouped-query causal attention over the S tokens of each sequence (nanotron §9.3
 * flash_attn_func(causal=True); verl §2 eager softmax(q k^T / sqrt(d)) v; llama3 结构详解 §3.2 GQA):
 *   o[b, i, h*d:(h+1)*d] = sum_{j <= i} softmax_j(q'_{b,i,h} . k'_{b,j,c} / sqrt(d)) v_{b,j,c},
 *   c = h / (n_heads / n_kv_heads).
 * qkv  packed [B, S, (n_heads + 2 n_kv_heads) d], read only.
 * rope NULL: q and k are already rotated; otherwise q and k are rotated as they are loaded, at
 *      position_ids[b, s] (kv_seq_len as in llama_layer_forward).
 * o    [B, S, n_heads d].
 * k_cache, v_cache: NULL, or [B, ctx, n_kv_heads, d]: rotated K and V of token (b, s) are stored at
 *      slot position_ids[b, s] (position_ids then required even when rope is NULL). */
ll_status gqa_attn_prefill(const void* qkv, const ll_rope* rope, const int64_t* position_ids,
                           int64_t kv_seq_len, void* o, void* k_cache, void* v_cache, int64_t ctx,
                           int64_t B, int64_t S, int64_t n_heads, int64_t n_kv_heads, int64_t head_dim,
                           int32_t dtype, void* stream);

/* Attention step of chunked prefill on a cache prefix (llama3 结构详解 §3.2 cache_k[:, start_pos :
 * start_pos + seqlen] = xk, keys = cache_k[:, : start_pos + seqlen]; CSDN answer "#### 5." mask with
 * start_pos zero columns):
 *   k_cache[b, p] = k_{b,s}, v_cache[b, p] = v_{b,s} with p = position_ids[b, s], then
 *   o[b, s, h*d:(h+1)*d] = sum_{j <= p} softmax_j(q_{b,s,h} . k_cache[b,j,c] / sqrt(d)) v_cache[b,j,c].
 * qkv packed [B, S, (n_heads + 2 n_kv_heads) d] with q and k already rotated, read only;
 * position_ids [B, S] int64, distinct per sequence, in [0, ctx); k_cache, v_cache [B, ctx, n_kv_heads, d]
 * (required; slots outside this chunk are read as stored); o [B, S, n_heads d].
 * workspace: device scratch owned by the caller, or NULL. With at least
 * gqa_attn_prefill_chunk_workspace_bytes bytes a small chunk shares each query block's keys out over
 * several workgroups (partial softmax records merged by a combine pass); with less, or NULL, every query
 * block is one workgroup (same results up to fp32 rounding order, slower for small chunks). */
size_t gqa_attn_prefill_chunk_workspace_bytes(int64_t B, int64_t S, int64_t n_heads, int64_t n_kv_heads,
                                              int64_t head_dim, int64_t ctx, int32_t dtype);
ll_status gqa_attn_prefill_chunk(const void* qkv, const int64_t* position_ids, void* o,
                                 void* k_cache, void* v_cache, int64_t ctx,
                                 int64_t B, int64_t S, int64_t n_heads, int64_t n_kv_heads, int64_t head_dim,
                                 int32_t dtype, void* workspace, size_t workspace_bytes, void* stream);

/* Padding-free causal attention over packed sequences (parallel_attention.py §3: flash_attn_varlen_func
 * with cu_seqlens_q = cu_seqlens_k = cu_seqlens, max_seqlen, causal=True):
 *   o[t, h*d:(h+1)*d] = sum_{cu[i] <= j <= t} softmax_j(q_{t,h} . k_{j,c} / sqrt(d)) v_{j,c},
 *   for the sequence i with cu[i] <= t < cu[i+1].
 * qkv packed [total_tokens, (n_heads + 2 n_kv_heads) d] with q and k already rotated (read only);
 * cu_seqlens, max_seqlen as in llama_layer_forward_varlen; o [total_tokens, n_heads d]. */
ll_status gqa_attn_prefill_varlen(const void* qkv, const int32_t* cu_seqlens, int64_t n_seqs,
                                  int64_t max_seqlen, int64_t total_tokens, void* o,
                                  int64_t n_heads, int64_t n_kv_heads, int64_t head_dim,
                                  int32_t dtype, void* stream);

/* Bytes of workspace gqa_attn_decode needs. */
size_t gqa_attn_decode_workspace_bytes(int64_t B, int64_t n_heads, int64_t head_dim, int64_t ctx);

/* One decode step of grouped-query attention against a KV cache (llama3 结构详解 §3.2 with
 * seqlen = 1, start_pos = pos[b]; CSDN answer "#### 3." KV cache):
 *   k_cache[b, pos[b]] = rope(k_new), v_cache[b, pos[b]] = v_new, then
 *   o[b, h*d:(h+1)*d] = sum_{j <= pos[b]} softmax_j(q'_{b,h} . k_cache[b,j,c] / sqrt(d)) v_cache[b,j,c].
 * qkv  [B, (n_heads + 2 n_kv_heads) d] (one token per sequence); pos [B] int64 in [0, ctx) and
 * below kv_seq_len; rope NULL means q and k are already rotated. o [B, n_heads d]. */
ll_status gqa_attn_decode(const void* qkv, const ll_rope* rope, const int64_t* pos, int64_t kv_seq_len,
                          void* k_cache, void* v_cache, int64_t ctx, void* o,
                          int64_t B, int64_t n_heads, int64_t n_kv_heads, int64_t head_dim,
                          int32_t dtype, void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace swiglu_mlp needs for M rows. */
size_t swiglu_mlp_workspace_bytes(int64_t M, int64_t hidden, int64_t intermediate, int32_t dtype);

/* SwiGLU MLP (nanotron §9.4; CSDN answer "#### 4." w2(silu(w1 x) * w3 x); NJU lecture 5 "SwiGLU模块"):
 *   out = residual + (silu(x W_gate^T) * (x W_up^T)) W_down^T,  silu(z) = z / (1 + e^-z).
 * x [M, hidden] (already normalised by the caller), w_gate_up [2 I, hidden], w_down [hidden, I],
 * residual NULL (no add) or [M, hidden]; out [M, hidden] (out may equal residual, not x). */
ll_status swiglu_mlp(const void* x, const void* w_gate_up, const void* w_down, const void* residual,
                     void* out, int64_t M, int64_t hidden, int64_t intermediate, int32_t dtype,
                     void* workspace, size_t workspace_bytes, void* stream);

/* Text of the last non-OK status returned on the calling thread ("" if none). */
const char* ll_last_error(void);

/* Frees the library-owned RoPE tables of every device and stream. Not safe while work that reads them
 * is still pending on any stream. */
void ll_release_caches(void);

/* Per-stage timing of llama_layer_forward, for benchmarking. ll_profile_begin() enables HIP event
 * markers between the stages of every later llama_layer_forward on the calling thread, clears the
 * totals and creates the events for reserve_calls calls up front (more are created on demand).
 * ll_profile_begin_stages() does the same for the stages whose bits are set in stage_mask (bit s =
 * stage s, 0 .. 6; LL_EINVAL for an empty mask or higher bits): only the markers those stages need
 * are recorded, since each marker between two kernels delays the second by a few microseconds.
 * ll_profile_begin(r) is ll_profile_begin_stages(r, 0x7F).
 * ll_profile_end() waits for the recorded events, writes the summed milliseconds and call counts of
 * up to max_stages stages (stage names from ll_profile_stage_name; stages not timed report 0 ms in
 * 0 calls) and disables the markers. It returns the number of stages written, or -1 on error. */
ll_status   ll_profile_begin(int32_t reserve_calls);
ll_status   ll_profile_begin_stages(int32_t reserve_calls, uint32_t stage_mask);
int32_t     ll_profile_end(double* stage_ms, int64_t* stage_calls, int32_t max_stages);
const char* ll_profile_stage_name(int32_t stage);

/* Library version string. */
const char* ll_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LLAMA_LAYER_H */
