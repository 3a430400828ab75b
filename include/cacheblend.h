/*
 * cacheblend.h — C ABI of libcacheblend.so: fusion of independently
 * precomputed per-chunk KV caches with selective recompute, on one AMD
 * Instinct MI355X (gfx950).
 *
 * The operation (pages cited by title and section):
 *  - "論文解説: CacheBlend — RAGシステム向けKV Cache融合による高速LLMサービング"
 *    (0h-n0.github.io), section "選択的再計算": each layer recomputes Q/K/V
 *    for a selected token set only, merges the recomputed K/V of that set
 *    with the precomputed K/V of the other tokens, and runs ordinary attention;
 *    section "HKVD（High KV Deviation）トークン選定": the set is chosen by
 *    per-token KV deviation and narrowed layer by layer (gradual filtering);
 *    section "RoPE（Rotary Position Embedding）との整合性": rotation R(m);
 *    section "vLLM統合": the serving interface is fetch-per-layer,
 *    prefill-per-layer and synchronize, mirrored by cb_fetch_kv,
 *    cb_prefill_layer and cb_synchronize; section "設定パラメータ": check
 *    layer, recompute ratio and minimum token count.
 *  - "CacheBlend" explainer (abeam.tech), section "チャンク単位でKVを保存す
 *    る": chunk caches are computed alone and their positions are corrected
 *    to the real input positions at reuse.
 *  - "論文解説: Prompt Cache" (0h-n0.github.io), section "RoPEにおける位置調整":
 *    a key encoded at p' moves to p by the rotation R(p - p').
 *
 * Conventions used by every call:
 *  - Pointers are plain addresses.  "device" = HIP device memory on the
 *    current device; "host" = ordinary host memory; "pinned" = page-locked
 *    host memory from hipHostMalloc.  The caller allocates and owns every
 *    buffer passed in; the library never frees caller memory.
 *  - Element type of weights, chunk KVs, x0 and the fused KV is the model
 *    dtype (CB_F32 = IEEE float32, CB_BF16 = bfloat16); deviations and
 *    hidden outputs are float32; indices are int32.
 *  - Layouts are row-major.  A KV row is [H_kv][d_head]; a cache is
 *    [L][tokens][H_kv][d_head]; weight matrices are [out][in].
 *  - RoPE pairs are interleaved (2i, 2i+1) with theta_i = base^(-2i/d_head);
 *    cos/sin of pos*theta_i are evaluated in float64 and rounded once to
 *    float32.
 *  - `stream` is a hipStream_t (NULL = the null stream).  Work is queued
 *    asynchronously; results are ready once the stream has been synchronized.
 *  - Errors: every call returns cb_status.  Arguments are validated before
 *    anything is queued, so a failed call has no side effects.  The message
 *    of the last failure on the calling thread is cb_last_error().  No C++
 *    exception or abort crosses the ABI.  Faults of queued work surface at
 *    the next synchronizing call.
 */
#ifndef CACHEBLEND_H
#define CACHEBLEND_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CB_ABI_VERSION 6

typedef enum cb_status {
    CB_OK = 0,
    CB_E_INVALID = -1,     /* null pointer, bad enum, negative size       */
    CB_E_SHAPE = -2,       /* sizes that do not fit together / unsupported */
    CB_E_NOT_PINNED = -3,  /* host chunk KV is not page-locked             */
    CB_E_SCHEDULE = -4,    /* schedule not monotone / out of range         */
    CB_E_OOM = -5,         /* workspace allocation failed                  */
    CB_E_HIP = -6,         /* a HIP runtime call failed                    */
    CB_E_BAD_STATE = -7,   /* layer-stepped calls out of order             */
    CB_E_UNSUPPORTED = -8  /* valid request the library does not implement */
} cb_status;

typedef enum cb_dtype { CB_F32 = 0, CB_BF16 = 1 } cb_dtype;

/* Recompute schedule kinds (CacheBlend explainer (0h-n0), sections on HKVD
 * selection and configuration parameters).  With n = chunk tokens and r in
 * basis points, both give s[0] = s[1] = n (layer 0 recomputes every chunk
 * row; layer 1 is the check layer) and r = 0 gives s = 0 (full KV reuse):
 *  FIXED:   s[l] = max(1, floor(n r / 10000)) for l >= 2.
 *  GRADUAL: r1 = min(10000, floor(1.2 r)); for l >= 1,
 *           s[l+1] = max(1, floor(n (r 2^e + r1 - r) / (10000 2^e))),
 *           e = min(l-1, 30), clamped to be non-increasing. */
typedef enum cb_schedule_kind { CB_SCHED_GRADUAL = 0, CB_SCHED_FIXED = 1 } cb_schedule_kind;

/* Deviation measure: sum of squared differences between the recomputed row
 * and the re-rotated cached row, over K and V (default), K only or V only
 * (CacheBlend explainer (0h-n0), eq. 1 and the selection code).  GIVEN
 * ranks by per-token scores the caller supplies (given_scores) in place of
 * a measured deviation, through the same selection and gradual filtering:
 * for baselines such as random scores, or for scores computed outside the
 * library (e.g. query-aware ones, which the CacheBlend explainer's outlook
 * names as follow-up work). */
/* ATTN (bf16 models): at every layer whose candidates are all the chunk rows
 * (up to and including the check layer) rank by per-token attention
 * deviation, as the explainer's first-layer rule does (section "HKVD（High KV
 * Deviation）トークン選定", eq. 2 of "KVキャッシュの定義と偏差メトリクス"
 * taken row by row): for chunk row j, the sum over query heads and keys of
 * (p1 - p0)^2, p1 / p0 its causal softmax rows over the recomputed keys and
 * over the re-rotated cached keys of the chunk positions.  There every chunk
 * row is recomputed, so p1 is the full prefill's attention and p0 what full
 * KV reuse would attend with.  Later layers rank by the KV deviation. */
typedef enum cb_dev_mode {
    CB_DEV_KV = 0,
    CB_DEV_K = 1,
    CB_DEV_V = 2,
    CB_DEV_GIVEN = 3,
    CB_DEV_ATTN = 4
} cb_dev_mode;

typedef struct cb_model_cfg {
    int32_t n_layers;
    int32_t d_model;
    int32_t n_q_heads;
    int32_t n_kv_heads;   /* must divide n_q_heads (GQA)                 */
    int32_t head_dim;     /* even; 64 or 128                             */
    int32_t ffn_dim;
    double  rope_base;    /* e.g. 10000                                  */
    float   rms_eps;      /* e.g. 1e-5                                   */
    int32_t dtype;        /* cb_dtype                                    */
} cb_model_cfg;

/* One pre-norm Llama block.  All device pointers in the model dtype:
 * attn_norm[d], wq[Hq*dh][d], wk[Hkv*dh][d], wv[Hkv*dh][d], wo[d][Hq*dh],
 * mlp_norm[d], w_gate[F][d], w_up[F][d], w_down[d][F].  No biases. */
typedef struct cb_layer_weights {
    const void* attn_norm;
    const void* wq;
    const void* wk;
    const void* wv;
    const void* wo;
    const void* mlp_norm;
    const void* w_gate;
    const void* w_up;
    const void* w_down;
} cb_layer_weights;

/* Storage format of a chunk cache.  PLAIN: the model dtype.  U8 / U4:
 * per-channel quantized codes (CacheGen explainer (0h-n0), "技術的詳細",
 * step 1 "チャネル別量子化"; 8 and 4 bits from its trade-off table): for
 * each layer and each of the C = H_kv*d_head channels c, over the chunk's
 * tokens, zero z_c = min x, scale s_c = (max x - z_c) / (2^b - 1), code =
 * round-half-even((x - z_c) / s_c) clamped to [0, 2^b - 1] (code 0 where
 * s_c = 0), decided in float32.  The fused cache receives code * s_c + z_c
 * (K then rotated like PLAIN).  U8 stores one code per byte; U4 two per
 * byte, channel 2i in the low nibble and 2i+1 in the high nibble.
 * cb_quantize_kv produces both. */
typedef enum cb_kv_format { CB_KV_PLAIN = 0, CB_KV_U8 = 1, CB_KV_U4 = 2 } cb_kv_format;

/* A precomputed chunk cache at chunk-local positions 0..n_tokens-1.
 * k, v: [L][n_tokens][H_kv][d_head]; layer l starts at element (PLAIN) or
 * code (U8/U4) l * layer_stride (layer_stride >= n_tokens*H_kv*d_head),
 * which lets chunks live inside a larger pool.  on_host = 0: device memory;
 * 1: pinned host memory, copied to the device layer by layer on the
 * library's side stream.  Quantized chunks also pass qparams:
 * [L][4][H_kv*d_head] float32 (k scale, k zero, v scale, v zero of every
 * channel), in the same kind of memory as k and v.  k, v and qparams must
 * be 16-byte aligned, and the bytes of a layer stride a multiple of 16.
 *
 * Staging (host chunks only, all three or none): stage_k / stage_v
 * (device, [L][n_tokens][H_kv*d_head] dense, in the chunk's format) and,
 * for quantized chunks, stage_qparams (device [L][4][H_kv*d_head]).  Each
 * layer's fetch then copies the host layer there and reads it from there,
 * so after the fusion the staging buffers hold a device copy of the chunk
 * (the HBM tier, cb_cache_*, hands out such buffers). */
typedef struct cb_chunk_kv {
    const void* k;
    const void* v;
    int32_t n_tokens;
    int32_t on_host;
    int64_t layer_stride;
    int32_t kv_format;        /* cb_kv_format                              */
    int32_t reserved;         /* must be 0                                 */
    const float* qparams;     /* U8/U4: [L][4][H_kv*d_head]; PLAIN: NULL   */
    void* stage_k;            /* NULL, or device copy destinations         */
    void* stage_v;
    float* stage_qparams;
} cb_chunk_kv;

typedef struct cb_request {
    int32_t n_chunks;
    const cb_chunk_kv* chunks;      /* host [n_chunks]                      */
    const int32_t* chunk_offsets;   /* host [n_chunks]: 0, then contiguous  */
    int32_t n_suffix;               /* query tokens after the last chunk    */
    const void* x0;                 /* device [N][d]: layer-0 input rows of
                                       all N prompt tokens in fused order   */
    const int32_t* schedule;        /* host [L+1] or NULL: s[0..L] (see
                                       cb_schedule_kind); NULL = derive it
                                       from recompute_bp and schedule_kind  */
    int32_t recompute_bp;           /* r in basis points, 0..10000          */
    int32_t schedule_kind;          /* cb_schedule_kind                     */
    int32_t dev_mode;               /* cb_dev_mode                          */
    int32_t min_tokens;             /* N < min_tokens: plain full prefill   */
    const float* given_scores;      /* CB_DEV_GIVEN: device [N_c], the score
                                       of each chunk token by position;
                                       otherwise NULL                       */
} cb_request;

/* Outputs of a fusion.  N = chunk tokens N_c + suffix. */
typedef struct cb_outputs {
    void* fused_k;      /* device [L][N][H_kv][d_head], model dtype (required) */
    void* fused_v;      /* device [L][N][H_kv][d_head], model dtype (required) */
    int32_t* sel_idx;   /* device [L][N_c] or NULL: row l holds the positions
                           kept after layer l, ascending, first s[l+1] valid  */
    int32_t* sel_count; /* host [L] or NULL: s[l+1], written before return   */
    float* hidden_out;  /* device [N_s + s[L]][d] or NULL: output rows of the
                           last layer (kept chunk rows then suffix, by position) */
    float* deviation;   /* device [L][N_c] or NULL: per-token deviation where
                           measured, NaN elsewhere                            */
} cb_outputs;

typedef struct cb_model cb_model;
typedef struct cb_plan cb_plan;

/* ------------------------------------------------------------- basics */
int cb_abi_version(void);
/* Message of the last failed call on this thread ("" if none).  Valid until
 * the next failing call on the same thread. */
const char* cb_last_error(void);

/* Host helper: the integer schedule s[0..n_layers] into s_out (host). */
cb_status cb_schedule(int32_t n_chunk_tokens, int32_t recompute_bp, int32_t kind,
                      int32_t n_layers, int32_t* s_out);

/* ------------------------------------------------------------- model */
/* Validates cfg and copies the weight pointer table (not the weights: the
 * caller keeps them alive until cb_model_destroy).  final_norm: device [d]
 * in the model dtype, the gain of the RMSNorm before the LM head (used by
 * cb_lm_head when it is given no final_norm), or NULL.  Builds the RoPE
 * table on the current device.  *out receives the handle. */
cb_status cb_model_create(const cb_model_cfg* cfg, const cb_layer_weights* layers,
                          const void* final_norm, cb_model** out);
void cb_model_destroy(cb_model* model);

/* Workspace of the model's fusion plans (cb_blend, cb_blend_batch, the
 * layer-stepped plans, cb_prefill).  By default each plan allocates it in
 * the order of its stream from a memory pool of the model.
 *  ws != NULL: plans carve it from the caller's device buffer [ws, ws +
 *    bytes) (256-byte aligned) and allocate nothing; the caller keeps it
 *    alive and unused by anything else until the plans' work is done, and
 *    plans of the model that run at the same time (other streams) race on it.
 *  ws == NULL, bytes > 0: pool allocations, at most bytes per plan.
 *  ws == NULL, bytes == 0: pool allocations without a limit.
 * A plan whose workspace does not fit fails with CB_E_OOM before anything is
 * queued.  cb_workspace_size gives the bytes a request needs (validating it
 * as cb_plan_create does, allocating nothing). */
cb_status cb_model_set_workspace(cb_model* model, void* ws, int64_t bytes);
cb_status cb_workspace_size(cb_model* model, const cb_request* req, int64_t* bytes);

/* ------------------------------------------------------------- fusion */
/* One-shot fusion of a request: per layer, rotate the chunk caches to their
 * real positions, recompute the scheduled rows, measure deviation, keep the
 * top rows, merge them into the fused cache, attend over the whole fused
 * cache, finish the block.  Equivalent to cb_plan_create, then cb_fetch_kv
 * and cb_prefill_layer for every layer, then cb_plan_destroy.
 * (CacheBlend explainer (0h-n0), "選択的再計算" Steps 1-4 with the K/V merge
 * equations, and "HKVD（High KV Deviation）トークン選定" for the kept rows;
 * CacheBlend explainer (abeam.tech), "高いずれを持つトークンだけを再計算する":
 * Q/K/V of the selected tokens only, which attend over the whole input.) */
cb_status cb_blend(cb_model* model, const cb_request* req, const cb_outputs* out,
                   void* stream);

/* Layer-stepped form.  cb_plan_create validates everything and reserves the
 * workspace (stream-ordered on `stream`).  cb_fetch_kv(plan, l) queues the
 * load (pinned host -> device for host chunks) and rotation of layer l's
 * chunk caches into fused_k/v[l] on the plan's side stream and records an
 * event; layers may be fetched in any order, each at most once.
 * cb_prefill_layer(plan, l) must be called for l = 0, 1, ... in order; it
 * fetches layer l first if that was not done, makes `stream` wait for the
 * fetch, and queues the layer.  cb_synchronize blocks until all queued work
 * of the plan is done.  cb_plan_destroy releases the plan (it does not wait;
 * the workspace is freed in stream order). */
cb_status cb_plan_create(cb_model* model, const cb_request* req, const cb_outputs* out,
                         void* stream, cb_plan** plan);
cb_status cb_fetch_kv(cb_plan* plan, int32_t layer);
cb_status cb_prefill_layer(cb_plan* plan, int32_t layer);
cb_status cb_synchronize(cb_plan* plan);
void cb_plan_destroy(cb_plan* plan);

/* Full prefill (the reference the CacheBlend explainer (0h-n0) compares
 * against, section "KVキャッシュの定義と偏差メトリクス": KV^full; and the
 * per-chunk precompute of the abeam explainer's "チャンク単位でKVを保存する")
 * of n_tokens rows x0 (device [n][d], model dtype) at
 * positions pos0..pos0+n-1.  k_out/v_out: device [L][n][H_kv][d_head] model
 * dtype; hidden_out: device [n][d] float32 or NULL.  With pos0 = 0 this
 * precomputes a chunk cache at chunk-local positions. */
cb_status cb_prefill(cb_model* model, const void* x0, int32_t n_tokens, int32_t pos0,
                     void* k_out, void* v_out, float* hidden_out, void* stream);

/* ------------------------------------------------------------- first token
 * What the fused cache is used for next (CacheBlend explainer (abeam.tech),
 * "用語解説": the KV cache spares generation from recomputing past tokens;
 * TTFT is the time to the first output token).
 *
 * cb_lm_head: for each of `rows` rows of x (device float32 [rows][d], e.g.
 * the last row of hidden_out), logits[r] = W_lm rmsnorm(x[r]; final_norm)
 * (device float32 [rows][vocab]); final_norm [d] (NULL: the model's, from
 * cb_model_create) and w_lm [vocab][d] are device pointers in the model
 * dtype.  argmax (device int32 [rows] or
 * NULL): index of the largest logit, NaN above all, smallest index among
 * equals.
 *
 * cb_decode_step: one more token through every layer on top of a fused
 * cache.  x: device [d] model dtype (the new token's embedding) at position
 * n_ctx; fused_k / fused_v: device, layer l's rows 0..n_ctx-1 at element
 * l * layer_rows * H_kv*d_head (layer_rows >= n_ctx; a request inside a
 * batch passes its first row and the batch's total rows).  Per layer the
 * token's RoPE'd key and its value are written to k_new / v_new (device
 * [L][H_kv][d_head], model dtype), and it attends over the n_ctx cached
 * keys plus its own.  hidden_out: device float32 [d], the last layer's
 * output row (before the final norm). */
cb_status cb_lm_head(cb_model* model, const float* x, int32_t rows, const void* final_norm,
                     const void* w_lm, int32_t vocab, float* logits, int32_t* argmax,
                     void* stream);
cb_status cb_decode_step(cb_model* model, const void* x, int32_t n_ctx, const void* fused_k,
                         const void* fused_v, int64_t layer_rows, void* k_new, void* v_new,
                         float* hidden_out, void* stream);

/* ------------------------------------------------------------- batches
 * Several requests fused in one call (the serving case of the CacheBlend
 * explainer (0h-n0), section "vLLM統合": many RAG requests whose contexts
 * draw on a shared store of chunk caches).  Every request is fused exactly as
 * cb_blend would fuse it alone; the rows of all requests are stacked in each
 * projection, and attention, deviation and selection stay per request.
 *
 * Chunks come from a pool; a request lists pool indices in prompt order and
 * its chunk offsets are the running sums of their lengths (0, n_0,
 * n_0 + n_1, ...).  A pool chunk may be used by several requests or several
 * times in one request: a host-resident chunk is copied to the device once
 * per layer and rotated from there into every place it is used.
 *
 * Stacking: request b has N_b = N_c,b + N_s,b prompt tokens and owns rows
 * G_b .. G_b + N_b - 1 of every stacked [sum N] array, G_b = N_0 + ... +
 * N_{b-1}, in its own fused order.  Its chunk-token columns of [L][sum N_c]
 * outputs start at C_b = N_c,0 + ... + N_c,b-1.  Positions, sel_idx
 * entries and deviation columns are the request's own (0 = its first
 * token). */
typedef struct cb_batch_item {
    int32_t n_chunks;
    const int32_t* chunk_ids;     /* host [n_chunks]: indices into the pool   */
    int32_t n_suffix;             /* query tokens after the last chunk        */
    const int32_t* schedule;      /* host [L+1] or NULL: derive it from the
                                     batch's recompute_bp / schedule_kind     */
} cb_batch_item;

typedef struct cb_batch_request {
    int32_t n_pool;
    const cb_chunk_kv* pool;      /* host [n_pool]; only used entries are read */
    int32_t n_requests;
    const cb_batch_item* items;   /* host [n_requests]                        */
    const void* x0;               /* device [sum N][d], model dtype, stacked  */
    int32_t recompute_bp;
    int32_t schedule_kind;
    int32_t dev_mode;
    int32_t min_tokens;           /* per request: N_b < min_tokens -> full prefill */
    const float* given_scores;    /* CB_DEV_GIVEN: device [sum N_c], request b's
                                     scores by position at columns C_b..; else NULL */
} cb_batch_request;

typedef struct cb_batch_outputs {
    void* fused_k;      /* device [L][sum N][H_kv][d_head] (required)          */
    void* fused_v;      /* device [L][sum N][H_kv][d_head] (required)          */
    int32_t* sel_idx;   /* device [L][sum N_c] or NULL: request b's kept
                           positions after layer l at columns C_b.., ascending,
                           first s_b[l+1] valid                                */
    int32_t* sel_count; /* host [n_requests][L] or NULL: s_b[l+1]              */
    float* hidden_out;  /* device [sum (s_b[L] + N_s,b)][d] or NULL: last-layer
                           output rows, request by request (kept chunk rows,
                           then suffix, by position)                           */
    float* deviation;   /* device [L][sum N_c] or NULL: deviation by position
                           at columns C_b.., NaN where not measured            */
} cb_batch_outputs;

/* One-shot fusion of a batch; stream-ordered like cb_blend.  Per layer the
 * used host chunks are copied once on the side stream and rotated into
 * every request that uses them while the previous layer computes. */
cb_status cb_blend_batch(cb_model* model, const cb_batch_request* req,
                         const cb_batch_outputs* out, void* stream);

/* ------------------------------------------------------------- chunk store
 * Load controller (CacheBlend explainer (0h-n0), "パイプライン実行とロード
 * コントローラ"): recomputing a fraction r of the prompt costs r T_prefill,
 * loading the chunk caches costs T_load = per_token_kv_bytes * n_tokens /
 * throughput, and layer-wise pipelining hides the load when r T_prefill >=
 * T_load; the controller picks r* = max(r_min, T_load / T_prefill).
 * *r_bp_out = r* in basis points: the ratio to the nearest basis point
 * (halves up), at least r_min_bp, at most 10000.  Times in seconds, bytes
 * and throughput (bytes/s) positive and finite; host only. */
cb_status cb_controller_ratio(double t_prefill_s, double per_token_kv_bytes, int64_t n_tokens,
                              double throughput_bytes_per_s, int32_t r_min_bp,
                              int32_t* r_bp_out);

/* HBM tier in front of chunk caches held in pinned host memory
 * (CachedAttention explainer (0h-n0), "エビクションポリシー"; Prompt Cache
 * explainer (0h-n0), "キャッシュヒット率とエビクション"): whole chunk caches
 * are kept in device memory up to a byte budget; the least recently used
 * leave first.
 *
 * Protocol, all on one caller stream: cb_cache_resolve for the chunk uses
 * of a request or batch, the fusion with the resolved descriptors (queued
 * on the same stream), then cb_cache_commit.  A missed chunk is copied to
 * the device once, by the fusion's own per-layer fetch, into the entry the
 * lookup reserved for it (the staging fields of cb_chunk_kv); commit makes
 * those entries available to later lookups.  A key names one chunk cache
 * (content, length and format) for the life of the tier, e.g. a hash of
 * its text. */
typedef struct cb_chunk_cache cb_chunk_cache;

typedef struct cb_cache_stat {
    int64_t lookups;            /* host chunk uses looked up                 */
    int64_t hits;               /* of which served from HBM                  */
    int64_t admitted;           /* entries filled by fusions and committed   */
    int64_t evicted;            /* entries released                          */
    int64_t resident_entries;
    int64_t resident_bytes;     /* device bytes held by entries              */
    int64_t copied_bytes;       /* host -> device bytes staged into entries  */
} cb_cache_stat;

/* A tier on the current device for chunks of n_layers layers of row =
 * H_kv*d_head elements in dtype (quantized chunks are stored as codes plus
 * parameters); capacity_bytes of device memory for entries (0: nothing is
 * ever kept).  Entries come from a memory pool of the tier. */
cb_status cb_cache_create(int32_t n_layers, int32_t row, int32_t dtype, int64_t capacity_bytes,
                          cb_chunk_cache** out);
/* Waits for all work on the device, then releases every entry. */
void cb_cache_destroy(cb_chunk_cache* cache);
/* For each of n uses (keys and chunks host [n]), out (host [n]) receives:
 * for a pinned-host chunk whose key is resident, the descriptor of its HBM
 * copy (a hit, which becomes the most recently used); for another
 * pinned-host chunk, the chunk with staging buffers of a new entry, when
 * least recently used entries that this call does not use can be released
 * to make room (else the chunk unchanged); any other chunk unchanged.
 * hits (host [n] or NULL): 1 for a hit.  Entries are allocated and
 * released in the order of `stream`.  Entries reserved by an earlier
 * resolve that was not committed are released. */
cb_status cb_cache_resolve(cb_chunk_cache* cache, int32_t n, const uint64_t* keys,
                           const cb_chunk_kv* chunks, cb_chunk_kv* out, int32_t* hits,
                           void* stream);
/* After the fusion that reads the resolved descriptors is queued: the
 * entries that resolve reserved for these keys become resident. */
cb_status cb_cache_commit(cb_chunk_cache* cache, int32_t n, const uint64_t* keys);
cb_status cb_cache_stats(cb_chunk_cache* cache, cb_cache_stat* out);
/* Host-only replay of the tier's policy on batches of uses (batch b has
 * batch_sizes[b] consecutive entries of keys / sizes in bytes), each batch
 * resolved and committed: hits_out [total uses] gets 1 for a hit;
 * evicted_per_batch [n_batches] the number of entries released in each
 * batch, and evicted_out (NULL, or room for one key per use) their keys in
 * release order.  For tests and capacity planning. */
cb_status cb_cache_replay(int64_t capacity_bytes, int32_t n_batches, const int32_t* batch_sizes,
                          const uint64_t* keys, const int64_t* sizes, int32_t* hits_out,
                          uint64_t* evicted_out, int32_t* evicted_per_batch);

/* ------------------------------------------------------------- timing
 * Per-kernel-class timing of the fusion path with HIP events recorded on the
 * stream each kernel runs on (the caller's stream, or the side stream for
 * rotation).  Off by default; while on, every launch of a plan on this model
 * is bracketed by an event pair.  Algorithmic work per launch is accumulated
 * from the launch shapes: flops for the projections, bytes moved for the
 * bandwidth-bound kernels (attention flops depend on the kept positions and
 * are left to the caller). */
typedef enum cb_kernel_class {
    CB_K_ROTATE = 0,    /* chunk K rotation + V copy into the fused cache   */
    CB_K_RMSNORM,
    CB_K_GEMM_QKV,
    CB_K_DEVIATION,
    CB_K_SELECT,        /* selection, and the kept positions of layers that keep
                           every row (copied after the last layer)               */
    CB_K_SCATTER,
    CB_K_ATTENTION,
    CB_K_GEMM_O,
    CB_K_GEMM_GATEUP,
    CB_K_GEMM_DOWN,
    CB_K_DECODE_GEMV,   /* decode step and LM head matrix-vector products */
    CB_K_DECODE_ATTN,   /* decode-step attention over the fused cache     */
    CB_K_COUNT
} cb_kernel_class;

typedef struct cb_kernel_stat {
    int64_t launches;
    double total_ms;    /* summed event-measured durations   */
    double flops;       /* summed algorithmic flops          */
    double bytes;       /* summed algorithmic bytes moved    */
} cb_kernel_stat;

/* enable != 0 turns timing on and clears the statistics; 0 turns it off. */
cb_status cb_profile_enable(cb_model* model, int32_t enable);
/* Waits for the timed work and writes stats[CB_K_COUNT] (host). */
cb_status cb_profile_read(cb_model* model, cb_kernel_stat* stats);

/* ------------------------------------------------------------- kernels
 * Single steps of the path, exposed for parity tests.  All pointers are
 * device pointers unless stated. */

/* RoPE re-alignment (Prompt Cache explainer, RoPE position adjustment):
 * k_out[t] = R(delta) k_in[t] for n_tokens rows of [n_heads][head_dim];
 * v_out[t] = v_in[t] when v_in is not NULL.  In-place (k_out == k_in) is
 * allowed; otherwise buffers must not overlap. */
cb_status cb_rope_rerotate(int32_t dtype, const void* k_in, void* k_out,
                           const void* v_in, void* v_out, int32_t n_tokens,
                           int32_t n_heads, int32_t head_dim, int32_t delta,
                           double rope_base, void* stream);

/* Per-channel quantization of one chunk tensor (K or V) in the format
 * described at cb_kv_format.  x: [n_layers][n_tokens][row] in dtype, layer
 * l at element l * x_layer_stride.  bits: 8 or 4.  codes: [n_layers]
 * [n_tokens][row * bits / 8] bytes, dense (layer l at byte l * n_tokens *
 * row * bits / 8).  scale, zero: float32, the row values of layer l at
 * element l * param_stride (param_stride = 4 * row with scale = qparams
 * and zero = qparams + row for K, + 2 row and + 3 row for V, gives the
 * qparams layout of cb_chunk_kv).  row must be a multiple of 8; pointers
 * 16-byte aligned; x must be finite. */
cb_status cb_quantize_kv(int32_t dtype, const void* x, int32_t n_layers, int32_t n_tokens,
                         int32_t row, int64_t x_layer_stride, int32_t bits, void* codes,
                         float* scale, float* zero, int64_t param_stride, void* stream);

/* Dequantization fused with RoPE re-alignment, for one layer:
 * k_out[t] = R(delta) (k_codes[t] * s_k + z_k), v_out[t] = v_codes[t] * s_v
 * + z_v (when v_codes is not NULL) for n_tokens rows of [n_heads][head_dim];
 * qparams: [4][n_heads*head_dim] (k scale, k zero, v scale, v zero);
 * kv_format CB_KV_U8 or CB_KV_U4; outputs in dtype. */
cb_status cb_dequant_rerotate(int32_t dtype, int32_t kv_format, const void* k_codes,
                              const void* v_codes, const float* qparams, void* k_out,
                              void* v_out, int32_t n_tokens, int32_t n_heads, int32_t head_dim,
                              int32_t delta, double rope_base, void* stream);

/* KV deviation (CacheBlend explainer (0h-n0), eq. 1 squared):
 * dev[i] = sum over the row of (k_new - k_cached)^2 (+ (v_new - v_cached)^2)
 * for n_rows rows of row_elems elements; fp32 accumulation. */
cb_status cb_deviation(int32_t dtype, const void* k_new, const void* v_new,
                       const void* k_cached, const void* v_cached, int32_t n_rows,
                       int32_t row_elems, int32_t dev_mode, float* dev_out, void* stream);

/* Per-token attention deviation (the CB_DEV_ATTN measure) of n rows at
 * positions 0..n-1, bf16 only: q [n][Hq][dh] (RoPE applied), k_new and
 * k_cached [n][Hkv][dh]; dev_out[j] = sum over query heads h and keys
 * k <= j of (p1 - p0)^2, p1 / p0 the softmax rows of q_j . k / sqrt(dh)
 * over k_new and over k_cached (query head h reads KV head h / (Hq/Hkv)).
 * Allocates a workspace of Hq * n floats in stream order. */
cb_status cb_attention_deviation(int32_t dtype, const void* q, const void* k_new,
                                 const void* k_cached, int32_t n, int32_t n_q_heads,
                                 int32_t n_kv_heads, int32_t head_dim, float* dev_out,
                                 void* stream);

/* HKVD selection (CacheBlend explainer (0h-n0), "HKVD（High KV Deviation）
 * トークン選定", selection code: the top k by deviation, re-sorted by
 * position): the k indices of the largest dev values under the total
 * order (NaN first, larger first, -0.0 == +0.0, then smaller index first),
 * written ascending to idx_out[0..k).  0 <= k <= n. */
cb_status cb_topk_select(const float* dev, int32_t n, int32_t k, int32_t* idx_out,
                         void* stream);

/* Step 1 (input masking: gather the selected rows) and Step 3 (K/V merge:
 * the recomputed rows of the selected tokens into the cached KV) of the
 * CacheBlend explainer (0h-n0), "選択的再計算":
 * dst row i = src row idx[i] (gather) / dst row idx[i] = src row i (scatter);
 * rows of row_bytes bytes (a multiple of 4); idx device int32[n_rows]. */
cb_status cb_gather_rows(const void* src, void* dst, const int32_t* idx, int32_t n_rows,
                         int64_t row_bytes, void* stream);
cb_status cb_scatter_rows(const void* src, void* dst, const int32_t* idx, int32_t n_rows,
                          int64_t row_bytes, void* stream);

/* y = x / sqrt(mean(x^2) + eps) * g over rows of d; x float32 or model
 * dtype (x_dtype), g and y in y_dtype. */
cb_status cb_rmsnorm(int32_t x_dtype, const void* x, int32_t y_dtype, const void* g,
                     void* y, int32_t rows, int32_t d, float eps, void* stream);

/* c[m][n] = sum_k a[m][k] b[n][k] (float32 out) on the matrix cores.
 * k must be a multiple of 64 (bf16) or 32 (f32). */
cb_status cb_gemm(int32_t dtype, const void* a, const void* b, float* c, int32_t m,
                  int32_t n, int32_t k, void* stream);

/* Step 4 of the CacheBlend explainer (0h-n0), "選択的再計算" (ordinary
 * attention; the selected tokens attend over the whole input, abeam
 * explainer, "高いずれを持つトークンだけを再計算する").
 * Causal attention by real position: n_q query rows q [n_q][Hq][dh] at
 * positions q_pos (device int32, ascending) over keys k, v [n_kv][Hkv][dh] at
 * positions 0..n_kv-1; key j visible to query i iff j <= q_pos[i]; query
 * head h reads KV head h / (Hq/Hkv); out [n_q][Hq][dh] in dtype. */
cb_status cb_attention(int32_t dtype, const void* q, const int32_t* q_pos, int32_t n_q,
                       const void* k, const void* v, int32_t n_kv, int32_t n_q_heads,
                       int32_t n_kv_heads, int32_t head_dim, void* out, void* stream);

/* ------------------------------------------------------------- no allocation
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.
 *
 * cb_attention_noalloc computes exactly what cb_attention computes (same
 * arguments, same kernels, bit-identical results) but allocates nothing:
 * the split-key partials that cb_attention places in a per-call workspace
 * live in a fixed device array of CB_NOALLOC_SCRATCH_BYTES bytes inside the
 * library, one copy per GPU, held until the process ends.  A call whose
 * partials would not fit returns CB_E_SHAPE (cb_attention serves it).  Every
 * call on one GPU shares that array, so calls that overlap in time on one
 * GPU (other streams, other threads) race; calls ordered on one stream do
 * not.  The first call on a device looks up the array's address there. */
#define CB_NOALLOC_SCRATCH_BYTES (80ull << 20)
cb_status cb_attention_noalloc(int32_t dtype, const void* q, const int32_t* q_pos, int32_t n_q,
                               const void* k, const void* v, int32_t n_kv, int32_t n_q_heads,
                               int32_t n_kv_heads, int32_t head_dim, void* out, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* CACHEBLEND_H */
