// Launch wrappers of the gfx950 kernels (internal to libcacheblend.so).
// Every wrapper checks that its grid fits the buffers it is given before
// launching and returns the launch status.
#pragma once

#include "common.h"

namespace cb {

// ------------------------------------------------------------------ RoPE
// Table of (cos, sin)(pos * theta_i), float2 [n_pos][head_dim / 2].
struct RopeTab {
    const float2* tab = nullptr;
    int n_pos = 0;
    int half = 0;
};

// One chunk to move into the fused cache of one layer.
struct RotJob {
    const void* k_src;          // chunk K rows of layer 0 (nullptr: rotate k_dst in place)
    const void* v_src;          // chunk V rows of layer 0 (nullptr: V already in place)
    int64_t src_layer_stride;   // elements between consecutive layers of k_src/v_src
    int dst_row;                // first destination row (chunk offset)
    int n_tokens;
    int delta;                  // rotation amount (>= 0 or < 0)
    int pad_;
};

// Jobs travel by value in the kernel arguments (one launch per 64 chunks).
constexpr int kMaxRotJobs = 64;
struct RotJobs {
    RotJob j[kMaxRotJobs];
    int n;
    int max_tokens;
};

// For every job j and token t < n_tokens: K row (dst_row + t) of k_dst =
// R(delta) * K row t of the job's layer-`layer` source; V copied likewise.
hipError_t launch_rerotate(int dtype, const RotJobs& jobs, int layer, void* k_dst, void* v_dst,
                           int n_heads, int head_dim, const RopeTab& rope, hipStream_t s);

// ------------------------------------------------------------------ quantized chunks
// Per-channel quantized chunk caches (8- or 4-bit codes, a float32 scale and
// zero point per layer and channel; 4-bit codes two per byte, even channel
// in the low nibble).

// One quantized chunk to dequantize into the fused cache of one layer.
struct QRotJob {
    const uint8_t* k;           // K codes of layer 0
    const uint8_t* v;           // V codes of layer 0 (nullptr: no V)
    const float* qp;            // [4][row] of layer 0: k scale, k zero, v scale, v zero
    int64_t code_layer_stride;  // bytes between layers of k / v
    int64_t qp_layer_stride;    // floats between layers of qp
    int dst_row;                // first destination row (chunk offset)
    int n_tokens;
    int delta;                  // rotation amount
    int staged;                 // host bookkeeping: k/v/qp are offsets into a staging area
};

constexpr int kMaxQRotJobs = 32;
struct QRotJobs {
    QRotJob j[kMaxQRotJobs];
    int n;
    int max_tokens;
};

// For every job and token t: K row (dst_row + t) of k_dst = R(delta) *
// dequant(K codes row t of layer `layer`); V row = dequant(V codes row t).
hipError_t launch_dequant_rerotate(int dtype, int bits, const QRotJobs& jobs, int layer,
                                   void* k_dst, void* v_dst, int n_heads, int head_dim,
                                   const RopeTab& rope, hipStream_t s);

// Codes, scale and zero of x [n_layers][n_tokens][row] per layer and channel;
// ws: scratch of quantize_workspace() bytes (per-slice channel ranges).
size_t quantize_workspace(int n_layers, int n_tokens, int row);
hipError_t launch_quantize(int dtype, const void* x, int n_layers, int n_tokens, int row,
                           int64_t x_layer_stride, int bits, void* codes, float* scale,
                           float* zero, int64_t param_stride, void* ws, size_t ws_bytes,
                           hipStream_t s);

// p[i] = base + i for i < n.
hipError_t launch_iota(int* p, int n, int base, hipStream_t s);

// ------------------------------------------------------------------ rows
hipError_t launch_gather_rows(const void* src, void* dst, const int* idx, int n_rows,
                              int64_t row_bytes, hipStream_t s);
hipError_t launch_scatter_rows(const void* src, void* dst, const int* idx, int n_rows,
                               int64_t row_bytes, hipStream_t s);

// y[r] = rmsnorm(x[row(r)]) * g with row(r) = idx ? idx[r] : r.  When
// x_copy is not null the (gathered) input row is also stored there as f32.
hipError_t launch_rmsnorm(int x_dtype, const void* x, const int* idx, int y_dtype,
                          const void* g, void* y, float* x_copy, int rows, int d,
                          float eps, hipStream_t s);

// K/V rows of the recomputed set into the fused cache: for r < n_rows,
// fused row dst_row[r] receives k_new/v_new row src_idx[r].
hipError_t launch_scatter_kv(int dtype, const void* k_new, const void* v_new,
                             const int* src_idx, const int* dst_row, void* fk, void* fv,
                             int n_rows, int kv_dim, hipStream_t s);

// ------------------------------------------------------------------ requests
// Rows of several requests are stacked in every projection.  Per layer,
// request b owns the recomputed rows R[r_off .. r_off + n_c + n_s) (its n_c
// chunk rows by position, then its n_s suffix rows) and the query rows
// Q[q_off .. q_off + k + n_s) (the k chunk rows it keeps, then the suffix).
// Each stacked row carries a local position (RoPE, causality) and a global
// row of the fused cache.  Tables travel by value in kernel arguments,
// kMaxReq requests per launch.
constexpr int kMaxReq = 64;
struct ReqRows {
    int r_off, n_c, n_s, k;
    int q_off;
    int c_off;      // compact slot of the first chunk row in the deviation array
    int out_col;    // column of the request in per-layer [sum N_c] outputs
    int pad_;
};
struct ReqTab {
    ReqRows r[kMaxReq];
    int n;
    int max_c;      // largest n_c in the table
};

// Initial rows of request b: count rows from r_off with local positions
// lp0 + i and global rows g0 + i.
struct RowInit {
    int r_off, count, lp0, g0;
};
struct RowInitTab {
    RowInit r[kMaxReq];
    int n;
};
hipError_t launch_init_rows(const RowInitTab& t, int* pos, int* rows, hipStream_t s);

// Fills p[0..n) with the float value v.
hipError_t launch_fill(float* p, int64_t n, float v, hipStream_t s);

// Row copies within one int array of rows of row_len entries: row dst =
// row src for every pair (sources are never destinations of the same call).
constexpr int kMaxRowCopies = 64;
struct RowCopy {
    int dst, src;
};
struct IntRowCopies {
    RowCopy c[kMaxRowCopies];
    int n;
};
hipError_t launch_copy_int_rows(int* base, int64_t row_len, const IntRowCopies& t,
                                hipStream_t s);

// ------------------------------------------------------------------ selection
// For every request of the table and i < n_c: dev[c_off + i] = deviation of
// new row (r_off + i) against cached row crow = grow[r_off + i] (grow null:
// r_off + i).
hipError_t launch_deviation(int dtype, const void* k_new, const void* v_new,
                            const void* k_cached, const void* v_cached, const int* grow,
                            const ReqTab& t, int kv_dim, int mode, float* dev, hipStream_t s);

// Kernel-level top-k: idx_out[0..k) = kept indices, ascending.
hipError_t launch_topk(const float* dev, int n, int k, int* idx_out, hipStream_t s);

// Blend bookkeeping for one layer, one workgroup per request: keeps the k
// chunk rows with the largest deviation (all of them when k == n_c) and
// writes Q: sel_local[q_off + t] = stacked R index of kept row t (ascending
// position) then of the suffix rows; pos_q / row_q their local positions and
// global rows.  Optional: sel_pos[out_col + t] = kept local positions, and
// (when dev_out) dev_out[out_col + pos] = the deviation of every chunk row.
// dev[q.c_off + i] = scores[q.out_col + pos_r[q.r_off + i]] for the chunk
// rows of every request of the table (caller-given scores in place of a
// measured deviation).
hipError_t launch_given_scores(const float* scores, const ReqTab& t, const int* pos_r,
                               float* dev, hipStream_t s);

hipError_t launch_select(const float* dev, const ReqTab& t, const int* pos_r, const int* row_r,
                         int* sel_local, int* pos_q, int* row_q, int* sel_pos, float* dev_out,
                         hipStream_t s);

// ------------------------------------------------------------------ GEMM
enum Epi : int {
    EPI_STORE_F32 = 0,  // out0 (f32) [M][N] = acc
    EPI_QKV = 1,        // RoPE on q/k columns at pos[row]; q -> out0, k -> out1, v -> out2
    EPI_RESID = 2,      // out0 (f32) [M][N] = resid[ridx[row]] + acc
    EPI_SWIGLU = 3,     // out0 (T) [M][F] = silu(acc_gate) * acc_up
};

struct GemmArgs {
    const void* a;      // [M][K]
    const void* b0;     // weight rows [n0][K] (q / gate / plain B)
    const void* b1;     // weight rows [n1][K] (k / up)
    const void* b2;     // weight rows (v)
    int n0, n1;         // row counts of b0, b1 (b2 has N - n0 - n1)
    int M, N, K;        // for SWIGLU, N = F (output columns)
    void* out0;
    void* out1;
    void* out2;
    const float* resid; // EPI_RESID
    const int* ridx;    // EPI_RESID residual row map (nullptr = identity)
    const int* pos;     // EPI_QKV positions per row
    RopeTab rope;
    int head_dim;
    const int* kv_rows; // EPI_QKV: row of out1 / out2 that result row r of K / V goes to
                        // (nullptr = r; K and V then land straight in a cache)
};
hipError_t launch_gemm(int dtype, int epi, const GemmArgs& g, hipStream_t s);

// ------------------------------------------------------------------ decode
// One-row products y = W x for a decode step (W [N][K] row-major, x [K] in
// the model dtype), with the GEMM epilogues: EPI_QKV (q | k | v rows, RoPE
// at `pos` on q and k, model dtype outputs out0/out1/out2), EPI_RESID and
// EPI_STORE_F32 (f32 out0, + resid), EPI_SWIGLU (SiLU(b0 x) * (b1 x), N
// columns, model dtype out0).
struct GemvArgs {
    const void* x;
    const void* b0;
    const void* b1;
    const void* b2;
    int N, K;
    int n0, n1;
    void* out0;
    void* out1;
    void* out2;
    const float* resid;
    RopeTab rope;
    int pos;
    int head_dim;
};
hipError_t launch_gemv(int dtype, int epi, const GemvArgs& g, hipStream_t s);

// out[r] = argmax of row r of v ([rows][n], row stride `stride`): larger
// first, NaN above all, smaller index among equals.
hipError_t launch_argmax(const float* v, int rows, int n, int64_t stride, int* out, hipStream_t s);

// Attention of one query row (q [Hq][dh]) at position n_ctx over keys
// 0..n_ctx-1 of k / v ([n_ctx][Hkv][dh], model dtype) and its own key and
// value k_new / v_new ([Hkv][dh]); out [Hq][dh].  part_o [Hq][segments][dh]
// and part_ml [Hq][segments][2]: float scratch for the key segments.
struct DecodeAttnArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* k_new;
    const void* v_new;
    void* out;
    int n_ctx;
    int n_kv_heads;
    int group;          // query heads per KV head
    int head_dim;
    float scale;
    float* part_o;
    float* part_ml;
};
int decode_attention_segments(int n_ctx);
hipError_t launch_decode_attention(int dtype, const DecodeAttnArgs& a, hipStream_t s);

// ------------------------------------------------------------------ attention
// Causal attention of query rows over one request's keys.  A request range
// covers output rows q0..q0+nq-1 (row i reads q row qidx[i], qidx null: i,
// at position q_pos[i]); its keys/values are rows g0..g0+n_kv-1 of k/v at
// positions kv_pos0 + j.  The launcher cuts ranges into query tiles of the
// kernel's height, orders them longest first and passes them by value,
// kMaxAttnTiles per launch.
struct AttnRange {
    int q0, nq, g0, n_kv;
};
constexpr int kMaxAttnTiles = 128;
struct AttnTiles {
    AttnRange t[kMaxAttnTiles];   // nq <= tile height
    int n;
};

struct AttnArgs {
    const void* q;      // [*][Hq*dh]
    const int* qidx;    // row map into q (nullptr = identity)
    const int* q_pos;   // per output row
    const void* k;      // [*][Hkv*dh]
    const void* v;
    int kv_pos0;
    int n_q_heads, n_kv_heads, head_dim;
    void* out;          // [*][Hq*dh]
    // Split over keys (bf16 path): tiles whose visible keys exceed seg_keys
    // are cut into segments processed by separate workgroups; their
    // unnormalized partial outputs and (max, sum) go to part_o / part_ml and
    // a combine pass merges them.  Set by the launcher.
    int seg_keys;
    int max_seg;
    bf16* part_o;       // [tiles][Hq][max_seg][tile height][dh], normalized per segment
    float* part_ml;     // [tiles][Hq][max_seg][tile height][2]
    int* part_nk;       // [tiles] keys visible to each tile (written by its attention pass)
};

// Per-token attention deviation of requests whose every chunk row is
// recomputed (bf16).  Request i: its n chunk rows are query rows q_row0 ..
// (row j at position j, RoPE'd queries in q [*][Hq*dh]), their recomputed
// keys rows k_new_row0 .. of k_new and their cached (re-rotated) keys rows
// k_cached_row0 .. of k_cached ([*][Hkv*dh]); out[out0 + j] = sum over query
// heads and keys 0..j of the squared difference of the two softmax rows.
// part: workspace [Hq][part_stride] floats (query rows < part_stride).
struct AttnDevArgs {
    const void* q;
    const void* k_new;
    const void* k_cached;
    int n_q_heads, n_kv_heads, head_dim;
    float* part;
    int64_t part_stride;
};
struct AttnDevReq {
    int q_row0, n, k_new_row0, k_cached_row0, out0;
};
struct AttnDevTile {
    int q_row0, j0, nq, k_new_row0, k_cached_row0, n_keys;
};
struct AttnDevTiles {
    AttnDevTile t[kMaxAttnTiles];
    int n;
};
struct AttnDevSum {
    int row0, out0, n;
};
struct AttnDevSums {
    AttnDevSum r[kMaxReq];
    int n;
};
size_t attention_deviation_workspace(int n_q_heads, int64_t rows);
hipError_t launch_attention_deviation(int dtype, const AttnDevArgs& a, const AttnDevReq* r,
                                      int n_r, float* out, hipStream_t s);

// Workspace bytes the split partials of these ranges need (0: no split).
size_t attention_workspace(int dtype, const AttnRange* r, int n_r, int n_q_heads, int head_dim);

// Launches the attention of all ranges; `ws` holds at least
// attention_workspace(...) bytes.
hipError_t launch_attention(int dtype, const AttnArgs& a, const AttnRange* r, int n_r, void* ws,
                            size_t ws_bytes, hipStream_t s);

}  // namespace cb
