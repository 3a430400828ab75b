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

// Jobs travel by value in the kernel arguments (one launch per 16 chunks).
constexpr int kMaxRotJobs = 16;
struct RotJobs {
    RotJob j[kMaxRotJobs];
    int n;
    int max_tokens;
};

// For every job j and token t < n_tokens: K row (dst_row + t) of k_dst =
// R(delta) * K row t of the job's layer-`layer` source; V copied likewise.
hipError_t launch_rerotate(int dtype, const RotJobs& jobs, int layer, void* k_dst, void* v_dst,
                           int n_heads, int head_dim, const RopeTab& rope, hipStream_t s);

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
// fused row pos[src_idx[r]] (src_idx nullptr: identity; pos nullptr: the
// source row index) minus row_base receives k_new/v_new row src_idx[r].
hipError_t launch_scatter_kv(int dtype, const void* k_new, const void* v_new,
                             const int* src_idx, const int* pos, int row_base,
                             void* fk, void* fv, int n_rows, int kv_dim, hipStream_t s);

// ------------------------------------------------------------------ selection
// dev[r] = deviation of new row r against cached row crow(r) (crow = pos[r]
// - row_base, or r when pos is null); when dev_pos_out is not null also
// dev_pos_out[pos[r]] = dev[r].
hipError_t launch_deviation(int dtype, const void* k_new, const void* v_new,
                            const void* k_cached, const void* v_cached, const int* pos,
                            int row_base, int n_rows, int kv_dim, int mode, float* dev,
                            float* dev_pos_out, hipStream_t s);

// Kernel-level top-k: idx_out[0..k) = kept indices, ascending.
hipError_t launch_topk(const float* dev, int n, int k, int* idx_out, hipStream_t s);

// Blend bookkeeping for one layer.  R rows = n_c chunk rows then n_s suffix
// rows, positions pos_r.  Keeps the k chunk rows with largest dev (all when
// k == n_c), then writes sel_local[0..k+n_s) = kept R-row indices followed by
// the suffix rows, pos_q = their positions, sel_pos (optional) = kept chunk
// positions.
hipError_t launch_select(const float* dev, int n_c, int k, int n_s, const int* pos_r,
                         int* sel_local, int* pos_q, int* sel_pos, hipStream_t s);

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
};
hipError_t launch_gemm(int dtype, int epi, const GemmArgs& g, hipStream_t s);

// ------------------------------------------------------------------ attention
// out[i] = causal attention of q row qidx[i] (qidx null: i) at position
// q_pos[i] over keys/values rows 0..n_kv-1 at positions kv_pos0 + j.
struct AttnArgs {
    const void* q;      // [*][Hq*dh]
    const int* qidx;    // row map into q (nullptr = identity)
    const int* q_pos;   // [n_q]
    int n_q;
    const void* k;      // [n_kv][Hkv*dh]
    const void* v;
    int n_kv;
    int kv_pos0;
    int n_q_heads, n_kv_heads, head_dim;
    void* out;          // [n_q][Hq*dh]
    // Split over keys (bf16 path): query tiles whose visible keys exceed
    // seg_keys are cut into segments processed by separate workgroups; their
    // unnormalized partial outputs and (max, sum) go to part_o / part_ml and a
    // combine pass merges them.  seg_keys = 0 disables splitting.
    int seg_keys;
    int max_seg;
    float* part_o;      // [tiles][Hq][max_seg][64][dh]
    float* part_ml;     // [tiles][Hq][max_seg][64][2]
};
hipError_t launch_attention(int dtype, const AttnArgs& a, hipStream_t s);

// Split plan for n_q queries over n_kv keys: fills seg_keys / max_seg and
// returns the workspace bytes the partials need (0 when not split).
size_t attention_split_plan(int dtype, int n_q, int n_kv, int n_q_heads, int head_dim,
                            int* seg_keys, int* max_seg);

}  // namespace cb
