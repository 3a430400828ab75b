// KV deviation and HKVD (high KV deviation) selection.
//
// Deviation: CacheBlend explainer (0h-n0.github.io), section
// "KVキャッシュの定義と偏差メトリクス", eq. 1 (per-token L2 distance of the KV
// row), squared as in the section "HKVDトークン選定" selection code; it is
// measured between the recomputed row and the re-rotated cached row.
// Selection: the same section's code keeps the k rows of largest deviation
// and returns them in position order.  Ties are broken by position so the
// kept set is unique: order = (NaN first, larger value first, -0.0 == +0.0,
// smaller index first).
//
// The selection is exact integer work: every deviation maps to a 32-bit rank
// key (smaller = kept first); a 4-pass radix select over 8-bit digits finds
// the k-th smallest key T and how many rows equal to T are still needed; the
// kept rows are those below T plus the first `need` rows equal to T in
// index order; a block-wide scan writes them in ascending index order.
#include "kernels.h"

namespace cb {

namespace {

constexpr int kDevThreads = 256;
constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;

// a: a freshly computed row (likely still in L2); b: the cached row, read
// once with the non-temporal hint
template <typename T>
__device__ __forceinline__ float sq_diff8(const T* a, const T* b) {
    Frag<T> x = load_frag<T>(a);
    Frag<T> y = load_frag_nt<T>(b);
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float d = to_f32(x.v[i]) - to_f32(y.v[i]);
        s += d * d;
    }
    return s;
}

// One wave per row: lanes stride over the row in 8-element pieces.
// blockIdx.y = request of the table, blockIdx.x * 4 + wave = its chunk row.
template <typename T>
__global__ __launch_bounds__(kDevThreads) void deviation_kernel(
    const T* __restrict__ kn, const T* __restrict__ vn, const T* __restrict__ kc,
    const T* __restrict__ vc, const int* __restrict__ grow, const ReqTab t, int kv_dim,
    int mode, float* __restrict__ dev) {
    const ReqRows& q = t.r[blockIdx.y];
    const int lane = threadIdx.x & 63;
    const int i = blockIdx.x * (kDevThreads / 64) + (threadIdx.x >> 6);
    if (i >= q.n_c) return;
    const int r = q.r_off + i;
    const int64_t no = (int64_t)r * kv_dim;
    const int64_t co = (int64_t)(grow ? grow[r] : r) * kv_dim;
    float acc = 0.f;
    if (mode != 2)
        for (int c = lane * 8; c < kv_dim; c += 512) acc += sq_diff8(kn + no + c, kc + co + c);
    if (mode != 1)
        for (int c = lane * 8; c < kv_dim; c += 512) acc += sq_diff8(vn + no + c, vc + co + c);
    acc = warp_sum(acc);
    if (lane == 0) dev[q.c_off + i] = acc;
}

// One workgroup per row, for launches with few rows (a steady layer
// measures a few hundred): four waves split the row so that each thread has
// only a few independent 16-byte loads, all issued before any arithmetic,
// instead of one wave walking the whole row (latency-bound at ~145 rows).
// Partial sums are combined in a fixed order.
template <typename T>
__global__ __launch_bounds__(kDevThreads) void deviation_row_kernel(
    const T* __restrict__ kn, const T* __restrict__ vn, const T* __restrict__ kc,
    const T* __restrict__ vc, const int* __restrict__ grow, const ReqTab t, int kv_dim,
    int mode, float* __restrict__ dev) {
    __shared__ float part[kDevThreads / 64];
    const ReqRows& q = t.r[blockIdx.y];
    const int i = blockIdx.x;
    if (i >= q.n_c) return;                           // uniform over the workgroup
    const int r = q.r_off + i;
    const int64_t no = (int64_t)r * kv_dim;
    const int64_t co = (int64_t)(grow ? grow[r] : r) * kv_dim;
    float acc = 0.f;
    if (mode != 2)
        for (int c = threadIdx.x * 8; c < kv_dim; c += kDevThreads * 8)
            acc += sq_diff8(kn + no + c, kc + co + c);
    if (mode != 1)
        for (int c = threadIdx.x * 8; c < kv_dim; c += kDevThreads * 8)
            acc += sq_diff8(vn + no + c, vc + co + c);
    acc = warp_sum(acc);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        float sum = part[0];
#pragma unroll
        for (int w = 1; w < kDevThreads / 64; ++w) sum += part[w];
        dev[q.c_off + i] = sum;
    }
}

__global__ __launch_bounds__(kDevThreads) void given_scores_kernel(
    const float* __restrict__ scores, const ReqTab t, const int* __restrict__ pos_r,
    float* __restrict__ dev) {
    const ReqRows& q = t.r[blockIdx.y];
    const int i = blockIdx.x * kDevThreads + threadIdx.x;
    if (i < q.n_c) dev[q.c_off + i] = scores[q.out_col + pos_r[q.r_off + i]];
}

__device__ __forceinline__ uint32_t rank_key(float f) {
    if (f != f) return 0u;                      // NaN ranks above everything
    uint32_t b = __float_as_uint(f);
    if (f == 0.f) b = 0u;                       // -0.0 ranks with +0.0
    const uint32_t asc = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
    return ~asc;                                // larger value -> smaller key
}

// Exclusive scan of one int per thread over the block; returns the total too.
__device__ int block_exclusive_scan(int v, int* wsum, int& total) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    int inc = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(inc, o, 64);
        if (lane >= o) inc += t;
    }
    if (lane == 63) wsum[w] = inc;
    __syncthreads();
    if (threadIdx.x == 0) {
        int run = 0;
        for (int i = 0; i < kSelWaves; ++i) {
            const int t = wsum[i];
            wsum[i] = run;
            run += t;
        }
        wsum[kSelWaves] = run;
    }
    __syncthreads();
    const int ex = wsum[w] + inc - v;
    total = wsum[kSelWaves];
    __syncthreads();
    return ex;
}

// Marks the kept rows of dev[0..n) (k of them) and returns, per thread, the
// exclusive prefix of kept rows over its contiguous segment [beg, end).
struct SelState {
    uint32_t T;
    int need;
};

__device__ SelState radix_threshold(const float* __restrict__ dev, int n, int k,
                                    uint32_t* hist, int* bcast) {
    __shared__ int wtot[4];
    uint32_t prefix = 0, mask = 0;
    int kk = k;
    for (int shift = 24; shift >= 0; shift -= 8) {
        for (int i = threadIdx.x; i < 256; i += kSelThreads) hist[i] = 0;
        __syncthreads();
        for (int i = threadIdx.x; i < n; i += kSelThreads) {
            const uint32_t key = rank_key(dev[i]);
            if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
        }
        __syncthreads();
        // The digit is the first bin whose inclusive count reaches kk: a
        // scan over the 256 bins by the first four waves (one bin per lane).
        int h = 0, inc = 0;
        if (threadIdx.x < 256) {
            h = (int)hist[threadIdx.x];
            inc = h;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int t = __shfl_up(inc, o, 64);
                if ((threadIdx.x & 63) >= o) inc += t;
            }
            if ((threadIdx.x & 63) == 63) wtot[threadIdx.x >> 6] = inc;
        }
        __syncthreads();
        if (threadIdx.x < 256) {
            for (int w = 0; w < (int)(threadIdx.x >> 6); ++w) inc += wtot[w];
            const int exc = inc - h;
            if (exc < kk && inc >= kk) { bcast[0] = (int)threadIdx.x; bcast[1] = kk - exc; }
            if (threadIdx.x == 255 && inc < kk) { bcast[0] = 255; bcast[1] = kk - inc; }
        }
        __syncthreads();
        prefix |= (uint32_t)bcast[0] << shift;
        mask |= 0xFFu << shift;
        kk = bcast[1];
        __syncthreads();
    }
    return SelState{prefix, kk};
}

// Writes the kept indices (ascending) through `emit(slot, index)`.
template <typename Emit>
__device__ void select_rows(const float* __restrict__ dev, int n, int k, Emit emit) {
    __shared__ uint32_t hist[256];
    __shared__ int bcast[2];
    __shared__ int wsum[kSelWaves + 1];
    if (k <= 0) return;
    if (k >= n) {
        for (int i = threadIdx.x; i < n; i += kSelThreads) emit(i, i);
        return;
    }
    const SelState st = radix_threshold(dev, n, k, hist, bcast);
    const int per = (n + kSelThreads - 1) / kSelThreads;
    const int beg = min(n, (int)threadIdx.x * per), end = min(n, beg + per);
    int eq = 0;
    for (int i = beg; i < end; ++i) eq += rank_key(dev[i]) == st.T;
    int tot;
    int e = block_exclusive_scan(eq, wsum, tot);
    int cnt = 0;
    for (int i = beg; i < end; ++i) {
        const uint32_t key = rank_key(dev[i]);
        cnt += key < st.T || (key == st.T && e++ < st.need);
    }
    e -= eq;   // back to this segment's first equal-key rank
    int slot = block_exclusive_scan(cnt, wsum, tot);
    for (int i = beg; i < end; ++i) {
        const uint32_t key = rank_key(dev[i]);
        if (key < st.T || (key == st.T && e++ < st.need)) emit(slot++, i);
    }
}

__global__ __launch_bounds__(kSelThreads) void topk_kernel(const float* __restrict__ dev, int n,
                                                          int k, int* __restrict__ out) {
    select_rows(dev, n, k, [&](int slot, int i) { out[slot] = i; });
}

// One workgroup per request of the table.
__global__ __launch_bounds__(kSelThreads) void blend_select_kernel(
    const float* __restrict__ dev, const ReqTab t, const int* __restrict__ pos_r,
    const int* __restrict__ row_r, int* __restrict__ sel_local, int* __restrict__ pos_q,
    int* __restrict__ row_q, int* __restrict__ sel_pos, float* __restrict__ dev_out) {
    const ReqRows& q = t.r[blockIdx.x];
    const float* d = dev + q.c_off;
    select_rows(d, q.n_c, q.k, [&](int slot, int i) {
        const int r = q.r_off + i;
        const int p = pos_r[r];
        sel_local[q.q_off + slot] = r;
        pos_q[q.q_off + slot] = p;
        row_q[q.q_off + slot] = row_r[r];
        if (sel_pos) sel_pos[q.out_col + slot] = p;
    });
    for (int s = threadIdx.x; s < q.n_s; s += kSelThreads) {
        const int r = q.r_off + q.n_c + s;
        sel_local[q.q_off + q.k + s] = r;
        pos_q[q.q_off + q.k + s] = pos_r[r];
        row_q[q.q_off + q.k + s] = row_r[r];
    }
    if (dev_out)
        for (int i = threadIdx.x; i < q.n_c; i += kSelThreads)
            dev_out[q.out_col + pos_r[q.r_off + i]] = d[i];
}

}  // namespace

hipError_t launch_deviation(int dtype, const void* k_new, const void* v_new,
                            const void* k_cached, const void* v_cached, const int* grow,
                            const ReqTab& t, int kv_dim, int mode, float* dev, hipStream_t s) {
    if (t.n <= 0 || t.max_c <= 0) return hipSuccess;
    if (t.n > kMaxReq || kv_dim % 8 != 0) return hipErrorInvalidValue;
    for (int b = 0; b < t.n; ++b)
        if (t.r[b].n_c > t.max_c || t.r[b].n_c < 0) return hipErrorInvalidValue;
    // few rows: a workgroup per row; many rows: a wave per row
    if ((int64_t)t.max_c * t.n < 1024) {
        dim3 grid(t.max_c, t.n), block(kDevThreads);
        if (dtype == BF16)
            hipLaunchKernelGGL(deviation_row_kernel<bf16>, grid, block, 0, s, (const bf16*)k_new,
                               (const bf16*)v_new, (const bf16*)k_cached, (const bf16*)v_cached,
                               grow, t, kv_dim, mode, dev);
        else
            hipLaunchKernelGGL(deviation_row_kernel<float>, grid, block, 0, s, (const float*)k_new,
                               (const float*)v_new, (const float*)k_cached,
                               (const float*)v_cached, grow, t, kv_dim, mode, dev);
        return hipGetLastError();
    }
    const int per = kDevThreads / 64;
    dim3 grid((t.max_c + per - 1) / per, t.n), block(kDevThreads);
    if (dtype == BF16)
        hipLaunchKernelGGL(deviation_kernel<bf16>, grid, block, 0, s, (const bf16*)k_new,
                           (const bf16*)v_new, (const bf16*)k_cached, (const bf16*)v_cached, grow,
                           t, kv_dim, mode, dev);
    else
        hipLaunchKernelGGL(deviation_kernel<float>, grid, block, 0, s, (const float*)k_new,
                           (const float*)v_new, (const float*)k_cached,
                           (const float*)v_cached, grow, t, kv_dim, mode, dev);
    return hipGetLastError();
}

hipError_t launch_given_scores(const float* scores, const ReqTab& t, const int* pos_r,
                               float* dev, hipStream_t s) {
    if (t.n <= 0 || t.max_c <= 0) return hipSuccess;
    if (t.n > kMaxReq || !scores) return hipErrorInvalidValue;
    dim3 grid((t.max_c + kDevThreads - 1) / kDevThreads, t.n);
    hipLaunchKernelGGL(given_scores_kernel, grid, dim3(kDevThreads), 0, s, scores, t, pos_r, dev);
    return hipGetLastError();
}

hipError_t launch_topk(const float* dev, int n, int k, int* idx_out, hipStream_t s) {
    if (n <= 0 || k <= 0) return hipSuccess;
    hipLaunchKernelGGL(topk_kernel, dim3(1), dim3(kSelThreads), 0, s, dev, n, k, idx_out);
    return hipGetLastError();
}

hipError_t launch_select(const float* dev, const ReqTab& t, const int* pos_r, const int* row_r,
                         int* sel_local, int* pos_q, int* row_q, int* sel_pos, float* dev_out,
                         hipStream_t s) {
    if (t.n <= 0) return hipSuccess;
    if (t.n > kMaxReq) return hipErrorInvalidValue;
    for (int b = 0; b < t.n; ++b) {
        const ReqRows& q = t.r[b];
        if (q.k > q.n_c || q.k < 0 || q.n_s < 0) return hipErrorInvalidValue;
    }
    hipLaunchKernelGGL(blend_select_kernel, dim3(t.n), dim3(kSelThreads), 0, s, dev, t, pos_r,
                       row_r, sel_local, pos_q, row_q, sel_pos, dev_out);
    return hipGetLastError();
}

}  // namespace cb

