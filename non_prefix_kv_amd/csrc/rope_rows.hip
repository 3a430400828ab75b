// Bandwidth-bound kernels: RoPE re-alignment of cached keys, row gather /
// scatter, K/V merge into the fused cache, RMSNorm.
//
// RoPE re-alignment follows the Prompt Cache explainer (0h-n0.github.io),
// section "RoPEにおける位置調整": a key encoded at chunk-local position p'
// is moved to its real position p = p' + delta by the pair rotation
// R(delta * theta_i); the CacheBlend explainer's RoPE section fixes R and
// theta_i.  Values are not rotated.
#include <algorithm>

#include "kernels.h"

namespace cb {

namespace {

constexpr int kThreads = 256;

// One thread moves 8 consecutive elements of one K row (4 rotation pairs)
// and the matching 8 elements of the V row.  Consecutive threads cover
// consecutive 16/32-byte pieces of a row, so every wave reads and writes
// whole contiguous segments.
template <typename T>
__global__ __launch_bounds__(kThreads) void rerotate_kernel(
    const RotJobs jobs, int layer, T* __restrict__ kd, T* __restrict__ vd,
    int row_elems, int head_dim, const float2* __restrict__ tab, int half) {
    const RotJob& j = jobs.j[blockIdx.y];
    const int vecs = row_elems >> 3;
    const int64_t u = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (u >= (int64_t)j.n_tokens * vecs) return;
    const int t = (int)(u / vecs);
    const int c = (int)(u - (int64_t)t * vecs) * 8;
    const int64_t d_off = (int64_t)(j.dst_row + t) * row_elems + c;
    const int64_t s_off = (int64_t)layer * j.src_layer_stride + (int64_t)t * row_elems + c;
    const T* ks = j.k_src ? static_cast<const T*>(j.k_src) + s_off : kd + d_off;

    float x[8];
    if (j.k_src) {          // a chunk cache row: read once, not again soon
        const Frag<T> f = load_frag_nt<T>(ks);
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = to_f32(f.v[i]);
    } else {
        Vec8<T>::load(ks, x);
    }
    const int ad = j.delta < 0 ? -j.delta : j.delta;
    const float sg = j.delta < 0 ? -1.f : 1.f;
    const float2* tr = tab + (int64_t)ad * half + ((c % head_dim) >> 1);
    float y[8];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const float2 cs = tr[p];
        const float sn = sg * cs.y;
        y[2 * p] = x[2 * p] * cs.x - x[2 * p + 1] * sn;
        y[2 * p + 1] = x[2 * p] * sn + x[2 * p + 1] * cs.x;
    }
    // the fused rows are read again only by later layers' kernels: written
    // with the non-temporal hint, like the chunk rows are read
    Vec8<T>::store_nt(kd + d_off, y);
    if (j.v_src) {
        const u32x4* vs = reinterpret_cast<const u32x4*>(static_cast<const T*>(j.v_src) + s_off);
        u32x4* vo = reinterpret_cast<u32x4*>(vd + d_off);
#pragma unroll
        for (int w = 0; w < (int)sizeof(T) / 2; ++w)
            __builtin_nontemporal_store(__builtin_nontemporal_load(vs + w), vo + w);
    }
}

__global__ __launch_bounds__(kThreads) void move_rows_kernel(
    const char* __restrict__ src, char* __restrict__ dst, const int* __restrict__ idx,
    int64_t row_bytes, int scatter) {
    const int r = blockIdx.x;
    const int64_t srow = scatter ? r : idx[r];
    const int64_t drow = scatter ? idx[r] : r;
    const char* s = src + srow * row_bytes;
    char* d = dst + drow * row_bytes;
    if ((row_bytes & 15) == 0) {
        for (int64_t o = (int64_t)threadIdx.x * 16; o < row_bytes; o += kThreads * 16)
            *reinterpret_cast<u32x4*>(d + o) = *reinterpret_cast<const u32x4*>(s + o);
    } else {
        for (int64_t o = (int64_t)threadIdx.x * 4; o < row_bytes; o += kThreads * 4)
            *reinterpret_cast<uint32_t*>(d + o) = *reinterpret_cast<const uint32_t*>(s + o);
    }
}

template <typename T>
__global__ __launch_bounds__(kThreads) void scatter_kv_kernel(
    const T* __restrict__ kn, const T* __restrict__ vn, const int* __restrict__ sidx,
    const int* __restrict__ drow, T* __restrict__ fk, T* __restrict__ fv, int kv_dim) {
    const int r = blockIdx.x;
    const int s = sidx ? sidx[r] : r;
    const int64_t d = (int64_t)(drow ? drow[r] : r) * kv_dim;
    const int64_t so = (int64_t)s * kv_dim;
    for (int c = threadIdx.x * 8; c < kv_dim; c += kThreads * 8) {
        Vec8<T>::copy(kn + so + c, fk + d + c);
        Vec8<T>::copy(vn + so + c, fv + d + c);
    }
}

__device__ __forceinline__ float block_sum(float v, float* red) {
    v = warp_sum(v);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    float t = 0.f;
#pragma unroll
    for (int i = 0; i < kThreads / 64; ++i) t += red[i];
    return t;
}

template <typename TX, typename TY>
__global__ __launch_bounds__(kThreads) void rmsnorm_kernel(
    const TX* __restrict__ x, const int* __restrict__ idx, const TY* __restrict__ g,
    TY* __restrict__ y, float* __restrict__ xc, int d, float eps) {
    __shared__ float red[kThreads / 64];
    const int r = blockIdx.x;
    const TX* xr = x + (int64_t)(idx ? idx[r] : r) * d;
    float ss = 0.f;
    for (int c = threadIdx.x; c < d; c += kThreads) {
        const float v = to_f32(xr[c]);
        ss += v * v;
    }
    ss = block_sum(ss, red);
    const float inv = 1.0f / sqrtf(ss / (float)d + eps);
    TY* yr = y + (int64_t)r * d;
    float* xcr = xc ? xc + (int64_t)r * d : nullptr;
    for (int c = threadIdx.x; c < d; c += kThreads) {
        const float v = to_f32(xr[c]);
        yr[c] = from_f32<TY>(v * inv * to_f32(g[c]));
        if (xcr) xcr[c] = v;
    }
}

// Row held in registers (8 consecutive elements per thread and step, up to
// 4 steps = 8192 elements): one read of x, one write of y.
template <typename TX, typename TY>
__global__ __launch_bounds__(kThreads) void rmsnorm_vec_kernel(
    const TX* __restrict__ x, const int* __restrict__ idx, const TY* __restrict__ g,
    TY* __restrict__ y, float* __restrict__ xc, int d, float eps) {
    constexpr int MAXV = 4;
    __shared__ float red[kThreads / 64];
    const int r = blockIdx.x;
    const TX* xr = x + (int64_t)(idx ? idx[r] : r) * d;
    float v[MAXV][8], gv[MAXV][8];
    float ss = 0.f;
    // the gains are loaded with the row, before the block-wide sum, so that
    // the sum's barrier is the only wait between the loads and the stores
#pragma unroll
    for (int k = 0; k < MAXV; ++k) {
        const int c = (k * kThreads + threadIdx.x) * 8;
        if (c < d) {
            Vec8<TX>::load(xr + c, v[k]);
            Vec8<TY>::load(g + c, gv[k]);
#pragma unroll
            for (int i = 0; i < 8; ++i) ss += v[k][i] * v[k][i];
        }
    }
    ss = block_sum(ss, red);
    const float inv = 1.0f / sqrtf(ss / (float)d + eps);
    TY* yr = y + (int64_t)r * d;
    float* xcr = xc ? xc + (int64_t)r * d : nullptr;
#pragma unroll
    for (int k = 0; k < MAXV; ++k) {
        const int c = (k * kThreads + threadIdx.x) * 8;
        if (c < d) {
            float o[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) o[i] = v[k][i] * inv * gv[k][i];
            Vec8<TY>::store(yr + c, o);
            if (xcr) Vec8<float>::store(xcr + c, v[k]);
        }
    }
}

__global__ void iota_kernel(int* p, int n, int base) {
    const int i = blockIdx.x * kThreads + threadIdx.x;
    if (i < n) p[i] = base + i;
}

// blockIdx.y = request of the table.
__global__ __launch_bounds__(kThreads) void init_rows_kernel(const RowInitTab t, int* pos,
                                                            int* rows) {
    const RowInit& q = t.r[blockIdx.y];
    for (int i = blockIdx.x * kThreads + threadIdx.x; i < q.count; i += gridDim.x * kThreads) {
        pos[q.r_off + i] = q.lp0 + i;
        rows[q.r_off + i] = q.g0 + i;
    }
}

__global__ __launch_bounds__(kThreads) void fill_kernel(float* p, int64_t n, float v) {
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * kThreads)
        p[i] = v;
}

// Row copies inside one int array of rows of row_len entries.
__global__ __launch_bounds__(kThreads) void copy_int_rows_kernel(int* __restrict__ base,
                                                                  int64_t row_len,
                                                                  const IntRowCopies t) {
    const RowCopy c = t.c[blockIdx.y];
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i < row_len) base[c.dst * row_len + i] = base[c.src * row_len + i];
}

}  // namespace

hipError_t launch_rerotate(int dtype, const RotJobs& jobs, int layer, void* k_dst, void* v_dst,
                           int n_heads, int head_dim, const RopeTab& rope, hipStream_t s) {
    if (jobs.n <= 0 || jobs.max_tokens <= 0) return hipSuccess;
    if (jobs.n > kMaxRotJobs) return hipErrorInvalidValue;
    const int row = n_heads * head_dim;
    if (head_dim % 8 != 0 || rope.half != head_dim / 2) return hipErrorInvalidValue;
    for (int i = 0; i < jobs.n; ++i) {
        const int ad = jobs.j[i].delta < 0 ? -jobs.j[i].delta : jobs.j[i].delta;
        if (ad >= rope.n_pos || jobs.j[i].n_tokens > jobs.max_tokens) return hipErrorInvalidValue;
    }
    const int64_t units = (int64_t)jobs.max_tokens * (row / 8);
    dim3 grid((unsigned)((units + kThreads - 1) / kThreads), (unsigned)jobs.n);
    if (dtype == BF16)
        hipLaunchKernelGGL(rerotate_kernel<bf16>, grid, dim3(kThreads), 0, s, jobs, layer,
                           (bf16*)k_dst, (bf16*)v_dst, row, head_dim, rope.tab, rope.half);
    else
        hipLaunchKernelGGL(rerotate_kernel<float>, grid, dim3(kThreads), 0, s, jobs, layer,
                           (float*)k_dst, (float*)v_dst, row, head_dim, rope.tab, rope.half);
    return hipGetLastError();
}

hipError_t launch_iota(int* p, int n, int base, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(iota_kernel, dim3((n + kThreads - 1) / kThreads), dim3(kThreads), 0, s, p, n,
                       base);
    return hipGetLastError();
}

hipError_t launch_init_rows(const RowInitTab& t, int* pos, int* rows, hipStream_t s) {
    if (t.n <= 0) return hipSuccess;
    if (t.n > kMaxReq) return hipErrorInvalidValue;
    int mx = 0;
    for (int b = 0; b < t.n; ++b) {
        if (t.r[b].count < 0) return hipErrorInvalidValue;
        mx = std::max(mx, t.r[b].count);
    }
    if (mx == 0) return hipSuccess;
    const int gx = std::min((mx + kThreads - 1) / kThreads, 1024);
    hipLaunchKernelGGL(init_rows_kernel, dim3(gx, t.n), dim3(kThreads), 0, s, t, pos, rows);
    return hipGetLastError();
}

hipError_t launch_fill(float* p, int64_t n, float v, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    const int64_t gx = std::min<int64_t>((n + kThreads - 1) / kThreads, 4096);
    hipLaunchKernelGGL(fill_kernel, dim3((unsigned)gx), dim3(kThreads), 0, s, p, n, v);
    return hipGetLastError();
}

hipError_t launch_gather_rows(const void* src, void* dst, const int* idx, int n_rows,
                              int64_t row_bytes, hipStream_t s) {
    if (n_rows <= 0) return hipSuccess;
    hipLaunchKernelGGL(move_rows_kernel, dim3(n_rows), dim3(kThreads), 0, s, (const char*)src,
                       (char*)dst, idx, row_bytes, 0);
    return hipGetLastError();
}

hipError_t launch_scatter_rows(const void* src, void* dst, const int* idx, int n_rows,
                               int64_t row_bytes, hipStream_t s) {
    if (n_rows <= 0) return hipSuccess;
    hipLaunchKernelGGL(move_rows_kernel, dim3(n_rows), dim3(kThreads), 0, s, (const char*)src,
                       (char*)dst, idx, row_bytes, 1);
    return hipGetLastError();
}

hipError_t launch_scatter_kv(int dtype, const void* k_new, const void* v_new,
                             const int* src_idx, const int* dst_row, void* fk, void* fv,
                             int n_rows, int kv_dim, hipStream_t s) {
    if (n_rows <= 0) return hipSuccess;
    if (kv_dim % 8 != 0) return hipErrorInvalidValue;
    if (dtype == BF16)
        hipLaunchKernelGGL(scatter_kv_kernel<bf16>, dim3(n_rows), dim3(kThreads), 0, s,
                           (const bf16*)k_new, (const bf16*)v_new, src_idx, dst_row, (bf16*)fk,
                           (bf16*)fv, kv_dim);
    else
        hipLaunchKernelGGL(scatter_kv_kernel<float>, dim3(n_rows), dim3(kThreads), 0, s,
                           (const float*)k_new, (const float*)v_new, src_idx, dst_row,
                           (float*)fk, (float*)fv, kv_dim);
    return hipGetLastError();
}

hipError_t launch_rmsnorm(int x_dtype, const void* x, const int* idx, int y_dtype,
                          const void* g, void* y, float* x_copy, int rows, int d, float eps,
                          hipStream_t s) {
    if (rows <= 0) return hipSuccess;
    dim3 grid(rows), block(kThreads);
    const bool vec = d % 8 == 0 && d <= 4 * kThreads * 8 && ((uintptr_t)x % 16) == 0 &&
                     ((uintptr_t)g % 16) == 0 && ((uintptr_t)y % 16) == 0 &&
                     ((uintptr_t)x_copy % 16) == 0;
    if (vec) {
        if (x_dtype == F32 && y_dtype == F32)
            hipLaunchKernelGGL((rmsnorm_vec_kernel<float, float>), grid, block, 0, s,
                               (const float*)x, idx, (const float*)g, (float*)y, x_copy, d, eps);
        else if (x_dtype == F32 && y_dtype == BF16)
            hipLaunchKernelGGL((rmsnorm_vec_kernel<float, bf16>), grid, block, 0, s,
                               (const float*)x, idx, (const bf16*)g, (bf16*)y, x_copy, d, eps);
        else if (x_dtype == BF16 && y_dtype == BF16)
            hipLaunchKernelGGL((rmsnorm_vec_kernel<bf16, bf16>), grid, block, 0, s,
                               (const bf16*)x, idx, (const bf16*)g, (bf16*)y, x_copy, d, eps);
        else
            hipLaunchKernelGGL((rmsnorm_vec_kernel<bf16, float>), grid, block, 0, s,
                               (const bf16*)x, idx, (const float*)g, (float*)y, x_copy, d, eps);
        return hipGetLastError();
    }
    if (x_dtype == F32 && y_dtype == F32)
        hipLaunchKernelGGL((rmsnorm_kernel<float, float>), grid, block, 0, s, (const float*)x,
                           idx, (const float*)g, (float*)y, x_copy, d, eps);
    else if (x_dtype == F32 && y_dtype == BF16)
        hipLaunchKernelGGL((rmsnorm_kernel<float, bf16>), grid, block, 0, s, (const float*)x,
                           idx, (const bf16*)g, (bf16*)y, x_copy, d, eps);
    else if (x_dtype == BF16 && y_dtype == BF16)
        hipLaunchKernelGGL((rmsnorm_kernel<bf16, bf16>), grid, block, 0, s, (const bf16*)x,
                           idx, (const bf16*)g, (bf16*)y, x_copy, d, eps);
    else
        hipLaunchKernelGGL((rmsnorm_kernel<bf16, float>), grid, block, 0, s, (const bf16*)x,
                           idx, (const float*)g, (float*)y, x_copy, d, eps);
    return hipGetLastError();
}

hipError_t launch_copy_int_rows(int* base, int64_t row_len, const IntRowCopies& t,
                                hipStream_t s) {
    if (t.n <= 0 || row_len <= 0) return hipSuccess;
    if (t.n > kMaxRowCopies) return hipErrorInvalidValue;
    for (int i = 0; i < t.n; ++i)
        if (t.c[i].dst < 0 || t.c[i].src < 0 || t.c[i].dst == t.c[i].src)
            return hipErrorInvalidValue;
    dim3 grid((unsigned)((row_len + kThreads - 1) / kThreads), t.n);
    hipLaunchKernelGGL(copy_int_rows_kernel, grid, dim3(kThreads), 0, s, base, row_len, t);
    return hipGetLastError();
}

}  // namespace cb
