// Per-channel quantized chunk caches: encoding, and decoding fused with the
// RoPE re-alignment of the fetch.
//
// Format: CacheGen explainer (0h-n0.github.io), "技術的詳細", step 1
// "チャネル別量子化": for every channel c of a layer, over the chunk's tokens,
// zero point z_c = min x, scale s_c = (max x - z_c) / (2^b - 1), code =
// round((x - z_c) / s_c); the decoder restores code * s_c + z_c.  Rounding
// is half to even, codes are clamped to [0, 2^b - 1] and a channel whose
// tokens are all equal (s_c = 0) gets code 0.  The decision is taken in
// float32 with IEEE operations (correctly rounded division, no contraction),
// so a float32 reference reproduces every code.
//
// All kernels are bound by HBM: encoding reads x twice (once for the
// per-channel range, once to encode) and writes b/8 bytes per element;
// decoding reads b/8 bytes and writes the model dtype.
#include <algorithm>

#include "kernels.h"

namespace cb {

namespace {

constexpr int kThreads = 256;
constexpr int kQuantWaves = 4;
constexpr int kChanPerBlock = 64 * 8;   // one wave covers 512 channels, 8 per lane
constexpr int kTokPerThread = 8;        // decode: tokens per thread (params loaded once)

template <int BITS>
__device__ __forceinline__ void store_codes(uint8_t* p, const float* q) {
    if constexpr (BITS == 8) {
        u32x2 w;
        w[0] = (uint32_t)q[0] | ((uint32_t)q[1] << 8) | ((uint32_t)q[2] << 16) | ((uint32_t)q[3] << 24);
        w[1] = (uint32_t)q[4] | ((uint32_t)q[5] << 8) | ((uint32_t)q[6] << 16) | ((uint32_t)q[7] << 24);
        *reinterpret_cast<u32x2*>(p) = w;
    } else {
        uint32_t w = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) w |= (uint32_t)q[i] << (4 * i);
        *reinterpret_cast<uint32_t*>(p) = w;
    }
}

template <int BITS>
__device__ __forceinline__ void load_codes(const uint8_t* p, float* x) {
    if constexpr (BITS == 8) {
        const u32x2 w = *reinterpret_cast<const u32x2*>(p);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[i] = (float)((w[0] >> (8 * i)) & 255u);
            x[4 + i] = (float)((w[1] >> (8 * i)) & 255u);
        }
    } else {
        const uint32_t w = *reinterpret_cast<const uint32_t*>(p);
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = (float)((w >> (4 * i)) & 15u);
    }
}

// Encoding runs in two launches over a grid (ceil(row / 512), n_layers,
// splits): each workgroup owns 512 channels (8 per lane) of one layer and a
// contiguous slice of the tokens, its 4 waves taking every 4th token.
// minmax_kernel writes the slice's per-channel minima and maxima; codes_kernel
// combines the partials of all slices (min / max are exact in any order),
// derives scale and zero, and encodes its slice.
template <typename T>
__global__ __launch_bounds__(kThreads) void minmax_kernel(
    const T* __restrict__ x, int n_tokens, int row, int64_t x_ls, int tok_per_split,
    float* __restrict__ part) {
    __shared__ float red_lo[kQuantWaves][kChanPerBlock], red_hi[kQuantWaves][kChanPerBlock];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, l = blockIdx.y, sp = blockIdx.z;
    const int c = blockIdx.x * kChanPerBlock + lane * 8;
    const bool live = c < row;
    const T* xl = x + (int64_t)l * x_ls;
    const int t0 = sp * tok_per_split, t1 = min(n_tokens, t0 + tok_per_split);
    float lo[8], hi[8], v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) { lo[i] = INFINITY; hi[i] = -INFINITY; }
    if (live)
        for (int t = t0 + w; t < t1; t += kQuantWaves) {
            Vec8<T>::load(xl + (int64_t)t * row + c, v);
#pragma unroll
            for (int i = 0; i < 8; ++i) { lo[i] = fminf(lo[i], v[i]); hi[i] = fmaxf(hi[i], v[i]); }
        }
#pragma unroll
    for (int i = 0; i < 8; ++i) { red_lo[w][lane * 8 + i] = lo[i]; red_hi[w][lane * 8 + i] = hi[i]; }
    __syncthreads();
    if (w != 0 || !live) return;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int u = 1; u < kQuantWaves; ++u) {
            lo[i] = fminf(lo[i], red_lo[u][lane * 8 + i]);
            hi[i] = fmaxf(hi[i], red_hi[u][lane * 8 + i]);
        }
    // partials: [layer][split][2][row]
    float* p = part + ((int64_t)l * gridDim.z + sp) * 2 * row + c;
    Vec8<float>::store(p, lo);
    Vec8<float>::store(p + row, hi);
}

template <typename T, int BITS>
__global__ __launch_bounds__(kThreads) void codes_kernel(
    const T* __restrict__ x, int n_tokens, int row, int64_t x_ls, int tok_per_split,
    const float* __restrict__ part, uint8_t* __restrict__ codes, float* __restrict__ scale,
    float* __restrict__ zero, int64_t ps) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, l = blockIdx.y, sp = blockIdx.z;
    const int c = blockIdx.x * kChanPerBlock + lane * 8;
    if (c >= row) return;
    float lo[8], hi[8], v[8], s[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) { lo[i] = INFINITY; hi[i] = -INFINITY; }
    const float* p = part + (int64_t)l * gridDim.z * 2 * row + c;
    for (int u = 0; u < (int)gridDim.z; ++u) {
        Vec8<float>::load(p + (int64_t)u * 2 * row, v);
#pragma unroll
        for (int i = 0; i < 8; ++i) lo[i] = fminf(lo[i], v[i]);
        Vec8<float>::load(p + (int64_t)u * 2 * row + row, v);
#pragma unroll
        for (int i = 0; i < 8; ++i) hi[i] = fmaxf(hi[i], v[i]);
    }
    const float levels = (float)((1 << BITS) - 1);
#pragma unroll
    for (int i = 0; i < 8; ++i) s[i] = __fsub_rn(hi[i], lo[i]) / levels;
    if (sp == 0 && w == 0) {
        Vec8<float>::store(scale + (int64_t)l * ps + c, s);
        Vec8<float>::store(zero + (int64_t)l * ps + c, lo);
    }
    const T* xl = x + (int64_t)l * x_ls;
    uint8_t* cl = codes + (int64_t)l * n_tokens * row * BITS / 8;
    const int t0 = sp * tok_per_split, t1 = min(n_tokens, t0 + tok_per_split);
    for (int t = t0 + w; t < t1; t += kQuantWaves) {
        Vec8<T>::load(xl + (int64_t)t * row + c, v);
        float q[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            q[i] = s[i] > 0.f ? fminf(fmaxf(rintf(__fsub_rn(v[i], lo[i]) / s[i]), 0.f), levels) : 0.f;
        store_codes<BITS>(cl + ((int64_t)t * row + c) * BITS / 8, q);
    }
}

// One thread decodes channels c .. c+7 of up to 8 consecutive tokens of one
// job (scale, zero and rotation factors loaded once); consecutive threads
// take consecutive 8-channel pieces of a row.
template <typename T, int BITS>
__global__ __launch_bounds__(kThreads) void dequant_rerotate_kernel(
    const QRotJobs jobs, int layer, T* __restrict__ kd, T* __restrict__ vd, int row,
    int head_dim, const float2* __restrict__ tab, int half) {
    const QRotJob& j = jobs.j[blockIdx.y];
    const int vecs = row >> 3;
    const int groups = (j.n_tokens + kTokPerThread - 1) / kTokPerThread;
    const int64_t u = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (u >= (int64_t)groups * vecs) return;
    const int g = (int)(u / vecs);
    const int c = (int)(u - (int64_t)g * vecs) * 8;
    const int t0 = g * kTokPerThread, t1 = min(j.n_tokens, t0 + kTokPerThread);
    const float* qp = j.qp + (int64_t)layer * j.qp_layer_stride;
    float ks[8], kz[8];
    Vec8<float>::load(qp + c, ks);
    Vec8<float>::load(qp + row + c, kz);
    const int ad = j.delta < 0 ? -j.delta : j.delta;
    const float sg = j.delta < 0 ? -1.f : 1.f;
    const float2* tr = tab + (int64_t)ad * half + ((c % head_dim) >> 1);
    float2 cs[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) cs[p] = float2{tr[p].x, sg * tr[p].y};
    const int64_t cl = (int64_t)layer * j.code_layer_stride;
    for (int t = t0; t < t1; ++t) {
        const int64_t co = cl + ((int64_t)t * row + c) * BITS / 8;
        const int64_t d_off = (int64_t)(j.dst_row + t) * row + c;
        float x[8], y[8];
        load_codes<BITS>(j.k + co, x);
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = fmaf(x[i], ks[i], kz[i]);
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            y[2 * p] = x[2 * p] * cs[p].x - x[2 * p + 1] * cs[p].y;
            y[2 * p + 1] = x[2 * p] * cs[p].y + x[2 * p + 1] * cs[p].x;
        }
        Vec8<T>::store(kd + d_off, y);
    }
    if (!j.v) return;
    float vs[8], vz[8];
    Vec8<float>::load(qp + 2 * row + c, vs);
    Vec8<float>::load(qp + 3 * row + c, vz);
    for (int t = t0; t < t1; ++t) {
        const int64_t co = cl + ((int64_t)t * row + c) * BITS / 8;
        float x[8];
        load_codes<BITS>(j.v + co, x);
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = fmaf(x[i], vs[i], vz[i]);
        Vec8<T>::store(vd + (int64_t)(j.dst_row + t) * row + c, x);
    }
}

constexpr int kTokPerSplit = 64;
constexpr int kMaxSplits = 256;

int quant_splits(int n_tokens) {
    return std::min(kMaxSplits, (n_tokens + kTokPerSplit - 1) / kTokPerSplit);
}

template <int BITS>
hipError_t launch_quantize_bits(int dtype, const void* x, int n_layers, int n_tokens, int row,
                                int64_t x_ls, void* codes, float* scale, float* zero, int64_t ps,
                                float* part, hipStream_t s) {
    const int splits = quant_splits(n_tokens);
    const int per = (n_tokens + splits - 1) / splits;
    dim3 grid((row + kChanPerBlock - 1) / kChanPerBlock, n_layers, splits);
    if (dtype == BF16) {
        hipLaunchKernelGGL(minmax_kernel<bf16>, grid, dim3(kThreads), 0, s, (const bf16*)x,
                           n_tokens, row, x_ls, per, part);
        hipLaunchKernelGGL((codes_kernel<bf16, BITS>), grid, dim3(kThreads), 0, s,
                           (const bf16*)x, n_tokens, row, x_ls, per, (const float*)part,
                           (uint8_t*)codes, scale, zero, ps);
    } else {
        hipLaunchKernelGGL(minmax_kernel<float>, grid, dim3(kThreads), 0, s, (const float*)x,
                           n_tokens, row, x_ls, per, part);
        hipLaunchKernelGGL((codes_kernel<float, BITS>), grid, dim3(kThreads), 0, s,
                           (const float*)x, n_tokens, row, x_ls, per, (const float*)part,
                           (uint8_t*)codes, scale, zero, ps);
    }
    return hipGetLastError();
}

template <int BITS>
hipError_t launch_dequant_bits(int dtype, const QRotJobs& jobs, int layer, void* k_dst,
                               void* v_dst, int row, int head_dim, const RopeTab& rope,
                               hipStream_t s) {
    const int64_t groups = (jobs.max_tokens + kTokPerThread - 1) / kTokPerThread;
    const int64_t units = groups * (row / 8);
    dim3 grid((unsigned)((units + kThreads - 1) / kThreads), (unsigned)jobs.n);
    if (dtype == BF16)
        hipLaunchKernelGGL((dequant_rerotate_kernel<bf16, BITS>), grid, dim3(kThreads), 0, s, jobs,
                           layer, (bf16*)k_dst, (bf16*)v_dst, row, head_dim, rope.tab, rope.half);
    else
        hipLaunchKernelGGL((dequant_rerotate_kernel<float, BITS>), grid, dim3(kThreads), 0, s,
                           jobs, layer, (float*)k_dst, (float*)v_dst, row, head_dim, rope.tab,
                           rope.half);
    return hipGetLastError();
}

}  // namespace

size_t quantize_workspace(int n_layers, int n_tokens, int row) {
    if (n_layers <= 0 || n_tokens <= 0 || row <= 0) return 0;
    return (size_t)n_layers * quant_splits(n_tokens) * 2 * row * sizeof(float);
}

hipError_t launch_quantize(int dtype, const void* x, int n_layers, int n_tokens, int row,
                           int64_t x_layer_stride, int bits, void* codes, float* scale,
                           float* zero, int64_t param_stride, void* ws, size_t ws_bytes,
                           hipStream_t s) {
    if (n_layers <= 0 || n_tokens <= 0) return hipSuccess;
    if (row <= 0 || row % 8 || param_stride < row || x_layer_stride < (int64_t)n_tokens * row ||
        !ws || ws_bytes < quantize_workspace(n_layers, n_tokens, row))
        return hipErrorInvalidValue;
    if (bits == 8)
        return launch_quantize_bits<8>(dtype, x, n_layers, n_tokens, row, x_layer_stride, codes,
                                       scale, zero, param_stride, (float*)ws, s);
    if (bits == 4)
        return launch_quantize_bits<4>(dtype, x, n_layers, n_tokens, row, x_layer_stride, codes,
                                       scale, zero, param_stride, (float*)ws, s);
    return hipErrorInvalidValue;
}

hipError_t launch_dequant_rerotate(int dtype, int bits, const QRotJobs& jobs, int layer,
                                   void* k_dst, void* v_dst, int n_heads, int head_dim,
                                   const RopeTab& rope, hipStream_t s) {
    if (jobs.n <= 0 || jobs.max_tokens <= 0) return hipSuccess;
    if (jobs.n > kMaxQRotJobs) return hipErrorInvalidValue;
    const int row = n_heads * head_dim;
    if (head_dim % 8 != 0 || rope.half != head_dim / 2) return hipErrorInvalidValue;
    for (int i = 0; i < jobs.n; ++i) {
        const QRotJob& j = jobs.j[i];
        const int ad = j.delta < 0 ? -j.delta : j.delta;
        if (ad >= rope.n_pos || j.n_tokens > jobs.max_tokens || j.n_tokens < 0 || !j.k || !j.qp ||
            j.staged)
            return hipErrorInvalidValue;
    }
    if (bits == 8) return launch_dequant_bits<8>(dtype, jobs, layer, k_dst, v_dst, row, head_dim, rope, s);
    if (bits == 4) return launch_dequant_bits<4>(dtype, jobs, layer, k_dst, v_dst, row, head_dim, rope, s);
    return hipErrorInvalidValue;
}

}  // namespace cb
