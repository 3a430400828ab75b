// First token and one decode step on a fused cache: matrix-vector products
// for one row, a split-key attention of one query over the fused keys, and
// an argmax over the vocabulary.
//
// The decode step is what the fused cache is for: the CacheBlend explainer
// (abeam.tech), section "用語解説", describes the KV cache as what lets
// generation avoid recomputing past tokens, and TTFT as the time until the
// first output token, which the prefill (here the fusion) dominates.
//
// Everything here reads each weight (or cached key / value) once per step,
// so it is bound by HBM bandwidth: every wave streams whole contiguous weight
// rows with 16-byte loads, many waves per CU keep enough bytes in flight, and
// the epilogues (RoPE, residual, SwiGLU) run on the reduced dot products.
#include <type_traits>

#include "kernels.h"

namespace cb {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kSegKeys = 64;               // keys per decode-attention workgroup
constexpr int kGemvUnits = 1;              // output units per GEMV wave group

// Order of the argmax: larger first, NaN above everything, smaller index
// first among equals (so the result is unique).
__device__ __forceinline__ bool better(float a, int ia, float b, int ib) {
    const bool na = a != a, nb = b != b;
    if (na != nb) return na;
    if (!na && a != b) return a > b;
    return ia < ib;
}

__global__ __launch_bounds__(1024) void argmax_kernel(const float* __restrict__ v, int n,
                                                      int64_t stride, int* __restrict__ out) {
    __shared__ float bv[16];
    __shared__ int bi[16];
    const float* row = v + blockIdx.x * stride;
    float best = -INFINITY;
    int idx = n;                       // sentinel: loses to every real entry
    for (int i = threadIdx.x; i < n; i += 1024)
        if (idx == n || better(row[i], i, best, idx)) { best = row[i]; idx = i; }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float ob = __shfl_xor(best, o, 64);
        const int oi = __shfl_xor(idx, o, 64);
        if (oi != n && (idx == n || better(ob, oi, best, idx))) { best = ob; idx = oi; }
    }
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) { bv[w] = best; bi[w] = idx; }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int k = 1; k < 16; ++k)
            if (bi[k] != n && (bi[0] == n || better(bv[k], bi[k], bv[0], bi[0]))) {
                bv[0] = bv[k];
                bi[0] = bi[k];
            }
        out[blockIdx.x] = bi[0] == n ? 0 : bi[0];
    }
}

// Sum over the N (2, 4, 8 or 16) lanes of a row group with DPP lane moves
// (full-rate VALU): swap neighbours, swap pairs, mirror within 8, mirror
// within 16.  Every lane of the group ends with the group's sum.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                 CTRL, 0xF, 0xF, false));
}
// Reduction (sum, or max when MAX) over the N lanes of a row group.
template <int N, bool MAX = false>
__device__ __forceinline__ float group_reduce(float v) {
    auto op = [](float a, float b) { return MAX ? fmaxf(a, b) : a + b; };
    if constexpr (N >= 2) v = op(v, dpp<0xB1>(v));      // quad_perm 1,0,3,2
    if constexpr (N >= 4) v = op(v, dpp<0x4E>(v));      // quad_perm 2,3,0,1
    if constexpr (N >= 8) v = op(v, dpp<0x141>(v));     // row_half_mirror
    if constexpr (N >= 16) v = op(v, dpp<0x140>(v));    // row_mirror
    return v;
}
template <int N>
__device__ __forceinline__ float group_sum(float v) { return group_reduce<N, false>(v); }

// Reduction over the whole wave: rows of 16 by DPP, then the four row
// results read into scalar registers.
template <bool MAX>
__device__ __forceinline__ float wave_reduce(float v) {
    v = group_reduce<16, MAX>(v);
    const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
    const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
    const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
    return MAX ? fmaxf(fmaxf(r0, r1), fmaxf(r2, r3)) : (r0 + r1) + (r2 + r3);
}

// R dot products of length K between x and weight rows w[0..R-1] (a null
// row reads as zero), taken by WPU waves together: wave `part` of them reads
// the 512-element pieces part, part + WPU, ... of the rows, each piece of x
// once for all R rows.  Returns the whole products in every lane of a wave
// when WPU = 1, else the wave's partial sums.
template <typename T, int WPU, int R>
__device__ __forceinline__ void dot_rows(const T* __restrict__ x, const T* const (&w)[R], int K,
                                         int lane, int part, float (&s)[R]) {
    // a group past the last unit loads nothing; in a live group (its first
    // row is live) a null row reads the first row instead, with no branch
    // between the loads, and its sum is dropped at the end
    if (!w[0]) {
#pragma unroll
        for (int r = 0; r < R; ++r) s[r] = 0.f;
        return;
    }
    const T* wr[R];
#pragma unroll
    for (int r = 0; r < R; ++r) wr[r] = w[r] ? w[r] : w[0];
    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = 0.f;
#pragma unroll 2
    for (int k = part * 512 + lane * 8; k < K; k += 512 * WPU) {
        float xv[8], wv[R][8];
        Vec8<T>::load(x + k, xv);
#pragma unroll
        for (int r = 0; r < R; ++r) Vec8<T>::load_nt(wr[r] + k, wv[r]);   // weights: once per step
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[r] += xv[i] * wv[r][i];
    }
#pragma unroll
    for (int r = 0; r < R; ++r) s[r] = w[r] ? wave_reduce<false>(acc[r]) : 0.f;
}

// A workgroup of 4 waves computes 4 / WPU groups of U units (WPU waves per
// group, which split K); a unit is a pair of output rows, or one SwiGLU
// column.  The U units of a group share every load of x.
template <typename T, int EPI, int WPU, int U>
__global__ __launch_bounds__(kThreads) void gemv_kernel(GemvArgs g) {
    constexpr int R = 2 * U;
    __shared__ float part_s[kWaves][R];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int grp = blockIdx.x * (kWaves / WPU) + wave / WPU, part = wave % WPU;
    const int units = EPI == EPI_SWIGLU ? g.N : (g.N + 1) / 2;
    const T* x = static_cast<const T*>(g.x);
    const int64_t K = g.K;
    const T* w[R];
    int local[U];
    void* out[U];
    bool rope[U], two[U], live[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
        const int u = grp * U + j;
        live[j] = u < units;
        w[2 * j] = w[2 * j + 1] = nullptr;
        local[j] = 0;
        out[j] = nullptr;
        rope[j] = false;
        two[j] = true;
        if (!live[j]) continue;
        if constexpr (EPI == EPI_SWIGLU) {
            w[2 * j] = static_cast<const T*>(g.b0) + u * K;
            w[2 * j + 1] = static_cast<const T*>(g.b1) + u * K;
        } else {
            const int r0 = 2 * u;
            two[j] = r0 + 1 < g.N;
            const T* m;
            if (EPI == EPI_QKV && r0 >= g.n0 + g.n1) {
                m = static_cast<const T*>(g.b2); local[j] = r0 - g.n0 - g.n1; out[j] = g.out2;
            } else if (EPI == EPI_QKV && r0 >= g.n0) {
                m = static_cast<const T*>(g.b1); local[j] = r0 - g.n0; out[j] = g.out1; rope[j] = true;
            } else {
                m = static_cast<const T*>(g.b0); local[j] = r0; out[j] = g.out0; rope[j] = EPI == EPI_QKV;
            }
            w[2 * j] = m + local[j] * K;
            w[2 * j + 1] = two[j] ? m + (local[j] + 1) * K : nullptr;
        }
    }
    float s[R];
    dot_rows<T, WPU, R>(x, w, g.K, lane, part, s);
    if constexpr (WPU > 1) {
        if (lane == 0)
#pragma unroll
            for (int r = 0; r < R; ++r) part_s[wave][r] = s[r];
        __syncthreads();
        if (part != 0) return;
#pragma unroll
        for (int p = 1; p < WPU; ++p)
#pragma unroll
            for (int r = 0; r < R; ++r) s[r] += part_s[wave + p][r];
    }
    // lane j stores unit j
#pragma unroll
    for (int j = 0; j < U; ++j) {
        if (lane != j || !live[j]) continue;
        const float a = s[2 * j], b = s[2 * j + 1];
        const int u = grp * U + j;
        if constexpr (EPI == EPI_SWIGLU) {
            static_cast<T*>(g.out0)[u] = from_f32<T>(a / (1.f + __expf(-a)) * b);
        } else if constexpr (EPI == EPI_QKV) {
            float y0 = a, y1 = b;
            if (rope[j]) {
                const float2 cs = g.rope.tab[(int64_t)g.pos * g.rope.half + ((local[j] % g.head_dim) >> 1)];
                y0 = a * cs.x - b * cs.y;
                y1 = a * cs.y + b * cs.x;
            }
            static_cast<T*>(out[j])[local[j]] = from_f32<T>(y0);
            static_cast<T*>(out[j])[local[j] + 1] = from_f32<T>(y1);
        } else {
            const int r0 = 2 * u;
            float* o = static_cast<float*>(g.out0);
            float y0 = a, y1 = b;
            if (EPI == EPI_RESID) {
                y0 += g.resid[r0];
                if (two[j]) y1 += g.resid[r0 + 1];
            }
            o[r0] = y0;
            if (two[j]) o[r0 + 1] = y1;
        }
    }
}

// Split-key attention of one query row (all query heads) over n_ctx cached
// keys plus the step's own key.  Grid (kv heads, key segments of 64); the G
// query heads that share a KV head are handled together, so each cached key
// and value row is read once.  A key row is spread over DH/8 lanes (8
// elements each); each wave owns 16 keys and issues all of their K and V
// loads before using them.  Output: per (query head, segment) the maximum,
// the sum of exponentials and the unnormalized output, merged by
// decode_combine_kernel.
template <typename T, int DH, int GMAX>
__global__ __launch_bounds__(kThreads) void decode_attention_kernel(DecodeAttnArgs a) {
    constexpr int LPK = DH / 8, KPI = 64 / LPK, PER_WAVE = kSegKeys / kWaves;
    constexpr int ITERS = PER_WAVE / KPI;
    static_assert(ITERS * KPI == PER_WAVE, "keys per wave");
    __shared__ float sc[GMAX][kSegKeys];
    __shared__ float stat[GMAX][2];
    __shared__ float osum[kWaves][KPI][GMAX][DH];     // per key subgroup partial outputs
    const int h = blockIdx.x, seg = blockIdx.y, nseg = gridDim.y;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int sub = lane / LPK, li = lane % LPK;
    const int G = GMAX == 1 ? 1 : a.group;
    const int kvd = a.n_kv_heads * DH;
    const int n_keys = a.n_ctx + 1;
    const int j0 = seg * kSegKeys + w * PER_WAVE;
    auto row = [&](const void* cache, const void* fresh, int j) -> const T* {
        return j < a.n_ctx ? static_cast<const T*>(cache) + (int64_t)j * kvd + h * DH + li * 8
                           : static_cast<const T*>(fresh) + h * DH + li * 8;
    };
    // every K and V load of this lane, issued first
    float kr[ITERS][8], vr[ITERS][8];
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
        const int j = j0 + it * KPI + sub;
        if (j < n_keys) {            // cached rows: read once per step
            Vec8<T>::load_nt(row(a.k, a.k_new, j), kr[it]);
            Vec8<T>::load_nt(row(a.v, a.v_new, j), vr[it]);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) kr[it][i] = vr[it][i] = 0.f;
        }
    }
    float q[GMAX][8];
#pragma unroll
    for (int g = 0; g < GMAX; ++g) {
        if (g < G) {
            Vec8<T>::load(static_cast<const T*>(a.q) + (int64_t)(h * G + g) * DH + li * 8, q[g]);
#pragma unroll
            for (int i = 0; i < 8; ++i) q[g][i] *= a.scale;
        }
    }
    // scores
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
        const int jl = w * PER_WAVE + it * KPI + sub;
        const bool ok = seg * kSegKeys + jl < n_keys;
#pragma unroll
        for (int g = 0; g < GMAX; ++g) {
            if (g >= G) break;
            float s = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) s += q[g][i] * kr[it][i];
            s = group_sum<LPK>(s);
            if (li == 0) sc[g][jl] = ok ? s : -INFINITY;
        }
    }
    __syncthreads();
    // softmax statistics of the segment: wave 0, lane t owns key t
    if (w == 0) {
#pragma unroll
        for (int g = 0; g < GMAX; ++g) {
            if (g >= G) break;
            const float s = sc[g][lane];
            const float m = wave_reduce<true>(s);
            const float p = s == -INFINITY ? 0.f : __expf(s - m);
            const float l = wave_reduce<false>(p);
            sc[g][lane] = p;
            if (lane == 0) { stat[g][0] = m; stat[g][1] = l; }
        }
    }
    __syncthreads();
    // values
    float o[GMAX][8];
#pragma unroll
    for (int g = 0; g < GMAX; ++g) {
        if (g >= G) break;
#pragma unroll
        for (int i = 0; i < 8; ++i) o[g][i] = 0.f;
#pragma unroll
        for (int it = 0; it < ITERS; ++it) {
            const float p = sc[g][w * PER_WAVE + it * KPI + sub];
#pragma unroll
            for (int i = 0; i < 8; ++i) o[g][i] += p * vr[it][i];
        }
        Vec8<float>::store(&osum[w][sub][g][li * 8], o[g]);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < G * DH; e += kThreads) {
        const int g = e / DH, d = e % DH;
        float sum = 0.f;
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww)
#pragma unroll
            for (int k = 0; k < KPI; ++k) sum += osum[ww][k][g][d];
        const int64_t slot = (int64_t)(h * G + g) * nseg + seg;
        a.part_o[slot * DH + d] = sum;
        if (d == 0) {
            a.part_ml[2 * slot] = stat[g][0];
            a.part_ml[2 * slot + 1] = stat[g][1];
        }
    }
}

// Decode attention on the matrix cores, for query-head groups (GQA): one
// wave per (KV head, 64-key segment), no workgroup barriers (each wave owns
// its LDS slice).  The group's query heads are the 16 columns of
// v_mfma_f32_16x16x32_bf16 (unused ones zero): S^T = K Q^T with K rows
// loaded straight into the A operand (lane l: key l % 16, dims
// 8 (l / 16) ..), then the softmax over each query column (4 keys per lane,
// 4 lanes per column), then O = P V with P taken from the score registers
// as the A operand (its keys ordered 4q+0..3, 16+4q+0..3 per 32-key step)
// and V read from LDS by transposing 8-byte reads that return exactly those
// 4-key runs for one dimension.  V reaches LDS by buffer_load ... lds into
// unpadded rows whose 16-byte chunks sit at chunk ^ key(row) so that the
// transposing reads of 16 rows x 2 chunks touch distinct banks.
// Output: the same per (query head, segment) maximum, sum of exponentials
// and unnormalized output as decode_attention_kernel.
typedef int i32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ i32x4_t dec_rsrc(const void* base, int bytes) {
    const uint64_t p = reinterpret_cast<uint64_t>(base);
    return i32x4_t{__builtin_amdgcn_readfirstlane((int)(uint32_t)p),
                   __builtin_amdgcn_readfirstlane((int)((p >> 32) & 0xFFFF)),
                   __builtin_amdgcn_readfirstlane(bytes), 0x00020000};
}
// 16 bytes per lane into LDS at m0 + 16 * lane, as in the prefill attention
// (the s_nop: one wait state after the write of M0).
__device__ __forceinline__ void dec_dma16(i32x4_t rsrc, int voff, uint32_t m0) {
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" : : "v"(voff), "s"(rsrc), "{m0}"(m0)
                 : "memory");
}
template <int DH> __device__ __forceinline__ int dec_vkey(int r) {
    return DH == 128 ? 2 * (r & 7) : 2 * ((r >> 1) & 3);
}

template <int DH>
__global__ __launch_bounds__(kThreads) void decode_attention_mfma_kernel(DecodeAttnArgs a) {
    constexpr int RB = DH * 2;                 // bytes per V row in LDS
    constexpr int CPR = RB / 16;               // 16-byte chunks per row
    constexpr int RPI = 64 / CPR;              // rows per copy instruction
    constexpr int NKS = DH / 32;               // 32-dim steps of the scores
    constexpr int NT = DH / 16;                // 16-dim output tiles
    __shared__ __attribute__((aligned(16))) unsigned char sv_all[kWaves][kSegKeys * RB];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int h = blockIdx.y, G = a.group;
    const int nseg = (a.n_ctx + 1 + kSegKeys - 1) / kSegKeys;
    const int seg = blockIdx.x * kWaves + wave;
    if (seg >= nseg) return;                   // wave-uniform; no barriers below
    const int kvd = a.n_kv_heads * DH;
    const int j0 = seg * kSegKeys, n_keys = a.n_ctx + 1;
    const int c16 = lane & 15, q4 = lane >> 4;
    unsigned char* sv = sv_all[wave];
    const bf16* vbase = static_cast<const bf16*>(a.v) + (int64_t)j0 * kvd + h * DH;
    // V rows of the cache into LDS (rows past the cache read as zero)
    {
        const int rows_c = min(kSegKeys, max(0, a.n_ctx - j0));
        const i32x4_t rs = dec_rsrc(vbase, rows_c * kvd * 2);
        const uint32_t l0 = (uint32_t)reinterpret_cast<uintptr_t>(sv);
#pragma unroll
        for (int c = 0; c < kSegKeys / RPI; ++c) {
            const int r = c * RPI + lane / CPR, slot = lane % CPR;
            dec_dma16(rs, r * kvd * 2 + ((slot ^ dec_vkey<DH>(r)) & (CPR - 1)) * 16, l0 + c * RPI * RB);
        }
    }
    // K rows straight into the A operand; Q of the group as the B operand
    bf16x8 kf[4][NKS], qf[NKS];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int j = j0 + 16 * t + c16;
        const bf16* kr = j < a.n_ctx ? static_cast<const bf16*>(a.k) + (int64_t)j * kvd + h * DH
                                     : static_cast<const bf16*>(a.k_new) + h * DH;
#pragma unroll
        for (int s = 0; s < NKS; ++s) {
            if (j < n_keys) kf[t][s] = *reinterpret_cast<const bf16x8*>(kr + 32 * s + 8 * q4);
            else
#pragma unroll
                for (int e = 0; e < 8; ++e) kf[t][s][e] = static_cast<bf16>(0.f);
        }
    }
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
        if (c16 < G)
            qf[s] = *reinterpret_cast<const bf16x8*>(static_cast<const bf16*>(a.q) +
                                                    (int64_t)(h * G + c16) * DH + 32 * s + 8 * q4);
        else
#pragma unroll
            for (int e = 0; e < 8; ++e) qf[s][e] = static_cast<bf16>(0.f);
    }
    floatx4 st[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        st[t] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < NKS; ++s)
            st[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[t][s], qf[s], st[t], 0, 0, 0);
    }
    // softmax of query column c16 over the segment's keys 16 t + 4 q4 + i
    float m = -INFINITY;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float s = j0 + 16 * t + 4 * q4 + i < n_keys ? st[t][i] * a.scale : -INFINITY;
            st[t][i] = s;
            m = fmaxf(m, s);
        }
    m = fmaxf(m, __shfl_xor(m, 16, 64));
    m = fmaxf(m, __shfl_xor(m, 32, 64));
    float l = 0.f;
    bf16x8 pa[2];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float p = st[t][i] == -INFINITY ? 0.f : __expf(st[t][i] - m);
            l += p;
            pa[t >> 1][(t & 1) * 4 + i] = static_cast<bf16>(p);
        }
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    // the new key's V row (not in the cache) goes to its slot by plain stores
    __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));   // vmcnt(0): the copies have landed
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    if (a.n_ctx >= j0 && a.n_ctx < j0 + kSegKeys && lane < CPR) {
        const int r = a.n_ctx - j0;
        *reinterpret_cast<u32x4*>(sv + r * RB + ((lane ^ dec_vkey<DH>(r)) & (CPR - 1)) * 16) =
            *reinterpret_cast<const u32x4*>(static_cast<const bf16*>(a.v_new) + h * DH + lane * 8);
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);                     // lgkmcnt(0): stores visible to the wave
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    // O = P V, 16 dims per tile, 32 keys per step
    floatx4 o[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) o[nt] = floatx4{0.f, 0.f, 0.f, 0.f};
    typedef short i16x4 __attribute__((ext_vector_type(4)));
    typedef short i16x8 __attribute__((ext_vector_type(8)));
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const int r = 32 * u + 4 * q4 + (c16 >> 2);           // + 16 for the second run
            const int col = 16 * nt + 4 * (c16 & 3);
            const int off = r * RB + ((((col >> 3) ^ dec_vkey<DH>(r)) & (CPR - 1)) << 4) + (col & 7) * 2;
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(sv + off));
            const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(sv + off + 16 * RB));
            const i16x8 w = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[u], __builtin_bit_cast(bf16x8, w), o[nt], 0, 0, 0);
        }
    // lane l holds O[query 4 q4 + i][dim 16 nt + c16]; stats of query c16 in every lane
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int g = 4 * q4 + i;
        if (g < G) {
            const int64_t slot = (int64_t)(h * G + g) * nseg + seg;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) a.part_o[slot * DH + 16 * nt + c16] = o[nt][i];
        }
    }
    if (q4 == 0 && c16 < G) {
        const int64_t slot = (int64_t)(h * G + c16) * nseg + seg;
        a.part_ml[2 * slot] = m;
        a.part_ml[2 * slot + 1] = l;
    }
}

// Merge of the key segments.  Workgroup (query head, 32-dimension slice):
// every thread first forms the largest segment maximum M and the weighted
// sum of exponentials over all segments (a few floats per segment), then the
// 256 threads = 32 dimensions x 8 segment slices accumulate the weighted
// segment outputs, and the 8 slices meet in LDS.
constexpr int kCombSlices = kThreads / 32;

template <typename T>
__global__ __launch_bounds__(kThreads) void decode_combine_kernel(DecodeAttnArgs a, int nseg,
                                                                  int dh) {
    __shared__ float red[kWaves];
    __shared__ float acc[kCombSlices][32];
    const int hq = blockIdx.x, d0 = blockIdx.y * 32, t = threadIdx.x, lane = t & 63, w = t >> 6;
    const float* ml = a.part_ml + (int64_t)hq * nseg * 2;
    const float* po = a.part_o + (int64_t)hq * nseg * dh;
    float mx = -INFINITY;
    for (int s = t; s < nseg; s += kThreads) mx = fmaxf(mx, ml[2 * s]);
    mx = wave_reduce<true>(mx);
    if (lane == 0) red[w] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    float den = 0.f;
    for (int s = t; s < nseg; s += kThreads) {
        const float m = ml[2 * s];
        den += m == -INFINITY ? 0.f : __expf(m - mx) * ml[2 * s + 1];
    }
    den = wave_reduce<false>(den);
    if (lane == 0) red[w] = den;
    __syncthreads();
    den = red[0] + red[1] + red[2] + red[3];
    const int d = d0 + (t & 31), sl = t >> 5;
    float num = 0.f;
    if (d < dh) {
#pragma unroll 4
        for (int s = sl; s < nseg; s += kCombSlices) {
            const float m = ml[2 * s];
            const float o = po[(int64_t)s * dh + d];
            num += (m == -INFINITY ? 0.f : __expf(m - mx)) * o;
        }
    }
    acc[sl][t & 31] = num;
    __syncthreads();
    if (t < 32 && d0 + t < dh) {
        float sum = 0.f;
#pragma unroll
        for (int k = 0; k < kCombSlices; ++k) sum += acc[k][t];
        static_cast<T*>(a.out)[(int64_t)hq * dh + d0 + t] = from_f32<T>(sum / den);
    }
}

template <typename T, int EPI>
hipError_t gemv_e(const GemvArgs& g, int units, hipStream_t s) {
    // K split over the 4 waves of a workgroup for every shape: short waves
    // leave a short tail when the last ones finish (measured on MI355X, 7B
    // decode step: 2.75 ms of GEMVs with 4 waves per unit, 2.86 with 2, 2.96
    // with 1 for the products of >= 8192 units).  One unit per workgroup:
    // 2.62 ms, against 2.88 with two units sharing the loads of x and 4.97
    // with four (fewer, longer workgroups keep fewer bytes in flight)
    hipLaunchKernelGGL((gemv_kernel<T, EPI, 4, kGemvUnits>), dim3((units + kGemvUnits - 1) / kGemvUnits),
                       dim3(kThreads), 0, s, g);
    return hipGetLastError();
}

template <typename T>
hipError_t gemv_t(int epi, const GemvArgs& g, hipStream_t s) {
    const int units = epi == EPI_SWIGLU ? g.N : (g.N + 1) / 2;
    switch (epi) {
        case EPI_STORE_F32: return gemv_e<T, EPI_STORE_F32>(g, units, s);
        case EPI_QKV: return gemv_e<T, EPI_QKV>(g, units, s);
        case EPI_RESID: return gemv_e<T, EPI_RESID>(g, units, s);
        case EPI_SWIGLU: return gemv_e<T, EPI_SWIGLU>(g, units, s);
    }
    return hipErrorInvalidValue;
}

template <typename T, int DH>
hipError_t decode_attn_t(const DecodeAttnArgs& a, hipStream_t s) {
    const int nseg = (a.n_ctx + 1 + kSegKeys - 1) / kSegKeys;
    const dim3 grid(a.n_kv_heads, nseg);
    if (std::is_same<T, bf16>::value && a.group > 1)
        hipLaunchKernelGGL((decode_attention_mfma_kernel<DH>), dim3((nseg + kWaves - 1) / kWaves, a.n_kv_heads),
                           dim3(kThreads), 0, s, a);
    else if (a.group == 1)
        hipLaunchKernelGGL((decode_attention_kernel<T, DH, 1>), grid, dim3(kThreads), 0, s, a);
    else
        hipLaunchKernelGGL((decode_attention_kernel<T, DH, 8>), grid, dim3(kThreads), 0, s, a);
    hipLaunchKernelGGL(decode_combine_kernel<T>, dim3(a.n_kv_heads * a.group, DH / 32),
                       dim3(kThreads), 0, s, a, nseg, DH);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv(int dtype, int epi, const GemvArgs& g, hipStream_t s) {
    if (g.N <= 0) return hipSuccess;
    if (g.K <= 0 || g.K % 8) return hipErrorInvalidValue;
    if (epi == EPI_QKV && (g.n0 % 2 || g.n1 % 2 || g.head_dim % 2 || !g.rope.tab || g.pos < 0 ||
                           g.pos >= g.rope.n_pos || g.rope.half != g.head_dim / 2))
        return hipErrorInvalidValue;
    return dtype == BF16 ? gemv_t<bf16>(epi, g, s) : gemv_t<float>(epi, g, s);
}

hipError_t launch_argmax(const float* v, int rows, int n, int64_t stride, int* out, hipStream_t s) {
    if (rows <= 0 || n <= 0) return hipSuccess;
    hipLaunchKernelGGL(argmax_kernel, dim3(rows), dim3(1024), 0, s, v, n, stride, out);
    return hipGetLastError();
}

int decode_attention_segments(int n_ctx) { return (n_ctx + 1 + kSegKeys - 1) / kSegKeys; }

hipError_t launch_decode_attention(int dtype, const DecodeAttnArgs& a, hipStream_t s) {
    if (a.n_ctx < 0 || a.group < 1 || a.group > 8 || !a.part_o || !a.part_ml)
        return hipErrorInvalidValue;
    if (a.head_dim == 128)
        return dtype == BF16 ? decode_attn_t<bf16, 128>(a, s) : decode_attn_t<float, 128>(a, s);
    if (a.head_dim == 64)
        return dtype == BF16 ? decode_attn_t<bf16, 64>(a, s) : decode_attn_t<float, 64>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace cb
