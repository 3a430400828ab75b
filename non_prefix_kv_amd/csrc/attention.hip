// Causal attention of the recomputed rows over the whole fused cache
// (CacheBlend explainer (0h-n0), section "選択的再計算", Step 4: ordinary
// attention on the merged K/V; abeam CacheBlend explainer: the selected
// tokens attend over the entire input).  Queries sit at scattered real
// positions; key j is visible to a query at position p iff its position
// kv_pos0 + j <= p.  GQA: query head h reads KV head h / (Hq / Hkv).
//
// gfx950 design: one workgroup = 64 query rows of one head (4 wave64s x 16
// queries), streaming key blocks through LDS with an online softmax (the
// rescaling scheme of FlashAttention, Dao et al.).  Scores are computed
// transposed, S^T = K Q^T, so each lane ends up holding the scores of one
// query for 16 keys; those probabilities are exactly the B operand of the
// next MFMA, O^T += V^T P^T, once V is stored transposed in LDS and the keys
// of each lane group are matched on both operands.  No probability tile goes
// through LDS.  Blocks whose keys all lie after a wave's last query position
// are skipped by that wave; blocks after the workgroup's last position are
// never loaded.  Tiles are issued longest-first.
#include "kernels.h"

namespace cb {

namespace {

constexpr int kThreads = 256;
constexpr int QT = 64;   // queries per workgroup

template <typename T> struct AttnCfg;
template <> struct AttnCfg<bf16> { static constexpr int KB = 64; };
template <> struct AttnCfg<float> { static constexpr int KB = 32; };

// Elements [0,4) and [16,20) of p as one fragment (two 4-element LDS reads).
__device__ __forceinline__ Frag<bf16> load_quad_pair(const bf16* p) {
    const u32x2 lo = *reinterpret_cast<const u32x2*>(p);
    const u32x2 hi = *reinterpret_cast<const u32x2*>(p + 16);
    const u32x4 w{lo[0], lo[1], hi[0], hi[1]};
    Frag<bf16> f;
    f.v = __builtin_bit_cast(bf16x8, w);
    return f;
}
__device__ __forceinline__ Frag<float> load_quad_pair(const float* p) {
    const floatx4 lo = *reinterpret_cast<const floatx4*>(p);
    const floatx4 hi = *reinterpret_cast<const floatx4*>(p + 16);
    Frag<float> f;
    f.v = floatx8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return f;
}

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void attention_kernel(AttnArgs a) {
    constexpr int KB = AttnCfg<T>::KB;
    constexpr int LDK = D + 16 / (int)sizeof(T);        // sK row stride (elements)
    constexpr int LDV = KB + 4;                          // sVt row stride (elements)
    constexpr int NKT = KB / 16;                         // 16-key tiles per block
    constexpr int NKS = KB / 32;                         // 32-key MFMA steps per block
    constexpr int NDS = D / 32;                          // 32-dim steps for S
    constexpr int NDT = D / 16;                          // 16-dim output tiles
    constexpr int VEC = 16 / (int)sizeof(T);
    __shared__ __attribute__((aligned(16))) T sK[KB * LDK];
    __shared__ __attribute__((aligned(16))) T sVt[D * LDV];
    __shared__ int sred[2][kThreads / 64];

    const int n_tiles = (a.n_q + QT - 1) / QT;
    const int qt = n_tiles - 1 - (int)blockIdx.x;      // longest tiles first
    const int h = blockIdx.y;
    const int hk = h / (a.n_q_heads / a.n_kv_heads);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int fr = lane & 15, g = lane >> 4;
    const int q_ld = a.n_q_heads * D, kv_ld = a.n_kv_heads * D;

    // This lane's query (column of S^T).
    const int qi_raw = qt * QT + wave * 16 + fr;
    const bool q_ok = qi_raw < a.n_q;
    const int qi = q_ok ? qi_raw : a.n_q - 1;
    const int qpos = a.q_pos[qi];
    // Workgroup / wave position range.
    int wmax = qpos, wmin = qpos;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
        wmax = max(wmax, __shfl_xor(wmax, o, 64));
        wmin = min(wmin, __shfl_xor(wmin, o, 64));
    }
    if (lane == 0) { sred[0][wave] = wmax; sred[1][wave] = wmin; }
    __syncthreads();
    int bmax = sred[0][0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) bmax = max(bmax, sred[0][w]);
    const int nk = min(a.n_kv, bmax - a.kv_pos0 + 1);
    const int n_kb = nk > 0 ? (nk + KB - 1) / KB : 0;

    // Q fragments (B operand of S^T = K Q^T), kept in registers.
    const int qrow = a.qidx ? a.qidx[qi] : qi;
    const T* qp = static_cast<const T*>(a.q) + (int64_t)qrow * q_ld + h * D;
    Frag<T> qf[NDS];
#pragma unroll
    for (int s = 0; s < NDS; ++s) qf[s] = load_frag<T>(qp + s * 32 + g * 8);

    floatx4 o[NDT];
#pragma unroll
    for (int t = 0; t < NDT; ++t) o[t] = floatx4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;
    const float sl2 = 1.4426950408889634f / sqrtf((float)D);   // log2(e) / sqrt(D)

    const T* kbase = static_cast<const T*>(a.k) + hk * D;
    const T* vbase = static_cast<const T*>(a.v) + hk * D;
    for (int kb = 0; kb < n_kb; ++kb) {
        const int k0 = kb * KB;
        // K block -> sK (row-major), V block -> sVt (transposed); rows past
        // n_kv are zero so masked probabilities never meet garbage values.
        for (int u = tid; u < KB * (D / VEC); u += kThreads) {
            const int r = u / (D / VEC), c = (u % (D / VEC)) * VEC;
            const bool ok = k0 + r < a.n_kv;
            u32x4 kv = ok ? *reinterpret_cast<const u32x4*>(kbase + (int64_t)(k0 + r) * kv_ld + c)
                          : u32x4{0, 0, 0, 0};
            *reinterpret_cast<u32x4*>(&sK[r * LDK + c]) = kv;
            u32x4 vv = ok ? *reinterpret_cast<const u32x4*>(vbase + (int64_t)(k0 + r) * kv_ld + c)
                          : u32x4{0, 0, 0, 0};
            const T* ve = reinterpret_cast<const T*>(&vv);
#pragma unroll
            for (int i = 0; i < VEC; ++i) sVt[(c + i) * LDV + r] = ve[i];
        }
        __syncthreads();
        if (a.kv_pos0 + k0 <= wmax) {     // wave-uniform: some key visible to this wave
            floatx4 st[NKT];
#pragma unroll
            for (int t = 0; t < NKT; ++t) {
                st[t] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < NDS; ++s) {
                    Frag<T> kf = load_frag<T>(&sK[(t * 16 + fr) * LDK + s * 32 + g * 8]);
                    mfma16(st[t], kf, qf[s]);
                }
            }
            const bool need_mask = (k0 + KB > a.n_kv) || (a.kv_pos0 + k0 + KB - 1 > wmin);
            float mloc = -INFINITY;
#pragma unroll
            for (int t = 0; t < NKT; ++t)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float sc = st[t][e] * sl2;
                    if (need_mask) {
                        const int kj = k0 + t * 16 + g * 4 + e;
                        if (kj >= a.n_kv || a.kv_pos0 + kj > qpos) sc = -INFINITY;
                    }
                    st[t][e] = sc;
                    mloc = fmaxf(mloc, sc);
                }
            mloc = fmaxf(mloc, __shfl_xor(mloc, 16, 64));
            mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
            const float m_new = fmaxf(m_run, mloc);
            const float m_use = m_new == -INFINITY ? 0.f : m_new;
            const float alpha = exp2f(m_run - m_use);
            m_run = m_new;
            l_run *= alpha;
#pragma unroll
            for (int t = 0; t < NDT; ++t) o[t] *= alpha;
            Frag<T> pf[NKS];
#pragma unroll
            for (int t = 0; t < NKT; ++t)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float p = exp2f(st[t][e] - m_use);
                    l_run += p;
                    pf[t >> 1].v[(t & 1) * 4 + e] = from_f32<T>(p);
                }
            // O^T += V^T P^T over this block's keys.
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
                for (int s2 = 0; s2 < NKS; ++s2) {
                    const T* vr = &sVt[(dt * 16 + fr) * LDV + s2 * 32 + g * 4];
                    mfma16(o[dt], load_quad_pair(vr), pf[s2]);
                }
            }
        }
        __syncthreads();
    }
    float l_tot = l_run + __shfl_xor(l_run, 16, 64);
    l_tot += __shfl_xor(l_tot, 32, 64);
    if (!q_ok) return;
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    T* op = static_cast<T*>(a.out) + (int64_t)qi * q_ld + h * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int e = 0; e < 4; ++e) op[dt * 16 + g * 4 + e] = from_f32<T>(o[dt][e] * inv);
}

template <typename T, int D>
hipError_t launch_t(const AttnArgs& a, hipStream_t s) {
    dim3 grid((a.n_q + QT - 1) / QT, a.n_q_heads);
    hipLaunchKernelGGL((attention_kernel<T, D>), grid, dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attention(int dtype, const AttnArgs& a, hipStream_t s) {
    if (a.n_q <= 0) return hipSuccess;
    if (a.n_kv_heads <= 0 || a.n_q_heads % a.n_kv_heads != 0) return hipErrorInvalidValue;
    if (a.head_dim == 128)
        return dtype == BF16 ? launch_t<bf16, 128>(a, s) : launch_t<float, 128>(a, s);
    if (a.head_dim == 64)
        return dtype == BF16 ? launch_t<bf16, 64>(a, s) : launch_t<float, 64>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace cb
