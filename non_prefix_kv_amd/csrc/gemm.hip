// Matrix-core GEMM for the projections of the recomputed rows:
// C[M][N] = A[M][K] * B[N][K]^T with both operands K-contiguous (activations
// row-major, weights [out][in]), fp32 accumulation, and fused epilogues:
//   EPI_QKV    q/k/v projections in one launch; RoPE applied to the q and k
//              columns at each row's real position (CacheBlend explainer
//              (0h-n0), RoPE section: R(m), theta_i); Q, K and V stored apart
//   EPI_RESID  O and down projections: fp32 residual (gathered by row map) + acc
//   EPI_SWIGLU gate/up projections: silu(gate) * up
//   EPI_STORE_F32 plain fp32 store (kernel-level entry point)
//
// Tiling for gfx950: a 128x128 output tile per 256-thread workgroup, four
// wave64s in a 2x2 grid, each wave 64x64 as 4x4 16x16 MFMA tiles.  K advances
// 128 bytes per step (64 bf16 / 32 f32) through double-buffered LDS.  LDS rows
// are unpadded 128-byte rows of eight 16-byte chunks stored at chunk index
// (chunk XOR row % 8): the fragment reads of 16 rows and the staging stores
// are then free of bank conflicts (measured: zero conflict cycles, versus a
// third of LDS cycles with 16-byte row padding).  Workgroups are renumbered
// so that consecutive tile ids (the row tiles that share one weight column
// block) land on the same XCD and reuse that XCD's L2.
#include "kernels.h"

namespace cb {

namespace {

constexpr int BM = 128, BN = 128, kThreads = 256;
constexpr int kRowBytes = 128;           // K-slice per stage, bytes per row

template <typename T> struct Tile {
    static constexpr int BK = kRowBytes / (int)sizeof(T);
    static constexpr int LDK = kRowBytes / (int)sizeof(T);                 // LDS row stride
    static constexpr int VEC = 16 / (int)sizeof(T);                        // elems per 16 B
};

// Element offset in a swizzled LDS tile of the 16-byte chunk that holds
// row r, element column c (c a multiple of 16 bytes' worth of elements).
template <typename T>
__device__ __forceinline__ int swz(int r, int c) {
    constexpr int VEC = Tile<T>::VEC;
    return r * Tile<T>::LDK + (((c / VEC) ^ r) & 7) * VEC;
}

// A fragment (8 consecutive reduction elements of one row) from a swizzled
// tile: one chunk for bf16, two chunks for f32.
template <typename T> __device__ __forceinline__ Frag<T> lds_frag(const T* s, int r, int c);
template <> __device__ __forceinline__ Frag<bf16> lds_frag<bf16>(const bf16* s, int r, int c) {
    return load_frag<bf16>(s + swz<bf16>(r, c));
}
template <> __device__ __forceinline__ Frag<float> lds_frag<float>(const float* s, int r, int c) {
    const floatx4 lo = *reinterpret_cast<const floatx4*>(s + swz<float>(r, c));
    const floatx4 hi = *reinterpret_cast<const floatx4*>(s + swz<float>(r, c + 4));
    Frag<float> f;
    f.v = floatx8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return f;
}

__device__ __forceinline__ float silu_f(float x) { return x / (1.0f + __expf(-x)); }

// Maps the hardware workgroup id to a logical tile id such that each XCD
// (ids are dealt round-robin over the 8 XCDs) receives a contiguous range.
__device__ __forceinline__ int xcd_remap(int hw, int total) {
    const int xcd = hw & 7, j = hw >> 3;
    const int base = total >> 3, rem = total & 7;
    return xcd * base + min(xcd, rem) + j;
}

// Row v (0..BN-1) of the block's B tile.  Rows past N are clamped to the
// last row: they only feed output columns that are never stored.
template <typename T, int EPI>
__device__ __forceinline__ const T* b_row_ptr(const GemmArgs& g, int v, int n_tile) {
    if (EPI == EPI_SWIGLU) {
        const int oc = min(n_tile * (BN / 2) + (v >> 5) * 16 + (v & 15), g.N - 1);
        return static_cast<const T*>((v & 16) ? g.b1 : g.b0) + (int64_t)oc * g.K;
    } else {
        const int n = min(n_tile * BN + v, g.N - 1);
        if (EPI == EPI_QKV) {
            if (n < g.n0) return static_cast<const T*>(g.b0) + (int64_t)n * g.K;
            if (n < g.n0 + g.n1) return static_cast<const T*>(g.b1) + (int64_t)(n - g.n0) * g.K;
            return static_cast<const T*>(g.b2) + (int64_t)(n - g.n0 - g.n1) * g.K;
        }
        return static_cast<const T*>(g.b0) + (int64_t)n * g.K;
    }
}

template <typename T, int EPI>
__global__ __launch_bounds__(kThreads, 2) void gemm_kernel(GemmArgs g) {
    using TL = Tile<T>;
    constexpr int BK = TL::BK, LDK = TL::LDK, VEC = TL::VEC;
    __shared__ __attribute__((aligned(16))) T sA[2][BM * LDK];
    __shared__ __attribute__((aligned(16))) T sB[2][BN * LDK];

    const int m_tiles = (g.M + BM - 1) / BM;
    const int n_cols_per_tile = (EPI == EPI_SWIGLU) ? BN / 2 : BN;
    const int n_tiles = (g.N + n_cols_per_tile - 1) / n_cols_per_tile;
    const int tile = xcd_remap(blockIdx.x, m_tiles * n_tiles);
    const int m_tile = tile % m_tiles, n_tile = tile / m_tiles;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    // Global -> register staging: each thread moves 4 x 16 B of A and of B
    // per stage, byte column (t%8)*16 of row t/8 + 32p.
    const int ld_row = tid >> 3;
    const int ld_col = (tid & 7) * VEC;
    const int st_off = swz<T>(ld_row, ld_col);          // + 32 rows per p
    const T* a_src[4];
    const T* b_src[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int r = ld_row + 32 * p;
        const int m = min(m_tile * BM + r, g.M - 1);
        a_src[p] = static_cast<const T*>(g.a) + (int64_t)m * g.K + ld_col;
        b_src[p] = b_row_ptr<T, EPI>(g, r, n_tile) + ld_col;
    }
    // Two register stage sets: while stage kt is multiplied out of LDS,
    // stage kt+1 waits in registers for its LDS store and stage kt+2 is in
    // flight from memory (prefetch distance 2 hides global latency).
    u32x4 sa0[4], sb0[4], sa1[4], sb1[4];
    auto load_stage = [&](int kt, u32x4 (&ra)[4], u32x4 (&rb)[4]) {
        const int ko = kt * BK;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            ra[p] = *reinterpret_cast<const u32x4*>(a_src[p] + ko);
            rb[p] = *reinterpret_cast<const u32x4*>(b_src[p] + ko);
        }
    };
    auto store_stage = [&](int buf, const u32x4 (&ra)[4], const u32x4 (&rb)[4]) {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            *reinterpret_cast<u32x4*>(&sA[buf][st_off + 32 * p * LDK]) = ra[p];
            *reinterpret_cast<u32x4*>(&sB[buf][st_off + 32 * p * LDK]) = rb[p];
        }
    };

    floatx4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    const int KT = g.K / BK;
    const int fr = lane & 15, fk = (lane >> 4) * 8;
    auto compute = [&](int buf) {
#pragma unroll
        for (int ks = 0; ks < BK; ks += 32) {
            Frag<T> af[4], bfr[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) af[i] = lds_frag<T>(sA[buf], wm * 64 + i * 16 + fr, ks + fk);
#pragma unroll
            for (int j = 0; j < 4; ++j) bfr[j] = lds_frag<T>(sB[buf], wn * 64 + j * 16 + fr, ks + fk);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) mfma16(acc[i][j], af[i], bfr[j]);
        }
    };
    // Steady state, unrolled by two so buffers and register sets are static:
    // on entry stage kt is in LDS buffer 0 and stage kt+1 in set 1.
    load_stage(0, sa0, sb0);
    if (KT > 1) load_stage(1, sa1, sb1);
    store_stage(0, sa0, sb0);
    __syncthreads();
    int kt = 0;
    for (; kt + 3 < KT; kt += 2) {
        load_stage(kt + 2, sa0, sb0);
        __builtin_amdgcn_sched_barrier(0);   // issue the loads before the math
        compute(0);
        store_stage(1, sa1, sb1);
        __syncthreads();
        load_stage(kt + 3, sa1, sb1);
        __builtin_amdgcn_sched_barrier(0);
        compute(1);
        store_stage(0, sa0, sb0);
        __syncthreads();
    }
    // One to three stages remain.
    if (kt + 2 < KT) {
        load_stage(kt + 2, sa0, sb0);
        compute(0);
        store_stage(1, sa1, sb1);
        __syncthreads();
        compute(1);
        store_stage(0, sa0, sb0);
        __syncthreads();
        compute(0);
    } else if (kt + 1 < KT) {
        compute(0);
        store_stage(1, sa1, sb1);
        __syncthreads();
        compute(1);
    } else {
        compute(0);
    }

    // Epilogue.  acc[i][j][e] = C[row][col] with
    // row = m_tile*128 + wm*64 + i*16 + 4*(lane/16) + e, col = ... + j*16 + lane%16.
    const int row0 = m_tile * BM + wm * 64 + (lane >> 4) * 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int row = row0 + i * 16 + e;
            const bool row_ok = row < g.M;
            if (EPI == EPI_SWIGLU) {
#pragma unroll
                for (int jj = 0; jj < 2; ++jj) {
                    const int oc = n_tile * (BN / 2) + wn * 32 + jj * 16 + fr;
                    if (row_ok && oc < g.N) {
                        const float gt = acc[i][2 * jj][e], up = acc[i][2 * jj + 1][e];
                        static_cast<T*>(g.out0)[(int64_t)row * g.N + oc] =
                            from_f32<T>(silu_f(gt) * up);
                    }
                }
            } else if (EPI == EPI_QKV) {
                const int p = row_ok ? g.pos[row] : 0;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int col = n_tile * BN + wn * 64 + j * 16 + fr;
                    const float x = acc[i][j][e];
                    const float partner = __shfl_xor(x, 1, 64);
                    if (!row_ok || col >= g.N) continue;
                    float y = x;
                    T* dst;
                    int64_t off;
                    int seg_col;
                    if (col < g.n0) {
                        dst = static_cast<T*>(g.out0); seg_col = col;
                        off = (int64_t)row * g.n0 + seg_col;
                    } else if (col < g.n0 + g.n1) {
                        dst = static_cast<T*>(g.out1); seg_col = col - g.n0;
                        off = (int64_t)row * g.n1 + seg_col;
                    } else {
                        dst = static_cast<T*>(g.out2); seg_col = col - g.n0 - g.n1;
                        off = (int64_t)row * (g.N - g.n0 - g.n1) + seg_col;
                    }
                    if (col < g.n0 + g.n1) {
                        const int d = seg_col % g.head_dim;
                        const float2 cs = g.rope.tab[(int64_t)p * g.rope.half + (d >> 1)];
                        y = (d & 1) ? partner * cs.y + x * cs.x : x * cs.x - partner * cs.y;
                    }
                    dst[off] = from_f32<T>(y);
                }
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int col = n_tile * BN + wn * 64 + j * 16 + fr;
                    if (!row_ok || col >= g.N) continue;
                    float y = acc[i][j][e];
                    if (EPI == EPI_RESID) {
                        const int rr = g.ridx ? g.ridx[row] : row;
                        y += g.resid[(int64_t)rr * g.N + col];
                    }
                    static_cast<float*>(g.out0)[(int64_t)row * g.N + col] = y;
                }
            }
        }
    }
}

template <typename T, int EPI>
hipError_t launch_t(const GemmArgs& g, hipStream_t s) {
    const int m_tiles = (g.M + BM - 1) / BM;
    const int cols = (EPI == EPI_SWIGLU) ? BN / 2 : BN;
    const int n_tiles = (g.N + cols - 1) / cols;
    hipLaunchKernelGGL((gemm_kernel<T, EPI>), dim3(m_tiles * n_tiles), dim3(kThreads), 0, s, g);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_dtype(int epi, const GemmArgs& g, hipStream_t s) {
    switch (epi) {
        case EPI_STORE_F32: return launch_t<T, EPI_STORE_F32>(g, s);
        case EPI_QKV: return launch_t<T, EPI_QKV>(g, s);
        case EPI_RESID: return launch_t<T, EPI_RESID>(g, s);
        case EPI_SWIGLU: return launch_t<T, EPI_SWIGLU>(g, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gemm(int dtype, int epi, const GemmArgs& g, hipStream_t s) {
    if (g.M <= 0 || g.N <= 0) return hipSuccess;
    const int bk = dtype == BF16 ? Tile<bf16>::BK : Tile<float>::BK;
    if (g.K <= 0 || g.K % bk != 0) return hipErrorInvalidValue;
    if (epi == EPI_QKV && (g.n0 % 16 || g.n1 % 16 || g.head_dim % 2 || !g.pos || !g.rope.tab))
        return hipErrorInvalidValue;
    return dtype == BF16 ? launch_dtype<bf16>(epi, g, s) : launch_dtype<float>(epi, g, s);
}

}  // namespace cb
