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
// wave64s in a 2x2 grid, each wave 64x64: 2x2 32x32x16 MFMA tiles for bf16
// (in register-only loops at one wave per SIMD the 32x32 form runs at about
// 1.95 PFLOP/s, the 16x16x32 form at 1.86 with an 8x8 accumulator grid), 4x4
// 16x16 tiles of 16x16x4 f32 MFMAs for f32.  K advances
// 128 bytes per step (64 bf16 / 32 f32) through double-buffered LDS.  LDS rows
// are unpadded 128-byte rows of eight 16-byte chunks stored at a swizzled
// chunk index (see swz): fragment reads and staging stores are then free of
// bank conflicts (measured: zero conflict cycles, versus a third of LDS
// cycles with 16-byte row padding).  Workgroups are renumbered
// so that consecutive tile ids (the row tiles that share one weight column
// block) land on the same XCD and reuse that XCD's L2.
#include <type_traits>

#include "kernels.h"

namespace cb {

namespace {

constexpr int BM = 128, BN = 128, kThreads = 256;
constexpr int kGroupM = 8;               // row tiles per rasterization group
constexpr int kRowBytes = 128;           // K-slice per stage, bytes per row

template <typename T> struct Tile {
    static constexpr int BK = kRowBytes / (int)sizeof(T);
    static constexpr int LDK = kRowBytes / (int)sizeof(T);                 // LDS row stride
    static constexpr int VEC = 16 / (int)sizeof(T);                        // elems per 16 B
};

// Element offset in a swizzled LDS tile of the 16-byte chunk that holds
// row r, element column c (c a multiple of 16 bytes' worth of elements).
// The chunk index is XORed with a function of the row chosen so that the
// fragment reads are free of bank conflicts (measured with
// SQ_LDS_BANK_CONFLICT): rows 0..15 of one chunk column for the 16x16 f32
// fragments (key: row % 8), rows 0..31 of two chunk columns for the 32x32
// bf16 fragments (key: (row / 2) % 8; row % 8 gives a 2-way conflict there).
template <typename T>
__device__ __forceinline__ int swz(int r, int c) {
    constexpr int VEC = Tile<T>::VEC;
    const int key = sizeof(T) == 2 ? (r >> 1) : r;
    return r * Tile<T>::LDK + (((c / VEC) ^ key) & 7) * VEC;
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

// Output row of q/k/v result row `row`: K and V rows go to kv_rows[row] when
// a row map is given; Q rows stay in result order.
__device__ __forceinline__ int64_t qkv_out_row(const GemmArgs& g, int row, bool kv) {
    return (kv && g.kv_rows) ? (int64_t)g.kv_rows[row] : (int64_t)row;
}

// Maps the hardware workgroup id to a logical tile id such that each XCD
// (ids are dealt round-robin over the 8 XCDs) receives a contiguous range.
__device__ __forceinline__ int xcd_remap(int hw, int total) {
    const int xcd = hw & 7, j = hw >> 3;
    const int base = total >> 3, rem = total & 7;
    return xcd * base + min(xcd, rem) + j;
}

typedef float floatx16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ void mfma32(floatx16& acc, const bf16x8& a, const bf16x8& b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
}

template <typename T> constexpr bool is_bf16() { return sizeof(T) == 2; }

// Row v (0..BN-1) of the block's B tile.  Rows past N are clamped to the
// last row: they only feed output columns that are never stored.  For the
// gate/up launch the tile interleaves gate and up rows so that each wave's
// two MFMA column tiles (32 wide for bf16, pairs of 16 for f32) hold gate
// and up of the same output columns.
template <typename T, int EPI>
__device__ __forceinline__ const T* b_row_ptr(const GemmArgs& g, int v, int n_tile) {
    if (EPI == EPI_SWIGLU) {
        constexpr int W = is_bf16<T>() ? 32 : 16;
        const int oc = min(n_tile * (BN / 2) + (v / (2 * W)) * W + (v % W), g.N - 1);
        return static_cast<const T*>((v & W) ? g.b1 : g.b0) + (int64_t)oc * g.K;
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

// Epilogue of one wave's 64x64 block.  Element e of accumulator (i, j) is
// C[row][col] with
//   bf16: row = wm*64 + i*32 + 8*(e/4) + 4*(lane/32) + e%4, col = wn*64 + j*32 + lane%32
//   f32:  row = wm*64 + i*16 + 4*(lane/16) + e,            col = wn*64 + j*16 + lane%16
// (offsets within the block tile).  One output column per lane.
template <typename T, int EPI, typename Acc, int NT>
__device__ __forceinline__ void epilogue(const GemmArgs& g, const Acc (&acc)[NT][NT], int m_tile,
                                         int n_tile, int wm, int wn, int lane) {
    constexpr int TW = is_bf16<T>() ? 32 : 16;          // MFMA tile width
    constexpr int NE = (int)(sizeof(Acc) / 4);
    const int cl = lane % TW;
#pragma unroll
    for (int i = 0; i < NT; ++i) {
#pragma unroll
        for (int e = 0; e < NE; ++e) {
            const int row = m_tile * BM + wm * 64 + i * TW +
                            (is_bf16<T>() ? 8 * (e / 4) + 4 * (lane / 32) + e % 4
                                          : 4 * (lane / 16) + e);
            const bool row_ok = row < g.M;
            if (EPI == EPI_SWIGLU) {
#pragma unroll
                for (int jj = 0; jj < NT / 2; ++jj) {
                    const int oc = n_tile * (BN / 2) + wn * 32 + jj * TW + cl;
                    if (row_ok && oc < g.N) {
                        const float gt = acc[i][2 * jj][e], up = acc[i][2 * jj + 1][e];
                        static_cast<T*>(g.out0)[(int64_t)row * g.N + oc] =
                            from_f32<T>(silu_f(gt) * up);
                    }
                }
            } else if (EPI == EPI_QKV) {
                const int p = row_ok ? g.pos[row] : 0;
#pragma unroll
                for (int j = 0; j < NT; ++j) {
                    const int col = n_tile * BN + wn * 64 + j * TW + cl;
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
                        off = qkv_out_row(g, row, true) * g.n1 + seg_col;
                    } else {
                        dst = static_cast<T*>(g.out2); seg_col = col - g.n0 - g.n1;
                        off = qkv_out_row(g, row, true) * (g.N - g.n0 - g.n1) + seg_col;
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
                for (int j = 0; j < NT; ++j) {
                    const int col = n_tile * BN + wn * 64 + j * TW + cl;
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
__global__ __launch_bounds__(kThreads, 2) void gemm_kernel(GemmArgs g) {
    using TL = Tile<T>;
    constexpr int BK = TL::BK, LDK = TL::LDK, VEC = TL::VEC;
    __shared__ __attribute__((aligned(16))) T sA[2][BM * LDK];
    __shared__ __attribute__((aligned(16))) T sB[2][BN * LDK];

    const int m_tiles = (g.M + BM - 1) / BM;
    const int n_cols_per_tile = (EPI == EPI_SWIGLU) ? BN / 2 : BN;
    const int n_tiles = (g.N + n_cols_per_tile - 1) / n_cols_per_tile;
    // Logical tiles in groups of kGroupM row tiles: the workgroups resident
    // on one XCD at a time cover a kGroupM x (64 / kGroupM) patch of output
    // tiles, so each K slice of A and of B they load is shared in that XCD's
    // L2 by several of them.
    const int tile = xcd_remap(blockIdx.x, m_tiles * n_tiles);
    const int group = tile / (kGroupM * n_tiles);
    const int first_m = group * kGroupM;
    const int gm = min(m_tiles - first_m, kGroupM);
    const int in_group = tile - group * kGroupM * n_tiles;
    const int m_tile = first_m + in_group % gm, n_tile = in_group / gm;

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

    // Accumulators: bf16 2x2 32x32 tiles, f32 4x4 16x16 tiles (64 floats per lane).
    constexpr int NT = is_bf16<T>() ? 2 : 4;
    using Acc = typename std::conditional<is_bf16<T>(), floatx16, floatx4>::type;
    Acc acc[NT][NT];
#pragma unroll
    for (int i = 0; i < NT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
            for (int e = 0; e < (int)(sizeof(Acc) / 4); ++e) acc[i][j][e] = 0.f;

    const int KT = g.K / BK;
    auto compute = [&](int buf) {
        if constexpr (is_bf16<T>()) {
            // lane l: row l % 32 of the tile, reduction elements 8 (l / 32) + 0..7
            const int fr = lane & 31, fk = (lane >> 5) * 8;
#pragma unroll
            for (int ks = 0; ks < BK; ks += 16) {
                bf16x8 af[2], bfr[2];
#pragma unroll
                for (int i = 0; i < 2; ++i)
                    af[i] = *reinterpret_cast<const bf16x8*>(
                        &sA[buf][swz<T>(wm * 64 + i * 32 + fr, ks + fk)]);
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    bfr[j] = *reinterpret_cast<const bf16x8*>(
                        &sB[buf][swz<T>(wn * 64 + j * 32 + fr, ks + fk)]);
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j) mfma32(acc[i][j], af[i], bfr[j]);
            }
        } else {
            const int fr = lane & 15, fk = (lane >> 4) * 8;
#pragma unroll
            for (int ks = 0; ks < BK; ks += 32) {
                Frag<T> af[4], bfr[4];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    af[i] = lds_frag<T>(sA[buf], wm * 64 + i * 16 + fr, ks + fk);
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    bfr[j] = lds_frag<T>(sB[buf], wn * 64 + j * 16 + fr, ks + fk);
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j) mfma16(acc[i][j], af[i], bfr[j]);
            }
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

    epilogue<T, EPI>(g, acc, m_tile, n_tile, wm, wn, lane);
}

// ---------------------------------------------------------------------------
// bf16 path with direct-to-LDS loads (the four-wave 128x128 kernel above
// remains the f32 path and the fallback for K not a multiple of 64).  Each
// buffer_load ... lds of a wave
// writes 64 x 16 B to consecutive LDS bytes: the 8 lanes of one tile row
// fetch that row's 16-byte chunks in swizzled order, so the LDS image is the
// same conflict-free layout as above without staging registers or LDS store
// instructions.  S stages of A and B (32 KB each) form a ring: while stage kt
// is multiplied out, stages kt+1 .. kt+S-1 are in flight.  Rows past M (or
// past the end of a weight matrix) lie outside the buffer resource's range
// and read as zero.  Fragments of the next 16-wide K step are read from LDS
// while the current step's MFMAs run.
typedef int i32x4 __attribute__((ext_vector_type(4)));

// Raw buffer descriptor: base address, stride 0, range `bytes` (uniform
// values; read from the first lane so the descriptor lives in SGPRs).
__device__ __forceinline__ i32x4 make_rsrc(const void* base, int bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    return i32x4{__builtin_amdgcn_readfirstlane((int)(uint32_t)a),
                 __builtin_amdgcn_readfirstlane((int)((a >> 32) & 0xFFFF)),
                 __builtin_amdgcn_readfirstlane(bytes), 0x00020000};
}

// 16 bytes per lane from buffer offset voff + soff into LDS at m0 + 16 * lane.
// Issued as inline assembly so that the compiler's memory model does not see
// a store to LDS (it would otherwise wait for every outstanding copy before
// any LDS read); completion is tracked by the explicit vmcnt waits below and
// the "memory" clobber keeps LDS reads from moving across the copy.  The
// hazard recognizer cannot see inside the statement: the s_nop is the one
// wait state the load needs after the scalar write of M0.  A descriptor or
// offset word written by v_readfirstlane needs five before the load; the
// kernels make their byte counts scalar (uniform_int) once, before the K
// loops that rebuild descriptors, so that no such write sits near a copy.
__device__ __forceinline__ void dma16(i32x4 rsrc, int voff, int soff, uint32_t m0) {
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
                 :
                 : "v"(voff), "s"(rsrc), "s"(soff), "{m0}"(m0)
                 : "memory");
}

// A value the whole wave agrees on, held in a scalar register from here on
// (the descriptors built from it in a K loop then need no v_readfirstlane).
__device__ __forceinline__ int uniform_int(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Byte range of the wave's 32-row slice: rows left (clamped to 0..32) x row bytes.
__device__ __forceinline__ int slice_bytes(int64_t rows_left, int row_bytes) {
    const int r = rows_left < 0 ? 0 : (rows_left > 32 ? 32 : (int)rows_left);
    return r * row_bytes;
}

// s_waitcnt with only the vector-memory counter limited to n (n < 64).
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Epilogue of the direct-to-LDS kernels, staged through LDS so that global
// traffic is row-contiguous: every wave writes (or adds) its 64x64 fp32
// block into a row-major 128 x (128 + 8) tile (the 8-float pad puts the two
// half-waves of a store on disjoint banks), then each thread finishes 4
// consecutive columns of 128 / (NTH / 32) rows: one 16-byte residual /
// RoPE-table load and one vector store per row.  `lds` is free, 16-byte
// aligned memory of >= 128*136 floats.
constexpr int kEpiLd = BN + 8;
template <bool ADD>
__device__ __forceinline__ void stage_acc(const floatx16 (&acc)[2][2], int wm, int wn, int lane,
                                          float* lds) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int r = wm * 64 + i * 32 + 8 * (e / 4) + 4 * (lane / 32) + e % 4;
                const int c = wn * 64 + j * 32 + lane % 32;
                if (ADD) lds[r * kEpiLd + c] += acc[i][j][e];
                else lds[r * kEpiLd + c] = acc[i][j][e];
            }
}

template <int EPI, int NTH>
__device__ __forceinline__ void epilogue_finish(const GemmArgs& g, int m_tile, int n_tile,
                                                const float* lds) {
    constexpr int RS = NTH / 32;                  // rows per pass
    constexpr int NP = BM / RS;                   // passes
    const int t = threadIdx.x;
    const int cc = (t % 32) * 4;                  // first of this thread's 4 columns
    const int row0 = m_tile * BM + t / 32;
    if (EPI == EPI_SWIGLU) {
        // output columns oc, oc+1 of the tile's 64: gate at LDS column
        // (oc/32)*64 + oc%32, up 32 columns further
        const int oc = (t % 32) * 2;
        const int gc = (oc / 32) * 64 + oc % 32;
        const int col = n_tile * (BN / 2) + oc;
#pragma unroll 4
        for (int p = 0; p < NP; ++p) {
            const int rl = t / 32 + RS * p, row = row0 + RS * p;
            if (row >= g.M) break;
            const float2 gt = *reinterpret_cast<const float2*>(&lds[rl * kEpiLd + gc]);
            const float2 up = *reinterpret_cast<const float2*>(&lds[rl * kEpiLd + gc + 32]);
            bf16* dst = static_cast<bf16*>(g.out0) + (int64_t)row * g.N + col;
            if (col + 1 < g.N) {
                typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
                *reinterpret_cast<bf16x2*>(dst) =
                    bf16x2{static_cast<bf16>(silu_f(gt.x) * up.x), static_cast<bf16>(silu_f(gt.y) * up.y)};
            } else if (col < g.N) {
                dst[0] = static_cast<bf16>(silu_f(gt.x) * up.x);
            }
        }
        return;
    }
    const int col = n_tile * BN + cc;
    if (EPI == EPI_QKV) {
        // the tile lies in one of q, k, v (checked by the launcher)
        const int c0 = n_tile * BN;
        bf16* base;
        int width, local;
        bool rope, kv = true;
        if (c0 < g.n0) { base = static_cast<bf16*>(g.out0); width = g.n0; local = col; rope = true; kv = false; }
        else if (c0 < g.n0 + g.n1) {
            base = static_cast<bf16*>(g.out1); width = g.n1; local = col - g.n0; rope = true;
        } else {
            base = static_cast<bf16*>(g.out2); width = g.N - g.n0 - g.n1; local = col - g.n0 - g.n1;
            rope = false;
        }
        const int hd = local % g.head_dim;         // multiple of 4: pairs (hd, hd+1), (hd+2, hd+3)
        // positions and output rows of all the thread's rows, then their
        // RoPE factors, before the first store (two dependent round trips)
        int pr[NP], orow[NP];
        floatx4 cs[NP];
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const int row = row0 + RS * p;
            pr[p] = row < g.M && rope ? g.pos[row] : 0;
            orow[p] = row < g.M ? (int)qkv_out_row(g, row, kv) : 0;
        }
        if (rope) {
#pragma unroll
            for (int p = 0; p < NP; ++p)
                cs[p] = *reinterpret_cast<const floatx4*>(
                    &g.rope.tab[(int64_t)pr[p] * g.rope.half + (hd >> 1)]);
        }
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const int rl = t / 32 + RS * p, row = row0 + RS * p;
            if (row >= g.M) break;
            const floatx4 x = *reinterpret_cast<const floatx4*>(&lds[rl * kEpiLd + cc]);
            floatx4 y = x;
            if (rope) {
                y[0] = x[0] * cs[p][0] - x[1] * cs[p][1];
                y[1] = x[0] * cs[p][1] + x[1] * cs[p][0];
                y[2] = x[2] * cs[p][2] - x[3] * cs[p][3];
                y[3] = x[2] * cs[p][3] + x[3] * cs[p][2];
            }
            *reinterpret_cast<bf16x4*>(base + (int64_t)orow[p] * width + local) =
                bf16x4{static_cast<bf16>(y[0]), static_cast<bf16>(y[1]), static_cast<bf16>(y[2]),
                       static_cast<bf16>(y[3])};
        }
        return;
    }
    // STORE_F32 / RESID: fp32 rows; vector path when the row length allows
    const bool vec = (g.N % 4) == 0;
    if (EPI == EPI_RESID && vec && col + 3 < g.N) {
        // residual row indices of all the thread's rows, then the residual
        // values, before the first store (two dependent round trips)
        int rr[NP];
        floatx4 rv[NP];
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const int row = row0 + RS * p;
            rr[p] = row < g.M ? (g.ridx ? g.ridx[row] : row) : -1;
        }
#pragma unroll
        for (int p = 0; p < NP; ++p)
            rv[p] = rr[p] >= 0 ? *reinterpret_cast<const floatx4*>(g.resid + (int64_t)rr[p] * g.N + col)
                               : floatx4{};
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const int rl = t / 32 + RS * p, row = row0 + RS * p;
            if (row >= g.M) break;
            const floatx4 y = *reinterpret_cast<const floatx4*>(&lds[rl * kEpiLd + cc]) + rv[p];
            *reinterpret_cast<floatx4*>(static_cast<float*>(g.out0) + (int64_t)row * g.N + col) = y;
        }
        return;
    }
#pragma unroll 4
    for (int p = 0; p < NP; ++p) {
        const int rl = t / 32 + RS * p, row = row0 + RS * p;
        if (row >= g.M) break;
        floatx4 y = *reinterpret_cast<const floatx4*>(&lds[rl * kEpiLd + cc]);
        float* dst = static_cast<float*>(g.out0) + (int64_t)row * g.N + col;
        const float* res = nullptr;
        if (EPI == EPI_RESID)
            res = g.resid + (int64_t)(g.ridx ? g.ridx[row] : row) * g.N + col;
        if (vec && col + 3 < g.N) {
            if (EPI == EPI_RESID) y += *reinterpret_cast<const floatx4*>(res);
            *reinterpret_cast<floatx4*>(dst) = y;
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k)
                if (col + k < g.N) dst[k] = y[k] + (EPI == EPI_RESID ? res[k] : 0.f);
        }
    }
}



// The direct-to-LDS kernel: a 128x128 tile per workgroup of eight waves, two
// per SIMD, and a ring of S x 32 KB stages (S = 5 fills the 160 KB of LDS:
// 3-4 stages in flight; against 4 stages, 2% off the 7B step).  K need not
// be a multiple of S: the stages past the last full turn run in a tail.  Waves w and w + 4 compute the same 64x64
// block over different halves of every K stage (16-wide steps 0-1 and 2-3),
// so while one waits for fragments or at the barrier the other keeps the
// SIMD's matrix unit busy; the two partial blocks are added in LDS before
// the epilogue.  LDS bytes per MFMA are those of four waves of 64x64 over
// whole stages, and each wave issues 4 of the stage's 32 copies.  Measured
// on MI355X against that four-wave form: 832 x 4096 x 11008 955 vs 890
// TFLOP/s, 832 x 22016 x 4096 788 vs 761; one wave per SIMD left the matrix
// units idle in every s_waitcnt and barrier (40% busy).  Also measured and
// dropped: register-staged copies into four LDS buffers with two register
// sets (five stages in flight), on the 7B step O 1.42 -> 1.53 ms and down
// 3.31 -> 3.43 ms per step.
constexpr int kThreads8 = 512;
template <int EPI, int S>
__global__ __launch_bounds__(kThreads8, 1) void gemm_dma8_kernel(GemmArgs g) {
    static_assert(S >= 3 && S <= 5, "stages");
    constexpr int BK = 64;                    // bf16 per stage row (128 B)
    constexpr int HALF = BM * BK;             // elements of the A (then B) part of a stage
    constexpr int DPS = 4;                    // copies per wave per stage
    __shared__ __attribute__((aligned(16))) bf16 sm0[S * 2 * HALF];   // stage ring
    auto stage = [&](auto ic) -> bf16* { return sm0 + decltype(ic)::value * 2 * HALF; };

    const int m_tiles = (g.M + BM - 1) / BM;
    const int n_cols_per_tile = (EPI == EPI_SWIGLU) ? BN / 2 : BN;
    const int n_tiles = (g.N + n_cols_per_tile - 1) / n_cols_per_tile;
    const int tile = xcd_remap(blockIdx.x, m_tiles * n_tiles);
    // rasterization groups: 4 row tiles for q/k/v (measured 2% faster than 8
    // there, 3% slower for gate/up)
    constexpr int GM = EPI == EPI_QKV ? 4 : kGroupM;
    const int group = tile / (GM * n_tiles);
    const int first_m = group * GM;
    const int gm = min(m_tiles - first_m, GM);
    const int in_group = tile - group * GM * n_tiles;
    const int m_tile = first_m + in_group % gm, n_tile = in_group / gm;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar descriptors
    const int kh = wave >> 2;                 // which half of each K stage
    const int wm = (wave >> 1) & 1, wn = wave & 1;
    const int Kb = g.K * 2;                   // bytes per row

    // This wave copies rows 16*wave .. +15 of the A tile and of the B tile.
    const bf16* a_base = static_cast<const bf16*>(g.a) + ((int64_t)m_tile * BM + 16 * wave) * g.K;
    const int64_t a_left = (int64_t)g.M - (int64_t)m_tile * BM - 16 * wave;
    const bf16* b_base;
    int64_t b_left;
    if (EPI == EPI_SWIGLU) {
        // B rows 32 s .. 32 s + 31 of the tile: gate (s even) or up (s odd)
        // rows of output columns n_tile*64 + (s/2)*32 ..; this wave's 16 rows
        // are the (wave % 2)-th half of slice s = wave / 2
        const int s = wave >> 1;
        const int oc0 = n_tile * (BN / 2) + (s >> 1) * 32 + (wave & 1) * 16;
        b_base = static_cast<const bf16*>((s & 1) ? g.b1 : g.b0) + (int64_t)oc0 * g.K;
        b_left = g.N - oc0;
    } else if (EPI == EPI_QKV) {
        const int c0 = n_tile * BN;
        const void* mat;
        int local, rows;
        if (c0 < g.n0) { mat = g.b0; local = c0; rows = g.n0; }
        else if (c0 < g.n0 + g.n1) { mat = g.b1; local = c0 - g.n0; rows = g.n1; }
        else { mat = g.b2; local = c0 - g.n0 - g.n1; rows = g.N - g.n0 - g.n1; }
        b_base = static_cast<const bf16*>(mat) + ((int64_t)local + 16 * wave) * g.K;
        b_left = rows - local - 16 * wave;
    } else {
        b_base = static_cast<const bf16*>(g.b0) + ((int64_t)n_tile * BN + 16 * wave) * g.K;
        b_left = g.N - (int64_t)n_tile * BN - 16 * wave;
    }
    const int a_bytes = uniform_int((int)(a_left < 0 ? 0 : (a_left > 16 ? 16 : a_left)) * Kb);
    const int b_bytes = uniform_int((int)(b_left < 0 ? 0 : (b_left > 16 ? 16 : b_left)) * Kb);

    // Lane i fetches row i/8 (of 8) at LDS slot i%8, i.e. global chunk
    // slot ^ key(row), key(r) = (r/2) % 8; the second 8 rows of the wave's
    // 16 differ in key by 4.
    const int r8 = lane >> 3, slot = lane & 7;
    const int v_even = r8 * Kb + ((slot ^ (r8 >> 1)) & 7) * 16;
    const int v_odd = r8 * Kb + ((slot ^ ((r8 >> 1) + 4)) & 7) * 16;

    const int KT = g.K / BK;
    auto issue = [&](int kt, bf16* buf) {
        const bool live = kt < KT;            // stages past the end read nothing
        const i32x4 xa = make_rsrc(a_base, live ? a_bytes : 0);
        const i32x4 xb = make_rsrc(b_base, live ? b_bytes : 0);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int vo = j ? v_odd : v_even;
            const int so = kt * 128 + 8 * j * Kb;
            const uint32_t da = (uint32_t)reinterpret_cast<uintptr_t>(buf + (16 * wave + 8 * j) * BK);
            dma16(xa, vo, so, da);
            dma16(xb, vo, so, da + HALF * 2);
        }
    };

    floatx16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    const int fr = lane & 31, fk = (lane >> 5) * 8;
    const int ka = 32 * kh, kb2 = 32 * kh + 16;    // this wave's two 16-wide steps
    auto read_frags = [&](const bf16* buf, int ks, bf16x8 (&fa)[2], bf16x8 (&fb)[2]) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
            fa[i] = *reinterpret_cast<const bf16x8*>(&buf[swz<bf16>(wm * 64 + i * 32 + fr, ks + fk)]);
#pragma unroll
        for (int j = 0; j < 2; ++j)
            fb[j] = *reinterpret_cast<const bf16x8*>(
                &buf[HALF + swz<bf16>(wn * 64 + j * 32 + fr, ks + fk)]);
    };
    auto mfma_step = [&](const bf16x8 (&fa)[2], const bf16x8 (&fb)[2]) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) mfma32(acc[i][j], fa[i], fb[j]);
    };
    auto interleave = [&]() {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
        }
    };
    bf16x8 fa0[2], fb0[2], fa1[2], fb1[2];
    // One K stage out of buffer I (this wave's first fragments already in
    // fa0/fb0): the second step's fragments are read under the first step's
    // MFMAs; the barrier publishing stage kt+1 follows; the copies of stage
    // kt+S-1 go out between the second step's MFMAs, and the next stage's
    // first fragments are read last.
    auto step = [&](auto ic, int kt) {
        constexpr int I = decltype(ic)::value;
        const bf16* buf = stage(ic);
        read_frags(buf, kb2, fa1, fb1);
        mfma_step(fa0, fb0);
        interleave();
        __builtin_amdgcn_sched_barrier(0);
        wait_vm<(S - 3) * DPS>();
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        {
            const int kn = kt + S - 1;
            bf16* dst = stage(std::integral_constant<int, (I + S - 1) % S>{});
            const bool live = kn < KT;
            const i32x4 xa = make_rsrc(a_base, live ? a_bytes : 0);
            const i32x4 xb = make_rsrc(b_base, live ? b_bytes : 0);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                mfma32(acc[t >> 1][t & 1], fa1[t >> 1], fb1[t & 1]);
                if (t < 2) {
                    const int vo = t ? v_odd : v_even;
                    const int so = kn * 128 + 8 * t * Kb;
                    const uint32_t da =
                        (uint32_t)reinterpret_cast<uintptr_t>(dst + (16 * wave + 8 * t) * BK);
                    dma16(xa, vo, so, da);
                    dma16(xb, vo, so, da + HALF * 2);
                }
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        // (after the last stage this reads a buffer that is never used)
        read_frags(stage(std::integral_constant<int, (I + 1) % S>{}), ka, fa0, fb0);
    };
    issue(0, stage(std::integral_constant<int, 0>{}));
    issue(1, stage(std::integral_constant<int, 1>{}));
    if constexpr (S > 3) issue(2, stage(std::integral_constant<int, 2>{}));
    if constexpr (S > 4) issue(3, stage(std::integral_constant<int, 3>{}));
    wait_vm<(S - 2) * DPS>();
    __builtin_amdgcn_s_barrier();
    read_frags(sm0, ka, fa0, fb0);
    int kt = 0;
    for (; kt + S <= KT; kt += S) {
        step(std::integral_constant<int, 0>{}, kt);
        step(std::integral_constant<int, 1>{}, kt + 1);
        step(std::integral_constant<int, 2>{}, kt + 2);
        if constexpr (S > 3) step(std::integral_constant<int, 3>{}, kt + 3);
        if constexpr (S > 4) step(std::integral_constant<int, 4>{}, kt + 4);
    }
    if (kt < KT) step(std::integral_constant<int, 0>{}, kt);
    if (kt + 1 < KT) step(std::integral_constant<int, 1>{}, kt + 1);
    if constexpr (S > 3) if (kt + 2 < KT) step(std::integral_constant<int, 2>{}, kt + 2);
    if constexpr (S > 4) if (kt + 3 < KT) step(std::integral_constant<int, 3>{}, kt + 3);
    // the trailing copies (empty ranges) still write LDS: let them land, and
    // let every wave finish its last fragment reads, before reusing LDS
    wait_vm<0>();
    __syncthreads();
    static_assert(S * 2 * HALF * 2 >= BM * kEpiLd * 4, "epilogue staging fits the stage ring");
    float* lds = reinterpret_cast<float*>(sm0);
    if (kh == 1) stage_acc<false>(acc, wm, wn, lane, lds);
    __syncthreads();
    if (kh == 0) stage_acc<true>(acc, wm, wn, lane, lds);
    __syncthreads();
    epilogue_finish<EPI, kThreads8>(g, m_tile, n_tile, lds);
}

template <typename T, int EPI>
hipError_t launch_t(const GemmArgs& g, hipStream_t s) {
    const int m_tiles = (g.M + BM - 1) / BM;
    const int cols = (EPI == EPI_SWIGLU) ? BN / 2 : BN;
    const int n_tiles = (g.N + cols - 1) / cols;
    hipLaunchKernelGGL((gemm_kernel<T, EPI>), dim3(m_tiles * n_tiles), dim3(kThreads), 0, s, g);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Large tiles for large products: 256x256 per workgroup, four waves of
// 128x128 (4x4 MFMA tiles of 32x32x16), K stages of 32 (64-byte LDS rows).
// Per K element this halves both the L2 -> LDS traffic and the LDS fragment
// reads of the 128x128 kernel, which bound that kernel on large shapes.
// LDS rows are 4 chunks of 16 bytes stored at chunk ^ ((row / 4) % 4) (zero
// bank conflicts for 32x32 fragment reads, measured).  A 5-stage ring (all
// 160 KB) filled in pairs of stages that share 128-byte lines (7B step
// 18.61 -> 18.47 ms, 13B 68.8 -> 67.3 ms against a 4-stage ring filled one
// stage per step), a mid-stage barrier and a staged epilogue, as in the
// 128x128 kernel; the epilogue goes through LDS in four passes of 64 rows.
constexpr int BBM = 256, BBN = 256, BBK = 32, kBigStages = 5;
constexpr int kBigLd = BBN + 8;

__device__ __forceinline__ int big_swz(int r, int chunk) {     // byte offset in a stage half
    return r * 64 + ((chunk ^ (r >> 2)) & 3) * 16;
}

template <int EPI>
__device__ __forceinline__ void big_epilogue(const GemmArgs& g, const floatx16 (&acc)[4][4],
                                             int m_tile, int n_tile, int wm, int wn, int lane,
                                             float* lds) {
    const int t = threadIdx.x;
#pragma unroll
    for (int q = 0; q < 4; ++q) {                 // rows 64q .. 64q+63 of the tile
        if (wm == q / 2) {
#pragma unroll
            for (int ii = 0; ii < 2; ++ii) {
                const int i = 2 * (q % 2) + ii;
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int r = ii * 32 + 8 * (e / 4) + 4 * (lane / 32) + e % 4;
                        const int c = wn * 128 + j * 32 + lane % 32;
                        lds[r * kBigLd + c] = acc[i][j][e];
                    }
            }
        }
        __syncthreads();
        const int row0 = m_tile * BBM + 64 * q + t / 64;
        if (EPI == EPI_SWIGLU) {
            const int oc = (t % 64) * 2;               // of the tile's 128 output columns
            const int gc = (oc / 32) * 64 + oc % 32;
            const int col = n_tile * (BBN / 2) + oc;
#pragma unroll 4
            for (int p = 0; p < 16; ++p) {
                const int rl = t / 64 + 4 * p, row = row0 + 4 * p;
                if (row < g.M) {
                    const float2 gt = *reinterpret_cast<const float2*>(&lds[rl * kBigLd + gc]);
                    const float2 up = *reinterpret_cast<const float2*>(&lds[rl * kBigLd + gc + 32]);
                    bf16* dst = static_cast<bf16*>(g.out0) + (int64_t)row * g.N + col;
                    if (col + 1 < g.N) {
                        typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
                        *reinterpret_cast<bf16x2*>(dst) = bf16x2{
                            static_cast<bf16>(silu_f(gt.x) * up.x), static_cast<bf16>(silu_f(gt.y) * up.y)};
                    } else if (col < g.N) {
                        dst[0] = static_cast<bf16>(silu_f(gt.x) * up.x);
                    }
                }
            }
        } else {
            const int cc = (t % 64) * 4;
            const int col = n_tile * BBN + cc;
            if (EPI == EPI_QKV) {
                const int c0 = n_tile * BBN;
                bf16* base;
                int width, local;
                bool rope, kv = true;
                if (c0 < g.n0) { base = static_cast<bf16*>(g.out0); width = g.n0; local = col; rope = true; kv = false; }
                else if (c0 < g.n0 + g.n1) {
                    base = static_cast<bf16*>(g.out1); width = g.n1; local = col - g.n0; rope = true;
                } else {
                    base = static_cast<bf16*>(g.out2); width = g.N - g.n0 - g.n1;
                    local = col - g.n0 - g.n1; rope = false;
                }
                const int hd = local % g.head_dim;
                // positions and output rows of the thread's 16 rows, then
                // their RoPE factors, before the first store
                int pr[16], orow[16];
                floatx4 cs[16];
#pragma unroll
                for (int p = 0; p < 16; ++p) {
                    const int row = row0 + 4 * p;
                    pr[p] = row < g.M && rope ? g.pos[row] : 0;
                    orow[p] = row < g.M ? (int)qkv_out_row(g, row, kv) : 0;
                }
                if (rope) {
#pragma unroll
                    for (int p = 0; p < 16; ++p)
                        cs[p] = *reinterpret_cast<const floatx4*>(
                            &g.rope.tab[(int64_t)pr[p] * g.rope.half + (hd >> 1)]);
                }
#pragma unroll
                for (int p = 0; p < 16; ++p) {
                    const int rl = t / 64 + 4 * p, row = row0 + 4 * p;
                    if (row < g.M) {
                        const floatx4 x = *reinterpret_cast<const floatx4*>(&lds[rl * kBigLd + cc]);
                        floatx4 y = x;
                        if (rope) {
                            y[0] = x[0] * cs[p][0] - x[1] * cs[p][1];
                            y[1] = x[0] * cs[p][1] + x[1] * cs[p][0];
                            y[2] = x[2] * cs[p][2] - x[3] * cs[p][3];
                            y[3] = x[2] * cs[p][3] + x[3] * cs[p][2];
                        }
                        *reinterpret_cast<bf16x4*>(base + (int64_t)orow[p] * width + local) =
                            bf16x4{static_cast<bf16>(y[0]), static_cast<bf16>(y[1]),
                                   static_cast<bf16>(y[2]), static_cast<bf16>(y[3])};
                    }
                }
            } else {
                const bool vec = (g.N % 4) == 0;
                if (EPI == EPI_RESID && vec && col + 3 < g.N) {
                    // residual row indices of the thread's 16 rows, then
                    // the residual values, before the first store
                    int rr[16];
                    floatx4 rv[16];
#pragma unroll
                    for (int p = 0; p < 16; ++p) {
                        const int row = row0 + 4 * p;
                        rr[p] = row < g.M ? (g.ridx ? g.ridx[row] : row) : -1;
                    }
#pragma unroll
                    for (int p = 0; p < 16; ++p)
                        rv[p] = rr[p] >= 0
                                    ? *reinterpret_cast<const floatx4*>(g.resid + (int64_t)rr[p] * g.N + col)
                                    : floatx4{};
#pragma unroll
                    for (int p = 0; p < 16; ++p) {
                        const int rl = t / 64 + 4 * p, row = row0 + 4 * p;
                        if (row < g.M)
                            *reinterpret_cast<floatx4*>(static_cast<float*>(g.out0) + (int64_t)row * g.N + col) =
                                *reinterpret_cast<const floatx4*>(&lds[rl * kBigLd + cc]) + rv[p];
                    }
                } else {
#pragma unroll 4
                    for (int p = 0; p < 16; ++p) {
                        const int rl = t / 64 + 4 * p, row = row0 + 4 * p;
                        if (row < g.M) {
                            floatx4 y = *reinterpret_cast<const floatx4*>(&lds[rl * kBigLd + cc]);
                            float* dst = static_cast<float*>(g.out0) + (int64_t)row * g.N + col;
                            const float* res = nullptr;
                            if (EPI == EPI_RESID)
                                res = g.resid + (int64_t)(g.ridx ? g.ridx[row] : row) * g.N + col;
                            if (vec && col + 3 < g.N) {
                                if (EPI == EPI_RESID) y += *reinterpret_cast<const floatx4*>(res);
                                *reinterpret_cast<floatx4*>(dst) = y;
                            } else {
#pragma unroll
                                for (int k = 0; k < 4; ++k)
                                    if (col + k < g.N) dst[k] = y[k] + (EPI == EPI_RESID ? res[k] : 0.f);
                            }
                        }
                    }
                }
            }
        }
        __syncthreads();
    }
}

// The same tile with a 4-stage ring filled one stage per step, fully
// unrolled with compile-time slots (K a multiple of 128).  Faster than the
// paired 5-stage kernel when many rounds of workgroups reuse the weights
// (the 32-request batch: 416.6 vs 428.3 ms per step); the paired kernel wins
// at 4 rounds or fewer, where the weights stream from HBM.
constexpr int kBig4Stages = 4;

template <int EPI>
__global__ __launch_bounds__(kThreads, 1) void gemm_big4_kernel(GemmArgs g) {
    constexpr int S = kBig4Stages;
    constexpr int HALF_B = BBM * BBK * 2;         // bytes of the A (then B) part of a stage
    constexpr int STAGE_B = 2 * HALF_B;
    __shared__ __attribute__((aligned(16))) char smem[S * STAGE_B];   // 128 KB
    const uint32_t lds0 = (uint32_t)reinterpret_cast<uintptr_t>(smem);

    const int m_tiles = (g.M + BBM - 1) / BBM;
    const int n_cols_per_tile = (EPI == EPI_SWIGLU) ? BBN / 2 : BBN;
    const int n_tiles = (g.N + n_cols_per_tile - 1) / n_cols_per_tile;
    const int tile = xcd_remap(blockIdx.x, m_tiles * n_tiles);
    const int group = tile / (kGroupM * n_tiles);
    const int first_m = group * kGroupM;
    const int gm = min(m_tiles - first_m, kGroupM);
    const int in_group = tile - group * kGroupM * n_tiles;
    const int m_tile = first_m + in_group % gm, n_tile = in_group / gm;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int Kb = g.K * 2;

    // This wave copies rows 64*wave .. +63 of the A tile and of the B tile.
    const bf16* a_base = static_cast<const bf16*>(g.a) + ((int64_t)m_tile * BBM + 64 * wave) * g.K;
    const int64_t a_rows = (int64_t)g.M - (int64_t)m_tile * BBM - 64 * wave;
    const int a_bytes = uniform_int((a_rows < 0 ? 0 : (a_rows > 64 ? 64 : (int)a_rows)) * Kb);
    // B: two 32-row halves (for gate/up they come from different matrices)
    const bf16* b_base[2];
    int b_bytes[2];
    if (EPI == EPI_SWIGLU) {
        const int oc0 = n_tile * (BBN / 2) + wave * 32;
        const int64_t rows = g.N - oc0;
        const int by = uniform_int((rows < 0 ? 0 : (rows > 32 ? 32 : (int)rows)) * Kb);
        b_base[0] = static_cast<const bf16*>(g.b0) + (int64_t)oc0 * g.K;
        b_base[1] = static_cast<const bf16*>(g.b1) + (int64_t)oc0 * g.K;
        b_bytes[0] = b_bytes[1] = by;
    } else {
        const void* mat = g.b0;
        int64_t local = (int64_t)n_tile * BBN, rows = g.N;
        if (EPI == EPI_QKV) {
            const int c0 = n_tile * BBN;
            if (c0 < g.n0) { mat = g.b0; local = c0; rows = g.n0; }
            else if (c0 < g.n0 + g.n1) { mat = g.b1; local = c0 - g.n0; rows = g.n1; }
            else { mat = g.b2; local = c0 - g.n0 - g.n1; rows = g.N - g.n0 - g.n1; }
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int64_t r0 = local + 64 * wave + 32 * h;
            const int64_t left = rows - r0;
            b_base[h] = static_cast<const bf16*>(mat) + r0 * g.K;
            b_bytes[h] = uniform_int((left < 0 ? 0 : (left > 32 ? 32 : (int)left)) * Kb);
        }
    }
    // Lane i copies row i/4 (of 16) into LDS slot i%4: global chunk slot ^ key,
    // key = (row/4) % 4 (the same for every 16-row block of the wave).
    const int r16 = lane >> 2, slot = lane & 3;
    const int voff = r16 * Kb + ((slot ^ (r16 >> 2)) & 3) * 16;
    const int KT = g.K / BBK;

    // Copies of stage kt into ring slot `buf`, 8 per wave; with `t` the
    // copies are spread over the MFMA steps (see big_copy_part).
    auto copy_part = [&](int kt, int buf, int part) {       // part 0..7
        const bool live = kt < KT;
        const int j = part & 3;                             // 16-row block within the 64
        const uint32_t dst = lds0 + buf * STAGE_B + (part < 4 ? 0 : HALF_B) + (64 * wave + 16 * j) * 64;
        const int so = kt * 64 + 16 * (j & 1) * Kb;
        if (part < 4) {
            const i32x4 r = make_rsrc(a_base, live ? a_bytes : 0);
            dma16(r, voff, kt * 64 + 16 * j * Kb, dst);
        } else {
            const int h = j >> 1;
            const i32x4 r = make_rsrc(b_base[h], live ? b_bytes[h] : 0);
            dma16(r, voff, so, dst);
        }
    };

    floatx16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    const int fr = lane & 31, fg = lane >> 5;
    auto read_frags = [&](int buf, int ks, bf16x8 (&fa)[4], bf16x8 (&fb)[4]) {
        const char* st = smem + buf * STAGE_B;
        const int chunk = ks * 2 + fg;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            fa[i] = *reinterpret_cast<const bf16x8*>(st + big_swz(wm * 128 + i * 32 + fr, chunk));
#pragma unroll
        for (int j = 0; j < 4; ++j)
            fb[j] = *reinterpret_cast<const bf16x8*>(st + HALF_B + big_swz(wn * 128 + j * 32 + fr, chunk));
    };
    // 16 MFMAs, with the 8 fragment reads of the next step one per two MFMAs.
    auto mfma_all = [&](const bf16x8 (&fa)[4], const bf16x8 (&fb)[4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) mfma32(acc[i][j], fa[i], fb[j]);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
    };
    bf16x8 fa0[4], fb0[4], fa1[4], fb1[4];
    auto step = [&](int kt, int buf) {
        read_frags(buf, 1, fa1, fb1);
        mfma_all(fa0, fb0);
        __builtin_amdgcn_sched_barrier(0);
        wait_vm<(S - 3) * 8>();
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        {
            // second half: per part 2 MFMAs, one copy of stage kt+S-1 and one
            // fragment read of stage kt+1 (after the last stage that reads a
            // slot of zeros that is never used)
            const int kn = kt + S - 1, nb = (buf + S - 1) % S;
            const char* st = smem + ((buf + 1) % S) * STAGE_B;
#pragma unroll
            for (int part = 0; part < 8; ++part) {
                mfma32(acc[part >> 1][2 * (part & 1)], fa1[part >> 1], fb1[2 * (part & 1)]);
                mfma32(acc[part >> 1][2 * (part & 1) + 1], fa1[part >> 1], fb1[2 * (part & 1) + 1]);
                copy_part(kn, nb, part);
                if (part < 4)
                    fa0[part] = *reinterpret_cast<const bf16x8*>(
                        st + big_swz(wm * 128 + part * 32 + fr, fg));
                else
                    fb0[part - 4] = *reinterpret_cast<const bf16x8*>(
                        st + HALF_B + big_swz(wn * 128 + (part - 4) * 32 + fr, fg));
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    };
#pragma unroll
    for (int s0 = 0; s0 < S - 1; ++s0)
#pragma unroll
        for (int part = 0; part < 8; ++part) copy_part(s0, s0, part);
    wait_vm<(S - 2) * 8>();
    __builtin_amdgcn_s_barrier();
    read_frags(0, 0, fa0, fb0);
    for (int kt = 0; kt < KT; kt += S) {       // KT is a multiple of S
#pragma unroll
        for (int b = 0; b < S; ++b) step(kt + b, b);
    }
    wait_vm<0>();
    __syncthreads();
    static_assert(S * STAGE_B >= 64 * kBigLd * 4, "epilogue staging fits the stage ring");
    big_epilogue<EPI>(g, acc, m_tile, n_tile, wm, wn, lane, reinterpret_cast<float*>(smem));
}

template <int EPI>
__global__ __launch_bounds__(kThreads, 1) void gemm_big_kernel(GemmArgs g) {
    constexpr int S = kBigStages;
    constexpr int HALF_B = BBM * BBK * 2;         // bytes of the A (then B) part of a stage
    constexpr int STAGE_B = 2 * HALF_B;
    static_assert(S == 5, "the paired copies and their vmcnt waits assume a 5-stage ring");
    __shared__ __attribute__((aligned(16))) char smem[S * STAGE_B];   // 160 KB
    const uint32_t lds0 = (uint32_t)reinterpret_cast<uintptr_t>(smem);

    const int m_tiles = (g.M + BBM - 1) / BBM;
    const int n_cols_per_tile = (EPI == EPI_SWIGLU) ? BBN / 2 : BBN;
    const int n_tiles = (g.N + n_cols_per_tile - 1) / n_cols_per_tile;
    const int tile = xcd_remap(blockIdx.x, m_tiles * n_tiles);
    const int group = tile / (kGroupM * n_tiles);
    const int first_m = group * kGroupM;
    const int gm = min(m_tiles - first_m, kGroupM);
    const int in_group = tile - group * kGroupM * n_tiles;
    const int m_tile = first_m + in_group % gm, n_tile = in_group / gm;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int Kb = g.K * 2;

    // This wave copies rows 64*wave .. +63 of the A tile and of the B tile.
    const bf16* a_base = static_cast<const bf16*>(g.a) + ((int64_t)m_tile * BBM + 64 * wave) * g.K;
    const int64_t a_rows = (int64_t)g.M - (int64_t)m_tile * BBM - 64 * wave;
    const int a_bytes = uniform_int((a_rows < 0 ? 0 : (a_rows > 64 ? 64 : (int)a_rows)) * Kb);
    // B: two 32-row halves (for gate/up they come from different matrices)
    const bf16* b_base[2];
    int b_bytes[2];
    if (EPI == EPI_SWIGLU) {
        const int oc0 = n_tile * (BBN / 2) + wave * 32;
        const int64_t rows = g.N - oc0;
        const int by = uniform_int((rows < 0 ? 0 : (rows > 32 ? 32 : (int)rows)) * Kb);
        b_base[0] = static_cast<const bf16*>(g.b0) + (int64_t)oc0 * g.K;
        b_base[1] = static_cast<const bf16*>(g.b1) + (int64_t)oc0 * g.K;
        b_bytes[0] = b_bytes[1] = by;
    } else {
        const void* mat = g.b0;
        int64_t local = (int64_t)n_tile * BBN, rows = g.N;
        if (EPI == EPI_QKV) {
            const int c0 = n_tile * BBN;
            if (c0 < g.n0) { mat = g.b0; local = c0; rows = g.n0; }
            else if (c0 < g.n0 + g.n1) { mat = g.b1; local = c0 - g.n0; rows = g.n1; }
            else { mat = g.b2; local = c0 - g.n0 - g.n1; rows = g.N - g.n0 - g.n1; }
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int64_t r0 = local + 64 * wave + 32 * h;
            const int64_t left = rows - r0;
            b_base[h] = static_cast<const bf16*>(mat) + r0 * g.K;
            b_bytes[h] = uniform_int((left < 0 ? 0 : (left > 32 ? 32 : (int)left)) * Kb);
        }
    }
    // Lane i copies row i/4 (of 16) into LDS slot i%4: global chunk slot ^ key,
    // key = (row/4) % 4 (the same for every 16-row block of the wave).
    const int r16 = lane >> 2, slot = lane & 3;
    const int voff = r16 * Kb + ((slot ^ (r16 >> 2)) & 3) * 16;
    const int KT = g.K / BBK;

    // Copies of stage kt into ring slot `buf`, 8 per wave; with `t` the
    // copies are spread over the MFMA steps (see big_copy_part).
    auto copy_part = [&](int kt, int buf, int part) {       // part 0..7
        const bool live = kt < KT;
        const int j = part & 3;                             // 16-row block within the 64
        const uint32_t dst = lds0 + buf * STAGE_B + (part < 4 ? 0 : HALF_B) + (64 * wave + 16 * j) * 64;
        const int so = kt * 64 + 16 * (j & 1) * Kb;
        if (part < 4) {
            const i32x4 r = make_rsrc(a_base, live ? a_bytes : 0);
            dma16(r, voff, kt * 64 + 16 * j * Kb, dst);
        } else {
            const int h = j >> 1;
            const i32x4 r = make_rsrc(b_base[h], live ? b_bytes[h] : 0);
            dma16(r, voff, so, dst);
        }
    };

    floatx16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    const int fr = lane & 31, fg = lane >> 5;
    auto read_frags = [&](int buf, int ks, bf16x8 (&fa)[4], bf16x8 (&fb)[4]) {
        const char* st = smem + buf * STAGE_B;
        const int chunk = ks * 2 + fg;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            fa[i] = *reinterpret_cast<const bf16x8*>(st + big_swz(wm * 128 + i * 32 + fr, chunk));
#pragma unroll
        for (int j = 0; j < 4; ++j)
            fb[j] = *reinterpret_cast<const bf16x8*>(st + HALF_B + big_swz(wn * 128 + j * 32 + fr, chunk));
    };
    // 16 MFMAs, with the 8 fragment reads of the next step one per two MFMAs.
    auto mfma_all = [&](const bf16x8 (&fa)[4], const bf16x8 (&fb)[4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) mfma32(acc[i][j], fa[i], fb[j]);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
    };
    bf16x8 fa0[4], fb0[4], fa1[4], fb1[4];
    // Copies go out in pairs of stages (2m, 2m + 1), whose 64-byte row pieces
    // are the two halves of the same 128-byte lines, back to back per copy:
    // an even step kt refills the slots of stages kt - 1 and kt with stages
    // kt + 4 and kt + 5 (stage kt's second-half fragments were read at the
    // start of the step; lgkmcnt(0) before the barrier makes every wave's
    // reads complete).  Slots are run-time values of a rolled loop.
    auto step = [&](auto ev, int kt, int buf) {
        constexpr bool EVEN = decltype(ev)::value;
        const int nbuf = buf + 1 == S ? 0 : buf + 1;
        const int fill = buf == 0 ? S - 1 : buf - 1;
        read_frags(buf, 1, fa1, fb1);
        mfma_all(fa0, fb0);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (EVEN) {
            // stage kt+1 landed: after its last copy come the 16 of the pair (kt+2, kt+3)
            __builtin_amdgcn_s_waitcnt((16 & 15) | ((16 >> 4) << 14) | (7 << 4) | (0 << 8));
        } else {
            // stage kt+1 landed: after its last copy come one of its partner and 16 more
            wait_vm<17>();
        }
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        {
            const char* st = smem + nbuf * STAGE_B;
#pragma unroll
            for (int part = 0; part < 8; ++part) {
                mfma32(acc[part >> 1][2 * (part & 1)], fa1[part >> 1], fb1[2 * (part & 1)]);
                mfma32(acc[part >> 1][2 * (part & 1) + 1], fa1[part >> 1], fb1[2 * (part & 1) + 1]);
                if (EVEN) {
                    copy_part(kt + S - 1, fill, part);
                    copy_part(kt + S, buf, part);
                }
                if (part < 4)
                    fa0[part] = *reinterpret_cast<const bf16x8*>(
                        st + big_swz(wm * 128 + part * 32 + fr, fg));
                else
                    fb0[part - 4] = *reinterpret_cast<const bf16x8*>(
                        st + HALF_B + big_swz(wn * 128 + (part - 4) * 32 + fr, fg));
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    };
#pragma unroll
    for (int part = 0; part < 8; ++part) { copy_part(0, 0, part); copy_part(1, 1, part); }
#pragma unroll
    for (int part = 0; part < 8; ++part) { copy_part(2, 2, part); copy_part(3, 3, part); }
    wait_vm<17>();                            // stage 0 landed
    __builtin_amdgcn_s_barrier();
    read_frags(0, 0, fa0, fb0);
    int ring = 0;
    for (int kt = 0; kt < KT; kt += 2) {      // KT is even
        step(std::true_type{}, kt, ring);
        ring = ring + 1 == S ? 0 : ring + 1;
        step(std::false_type{}, kt + 1, ring);
        ring = ring + 1 == S ? 0 : ring + 1;
    }
    wait_vm<0>();
    __syncthreads();
    static_assert(S * STAGE_B >= 64 * kBigLd * 4, "epilogue staging fits the stage ring");
    big_epilogue<EPI>(g, acc, m_tile, n_tile, wm, wn, lane, reinterpret_cast<float*>(smem));
}

// ---------------------------------------------------------------------------
// Mid-size tiles for products of roughly 800-900 rows: 224x192 per
// workgroup.  Four row tiles cover up to 896 rows (128-row tiles pad 832
// rows to 896 as well, 256-row tiles to 1024), and a 12288-wide q/k/v
// product is exactly 256 tiles, one round of workgroups.  Four waves in a
// 2x2 grid, each 112x96 as 7x6 blocks of v_mfma_f32_16x16x32_bf16; per
// output element this moves 0.58x the L2 -> LDS bytes of the 128x128 tile.
// K advances 32 per stage: one MFMA covers a whole stage, lane l supplying
// row l % 16 and the 16-byte chunk l / 16 of a 64-byte LDS row.  Rows are
// unpadded with chunk c stored at slot c ^ ((row / 2) % 4), so the eight
// rows a group of eight lanes reads fall on distinct banks.  A ring of 5
// stages (26 KB each) is filled by direct-to-LDS copies, 26 per stage (14
// A and 12 B blocks of 16 rows); wave w issues blocks w, w + 4, ..., so
// waves 2 and 3 pad their seventh copy with an empty one into a spare
// kilobyte, which keeps the vmcnt bookkeeping uniform.  The epilogue
// stages the accumulators through LDS in two passes of 112 rows.  This
// direct-to-LDS kernel serves K not a multiple of 128; otherwise the
// register-staged kernel below runs the same tile (measured on the 7B step:
// gate/up 5.54 -> 5.30 ms, q/k/v 3.57 -> 3.46 ms per step; bit-identical
// results, the K steps of each accumulator in the same order).
constexpr int MBM = 224, MBN = 192, MBK = 32;
constexpr int kMidStages = 5;
constexpr int kMidCopies = 7;                         // copies per wave per stage
constexpr int kMidABytes = MBM * MBK * 2;             // A part of a stage
constexpr int kMidStage = (MBM + MBN) * MBK * 2;      // bytes per stage
constexpr int kMidLd = MBN + 4;                       // epilogue staging row (floats)

__device__ __forceinline__ int mid_swz(int r, int chunk) {   // byte offset in a stage part
    return r * 64 + ((chunk ^ (r >> 1)) & 3) * 16;
}

// Accumulates in place: each MFMA's C operand and result are the same
// registers (the empty register pins after the main loop keep it so).
__device__ __forceinline__ void mfma16x32(floatx4& acc, const bf16x8& a, const bf16x8& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}

struct MidSrc {
    const bf16* p;      // first row of a 16-row copy block
    int64_t left;       // rows of its matrix from there on
};

// B rows 16 j .. 16 j + 15 of tile n_tile.  Gate/up: the 96 rows of wave
// column wn are 48 gate rows then the 48 up rows of the same output columns.
// q/k/v: blocks never straddle two matrices (row counts are multiples of 16).
template <int EPI>
__device__ __forceinline__ MidSrc mid_b_rows(const GemmArgs& g, int n_tile, int j) {
    if (EPI == EPI_SWIGLU) {
        const int wn = j / 6, jj = j % 6;
        const int oc0 = n_tile * (MBN / 2) + 48 * wn + 16 * (jj % 3);
        return {static_cast<const bf16*>(jj < 3 ? g.b0 : g.b1) + (int64_t)oc0 * g.K,
                (int64_t)g.N - oc0};
    }
    const int r0 = n_tile * MBN + 16 * j;
    if (EPI == EPI_QKV) {
        if (r0 < g.n0) return {static_cast<const bf16*>(g.b0) + (int64_t)r0 * g.K, (int64_t)g.n0 - r0};
        if (r0 < g.n0 + g.n1) {
            const int l = r0 - g.n0;
            return {static_cast<const bf16*>(g.b1) + (int64_t)l * g.K, (int64_t)g.n1 - l};
        }
        const int l = r0 - g.n0 - g.n1;
        return {static_cast<const bf16*>(g.b2) + (int64_t)l * g.K,
                (int64_t)(g.N - g.n0 - g.n1) - l};
    }
    return {static_cast<const bf16*>(g.b0) + (int64_t)r0 * g.K, (int64_t)g.N - r0};
}

// Rows row0 .. row0 + 111 of the tile, staged in LDS as [112][kMidLd] fp32.
// Each thread keeps one group of 4 columns (its output matrix, RoPE pair
// index and residual column are fixed) and walks every 5th row (every
// 10th for gate/up, whose groups are 4 output columns of 96), unrolled so
// that the position, RoPE-table and residual loads of several rows are in
// flight together.
template <int EPI>
__device__ __forceinline__ void mid_finish(const GemmArgs& g, int row0, int n_tile,
                                           const float* lds) {
    const int t = threadIdx.x;
    if (EPI == EPI_SWIGLU) {
        if (t >= 240) return;
        const int oc = 4 * (t % 24);                 // of the tile's 96 output columns
        const int lc = 96 * (oc / 48) + oc % 48;     // gate at lc, up at lc + 48
        const int col = n_tile * (MBN / 2) + oc;
        if (col >= g.N) return;
        const bool full = col + 3 < g.N;
#pragma unroll 4
        for (int rl = t / 24; rl < 112; rl += 10) {
            const int row = row0 + rl;
            if (row >= g.M) break;
            const floatx4 gt = *reinterpret_cast<const floatx4*>(&lds[rl * kMidLd + lc]);
            const floatx4 up = *reinterpret_cast<const floatx4*>(&lds[rl * kMidLd + lc + 48]);
            bf16* dst = static_cast<bf16*>(g.out0) + (int64_t)row * g.N + col;
            if (full) {
                *reinterpret_cast<bf16x4*>(dst) =
                    bf16x4{static_cast<bf16>(silu_f(gt[0]) * up[0]), static_cast<bf16>(silu_f(gt[1]) * up[1]),
                           static_cast<bf16>(silu_f(gt[2]) * up[2]), static_cast<bf16>(silu_f(gt[3]) * up[3])};
            } else {
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    if (col + k < g.N) dst[k] = static_cast<bf16>(silu_f(gt[k]) * up[k]);
            }
        }
        return;
    }
    if (t >= 240) return;
    const int cg = 4 * (t % 48);
    const int col = n_tile * MBN + cg;
    if (col >= g.N) return;
    if (EPI == EPI_QKV) {
        // the 4 columns lie in one of q, k, v (row counts are multiples of 16)
        bf16* base;
        int width, local;
        bool rope, kv = true;
        if (col < g.n0) { base = static_cast<bf16*>(g.out0); width = g.n0; local = col; rope = true; kv = false; }
        else if (col < g.n0 + g.n1) {
            base = static_cast<bf16*>(g.out1); width = g.n1; local = col - g.n0; rope = true;
        } else {
            base = static_cast<bf16*>(g.out2); width = g.N - g.n0 - g.n1;
            local = col - g.n0 - g.n1; rope = false;
        }
        const int pair = (local % g.head_dim) >> 1;   // even: pairs (pair, pair + 1)
        // The thread's rows rl = t / 48 + 5 i < 112.  Their positions and
        // output rows, then their RoPE factors, are all loaded before the
        // first store: two dependent round trips per half tile instead of
        // two or three per group of rows.
        constexpr int NR = 23;
        const int r0 = t / 48;
        int pr[NR], orow[NR];
        floatx4 cs[NR];
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            const int rl = r0 + 5 * i, row = row0 + rl;
            const bool ok = rl < 112 && row < g.M;
            pr[i] = ok && rope ? g.pos[row] : 0;
            orow[i] = ok ? (int)qkv_out_row(g, row, kv) : 0;
        }
        if (rope) {
#pragma unroll
            for (int i = 0; i < NR; ++i)
                cs[i] = *reinterpret_cast<const floatx4*>(
                    &g.rope.tab[(int64_t)pr[i] * g.rope.half + pair]);
        }
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            const int rl = r0 + 5 * i, row = row0 + rl;
            if (rl >= 112 || row >= g.M) break;
            const floatx4 x = *reinterpret_cast<const floatx4*>(&lds[rl * kMidLd + cg]);
            floatx4 y = x;
            if (rope) {
                y[0] = x[0] * cs[i][0] - x[1] * cs[i][1];
                y[1] = x[0] * cs[i][1] + x[1] * cs[i][0];
                y[2] = x[2] * cs[i][2] - x[3] * cs[i][3];
                y[3] = x[2] * cs[i][3] + x[3] * cs[i][2];
            }
            *reinterpret_cast<bf16x4*>(base + (int64_t)orow[i] * width + local) =
                bf16x4{static_cast<bf16>(y[0]), static_cast<bf16>(y[1]), static_cast<bf16>(y[2]),
                       static_cast<bf16>(y[3])};
        }
        return;
    }
    const bool vec = (g.N % 4) == 0 && col + 3 < g.N;
    if (EPI == EPI_RESID && vec) {
        // residual row indices of the thread's rows t / 48 + 5 i < 112, then
        // the residual values, before the first store
        constexpr int NR = 23;
        const int r0 = t / 48;
        int rr[NR];
        floatx4 rv[NR];
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            const int rl = r0 + 5 * i, row = row0 + rl;
            rr[i] = rl < 112 && row < g.M ? (g.ridx ? g.ridx[row] : row) : -1;
        }
#pragma unroll
        for (int i = 0; i < NR; ++i)
            rv[i] = rr[i] >= 0 ? *reinterpret_cast<const floatx4*>(g.resid + (int64_t)rr[i] * g.N + col)
                               : floatx4{};
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            const int rl = r0 + 5 * i, row = row0 + rl;
            if (rl >= 112 || row >= g.M) break;
            *reinterpret_cast<floatx4*>(static_cast<float*>(g.out0) + (int64_t)row * g.N + col) =
                *reinterpret_cast<const floatx4*>(&lds[rl * kMidLd + cg]) + rv[i];
        }
        return;
    }
#pragma unroll 4
    for (int rl = t / 48; rl < 112; rl += 5) {
        const int row = row0 + rl;
        if (row >= g.M) break;
        const floatx4 x = *reinterpret_cast<const floatx4*>(&lds[rl * kMidLd + cg]);
        float* dst = static_cast<float*>(g.out0) + (int64_t)row * g.N + col;
        const float* res = nullptr;
        if (EPI == EPI_RESID) res = g.resid + (int64_t)(g.ridx ? g.ridx[row] : row) * g.N + col;
        if (vec) {
            floatx4 y = x;
            if (EPI == EPI_RESID) y += *reinterpret_cast<const floatx4*>(res);
            *reinterpret_cast<floatx4*>(dst) = y;
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k)
                if (col + k < g.N) dst[k] = x[k] + (EPI == EPI_RESID ? res[k] : 0.f);
        }
    }
}

template <int EPI, int S>
__global__ __launch_bounds__(kThreads, 1) void gemm_mid_kernel(GemmArgs g) {
    static_assert(S == 5, "the paired copies and their vmcnt waits assume a 5-stage ring");
    __shared__ __attribute__((aligned(16))) char smem[S * kMidStage + 1024];
    const uint32_t lds0 = (uint32_t)reinterpret_cast<uintptr_t>(smem);
    const uint32_t spare = lds0 + S * kMidStage;         // target of the empty copies

    const int m_tiles = (g.M + MBM - 1) / MBM;
    const int cols = EPI == EPI_SWIGLU ? MBN / 2 : MBN;
    const int n_tiles = (g.N + cols - 1) / cols;
    const int tile = xcd_remap(blockIdx.x, m_tiles * n_tiles);
    const int group = tile / (kGroupM * n_tiles);
    const int first_m = group * kGroupM;
    const int gm = min(m_tiles - first_m, kGroupM);
    const int in_group = tile - group * kGroupM * n_tiles;
    const int m_tile = first_m + in_group % gm, n_tile = in_group / gm;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar descriptors
    const int wm = wave >> 1, wn = wave & 1;
    const int Kb = g.K * 2;

    // Copies 0-3 of this wave move A blocks 4 c + wave (rows 16 b .. 16 b + 15
    // of the tile; blocks 14 and 15 do not exist: they lie past the
    // descriptor's range, read as zero and land in the spare kilobyte);
    // copies 4-6 move B blocks 4 (c - 4) + wave.  One descriptor covers the
    // A tile, one per copy the B blocks (which may come from different
    // matrices).
    const int64_t a_left = (int64_t)g.M - (int64_t)m_tile * MBM;
    const i32x4 da = make_rsrc(static_cast<const bf16*>(g.a) + (int64_t)m_tile * MBM * g.K,
                               (int)(a_left <= 0 ? 0 : (a_left >= MBM ? MBM : a_left)) * Kb);
    const bf16* b_src[3];
    int b_bytes[3];
#pragma unroll
    for (int c = 0; c < 3; ++c) {
        const MidSrc sr = mid_b_rows<EPI>(g, n_tile, 4 * c + wave);
        b_src[c] = sr.p;
        b_bytes[c] = uniform_int((int)(sr.left <= 0 ? 0 : (sr.left >= 16 ? 16 : sr.left)) * Kb);
    }
    // Lane i copies row i / 4 of a block into slot i % 4: global chunk
    // slot ^ key(row), key(r) = (r / 2) % 4 (the same for every block).
    const int r4 = lane >> 2, sl = lane & 3;
    const int voff = r4 * Kb + ((sl ^ (r4 >> 1)) & 3) * 16;
    const int KT = g.K / MBK;
    const i32x4 none = make_rsrc(g.a, 0);
    auto copy = [&](int c, int kt, int slot) {
        const bool live = kt < KT;                       // stages past the end read nothing
        if (c < 4) {
            const int b = 4 * c + wave;
            const uint32_t d = b < 14 ? lds0 + slot * kMidStage + 16 * b * 64 : spare;
            dma16(live ? da : none, voff + 16 * b * Kb, kt * 64, d);
        } else {
            const int j = 4 * (c - 4) + wave;
            const i32x4 r = make_rsrc(b_src[c - 4], live ? b_bytes[c - 4] : 0);
            dma16(r, voff, kt * 64, lds0 + slot * kMidStage + kMidABytes + 16 * j * 64);
        }
    };

    floatx4 acc[7][6];
#pragma unroll
    for (int i = 0; i < 7; ++i)
#pragma unroll
        for (int j = 0; j < 6; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    const int fr = lane & 15, fq = lane >> 4;
    auto frag = [&](int off) { return *reinterpret_cast<const bf16x8*>(smem + off); };
    const int a_off = mid_swz(wm * 112 + fr, fq);             // + 16 i rows: + 1024 i bytes
    const int b_off = kMidABytes + mid_swz(wn * 96 + fr, fq); // + 16 j rows
    bf16x8 fa[7], fb[6], na[7], nb[6];
    // One K stage out of ring slot `slot`, its fragments in (ca, cb): the 42
    // MFMAs (A fragment i with B fragments 0-5) are interleaved with the 13
    // fragment reads of stage kt + 1 into (xa, xb).  Copies go out in pairs
    // of stages 2m, 2m + 1, whose 64-byte row pieces are the two halves of
    // the same 128-byte lines, issued back to back per block: an even step
    // kt refills the slots of stages kt - 1 and kt with stages kt + 4 and
    // kt + 5 (measured: 7B step 19.44 -> 18.80 ms against one stage per
    // step).  Slots are run-time values (a rolled loop keeps the
    // accumulators in place); they only offset LDS addresses.
    auto step = [&](auto ev, int kt, int slot, const bf16x8 (&ca)[7], const bf16x8 (&cb)[6],
                    bf16x8 (&xa)[7], bf16x8 (&xb)[6]) {
        constexpr bool EVEN = decltype(ev)::value;
        const int nxt = slot + 1 == S ? 0 : slot + 1;
        const int fill = slot == 0 ? S - 1 : slot - 1;
        const char* nbase = smem + nxt * kMidStage;
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (EVEN) {
            // stage kt+1 landed (only the pair kt+2, kt+3 may be in flight),
            // and this wave's reads of stage kt have completed: its slot is
            // refilled after the barrier
            constexpr int N = 2 * kMidCopies;
            __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (0 << 8));
        } else {
            // stage kt+1 landed: after its last copy come one copy of its
            // pair partner kt+2 and the 14 copies of the last even step
            wait_vm<2 * kMidCopies + 1>();
        }
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < 42; ++t) {
            mfma16x32(acc[t / 6][t % 6], ca[t / 6], cb[t % 6]);
            // one read per two MFMAs over the first 26, B fragments first:
            // the next stage's first six MFMAs use all of them, while A
            // fragment i is first used by its MFMA 6 i
            if (t % 2 == 1 && t / 2 < 13) {
                const int q = t / 2;
                if (q < 6) xb[q] = *reinterpret_cast<const bf16x8*>(nbase + b_off + 1024 * q);
                else xa[q - 6] = *reinterpret_cast<const bf16x8*>(nbase + a_off + 1024 * (q - 6));
            }
            if (EVEN && t % 6 == 5) {          // the two halves of the same 128-byte lines
                copy(t / 6, kt + S - 1, fill);
                copy(t / 6, kt + S, slot);
            }
        }
#pragma unroll
        for (int k = 0; k < 13; ++k) {
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);   // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);
        __builtin_amdgcn_sched_barrier(0);
    };
    // stages 0-3 as the pairs (0, 1), (2, 3); stage 0 has landed once at most
    // one copy of stage 1 and the 14 of (2, 3) are outstanding
#pragma unroll
    for (int c = 0; c < kMidCopies; ++c) { copy(c, 0, 0); copy(c, 1, 1); }
#pragma unroll
    for (int c = 0; c < kMidCopies; ++c) { copy(c, 2, 2); copy(c, 3, 3); }
    wait_vm<2 * kMidCopies + 1>();
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int i = 0; i < 7; ++i) fa[i] = frag(a_off + 1024 * i);
#pragma unroll
    for (int j = 0; j < 6; ++j) fb[j] = frag(b_off + 1024 * j);
    // KT is even (K is a multiple of 64): two stages per iteration, the
    // fragment registers alternating
    int slot = 0;
    for (int kt = 0; kt < KT; kt += 2) {
        step(std::true_type{}, kt, slot, fa, fb, na, nb);
        slot = slot + 1 == S ? 0 : slot + 1;
        step(std::false_type{}, kt + 1, slot, na, nb, fa, fb);
        slot = slot + 1 == S ? 0 : slot + 1;
    }
    // Empty statements that take each accumulator in AGPRs: without them the
    // register allocator gives 21 of the 42 MFMAs a result register other
    // than their C operand and copies the accumulators back once per loop
    // iteration (252 v_accvgpr_mov per two K stages).  They emit nothing;
    // the wait states between the last MFMA and the first read of its result
    // are placed by the compiler, which sees every MFMA.
#pragma unroll
    for (int i = 0; i < 7; ++i)
#pragma unroll
        for (int j = 0; j < 6; ++j) asm volatile("" : "+a"(acc[i][j]));
    // trailing (empty) copies still write LDS: let them land, and every
    // wave finish its fragment reads, before the ring becomes staging space
    wait_vm<0>();
    __syncthreads();
    static_assert(112 * kMidLd * 4 <= S * kMidStage, "epilogue staging fits the ring");
    float* lds = reinterpret_cast<float*>(smem);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        if (wm == q) {
#pragma unroll
            for (int i = 0; i < 7; ++i)
#pragma unroll
                for (int j = 0; j < 6; ++j)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        lds[(16 * i + 4 * fq + e) * kMidLd + 96 * wn + 16 * j + fr] = acc[i][j][e];
        }
        __syncthreads();
        mid_finish<EPI>(g, m_tile * MBM + 112 * q, n_tile, lds);
        __syncthreads();
    }
}

// The same 224x192 tile with register-staged copies: each thread loads its
// 13 16-byte chunks of a 64-wide K stage (7 of A, 6 of B; the 8 lanes of a
// row read one whole 128-byte line) into registers with buffer loads, and
// stores them to LDS one iteration later.  Three LDS buffers of 52 KB: while
// stage k is multiplied out, stage k + 2 is stored from the registers and
// the loads of stage k + 3 go out; one barrier per 64-wide stage.  Rows
// past M or past a weight matrix lie outside their buffer resource's range
// and read as zero.  LDS rows are 128 bytes with chunk c of row r at slot
// c ^ ((r / 2) % 8): the 16 rows of one fragment read and the 8 rows of one
// wave's store fall on distinct banks.  Measured and dropped: a second
// register set (loads two stages ahead), stores split evenly over both K
// steps of a stage, or all in the first (none changed the time), and B
// fragments loaded by each wave straight into its MFMA operand registers
// with only A through LDS (gate/up 5.05 -> 7.90 ms per 7B step).
constexpr int kRsK = 64;                              // K per stage
constexpr int kRsABytes = MBM * kRsK * 2;             // 28 KB
constexpr int kRsBuf = (MBM + MBN) * kRsK * 2;        // 52 KB
constexpr int kRsBufs = 3;

__device__ __forceinline__ u32x4 rs_load(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
}

// Workgroup barrier after this wave's LDS accesses have completed
// (lgkmcnt(0)), with compiler-only memory barriers on both sides.  Written
// out rather than __syncthreads(): with that call at the end of the loop
// body the register allocator moved about a hundred accumulator registers
// per stage (v_accvgpr_mov/read/write) instead of accumulating in place.
__device__ __forceinline__ void rs_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (0 << 8));   // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

template <int EPI>
__global__ __launch_bounds__(kThreads, 1) void gemm_rs_kernel(GemmArgs g) {
    __shared__ __attribute__((aligned(16))) char smem[kRsBufs * kRsBuf];

    const int m_tiles = (g.M + MBM - 1) / MBM;
    const int cols = EPI == EPI_SWIGLU ? MBN / 2 : MBN;
    const int n_tiles = (g.N + cols - 1) / cols;
    const int tile = xcd_remap(blockIdx.x, m_tiles * n_tiles);
    const int group = tile / (kGroupM * n_tiles);
    const int first_m = group * kGroupM;
    const int gm = min(m_tiles - first_m, kGroupM);
    const int in_group = tile - group * kGroupM * n_tiles;
    const int m_tile = first_m + in_group % gm, n_tile = in_group / gm;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int Kb = g.K * 2;
    const int KT = g.K / kRsK;

    // Copy chunks: thread t moves chunk t % 8 of rows t / 8 + 32 i (A rows
    // i = 0..6, B rows i = 0..5).  The B rows of (wave, i) all lie in the
    // 16-row block 2 i + wave / 2.
    const int crow = tid >> 3, cc = tid & 7;
    const int64_t a_left = (int64_t)g.M - (int64_t)m_tile * MBM;
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<bf16*>(static_cast<const bf16*>(g.a) + (int64_t)m_tile * MBM * g.K), (short)0,
        uniform_int((int)(a_left <= 0 ? 0 : (a_left >= MBM ? MBM : a_left)) * Kb), 0x00020000);
    __amdgpu_buffer_rsrc_t rb[6];
#pragma unroll
    for (int i = 0; i < 6; ++i) {
        const MidSrc sr = mid_b_rows<EPI>(g, n_tile, 2 * i + (wave >> 1));
        rb[i] = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<bf16*>(sr.p), (short)0,
            uniform_int((int)(sr.left <= 0 ? 0 : (sr.left >= 16 ? 16 : sr.left)) * Kb), 0x00020000);
    }
    const int a_voff = crow * Kb + cc * 16;                 // + 32 i rows
    const int b_voff = (crow & 15) * Kb + cc * 16;
    const int wr_off = crow * 128 + ((cc ^ ((crow >> 1) & 7)) << 4);   // + 4096 i
    u32x4 stg[13];
    auto load_stage = [&](int kt, u32x4 (&r)[13]) {
#pragma unroll
        for (int i = 0; i < 7; ++i) r[i] = rs_load(ra, a_voff + 32 * i * Kb, kt * 128);
#pragma unroll
        for (int i = 0; i < 6; ++i) r[7 + i] = rs_load(rb[i], b_voff, kt * 128);
    };
    auto store_one = [&](int buf, int i, const u32x4& v) {
        char* base = smem + buf * kRsBuf + (i < 7 ? 4096 * i : kRsABytes + 4096 * (i - 7));
        *reinterpret_cast<u32x4*>(base + wr_off) = v;
    };

    floatx4 acc[7][6];
#pragma unroll
    for (int i = 0; i < 7; ++i)
#pragma unroll
        for (int j = 0; j < 6; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    // fragment of row fr of a 16-row block, K chunk 4 s + fq of the stage
    const int fr = lane & 15, fq = lane >> 4;
    const int key = (fr >> 1) & 7;
    const int a_rd = (wm * 112 + fr) * 128;                 // + 2048 i
    const int b_rd = kRsABytes + (wn * 96 + fr) * 128;      // + 2048 j
    auto frag_off = [&](int s) { return ((4 * s + fq) ^ key) << 4; };
    bf16x8 fa[7], fb[6], na[7], nb[6];

    // Prologue: stages 0 and 1 stored, stage 2 in flight, stage 0's first
    // fragments read.
    {
        u32x4 s1[13];
        load_stage(0, stg);
        load_stage(min(1, KT - 1), s1);
#pragma unroll
        for (int i = 0; i < 13; ++i) store_one(0, i, stg[i]);
#pragma unroll
        for (int i = 0; i < 13; ++i) store_one(1, i, s1[i]);
        load_stage(min(2, KT - 1), stg);
    }
    rs_barrier();
    {
        const int o = frag_off(0);
#pragma unroll
        for (int i = 0; i < 7; ++i) fa[i] = *reinterpret_cast<const bf16x8*>(smem + a_rd + 2048 * i + o);
#pragma unroll
        for (int j = 0; j < 6; ++j) fb[j] = *reinterpret_cast<const bf16x8*>(smem + b_rd + 2048 * j + o);
    }

    // One 32-wide K step: 42 MFMAs on fragments (ca, cb) while the 13
    // fragments of the next step are read from `rbuf` (chunk column `o`)
    // into (xa, xb).  In a stage's second step (SECOND) the registers of
    // stage kt + 2 are also stored to buffer `fill` and stage kt + 3 is
    // loaded.  The barrier at the start of the next stage publishes these
    // stores; the one at the start of this stage freed their buffer (stage
    // kt - 1's, read last in that stage's first step).
    // Stage kt lives in buffer kt % 3; near the end the loads repeat the
    // last stage and the stores and reads go to buffers never read again,
    // so the loop body is the same for every stage.
    auto step = [&](auto sc, int kt, const char* rbuf, int o, int fill, const bf16x8 (&ca)[7],
                    const bf16x8 (&cb)[6], bf16x8 (&xa)[7], bf16x8 (&xb)[6]) {
        constexpr bool SECOND = decltype(sc)::value;
        const int soff3 = min(kt + 3, KT - 1) * 128;
        if (!SECOND) rs_barrier();
#pragma unroll
        for (int t = 0; t < 42; ++t) {
            mfma16x32(acc[t / 6][t % 6], ca[t / 6], cb[t % 6]);
            if (t % 3 == (SECOND ? 0 : 2) && t / 3 < 13) {
                const int q = t / 3;
                if (SECOND) {
                    store_one(fill, q, stg[q]);
                    if (q < 7) stg[q] = rs_load(ra, a_voff + 32 * q * Kb, soff3);
                    else stg[q] = rs_load(rb[q - 7], b_voff, soff3);
                }
                if (q < 6) xb[q] = *reinterpret_cast<const bf16x8*>(rbuf + b_rd + 2048 * q + o);
                else xa[q - 6] = *reinterpret_cast<const bf16x8*>(rbuf + a_rd + 2048 * (q - 6) + o);
            }
        }
#pragma unroll
        for (int q = 0; q < 13; ++q) {
            if (SECOND) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
                __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);   // DS write
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // VMEM read
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
            } else {
                __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
        __builtin_amdgcn_sched_barrier(0);
    };
    const int o0 = frag_off(0), o1 = frag_off(1);
    // KT is even (K is a multiple of 128): two stages per loop iteration
    int cur = 0;
    for (int kt = 0; kt < KT; kt += 2) {
        const int c1 = cur == 2 ? 0 : cur + 1, c2 = c1 == 2 ? 0 : c1 + 1;
        step(std::false_type{}, kt, smem + cur * kRsBuf, o1, 0, fa, fb, na, nb);
        step(std::true_type{}, kt, smem + c1 * kRsBuf, o0, c2, na, nb, fa, fb);
        step(std::false_type{}, kt + 1, smem + c1 * kRsBuf, o1, 0, fa, fb, na, nb);
        step(std::true_type{}, kt + 1, smem + c2 * kRsBuf, o0, cur, na, nb, fa, fb);
        cur = c2;
    }
    // the last (repeated) loads have landed and every wave's LDS reads and
    // stores are done before the buffers become staging space
    __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));   // vmcnt(0)
    rs_barrier();
#pragma unroll
    for (int i = 0; i < 7; ++i)
#pragma unroll
        for (int j = 0; j < 6; ++j) asm volatile("" : "+a"(acc[i][j]));
    static_assert(112 * kMidLd * 4 <= kRsBufs * kRsBuf, "epilogue staging fits the buffers");
    float* lds = reinterpret_cast<float*>(smem);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        if (wm == q) {
#pragma unroll
            for (int i = 0; i < 7; ++i)
#pragma unroll
                for (int j = 0; j < 6; ++j)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        lds[(16 * i + 4 * fq + e) * kMidLd + 96 * wn + 16 * j + fr] = acc[i][j][e];
        }
        __syncthreads();
        mid_finish<EPI>(g, m_tile * MBM + 112 * q, n_tile, lds);
        __syncthreads();
    }
}

template <int EPI>
hipError_t launch_mid(const GemmArgs& g, hipStream_t s) {
    const int m_tiles = (g.M + MBM - 1) / MBM;
    const int cols = (EPI == EPI_SWIGLU) ? MBN / 2 : MBN;
    const int n_tiles = (g.N + cols - 1) / cols;
    if (g.K % (2 * kRsK) == 0)
        hipLaunchKernelGGL((gemm_rs_kernel<EPI>), dim3(m_tiles * n_tiles), dim3(kThreads), 0, s, g);
    else
        hipLaunchKernelGGL((gemm_mid_kernel<EPI, kMidStages>), dim3(m_tiles * n_tiles),
                           dim3(kThreads), 0, s, g);
    return hipGetLastError();
}

constexpr int kDmaStages = 5;            // LDS ring depth of the bf16 kernel

int num_cus();

template <int EPI>
hipError_t launch_big(const GemmArgs& g, hipStream_t s) {
    const int m_tiles = (g.M + BBM - 1) / BBM;
    const int cols = (EPI == EPI_SWIGLU) ? BBN / 2 : BBN;
    const int n_tiles = (g.N + cols - 1) / cols;
    const int64_t tiles = (int64_t)m_tiles * n_tiles;
    if (tiles > 4 * (int64_t)num_cus() && g.K % (BBK * kBig4Stages) == 0)
        hipLaunchKernelGGL((gemm_big4_kernel<EPI>), dim3(tiles), dim3(kThreads), 0, s, g);
    else
        hipLaunchKernelGGL((gemm_big_kernel<EPI>), dim3(tiles), dim3(kThreads), 0, s, g);
    return hipGetLastError();
}

int num_cus() {
    static int n = [] {
        int dev = 0, c = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0)
            c = 256;
        return c;
    }();
    return n;
}

// Tile choice.  All three bf16 kernels run one workgroup per CU (256 at a
// time); compare whole rounds of workgroups, each round priced in units of
// one 128x128 tile.  A 256x256 tile costs about 3 of them (4x the work at
// ~1.3x the efficiency): 2.9, so that one round of 256x256 beats three of
// 128x128 (Yi-34B down projection, 1484 x 7168 x 20480: 616 vs 792 us;
// 34B step 154 -> 141 ms), 3.1 for the q/k/v product; a 224x192 tile
// kMidCost.  Ties go to the smaller tile.  Measured on MI355X (bf16): large
// products (>= 4096 rows) 1.2-1.3x faster on 256x256; N = 4096 products at
// ~832 rows lose badly there (340 vs 760 TF/s).
constexpr double kMidCost = 2.35;
enum TileKind { TILE_128, TILE_256, TILE_224x192 };

bool big_shape_ok(int epi, const GemmArgs& g) {
    if (g.K % (2 * BBK) != 0 || (int64_t)g.K * 2 * 64 + 64 >= (int64_t)1 << 31) return false;
    if (epi == EPI_QKV && (g.n0 % BBN != 0 || g.n1 % BBN != 0)) return false;
    return true;
}

bool mid_shape_ok(int epi, const GemmArgs& g) {
    // copy offsets reach 256 rows (16 blocks of 16) into the A tile
    if (g.K % (2 * MBK) != 0 || (int64_t)g.K * 2 * 256 >= (int64_t)1 << 31) return false;
    if (epi == EPI_QKV && g.head_dim % 4 != 0) return false;
    return true;
}

TileKind choose_tile(int epi, const GemmArgs& g) {
    const int64_t rows_b = epi == EPI_SWIGLU ? 2 * (int64_t)g.N : g.N;   // B rows
    const int64_t cus = num_cus();
    auto rounds = [&](int bm, int bn) {
        const int64_t tiles = ((g.M + bm - 1) / bm) * ((rows_b + bn - 1) / bn);
        return (double)((tiles + cus - 1) / cus);
    };
    TileKind best = TILE_128;
    double cost = rounds(BM, BN);
    if (mid_shape_ok(epi, g)) {
        const double c = kMidCost * rounds(MBM, MBN);
        if (c < cost) { cost = c; best = TILE_224x192; }
    }
    if (big_shape_ok(epi, g)) {
        const double c = (epi == EPI_QKV ? 3.1 : 2.9) * rounds(BBM, BBN);
        if (c < cost) { cost = c; best = TILE_256; }
    }
    return best;
}

template <int EPI>
hipError_t launch_dma(const GemmArgs& g, hipStream_t s) {
    const int m_tiles = (g.M + BM - 1) / BM;
    const int cols = (EPI == EPI_SWIGLU) ? BN / 2 : BN;
    const int n_tiles = (g.N + cols - 1) / cols;
    hipLaunchKernelGGL((gemm_dma8_kernel<EPI, kDmaStages>), dim3(m_tiles * n_tiles),
                       dim3(kThreads8), 0, s, g);
    return hipGetLastError();
}

// The direct-to-LDS kernel needs whole 64-element stages, buffer offsets
// below 2^31 and, for q/k/v, tiles that do not straddle matrices.
bool dma_ok(int epi, const GemmArgs& g) {
    if (g.K % 64 != 0 || (int64_t)g.K * 2 * 32 + 128 >= (int64_t)1 << 31)
        return false;
    if (epi == EPI_QKV && (g.n0 % BN != 0 || g.n1 % BN != 0)) return false;
    return true;
}

// The product restricted to result rows [r0, r0 + m), for the plain-store
// and SwiGLU epilogues: A and the output move by r0 rows.
GemmArgs row_slice(int epi, const GemmArgs& g, int r0, int m) {
    GemmArgs h = g;
    h.M = m;
    h.a = static_cast<const bf16*>(g.a) + (int64_t)r0 * g.K;
    if (epi == EPI_STORE_F32) h.out0 = static_cast<float*>(g.out0) + (int64_t)r0 * g.N;
    else h.out0 = static_cast<bf16*>(g.out0) + (int64_t)r0 * g.N;
    return h;
}

// A product a few rows taller than a whole number of 224-row tiles (947
// rows: layer 1's MLP and layer 2's q/k/v at 7B width, r = 15%) would spend
// a round of 224x192 tiles, or a larger tile, on its last rows.  Split: the
// whole 224-row tiles on 224x192 tiles, the remaining rows (at most
// kSplitRows) on 128x128 tiles, when the cost model prices the two launches
// below the best single one.  Only the plain-store and SwiGLU products
// take it: at the widths served here the q/k/v and residual products price a
// split above their single launch.
constexpr int kSplitRows = 64;

bool try_row_split(int epi, const GemmArgs& g, hipStream_t s, hipError_t* err) {
    const int rem = g.M % MBM, m_main = g.M - rem;
    if (epi != EPI_STORE_F32 && epi != EPI_SWIGLU) return false;
    if (m_main == 0 || rem == 0 || rem > kSplitRows) return false;
    if (!mid_shape_ok(epi, g) || !dma_ok(epi, g)) return false;
    const int64_t rows_b = epi == EPI_SWIGLU ? 2 * (int64_t)g.N : g.N;
    const int64_t cus = num_cus();
    auto rounds = [&](int64_t m, int bm, int bn) {
        const int64_t tiles = ((m + bm - 1) / bm) * ((rows_b + bn - 1) / bn);
        return (double)((tiles + cus - 1) / cus);
    };
    double best = rounds(g.M, BM, BN);
    best = std::min(best, kMidCost * rounds(g.M, MBM, MBN));
    if (big_shape_ok(epi, g))
        best = std::min(best, (epi == EPI_QKV ? 3.1 : 2.9) * rounds(g.M, BBM, BBN));
    const double split = kMidCost * rounds(m_main, MBM, MBN) + rounds(rem, BM, BN);
    if (!(split < best)) return false;
    const GemmArgs lo = row_slice(epi, g, 0, m_main), hi = row_slice(epi, g, m_main, rem);
    hipError_t e = epi == EPI_SWIGLU ? launch_mid<EPI_SWIGLU>(lo, s)
                                     : launch_mid<EPI_STORE_F32>(lo, s);
    if (e == hipSuccess)
        e = epi == EPI_SWIGLU ? launch_dma<EPI_SWIGLU>(hi, s) : launch_dma<EPI_STORE_F32>(hi, s);
    *err = e;
    return true;
}

template <typename T>
hipError_t launch_dtype(int epi, const GemmArgs& g, hipStream_t s) {
    if constexpr (is_bf16<T>()) {
        hipError_t split_err;
        if (try_row_split(epi, g, s, &split_err)) return split_err;
        const TileKind tk = choose_tile(epi, g);
        if (tk == TILE_224x192) {
            switch (epi) {
                case EPI_STORE_F32: return launch_mid<EPI_STORE_F32>(g, s);
                case EPI_QKV: return launch_mid<EPI_QKV>(g, s);
                case EPI_RESID: return launch_mid<EPI_RESID>(g, s);
                case EPI_SWIGLU: return launch_mid<EPI_SWIGLU>(g, s);
            }
            return hipErrorInvalidValue;
        }
        if (tk == TILE_256) {
            switch (epi) {
                case EPI_STORE_F32: return launch_big<EPI_STORE_F32>(g, s);
                case EPI_QKV: return launch_big<EPI_QKV>(g, s);
                case EPI_RESID: return launch_big<EPI_RESID>(g, s);
                case EPI_SWIGLU: return launch_big<EPI_SWIGLU>(g, s);
            }
            return hipErrorInvalidValue;
        }
        if (dma_ok(epi, g)) {
            switch (epi) {
                case EPI_STORE_F32: return launch_dma<EPI_STORE_F32>(g, s);
                case EPI_QKV: return launch_dma<EPI_QKV>(g, s);
                case EPI_RESID: return launch_dma<EPI_RESID>(g, s);
                case EPI_SWIGLU: return launch_dma<EPI_SWIGLU>(g, s);
            }
            return hipErrorInvalidValue;
        }
    }
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
