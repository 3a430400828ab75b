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
#include <algorithm>
#include <climits>
#include <utility>
#include <vector>

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

// Four keys of one V column packed for a single LDS store (sVt is [d][key]);
// rows[q] holds 16 bytes of key q.  Element extraction by shifts keeps the
// staging registers out of memory.
__device__ __forceinline__ uint32_t bf16_bits(const u32x4& r, int i) {
    return (r[i >> 1] >> ((i & 1) * 16)) & 0xFFFFu;
}
__device__ __forceinline__ void store_vt4(bf16* dst, const u32x4 (&rows)[4], int i) {
    const u32x2 w{bf16_bits(rows[0], i) | (bf16_bits(rows[1], i) << 16),
                  bf16_bits(rows[2], i) | (bf16_bits(rows[3], i) << 16)};
    *reinterpret_cast<u32x2*>(dst) = w;
}
__device__ __forceinline__ void store_vt4(float* dst, const u32x4 (&rows)[4], int i) {
    const u32x4 w{rows[0][i], rows[1][i], rows[2][i], rows[3][i]};
    *reinterpret_cast<u32x4*>(dst) = w;
}

template <typename T, int D>
__global__ __launch_bounds__(kThreads, 2) void attention_kernel(AttnArgs a, const AttnTiles tl) {
    constexpr int KB = AttnCfg<T>::KB;
    constexpr int LDK = D + 16 / (int)sizeof(T);        // sK row stride (elements)
    constexpr int LDV = KB + 4;                          // sVt row stride (elements)
    constexpr int NKT = KB / 16;                         // 16-key tiles per block
    constexpr int NKS = KB / 32;                         // 32-key MFMA steps per block
    constexpr int NDS = D / 32;                          // 32-dim steps for S
    constexpr int NDT = D / 16;                          // 16-dim output tiles
    constexpr int VEC = 16 / (int)sizeof(T);             // elements per 16-byte load
    constexpr int KU = KB * D / VEC / kThreads;          // K loads per thread per block
    constexpr int VUNITS = (KB / 4) * (D / VEC);         // V units of 4 keys x VEC dims
    static_assert(KU >= 1 && KB * D / VEC == KU * kThreads, "K tile split");
    static_assert(VUNITS <= kThreads, "V tile split");
    __shared__ __attribute__((aligned(16))) T sK[2][KB * LDK];
    __shared__ __attribute__((aligned(16))) T sVt[2][D * LDV];
    __shared__ int sred[2][kThreads / 64];

    const AttnRange& tile = tl.t[blockIdx.x];          // tiles come longest first
    const int n_kv = tile.n_kv;
    const int h = blockIdx.y;
    const int hk = h / (a.n_q_heads / a.n_kv_heads);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int fr = lane & 15, g = lane >> 4;
    const int q_ld = a.n_q_heads * D, kv_ld = a.n_kv_heads * D;

    // This lane's query (column of S^T).
    const int ql = wave * 16 + fr;
    const bool q_ok = ql < tile.nq;
    const int qi = tile.q0 + (q_ok ? ql : tile.nq - 1);
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
    const int nk = min(n_kv, bmax - a.kv_pos0 + 1);
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

    const T* kbase = static_cast<const T*>(a.k) + (int64_t)tile.g0 * kv_ld + hk * D;
    const T* vbase = static_cast<const T*>(a.v) + (int64_t)tile.g0 * kv_ld + hk * D;
    // Register staging of the next key block: K as KU 16-byte pieces of
    // single rows, V as 4 rows x 16 bytes so the transposed LDS image can be
    // written 4 keys at a time.  Rows past n_kv are clamped to the last key:
    // their scores are masked and the finite values they hold meet p = 0.
    u32x4 rk[KU], rv[4];
    const bool v_unit = tid < VUNITS;
    const int vr0 = (tid / (D / VEC)) * 4, vc = (tid % (D / VEC)) * VEC;
    auto load_block = [&](int kb) {
        const int k0 = kb * KB;
#pragma unroll
        for (int j = 0; j < KU; ++j) {
            const int u = tid + j * kThreads;
            const int r = u / (D / VEC), c = (u % (D / VEC)) * VEC;
            const int kr = min(k0 + r, n_kv - 1);
            rk[j] = *reinterpret_cast<const u32x4*>(kbase + (int64_t)kr * kv_ld + c);
        }
        if (v_unit) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int vr = min(k0 + vr0 + q, n_kv - 1);
                rv[q] = *reinterpret_cast<const u32x4*>(vbase + (int64_t)vr * kv_ld + vc);
            }
        }
    };
    auto store_block = [&](int buf) {
#pragma unroll
        for (int j = 0; j < KU; ++j) {
            const int u = tid + j * kThreads;
            const int r = u / (D / VEC), c = (u % (D / VEC)) * VEC;
            *reinterpret_cast<u32x4*>(&sK[buf][r * LDK + c]) = rk[j];
        }
        if (v_unit) {
#pragma unroll
            for (int i = 0; i < VEC; ++i) store_vt4(&sVt[buf][(vc + i) * LDV + vr0], rv, i);
        }
    };

    auto compute = [&](int cur, int kb) {
        const int k0 = kb * KB;
        if (a.kv_pos0 + k0 <= wmax) {     // wave-uniform: some key visible to this wave
            floatx4 st[NKT];
#pragma unroll
            for (int t = 0; t < NKT; ++t) {
                st[t] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < NDS; ++s) {
                    Frag<T> kf = load_frag<T>(&sK[cur][(t * 16 + fr) * LDK + s * 32 + g * 8]);
                    mfma16(st[t], kf, qf[s]);
                }
            }
            const bool need_mask = (k0 + KB > n_kv) || (a.kv_pos0 + k0 + KB - 1 > wmin);
            float mloc = -INFINITY;
#pragma unroll
            for (int t = 0; t < NKT; ++t)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float sc = st[t][e] * sl2;
                    if (need_mask) {
                        const int kj = k0 + t * 16 + g * 4 + e;
                        if (kj >= n_kv || a.kv_pos0 + kj > qpos) sc = -INFINITY;
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
                    const T* vr = &sVt[cur][(dt * 16 + fr) * LDV + s2 * 32 + g * 4];
                    mfma16(o[dt], load_quad_pair(vr), pf[s2]);
                }
            }
        }
    };
    // Steady state unrolled by two (static LDS buffers): on entry block kb is
    // in buffer 0; block kb+1 is fetched into registers during the math.
    if (n_kb > 0) {
        load_block(0);
        store_block(0);
    }
    __syncthreads();
    int kb = 0;
    for (; kb + 2 < n_kb; kb += 2) {
        load_block(kb + 1);
        __builtin_amdgcn_sched_barrier(0);
        compute(0, kb);
        store_block(1);
        __syncthreads();
        load_block(kb + 2);
        __builtin_amdgcn_sched_barrier(0);
        compute(1, kb + 1);
        store_block(0);
        __syncthreads();
    }
    if (kb + 1 < n_kb) {
        load_block(kb + 1);
        __builtin_amdgcn_sched_barrier(0);
        compute(0, kb);
        store_block(1);
        __syncthreads();
        compute(1, kb + 1);
    } else if (kb < n_kb) {
        compute(0, kb);
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

// ---------------------------------------------------------------------------
// bf16 path: 32 queries per wave on 32x32x16 MFMAs, four waves per
// workgroup (128 queries of one head), 64-key blocks.  Layout of
// v_mfma_f32_32x32x16_bf16: lane l supplies row (l % 32) of A and column
// (l % 32) of B with reduction elements 8 * (l / 32) + 0..7; accumulator
// element i of lane l is C[8 * (i / 4) + 4 * (l / 32) + i % 4][l % 32].
//
// K and V blocks go straight from memory into LDS (buffer_load ... lds: each
// instruction of a wave writes 64 x 16 B to consecutive LDS bytes), two
// stages: block kb+1 is copied while block kb is multiplied out.  LDS rows
// are unpadded; the 16-byte chunks of a row are stored at a swizzled slot
// (chunk ^ key(row)), and each lane fetches the global chunk that belongs in
// its slot.  A 64-key block gives each wave two independent 32-key score
// tiles (two MFMA chains in flight) and one softmax pass per 64 keys.
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void mfma32(floatx16& acc, const bf16x8& a, const bf16x8& b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
}

// Three-way maximum: the compiler forms v_max3_f32 from the pair of fmaxf
// (quieting only the first operands it cannot prove canonical), and, seeing
// that the scores come from MFMAs, places the wait states their results
// need before the first read.
__device__ __forceinline__ float vmax3(float a, float b, float c) {
    return fmaxf(fmaxf(a, b), c);
}

// max(x, x of lane ^ 32): the wave's two halves exchanged by a VALU permute
// (v_permlane32_swap: lanes 32-63 of the first operand trade places with
// lanes 0-31 of the second, here both x) instead of an LDS-routed shuffle.
__device__ __forceinline__ float max_xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

constexpr int kT32 = 256;   // threads per workgroup (4 waves)
constexpr int QT32 = 128;   // queries per workgroup
constexpr int KBL = 64;     // keys per block
constexpr float kLazyLog2 = 8.0f;   // rescale threshold of the running maximum (log2 units)
// (query tile, head, key segment) units wanted per launch.  Measured on
// MI355X, 832 queries x 4096 keys x 32 heads in the 7B step: 768 units
// (4 segments) 2.54 ms of attention + merge per step, 512 (3 segments)
// 2.58, 1024 (5 segments) 2.60, 1536 2.77; earlier, with a slower kernel,
// 2048 (8 segments) and 4096 (16 segments of 256 keys) were slower still.
constexpr int kSplitUnits = 768;
constexpr int kFewSegs = 4;   // the merge's one-round-trip path takes up to this many segments

// Hardware workgroup ids are dealt round-robin over the 8 XCDs; renumber so
// each XCD gets a contiguous logical range (blocks that read the same key
// segment of the same head then share one L2).
__device__ __forceinline__ int xcd_order(int hw, int total) {
    const int xcd = hw & 7, j = hw >> 3;
    const int base = total >> 3, rem = total & 7;
    return xcd * base + min(xcd, rem) + j;
}

// Raw buffer descriptor: base address, stride 0, range `bytes` (wave-uniform
// values, read from the first lane so the descriptor lives in SGPRs).
__device__ __forceinline__ i32x4 attn_rsrc(const void* base, int bytes) {
    const uint64_t p = reinterpret_cast<uint64_t>(base);
    return i32x4{__builtin_amdgcn_readfirstlane((int)(uint32_t)p),
                 __builtin_amdgcn_readfirstlane((int)((p >> 32) & 0xFFFF)),
                 __builtin_amdgcn_readfirstlane(bytes), 0x00020000};
}

// 16 bytes per lane from buffer offset voff into LDS at m0 + 16 * lane.
// Inline assembly keeps the compiler from treating it as an LDS store it
// must wait for; completion is tracked by explicit vmcnt waits and the
// "memory" clobber keeps LDS accesses from moving across the copy.  The
// s_nop is the one wait state the load needs after the write of M0, which
// the hazard recognizer cannot see inside the statement.
__device__ __forceinline__ void attn_dma16(i32x4 rsrc, int voff, uint32_t m0) {
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" : : "v"(voff), "s"(rsrc), "{m0}"(m0)
                 : "memory");
}

// Swizzle keys of the LDS rows (D*2 bytes each).  K is read as 16-byte
// fragments, 16 lanes at a time over 16 rows of one chunk column: the slots
// of 16 consecutive rows (D = 128) or of 8 rows of equal parity (D = 64,
// two rows per 256-byte bank window) must differ.  V is read by transposing
// 8-byte reads, 32 lanes at a time over 4 rows x 4 chunks: the 4 rows must
// move the chunk column by distinct multiples of 4 (D = 128) or, for D = 64,
// rows 2 apart (same bank half) must land in opposite 64-byte halves.
template <int D> __device__ __forceinline__ int k_key(int r) {
    return D == 128 ? (r & 15) : ((r >> 1) & 7);
}
template <int D> __device__ __forceinline__ int v_key(int r) {
    return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1);
}

template <int D>
__global__ __launch_bounds__(kT32, 2) void attention64_kernel(AttnArgs a, const AttnTiles tl) {
    constexpr int RB = D * 2;                  // bytes per LDS row
    constexpr int CPR = RB / 16;               // 16-byte chunks per row
    constexpr int RPI = 64 / CPR;              // rows per copy instruction
    constexpr int CPW = KBL / 4 / RPI;         // copy instructions per wave (K, and again V)
    constexpr int NDS = D / 16;                // 16-dim reduction steps for S
    constexpr int NDT = D / 32;                // 32-dim output tiles
    constexpr int BLK = KBL * RB;              // bytes of one K (or V) block
    static_assert(CPW >= 1 && CPW * RPI * 4 == KBL, "copy split");
    __shared__ __attribute__((aligned(16))) unsigned char smem[2 * 2 * BLK];   // [stage][K|V]
    __shared__ int sred[kT32 / 64];

    // logical id -> (tile, segment, head), tile fastest; tiles come longest first
    const int n_tiles = tl.n;
    const int n_segs = a.seg_keys > 0 ? a.max_seg : 1;
    const int logical = xcd_order(blockIdx.x, n_tiles * n_segs * a.n_q_heads);
    const int qt = logical % n_tiles;
    const int seg = (logical / n_tiles) % n_segs;
    const int h = logical / (n_tiles * n_segs);
    const AttnRange& tile = tl.t[qt];
    const int n_kv = tile.n_kv;
    const int hk = h / (a.n_q_heads / a.n_kv_heads);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int fr = lane & 31, g = lane >> 5;
    const int q_ld = a.n_q_heads * D, kv_ld = a.n_kv_heads * D;

    const int ql = wave * 32 + fr;
    const bool q_ok = ql < tile.nq;
    const int qi = tile.q0 + (q_ok ? ql : tile.nq - 1);
    const int qpos = a.q_pos[qi];
    int wmax = qpos, wmin = qpos;
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) {
        wmax = max(wmax, __shfl_xor(wmax, o, 64));
        wmin = min(wmin, __shfl_xor(wmin, o, 64));
    }
    if (lane == 0) sred[wave] = wmax;
    __syncthreads();
    int bmax = sred[0];
#pragma unroll
    for (int w = 1; w < kT32 / 64; ++w) bmax = max(bmax, sred[w]);
    const int nk = min(n_kv, bmax - a.kv_pos0 + 1);
    if (a.part_nk && seg == 0 && h == 0 && tid == 0) a.part_nk[qt] = nk;   // for the merge pass
    // Key segment of this workgroup (whole range when not split).
    const int n_seg = a.seg_keys > 0 ? max(1, (nk + a.seg_keys - 1) / a.seg_keys) : 1;
    if (seg >= n_seg) return;                          // uniform over the workgroup
    const int kb_beg = a.seg_keys > 0 ? seg * (a.seg_keys / KBL) : 0;
    const int k_end = a.seg_keys > 0 ? min(nk, (seg + 1) * a.seg_keys) : nk;
    const int n_kb = k_end > kb_beg * KBL ? (k_end - kb_beg * KBL + KBL - 1) / KBL : 0;

    const int qrow = a.qidx ? a.qidx[qi] : qi;
    const bf16* qp = static_cast<const bf16*>(a.q) + (int64_t)qrow * q_ld + h * D;
    bf16x8 qf[NDS];
#pragma unroll
    for (int s = 0; s < NDS; ++s) qf[s] = *reinterpret_cast<const bf16x8*>(qp + s * 16 + g * 8);

    floatx16 o[NDT];
#pragma unroll
    for (int t = 0; t < NDT; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[t][i] = 0.f;
    float m_run = -INFINITY;
    // Softmax denominator: the lane's share of its query's probabilities
    // (lanes l and l + 32 hold the two halves of every key block).
    float l_part = 0.f;
    const float sl2 = 1.4426950408889634f / sqrtf((float)D);

    const bf16* kbase = static_cast<const bf16*>(a.k) + (int64_t)tile.g0 * kv_ld + hk * D;
    const bf16* vbase = static_cast<const bf16*>(a.v) + (int64_t)tile.g0 * kv_ld + hk * D;
    // Copies: wave w fills rows 16 w .. 16 w + 15 of the K and V blocks, RPI
    // rows per instruction; lane l of instruction c goes to row
    // 16 w + RPI c + l / CPR, slot l % CPR, and fetches the chunk stored there.
    int k_voff[CPW], v_voff[CPW];
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
        const int r = 16 * wave + RPI * c + lane / CPR, slot = lane % CPR;
        k_voff[c] = r * kv_ld * 2 + ((slot ^ k_key<D>(r)) & (CPR - 1)) * 16;
        v_voff[c] = r * kv_ld * 2 + ((slot ^ v_key<D>(r)) & (CPR - 1)) * 16;
    }
    const uint32_t lds0 = (uint32_t)reinterpret_cast<uintptr_t>(smem);
    auto issue = [&](int kb, int st) {
        const int k0 = (kb_beg + kb) * KBL;
        const int rows = min(KBL, n_kv - k0);      // rows past the last key read as zero
        const i32x4 rk = attn_rsrc(kbase + (int64_t)k0 * kv_ld, rows * kv_ld * 2);
        const i32x4 rv = attn_rsrc(vbase + (int64_t)k0 * kv_ld, rows * kv_ld * 2);
        const uint32_t kd = lds0 + st * 2 * BLK + 16 * wave * RB;
#pragma unroll
        for (int c = 0; c < CPW; ++c) {
            attn_dma16(rk, k_voff[c], kd + c * RPI * RB);
            attn_dma16(rv, v_voff[c], kd + BLK + c * RPI * RB);
        }
    };
    // K fragment (row kr, dims 16 s + 8 g ..) and transposed V reads: within
    // each 16-lane group the transposing read hands lane j the j-th column of
    // the 4 x 16 block the group addresses (lane s points at row s / 4,
    // columns 4 (s % 4) .. +3), so lane l gets 4 consecutive keys of one dimension.
    const int kkey = k_key<D>(fr);                          // same for rows fr + 32
    const int tr_g = lane >> 4, tr_s = lane & 15;
    const int tr_row = 4 * (tr_g >> 1) + (tr_s >> 2);       // + 16 q4 (+ 8 for the upper half)
    const int tr_col = 16 * (tr_g & 1) + 4 * (tr_s & 3);    // + 32 dt
    const int vkey = v_key<D>(tr_row);                      // same for rows tr_row + 8 j
    // A wave whose 32 query slots all lie past the tile's last query (the
    // short last tile of a range) has nothing to compute; it still copies its
    // share of every block and meets every barrier.
    const bool wave_live = wave * 32 < tile.nq;
    auto compute = [&](int st, int kb) {
        const int k0 = (kb_beg + kb) * KBL;
        if (!wave_live || a.kv_pos0 + k0 > wmax) return;   // wave-uniform
        const unsigned char* sk = smem + st * 2 * BLK;
        const unsigned char* sv = sk + BLK;
        // S^T = K Q^T for the block's two 32-key halves: K fragments are read
        // two reduction steps ahead of their MFMAs so the LDS latency hides
        // behind the two independent MFMA chains.
        floatx16 s2[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int i = 0; i < 16; ++i) s2[hh][i] = 0.f;
        bf16x8 k_lo[3], k_hi[3];
        auto read_k = [&](int s) {
            const int off = fr * RB + (((2 * s + g) ^ kkey) & (CPR - 1)) * 16;
            k_lo[s % 3] = *reinterpret_cast<const bf16x8*>(sk + off);
            k_hi[s % 3] = *reinterpret_cast<const bf16x8*>(sk + off + 32 * RB);
        };
        read_k(0);
        read_k(1);
#pragma unroll
        for (int s = 0; s < NDS; ++s) {
            if (s + 2 < NDS) read_k(s + 2);
            mfma32(s2[0], k_lo[s % 3], qf[s]);
            mfma32(s2[1], k_hi[s % 3], qf[s]);
        }
        // keep that order: the scheduler would otherwise sink each read to
        // its MFMA and expose the LDS latency at every step
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);           // reads of steps 0, 1
#pragma unroll
        for (int s = 0; s < NDS; ++s) {
            if (s + 2 < NDS) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // step s + 2
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);                    // step s
        }
        // Scores stay unscaled; the running max is kept in scaled (log2)
        // units and the scale is folded into one FMA before v_exp_f32.
        const bool need_mask = (k0 + KBL > n_kv) || (a.kv_pos0 + k0 + KBL - 1 > wmin);
        if (need_mask) {
            // key k0 + 4 g + c (c a compile-time offset) is visible iff c <= lim
            const int lim = min(n_kv - 1, qpos - a.kv_pos0) - k0 - 4 * g;
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (32 * hh + 8 * (i >> 2) + (i & 3) > lim) s2[hh][i] = -INFINITY;
        }
        float mloc = vmax3(s2[0][0], s2[1][0], s2[0][1]);
#pragma unroll
        for (int i = 1; i < 16; ++i)
            mloc = i == 1 ? vmax3(mloc, s2[1][1], s2[1][1]) : vmax3(mloc, s2[0][i], s2[1][i]);
        mloc = max_xor32(mloc) * sl2;
        // The reference maximum only moves when a score exceeds it by more
        // than kLazyLog2 (probabilities then stay below 2^kLazyLog2): after
        // the first keys O and l are rarely rescaled.  Any reference gives
        // the same normalized result; the merge pass combines segments by
        // their own references.
        const bool grow = mloc > m_run + kLazyLog2;      // false for an all-masked block
        const float m_new = grow ? mloc : m_run;
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        if (__ballot(grow)) {
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
            l_part *= alpha;
#pragma unroll
            for (int t = 0; t < NDT; ++t) o[t] *= alpha;
        }
        m_run = m_new;
        // Per 16-key group q4: its transposed V reads first (they do not
        // depend on P), then the group's probabilities, added to the lane's
        // share of the denominator in fp32 before their rounding to bf16 for
        // the MFMAs (the two differ by the mean rounding error of the
        // probabilities, a relative 2^-9 / sqrt(keys)), then one MFMA per
        // 32-dim output tile (independent accumulators).
        // P^T slot j of group q4 = 2 hh + j / 8 holds key
        // 32 hh + 16 (j / 8) + 8 ((j % 8) / 4) + 4 g + j % 4: the key order
        // of the transposed V reads.
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            typedef short i16x4 __attribute__((ext_vector_type(4)));
            typedef short i16x8 __attribute__((ext_vector_type(8)));
            typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
            bf16x8 vf[NDT];
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
                const int col = dt * 32 + tr_col;
                const int off = (16 * q4 + tr_row) * RB + ((((col >> 3) ^ vkey) & (CPR - 1)) << 4) +
                                (col & 7) * 2;
                const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(sv + off));
                const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(sv + off + 8 * RB));
                vf[dt] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            }
            bf16x8 pf;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float e = __builtin_amdgcn_exp2f(fmaf(s2[q4 >> 1][(q4 & 1) * 8 + j], sl2, -m_use));
                l_part += e;
                pf[j] = static_cast<bf16>(e);
            }
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) mfma32(o[dt], vf[dt], pf);
        }
    };
    // Two stages: block kb+1 is copied into the other stage while block kb is
    // multiplied out; the wait + barrier at the end publishes it (and tells
    // every wave that stage kb's buffer is free again).
    if (n_kb > 0) {
        issue(0, 0);
        __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));   // vmcnt(0)
        __syncthreads();
    }
    for (int kb = 0; kb < n_kb; ++kb) {
        const int st = kb & 1;
        if (kb + 1 < n_kb) issue(kb + 1, st ^ 1);
        compute(st, kb);
        __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));   // vmcnt(0)
        __syncthreads();
    }
    const float l_tot = l_part + __shfl_xor(l_part, 32, 64);
    if (n_seg > 1) {
        // Partial of this segment: O normalized by the segment's own sum (bf16,
        // half the bytes of the unnormalized float sums), running max (log2
        // units) and sum.
        const int64_t slot = ((int64_t)qt * a.n_q_heads + h) * a.max_seg + seg;
        bf16* po = a.part_o + (slot * QT32 + ql) * D;
        const float inv_s = l_tot > 0.f ? 1.0f / l_tot : 0.f;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4)
                *reinterpret_cast<bf16x4*>(po + dt * 32 + 8 * i4 + 4 * g) =
                    bf16x4{static_cast<bf16>(o[dt][i4 * 4] * inv_s),
                           static_cast<bf16>(o[dt][i4 * 4 + 1] * inv_s),
                           static_cast<bf16>(o[dt][i4 * 4 + 2] * inv_s),
                           static_cast<bf16>(o[dt][i4 * 4 + 3] * inv_s)};
        if (g == 0) {
            float* pm = a.part_ml + (slot * QT32 + ql) * 2;
            pm[0] = m_run;
            pm[1] = l_tot;
        }
        return;
    }
    if (!q_ok) return;
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    bf16* op = static_cast<bf16*>(a.out) + (int64_t)qi * q_ld + h * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
            bf16x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = static_cast<bf16>(o[dt][i4 * 4 + e] * inv);
            *reinterpret_cast<bf16x4*>(op + dt * 32 + 8 * i4 + 4 * g) = v;
        }
}

// Merges the segment partials of split tiles: with per-segment max m_s and
// sum l_s, O = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s, M = max_s m_s.
// Tiles that were not split were finished by their only workgroup.  D/8
// threads per query, 8 output dims each (16-byte loads of the bf16
// partials); a workgroup covers 2048 / D queries of one tile and head, so
// the merge is spread over the whole GPU.  The number of segments of a tile
// comes from the visible-key count its attention workgroups recorded.
template <int D>
__global__ __launch_bounds__(256) void attention_combine_kernel(AttnArgs a, const AttnTiles tl) {
    constexpr int TPQ = D / 8;                      // threads per query
    constexpr int QPW = 256 / TPQ;                  // queries per workgroup
    const int per_tile = QT32 / QPW;
    const int qt = blockIdx.x / per_tile, qg = blockIdx.x % per_tile;
    const int h = blockIdx.y;
    const AttnRange& tile = tl.t[qt];
    const int ql = qg * QPW + (int)threadIdx.x / TPQ;
    if (ql >= tile.nq) return;
    const int c = ((int)threadIdx.x % TPQ) * 8;
    const int64_t slot0 = ((int64_t)qt * a.n_q_heads + h) * a.max_seg;
    bf16* dst = static_cast<bf16*>(a.out) + (int64_t)(tile.q0 + ql) * a.n_q_heads * D + h * D + c;
    if (a.max_seg <= kFewSegs) {
        // Up to kFewSegs segments: every slot's partial is loaded together
        // with the segment count, one round trip instead of three (slots
        // past max_seg repeat the last one and are never used).
        float2 ml[kFewSegs];
        bf16x8 ov[kFewSegs];
#pragma unroll
        for (int sg = 0; sg < kFewSegs; ++sg) {
            const int64_t sl = slot0 + min(sg, a.max_seg - 1);
            ml[sg] = *reinterpret_cast<const float2*>(a.part_ml + (sl * QT32 + ql) * 2);
            ov[sg] = *reinterpret_cast<const bf16x8*>(a.part_o + (sl * QT32 + ql) * D + c);
        }
        const int n_seg = max(1, (a.part_nk[qt] + a.seg_keys - 1) / a.seg_keys);
        if (n_seg <= 1) return;
        float M = -INFINITY;
#pragma unroll
        for (int sg = 0; sg < kFewSegs; ++sg)
            if (sg < n_seg) M = fmaxf(M, ml[sg].x);
        const float Mu = M == -INFINITY ? 0.f : M;
        float L = 0.f;
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int sg = 0; sg < kFewSegs; ++sg) {
            if (sg >= n_seg) break;
            const float wl = __builtin_amdgcn_exp2f(ml[sg].x - Mu) * ml[sg].y;
            L += wl;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] += wl * static_cast<float>(ov[sg][e]);
        }
        const float inv = L > 0.f ? 1.0f / L : 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] *= inv;
        Vec8<bf16>::store(dst, acc);
        return;
    }
    const int n_seg = max(1, (a.part_nk[qt] + a.seg_keys - 1) / a.seg_keys);
    if (n_seg <= 1) return;
    float M = -INFINITY;
    for (int sg = 0; sg < n_seg; ++sg)
        M = fmaxf(M, a.part_ml[((slot0 + sg) * QT32 + ql) * 2]);
    const float Mu = M == -INFINITY ? 0.f : M;
    float L = 0.f;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int sg = 0; sg < n_seg; ++sg) {
        const float* pm = a.part_ml + ((slot0 + sg) * QT32 + ql) * 2;
        float ov[8];
        Vec8<bf16>::load(a.part_o + ((slot0 + sg) * QT32 + ql) * D + c, ov);
        const float wl = __builtin_amdgcn_exp2f(pm[0] - Mu) * pm[1];   // weight x segment sum
        L += wl;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += wl * ov[e];
    }
    const float inv = L > 0.f ? 1.0f / L : 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= inv;
    Vec8<bf16>::store(dst, acc);
}

// Query tiles of height `qth` cut from the ranges, ordered by an estimate of
// their visible keys (rows of a range ascend in position, so later tiles of
// a range see more keys), longest first; stable for equal estimates.
std::vector<AttnRange> make_tiles(const AttnRange* r, int n_r, int qth) {
    std::vector<std::pair<double, AttnRange>> w;
    for (int i = 0; i < n_r; ++i) {
        const AttnRange& x = r[i];
        for (int q = 0; q < x.nq; q += qth) {
            const AttnRange t{x.q0 + q, std::min(qth, x.nq - q), x.g0, x.n_kv};
            w.push_back({(double)x.n_kv * (q + t.nq) / x.nq, t});
        }
    }
    std::stable_sort(w.begin(), w.end(),
                     [](const auto& a, const auto& b) { return a.first > b.first; });
    std::vector<AttnRange> out(w.size());
    for (size_t i = 0; i < w.size(); ++i) out[i] = w[i].second;
    return out;
}

// Split plan of one launch of n tiles: segments of 512 keys when the plain
// grid leaves the GPU short of workgroups.
struct SplitPlan {
    int seg_keys = 0, max_seg = 1;
    size_t bytes = 0;
};
SplitPlan split_plan(const AttnRange* t, int n, int n_q_heads, int head_dim) {
    SplitPlan p;
    int max_kv = 0;
    for (int i = 0; i < n; ++i) max_kv = std::max(max_kv, t[i].n_kv);
    const int64_t units = (int64_t)n * n_q_heads;
    if (units >= kSplitUnits || max_kv <= 1024) return p;
    // Enough segments for ~kSplitUnits work units (the partials cost HBM
    // traffic), each at least 512 keys long.
    const int want = (int)std::min<int64_t>((kSplitUnits + units - 1) / units,
                                            (max_kv + 511) / 512);
    p.seg_keys = ((max_kv + want - 1) / want + KBL - 1) / KBL * KBL;
    p.max_seg = (max_kv + p.seg_keys - 1) / p.seg_keys;
    if (p.max_seg <= 1) return SplitPlan{};
    p.bytes = (size_t)n * n_q_heads * p.max_seg * QT32 * (head_dim * sizeof(bf16) + 2 * sizeof(float)) +
              (size_t)n * sizeof(int);
    return p;
}

template <int D>
hipError_t launch32(const AttnArgs& a0, const AttnTiles& tl, void* ws, size_t ws_bytes,
                    hipStream_t s) {
    const SplitPlan sp = split_plan(tl.t, tl.n, a0.n_q_heads, D);
    AttnArgs a = a0;
    a.seg_keys = sp.seg_keys;
    a.max_seg = sp.max_seg;
    a.part_o = nullptr;
    a.part_ml = nullptr;
    a.part_nk = nullptr;
    if (sp.bytes) {
        if (!ws || ws_bytes < sp.bytes) return hipErrorInvalidValue;
        a.part_o = static_cast<bf16*>(ws);
        a.part_ml = reinterpret_cast<float*>(a.part_o + (size_t)tl.n * a.n_q_heads * sp.max_seg * QT32 * D);
        a.part_nk = reinterpret_cast<int*>(a.part_ml + (size_t)tl.n * a.n_q_heads * sp.max_seg * QT32 * 2);
    }
    const int64_t blocks = (int64_t)tl.n * a.n_q_heads * a.max_seg;
    if (blocks > INT_MAX) return hipErrorInvalidValue;
    hipLaunchKernelGGL((attention64_kernel<D>), dim3((unsigned)blocks), dim3(kT32), 0, s, a, tl);
    if (sp.bytes)
        hipLaunchKernelGGL((attention_combine_kernel<D>), dim3(tl.n * (QT32 / (256 / (D / 8))), a.n_q_heads),
                           dim3(256), 0, s, a, tl);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_t(const AttnArgs& a, const AttnTiles& tl, hipStream_t s) {
    hipLaunchKernelGGL((attention_kernel<T, D>), dim3(tl.n, a.n_q_heads), dim3(kThreads), 0, s, a,
                       tl);
    return hipGetLastError();
}

int tile_height(int dtype) { return dtype == BF16 ? QT32 : QT; }

// Per-token attention deviation (CacheBlend explainer (0h-n0), eq. 2 taken
// row by row, the first-layer rule of HKVD selection): for query row j of a
// request whose every chunk row is recomputed, and query head h,
//   dev_h[j] = sum_k (p1[k] - p0[k])^2,
// p1 / p0 the causal softmax rows of q_j over the recomputed keys and over
// the cached keys of the chunk positions 0..j.  One pass over the keys with
// the running maxima m1, m0 and sums l1 = sum e1, l0 = sum e0, A = sum e1^2,
// B = sum e1 e0, C = sum e0^2 (e = 2^(score - m), rescaled as m grows):
//   dev_h = A / l1^2 - 2 B / (l1 l0) + C / l0^2,
// which is sum (e1/l1 - e0/l0)^2 expanded.  Same tiles, LDS layout and
// score MFMAs as attention64_kernel, with the block of recomputed keys in
// place of V.  part[h][row] receives dev_h of every query row.
template <int D>
__global__ __launch_bounds__(kT32, 2) void attn_dev_kernel(AttnDevArgs a, const AttnDevTiles tl) {
    constexpr int RB = D * 2, CPR = RB / 16, RPI = 64 / CPR, CPW = KBL / 4 / RPI;
    constexpr int NDS = D / 16, BLK = KBL * RB;
    static_assert(CPW >= 1 && CPW * RPI * 4 == KBL, "copy split");
    __shared__ __attribute__((aligned(16))) unsigned char smem[2 * 2 * BLK];   // [stage][new|cached]
    __shared__ int sred[kT32 / 64];

    const int logical = xcd_order(blockIdx.x, tl.n * a.n_q_heads);
    const int qt = logical % tl.n, h = logical / tl.n;
    const AttnDevTile& tile = tl.t[qt];
    const int hk = h / (a.n_q_heads / a.n_kv_heads);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int fr = lane & 31, g = lane >> 5;
    const int q_ld = a.n_q_heads * D, kv_ld = a.n_kv_heads * D;

    // query j (= its position, 0-based within the request's chunk rows)
    const int ql = wave * 32 + fr;
    const bool q_ok = ql < tile.nq;
    const int qpos = tile.j0 + (q_ok ? ql : tile.nq - 1);
    int wmax = qpos, wmin = qpos;
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) {
        wmax = max(wmax, __shfl_xor(wmax, o, 64));
        wmin = min(wmin, __shfl_xor(wmin, o, 64));
    }
    if (lane == 0) sred[wave] = wmax;
    __syncthreads();
    int bmax = sred[0];
#pragma unroll
    for (int w = 1; w < kT32 / 64; ++w) bmax = max(bmax, sred[w]);
    const int nk = bmax + 1;                          // keys 0..bmax
    const int n_kb = (nk + KBL - 1) / KBL;

    const bf16* qp = static_cast<const bf16*>(a.q) + (int64_t)(tile.q_row0 + qpos) * q_ld + h * D;
    bf16x8 qf[NDS];
#pragma unroll
    for (int s = 0; s < NDS; ++s) qf[s] = *reinterpret_cast<const bf16x8*>(qp + s * 16 + g * 8);

    const bf16* k1base = static_cast<const bf16*>(a.k_new) + (int64_t)tile.k_new_row0 * kv_ld + hk * D;
    const bf16* k0base = static_cast<const bf16*>(a.k_cached) + (int64_t)tile.k_cached_row0 * kv_ld + hk * D;
    int k_voff[CPW];
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
        const int r = 16 * wave + RPI * c + lane / CPR, slot = lane % CPR;
        k_voff[c] = r * kv_ld * 2 + ((slot ^ k_key<D>(r)) & (CPR - 1)) * 16;
    }
    const uint32_t lds0 = (uint32_t)reinterpret_cast<uintptr_t>(smem);
    auto issue = [&](int kb, int st) {
        const int k0 = kb * KBL;
        const int rows = min(KBL, tile.n_keys - k0);   // rows past the last key read as zero
        const i32x4 r1 = attn_rsrc(k1base + (int64_t)k0 * kv_ld, rows * kv_ld * 2);
        const i32x4 r0 = attn_rsrc(k0base + (int64_t)k0 * kv_ld, rows * kv_ld * 2);
        const uint32_t d = lds0 + st * 2 * BLK + 16 * wave * RB;
#pragma unroll
        for (int c = 0; c < CPW; ++c) {
            attn_dma16(r1, k_voff[c], d + c * RPI * RB);
            attn_dma16(r0, k_voff[c], d + BLK + c * RPI * RB);
        }
    };
    const int kkey = k_key<D>(fr);
    const float sl2 = 1.4426950408889634f / sqrtf((float)D);
    float m1 = -INFINITY, m0 = -INFINITY, l1 = 0.f, l0 = 0.f, A = 0.f, B = 0.f, C = 0.f;
    auto scores = [&](const unsigned char* sk, floatx16 (&s2)[2]) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int i = 0; i < 16; ++i) s2[hh][i] = 0.f;
#pragma unroll
        for (int s = 0; s < NDS; ++s) {
            const int off = fr * RB + (((2 * s + g) ^ kkey) & (CPR - 1)) * 16;
            mfma32(s2[0], *reinterpret_cast<const bf16x8*>(sk + off), qf[s]);
            mfma32(s2[1], *reinterpret_cast<const bf16x8*>(sk + off + 32 * RB), qf[s]);
        }
    };
    auto compute = [&](int st, int kb) {
        const int k0 = kb * KBL;
        if (k0 > wmax) return;                          // wave-uniform: nothing visible
        floatx16 s1[2], s0[2];
        scores(smem + st * 2 * BLK, s1);
        scores(smem + st * 2 * BLK + BLK, s0);
        if (k0 + KBL - 1 > wmin) {
            // key k0 + 4 g + c is visible iff c <= lim (query j sees keys 0..j)
            const int lim = qpos - k0 - 4 * g;
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (32 * hh + 8 * (i >> 2) + (i & 3) > lim) {
                        s1[hh][i] = -INFINITY;
                        s0[hh][i] = -INFINITY;
                    }
        }
        // Scores in log2 units first, so that the largest key's term is
        // exactly 2^0, and both key sets through the same rounded operations
        // (no contraction into FMAs, which the compiler could apply to one
        // set and not the other): identical key sets give identical terms.
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                s1[hh][i] = __fmul_rn(s1[hh][i], sl2);
                s0[hh][i] = __fmul_rn(s0[hh][i], sl2);
            }
        float b1 = vmax3(s1[0][0], s1[1][0], s1[0][1]), b0 = vmax3(s0[0][0], s0[1][0], s0[0][1]);
#pragma unroll
        for (int i = 1; i < 16; ++i) {
            b1 = i == 1 ? vmax3(b1, s1[1][1], s1[1][1]) : vmax3(b1, s1[0][i], s1[1][i]);
            b0 = i == 1 ? vmax3(b0, s0[1][1], s0[1][1]) : vmax3(b0, s0[0][i], s0[1][i]);
        }
        b1 = fmaxf(b1, __shfl_xor(b1, 32, 64));
        b0 = fmaxf(b0, __shfl_xor(b0, 32, 64));
        // the query's own key is in the first block that reaches it, so
        // the maxima are finite from the first visible block on
        const float n1 = fmaxf(m1, b1), n0 = fmaxf(m0, b0);
        const float f1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - n1);
        const float f0 = m0 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m0 - n0);
        l1 = __fmul_rn(l1, f1);
        l0 = __fmul_rn(l0, f0);
        A = __fmul_rn(A, __fmul_rn(f1, f1));
        B = __fmul_rn(B, __fmul_rn(f1, f0));
        C = __fmul_rn(C, __fmul_rn(f0, f0));
        m1 = n1; m0 = n0;
        const float u1 = n1 == -INFINITY ? 0.f : n1, u0 = n0 == -INFINITY ? 0.f : n0;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float e1 = __builtin_amdgcn_exp2f(__fsub_rn(s1[hh][i], u1));
                const float e0 = __builtin_amdgcn_exp2f(__fsub_rn(s0[hh][i], u0));
                l1 += e1;
                l0 += e0;
                A = fmaf(e1, e1, A);
                B = fmaf(e1, e0, B);
                C = fmaf(e0, e0, C);
            }
    };
    if (n_kb > 0) {
        issue(0, 0);
        __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));   // vmcnt(0)
        __syncthreads();
    }
    for (int kb = 0; kb < n_kb; ++kb) {
        const int st = kb & 1;
        if (kb + 1 < n_kb) issue(kb + 1, st ^ 1);
        compute(st, kb);
        __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));   // vmcnt(0)
        __syncthreads();
    }
    // lanes l and l ^ 32 hold the same query's two halves of every block
    // (same maxima): add their sums
    l1 += __shfl_xor(l1, 32, 64);
    l0 += __shfl_xor(l0, 32, 64);
    A += __shfl_xor(A, 32, 64);
    B += __shfl_xor(B, 32, 64);
    C += __shfl_xor(C, 32, 64);
    if (!q_ok || g) return;
    // (A/l1^2 - B/(l1 l0)) + (C/l0^2 - B/(l1 l0)), each product rounded on its
    // own (no contraction): identical key sets give exactly zero
    const float i1 = 1.f / l1, i0 = 1.f / l0;
    const float ta = __fmul_rn(__fmul_rn(A, i1), i1);
    const float tb = __fmul_rn(__fmul_rn(B, i1), i0);
    const float tc = __fmul_rn(__fmul_rn(C, i0), i0);
    const float dev = fmaxf(0.f, __fadd_rn(__fsub_rn(ta, tb), __fsub_rn(tc, tb)));
    a.part[(int64_t)h * a.part_stride + tile.q_row0 + qpos] = dev;
}

// out[c_off + j] = sum over heads (in head order) of part[h][row0 + j].
__global__ __launch_bounds__(256) void attn_dev_sum_kernel(const float* __restrict__ part,
                                                           int64_t part_stride, int n_heads,
                                                           const AttnDevSums t,
                                                           float* __restrict__ out) {
    const AttnDevSum& r = t.r[blockIdx.y];
    const int j = blockIdx.x * 256 + threadIdx.x;
    if (j >= r.n) return;
    float s = 0.f;
    for (int h = 0; h < n_heads; ++h) s += part[(int64_t)h * part_stride + r.row0 + j];
    out[r.out0 + j] = s;
}

}  // namespace

size_t attention_workspace(int dtype, const AttnRange* r, int n_r, int n_q_heads, int head_dim) {
    if (dtype != BF16 || n_r <= 0) return 0;
    const std::vector<AttnRange> tiles = make_tiles(r, n_r, tile_height(dtype));
    size_t need = 0;
    for (size_t i = 0; i < tiles.size(); i += kMaxAttnTiles) {
        const int n = (int)std::min<size_t>(kMaxAttnTiles, tiles.size() - i);
        need = std::max(need, split_plan(&tiles[i], n, n_q_heads, head_dim).bytes);
    }
    return need;
}

hipError_t launch_attention(int dtype, const AttnArgs& a, const AttnRange* r, int n_r, void* ws,
                            size_t ws_bytes, hipStream_t s) {
    if (n_r <= 0) return hipSuccess;
    if (a.n_kv_heads <= 0 || a.n_q_heads % a.n_kv_heads != 0) return hipErrorInvalidValue;
    if (a.head_dim != 64 && a.head_dim != 128) return hipErrorInvalidValue;
    for (int i = 0; i < n_r; ++i)
        if (r[i].nq < 0 || (r[i].nq > 0 && r[i].n_kv <= 0)) return hipErrorInvalidValue;
    const std::vector<AttnRange> tiles = make_tiles(r, n_r, tile_height(dtype));
    for (size_t i = 0; i < tiles.size(); i += kMaxAttnTiles) {
        AttnTiles tl;
        tl.n = (int)std::min<size_t>(kMaxAttnTiles, tiles.size() - i);
        for (int j = 0; j < tl.n; ++j) tl.t[j] = tiles[i + j];
        hipError_t e;
        if (dtype == BF16)
            e = a.head_dim == 128 ? launch32<128>(a, tl, ws, ws_bytes, s)
                                  : launch32<64>(a, tl, ws, ws_bytes, s);
        else
            e = a.head_dim == 128 ? launch_t<float, 128>(a, tl, s) : launch_t<float, 64>(a, tl, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

size_t attention_deviation_workspace(int n_q_heads, int64_t rows) {
    return (size_t)n_q_heads * (size_t)std::max<int64_t>(rows, 1) * sizeof(float);
}

hipError_t launch_attention_deviation(int dtype, const AttnDevArgs& a0, const AttnDevReq* r,
                                      int n_r, float* out, hipStream_t s) {
    if (n_r <= 0) return hipSuccess;
    if (dtype != BF16 || (a0.head_dim != 64 && a0.head_dim != 128) || a0.n_kv_heads <= 0 ||
        a0.n_q_heads % a0.n_kv_heads != 0 || !a0.part || a0.part_stride <= 0)
        return hipErrorInvalidValue;
    std::vector<AttnDevTile> tiles;
    for (int i = 0; i < n_r; ++i) {
        if (r[i].n < 0 || (int64_t)r[i].q_row0 + r[i].n > a0.part_stride) return hipErrorInvalidValue;
        for (int j = 0; j < r[i].n; j += QT32)
            tiles.push_back(AttnDevTile{r[i].q_row0, j, std::min(QT32, r[i].n - j),
                                        r[i].k_new_row0, r[i].k_cached_row0, r[i].n});
    }
    // longest first (later tiles see more keys)
    std::stable_sort(tiles.begin(), tiles.end(), [](const AttnDevTile& x, const AttnDevTile& y) {
        return x.j0 + x.nq > y.j0 + y.nq;
    });
    for (size_t i = 0; i < tiles.size(); i += kMaxAttnTiles) {
        AttnDevTiles tl;
        tl.n = (int)std::min<size_t>(kMaxAttnTiles, tiles.size() - i);
        for (int j = 0; j < tl.n; ++j) tl.t[j] = tiles[i + j];
        const dim3 grid((unsigned)(tl.n * a0.n_q_heads));
        if (a0.head_dim == 128)
            hipLaunchKernelGGL((attn_dev_kernel<128>), grid, dim3(kT32), 0, s, a0, tl);
        else
            hipLaunchKernelGGL((attn_dev_kernel<64>), grid, dim3(kT32), 0, s, a0, tl);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    for (int i = 0; i < n_r; i += kMaxReq) {
        AttnDevSums t{};
        t.n = std::min(kMaxReq, n_r - i);
        int max_n = 0;
        for (int j = 0; j < t.n; ++j) {
            t.r[j] = AttnDevSum{r[i + j].q_row0, r[i + j].out0, r[i + j].n};
            max_n = std::max(max_n, r[i + j].n);
        }
        if (max_n == 0) continue;
        hipLaunchKernelGGL(attn_dev_sum_kernel, dim3((max_n + 255) / 256, t.n), dim3(256), 0, s,
                           a0.part, a0.part_stride, a0.n_q_heads, t, out);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace cb
