// Internal helpers shared by the gfx950 kernels and the runtime.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cb {

using bf16 = __bf16;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

enum DType : int { F32 = 0, BF16 = 1 };

__host__ __device__ inline int elem_size(int dtype) { return dtype == BF16 ? 2 : 4; }

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return static_cast<float>(x); }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
// gfx950 converts with round-to-nearest-even in hardware.
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return static_cast<bf16>(x); }

// A fragment: 8 consecutive reduction-dim elements held by one lane.
template <typename T> struct Frag;
template <> struct Frag<bf16> { bf16x8 v; };
template <> struct Frag<float> { floatx8 v; };

// 16x16 output tile += A(16 x 32) * B(32 x 16).  Lane l supplies row (l % 16)
// of A and column (l % 16) of B with the 8 reduction elements of lane group
// l / 16; the accumulator holds C[4 * (l / 16) + i][l % 16], i = 0..3.
// bf16: one v_mfma_f32_16x16x32_bf16.  f32: eight v_mfma_f32_16x16x4_f32,
// the j-th taking element j of every lane (a fixed permutation of the
// reduction index, identical on both operands).
__device__ __forceinline__ void mfma16(floatx4& acc, const Frag<bf16>& a, const Frag<bf16>& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, acc, 0, 0, 0);
}
__device__ __forceinline__ void mfma16(floatx4& acc, const Frag<float>& a, const Frag<float>& b) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[j], b.v[j], acc, 0, 0, 0);
}

template <typename T>
__device__ __forceinline__ Frag<T> load_frag(const T* p);   // 8 contiguous elements
template <> __device__ __forceinline__ Frag<bf16> load_frag<bf16>(const bf16* p) {
    Frag<bf16> f;
    f.v = *reinterpret_cast<const bf16x8*>(p);
    return f;
}
template <> __device__ __forceinline__ Frag<float> load_frag<float>(const float* p) {
    Frag<float> f;
    floatx4 a = *reinterpret_cast<const floatx4*>(p);
    floatx4 b = *reinterpret_cast<const floatx4*>(p + 4);
    f.v = floatx8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    return f;
}

// The same 8 elements read with the non-temporal hint, for operands that
// are streamed once and not read again soon (chunk caches, cached rows):
// they then displace less of what the next kernels read from the caches.
template <typename T>
__device__ __forceinline__ Frag<T> load_frag_nt(const T* p);
template <> __device__ __forceinline__ Frag<bf16> load_frag_nt<bf16>(const bf16* p) {
    Frag<bf16> f;
    f.v = __builtin_bit_cast(bf16x8, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)));
    return f;
}
template <> __device__ __forceinline__ Frag<float> load_frag_nt<float>(const float* p) {
    Frag<float> f;
    const floatx4 a = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(p));
    const floatx4 b = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(p + 4));
    f.v = floatx8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    return f;
}

// 8 consecutive elements of a row, loaded to / stored from float registers.
template <typename T> struct Vec8;
template <> struct Vec8<bf16> {
    static __device__ __forceinline__ void load(const bf16* p, float* x) {
        bf16x8 v = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = static_cast<float>(v[i]);
    }
    static __device__ __forceinline__ void store(bf16* p, const float* x) {
        bf16x8 v;
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = static_cast<bf16>(x[i]);
        *reinterpret_cast<bf16x8*>(p) = v;
    }
    static __device__ __forceinline__ void copy(const bf16* s, bf16* d) {
        *reinterpret_cast<u32x4*>(d) = *reinterpret_cast<const u32x4*>(s);
    }
    // with the non-temporal hint: rows read once in a pass
    static __device__ __forceinline__ void load_nt(const bf16* p, float* x) {
        const bf16x8 v = __builtin_bit_cast(bf16x8, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)));
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = static_cast<float>(v[i]);
    }
    // with the non-temporal hint: rows written once and not read again soon
    static __device__ __forceinline__ void store_nt(bf16* p, const float* x) {
        bf16x8 v;
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = static_cast<bf16>(x[i]);
        __builtin_nontemporal_store(__builtin_bit_cast(u32x4, v), reinterpret_cast<u32x4*>(p));
    }
};
template <> struct Vec8<float> {
    static __device__ __forceinline__ void load(const float* p, float* x) {
        floatx4 a = *reinterpret_cast<const floatx4*>(p);
        floatx4 b = *reinterpret_cast<const floatx4*>(p + 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) { x[i] = a[i]; x[4 + i] = b[i]; }
    }
    static __device__ __forceinline__ void store(float* p, const float* x) {
        *reinterpret_cast<floatx4*>(p) = floatx4{x[0], x[1], x[2], x[3]};
        *reinterpret_cast<floatx4*>(p + 4) = floatx4{x[4], x[5], x[6], x[7]};
    }
    static __device__ __forceinline__ void copy(const float* s, float* d) {
        *reinterpret_cast<u32x4*>(d) = *reinterpret_cast<const u32x4*>(s);
        *reinterpret_cast<u32x4*>(d + 4) = *reinterpret_cast<const u32x4*>(s + 4);
    }
    static __device__ __forceinline__ void load_nt(const float* p, float* x) {
        const floatx4 a = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(p));
        const floatx4 b = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(p + 4));
#pragma unroll
        for (int i = 0; i < 4; ++i) { x[i] = a[i]; x[4 + i] = b[i]; }
    }
    static __device__ __forceinline__ void store_nt(float* p, const float* x) {
        __builtin_nontemporal_store(floatx4{x[0], x[1], x[2], x[3]}, reinterpret_cast<floatx4*>(p));
        __builtin_nontemporal_store(floatx4{x[4], x[5], x[6], x[7]}, reinterpret_cast<floatx4*>(p + 4));
    }
};

__device__ __forceinline__ float warp_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

}  // namespace cb
