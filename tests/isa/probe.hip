// Small kernels whose only purpose is to show, in the compiler's gfx950
// output, how many wait states its hazard recognizer places between a
// producer and a consumer that it can see.  The checker of the library's
// own device code uses these counts as the required minimum.  Not part of
// the library; never launched.
#include <hip/hip_runtime.h>

typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f16v __attribute__((ext_vector_type(16)));
typedef __bf16 b8 __attribute__((ext_vector_type(8)));

// matrix result read by a vector ALU instruction
__global__ void probe_raw_valu_16(const b8* a, f4* o) {
    f4 c = {0, 0, 0, 0};
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[threadIdx.x], a[threadIdx.x + 64], c, 0, 0, 0);
    o[threadIdx.x] = c * 2.0f;
}
__global__ void probe_raw_valu_32(const b8* a, f16v* o) {
    f16v c = {};
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[threadIdx.x], a[threadIdx.x + 64], c, 0, 0, 0);
    o[threadIdx.x] = c * 2.0f;
}
// matrix result stored to memory / to LDS
__global__ void probe_raw_vmem_16(const b8* a, f4* o) {
    f4 c = {0, 0, 0, 0};
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[threadIdx.x], a[threadIdx.x + 64], c, 0, 0, 0);
    o[threadIdx.x] = c;
}
__global__ void probe_raw_lds_16(const b8* a, float* o) {
    __shared__ f4 s[64];
    f4 c = {0, 0, 0, 0};
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[threadIdx.x], a[threadIdx.x + 64], c, 0, 0, 0);
    s[threadIdx.x] = c;
    __syncthreads();
    o[threadIdx.x] = s[63 - threadIdx.x][1];
}
// matrix result used as the A operand of the next matrix op
__global__ void probe_raw_srca_16(const b8* a, f4* o) {
    f4 c = {0, 0, 0, 0}, d = {1, 1, 1, 1};
    const b8 y = a[threadIdx.x + 64];
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[threadIdx.x], y, c, 0, 0, 0);
    d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(b8, c), y, d, 0, 0, 0);
    o[threadIdx.x] = d;
}
// matrix result accumulated by the next matrix op (SrcC, same registers)
__global__ void probe_srcc_16(const b8* a, f4* o) {
    f4 c = {0, 0, 0, 0};
    const b8 x = a[threadIdx.x], y = a[threadIdx.x + 64];
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, y, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(y, x, c, 0, 0, 0);
    o[threadIdx.x] = c;
}
__global__ void probe_srcc_32(const b8* a, f16v* o) {
    f16v c = {};
    const b8 x = a[threadIdx.x], y = a[threadIdx.x + 64];
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, y, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(y, x, c, 0, 0, 0);
    o[threadIdx.x] = c;
}
// vector ALU result read by a matrix op
__global__ void probe_valu_to_xdl(const b8* a, f4* o, float s) {
    f4 c = {s, s, s, s};
    c = c * s + 1.0f;
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[threadIdx.x], a[threadIdx.x + 64], c, 0, 0, 0);
    o[threadIdx.x] = c;
}
// M0 written for a buffer load into LDS
__global__ void probe_m0_lds_dma(__amdgpu_buffer_rsrc_t r, float* o) {
    __shared__ float s[2048];
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r, (__attribute__((address_space(3))) void*)(s), 16, threadIdx.x * 16, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r, (__attribute__((address_space(3))) void*)(s + 1024), 16, threadIdx.x * 16, 0, 0, 0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    o[threadIdx.x] = s[threadIdx.x * 3];
}
// the single-precision matrix op of the float32 GEMM
__global__ void probe_raw_valu_f32(const float* a, f4* o) {
    f4 c = {0, 0, 0, 0};
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[threadIdx.x], a[threadIdx.x + 64], c, 0, 0, 0);
    o[threadIdx.x] = c * 2.0f;
}
__global__ void probe_srcc_f32(const float* a, f4* o) {
    f4 c = {0, 0, 0, 0};
    const float x = a[threadIdx.x], y = a[threadIdx.x + 64];
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(x, y, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(y, x, c, 0, 0, 0);
    o[threadIdx.x] = c;
}
// a scalar register written by a vector instruction, then read by a buffer load
__global__ void probe_valu_sgpr_vmem(const float* p, float* o, int n) {
    const int off = __builtin_amdgcn_readfirstlane(__float_as_int(p[threadIdx.x]) + n);
    __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)p, 0, 0x10000, 0x20000);
    o[threadIdx.x] = __builtin_amdgcn_raw_buffer_load_b32(r, threadIdx.x * 4, off, 0);
}
