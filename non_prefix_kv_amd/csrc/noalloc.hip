// cb_attention_noalloc: the kernel-level attention call for callers that
// cannot allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid hipMalloc).  It runs the same kernels as
// cb_attention; the split-key partials that cb_attention places in a
// workspace it allocates per call live here in a file-scope device array of
// fixed size, one copy per GPU, held until the process ends.
#include <mutex>

#include <hip/hip_runtime.h>

#include "../../include/cacheblend.h"
#include "host.h"
#include "kernels.h"

namespace {

constexpr size_t kScratchBytes = (size_t)80 << 20;   // CB_NOALLOC_SCRATCH_BYTES
static_assert(kScratchBytes == CB_NOALLOC_SCRATCH_BYTES, "header and library disagree");

// The array's name is only a host-side stand-in for the symbol: host code
// must use the address hipGetSymbolAddress returns for each device.
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's copy of `scratch` (looked up once per
// device, with that device current).
cb_status scratch_address(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return cb::set_error(CB_E_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return cb::set_error(CB_E_UNSUPPORTED, "device %d beyond the %d this library tracks", dev,
                             kMaxDevices);
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return cb::set_error(CB_E_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                                 hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return CB_OK;
}

}  // namespace

extern "C" cb_status cb_attention_noalloc(int32_t dtype, const void* q, const int32_t* q_pos,
                                          int32_t n_q, const void* k, const void* v,
                                          int32_t n_kv, int32_t n_q_heads, int32_t n_kv_heads,
                                          int32_t head_dim, void* out, void* stream) {
    using namespace cb;
    if (dtype != CB_F32 && dtype != CB_BF16) return set_error(CB_E_INVALID, "dtype %d", dtype);
    if (n_q < 0 || n_kv <= 0 || n_q_heads <= 0 || n_kv_heads <= 0 || n_q_heads % n_kv_heads)
        return set_error(CB_E_SHAPE, "bad sizes");
    if (head_dim != 64 && head_dim != 128)
        return set_error(CB_E_UNSUPPORTED, "head_dim %d", head_dim);
    if (n_q > 0 && (!q || !q_pos || !k || !v || !out)) return set_error(CB_E_INVALID, "NULL buffer");
    const AttnRange range{0, n_q, 0, n_kv};
    const size_t need = attention_workspace(dtype, &range, 1, n_q_heads, head_dim);
    if (need > kScratchBytes)
        return set_error(CB_E_SHAPE,
                         "split-key partials of %zu bytes exceed the fixed scratch of %zu bytes "
                         "(use cb_attention)", need, kScratchBytes);
    void* ws = nullptr;
    if (need) {
        const cb_status st = scratch_address(&ws);
        if (st != CB_OK) return st;
    }
    AttnArgs a{};
    a.q = q; a.q_pos = q_pos; a.k = k; a.v = v;
    a.n_q_heads = n_q_heads; a.n_kv_heads = n_kv_heads; a.head_dim = head_dim; a.out = out;
    const hipError_t e = launch_attention(dtype, a, &range, 1, ws, need,
                                          reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return set_error(CB_E_HIP, "attention launch: %s", hipGetErrorString(e));
    return CB_OK;
}
