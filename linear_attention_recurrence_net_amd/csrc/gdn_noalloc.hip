// gdn_noalloc.hip -- the general chunked prefill for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).  Its workspace is a fixed array of the
// library's own device memory instead of a caller buffer; everything else is
// gdn_prefill_chunked_ex.

#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "gdn.h"

namespace {

// The prefill workspace of every gdn_prefill_chunked_ex_noalloc call on a
// device.  Each device that loads the library holds its own copy until the
// process ends.  In host code this name is only a stand-in for the symbol:
// kernels and copies take the address scratch_address() returns.
static __device__ __align__(256) unsigned char scratch[GDN_PREFILL_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];  // device address of each device's array
std::mutex g_scratch_mu;

// The device address of the current device's scratch array, looked up once
// per device with that device current.
int scratch_address(void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return GDN_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return GDN_ERR_UNSUPPORTED;
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (p == nullptr) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
                return GDN_ERR_HIP;
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return GDN_OK;
}

}  // namespace

extern "C" {

int gdn_prefill_chunked_ex_noalloc(int32_t B, int32_t T, int32_t H, int32_t H_qk, int32_t head_map,
                                   int32_t d_k, int32_t d_v, int32_t chunk, int32_t qkv_dtype,
                                   int32_t gate, int32_t K, const void* q, const void* k,
                                   const void* v, const float* g, const float* beta, float* state,
                                   float* final_state, float* o, void* stream) {
    // Every argument check of gdn_prefill_chunked_ex, which launches nothing
    // when it reports a missing workspace; any other status (including OK
    // for problems that need no workspace) is final.
    const int st = gdn_prefill_chunked_ex(B, T, H, H_qk, head_map, d_k, d_v, chunk, qkv_dtype, gate, K,
                                          q, k, v, g, beta, state, final_state, o, nullptr, 0, stream);
    if (st != GDN_ERR_WORKSPACE) return st;
    const size_t need = gdn_prefill_workspace_size_ex(B, T, H, d_k, d_v, chunk, qkv_dtype, gate);
    if (need > static_cast<size_t>(GDN_PREFILL_SCRATCH_BYTES)) return GDN_ERR_SCRATCH;
    void* ws = nullptr;
    const int as = scratch_address(&ws);
    if (as != GDN_OK) return as;
    return gdn_prefill_chunked_ex(B, T, H, H_qk, head_map, d_k, d_v, chunk, qkv_dtype, gate, K, q, k,
                                  v, g, beta, state, final_state, o, ws,
                                  static_cast<size_t>(GDN_PREFILL_SCRATCH_BYTES), stream);
}

}  // extern "C"
