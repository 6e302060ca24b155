// noalloc.hip -- the forward for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc): bsattn_forward_noalloc runs bsattn_forward with a file-scope
// device array as its workspace.
//
// The array holds what bsattn_forward keeps in its workspace: the fp32
// partials of rows split across workgroups and their LSEs (and, for token and
// adaptive layouts, the gathered K/V tiles of the global tokens and the block
// sums).  None of it needs to start at zero.  Each device the library runs on
// holds its own copy of the array, at its own address, until the process
// ends; every call on one device shares that copy, so calls that overlap in
// time on one device race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../internal.h"

static __device__ __align__(256) unsigned char scratch[bsattn::kNoAllocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};   // the array's device address, per device

}  // namespace

namespace bsattn {

// In host code `scratch` names a host-side stand-in, not the device array: its
// device address comes from hipGetSymbolAddress, once per device, with that
// device current (the caller's).
hipError_t noalloc_scratch(void** ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> g(g_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch[dev] = p;
    }
    *ptr = g_scratch[dev];
    return hipSuccess;
}

}  // namespace bsattn

extern "C" bsattn_status bsattn_forward_noalloc(const bsattn_layout* layout, bsattn_dtype dtype, int32_t batch,
                                                int32_t num_heads, int32_t seq_len, int32_t head_dim,
                                                const void* q, const void* k, const void* v, void* out,
                                                float* lse, const int32_t* key_valid_len, float scale,
                                                hipStream_t stream) {
    if (!layout) return bsattn::set_failure(BSATTN_ERR_INVALID_ARG, "layout is NULL");
    size_t need = 0;
    bsattn_status st = bsattn_workspace_size(layout, batch, head_dim, 0, &need);
    if (st != BSATTN_OK) return st;
    if (need > bsattn::kNoAllocScratchBytes)
        return bsattn::set_failure(BSATTN_ERR_UNSUPPORTED,
                                   "this call needs more workspace than the 64 MiB of bsattn_forward_noalloc");
    void* ws = nullptr;
    const hipError_t e = bsattn::noalloc_scratch(&ws);
    if (e != hipSuccess) return bsattn::set_failure(BSATTN_ERR_HIP, hipGetErrorString(e));
    return bsattn::forward_prepared_only(layout, dtype, batch, num_heads, seq_len, head_dim, q, k, v, out, lse,
                                         key_valid_len, scale, ws, bsattn::kNoAllocScratchBytes, stream);
}
