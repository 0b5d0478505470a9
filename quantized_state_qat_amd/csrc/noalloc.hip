// Allocation-free variant of the straight-through backward.  Its workspace is a file-scope
// device array of fixed size, so a call allocates nothing: for callers that cannot call
// hipMalloc (code under HIP graph capture, tight serving loops, harnesses that forbid it).
//
// Each GPU the library runs on holds one copy of the array (kScratchBytes) until the process
// ends.  Every call on a GPU uses that GPU's copy, whose contents are whatever the last call
// left: the backward writes every workspace element it reads before reading it, so nothing
// needs clearing.  Calls that overlap in time on one GPU (two streams, two threads) race on
// the array; callers serialize them.
#include <mutex>

#include "la_internal.hpp"

namespace {

constexpr size_t kScratchBytes = static_cast<size_t>(128) << 20;  // 128 MiB per GPU

__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of `scratch` on the current device.  The array's name is a host-side
// stand-in in host code; its address on each device is looked up once, with that device
// current, and kept per device.
hipError_t scratch_on_current_device(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return hipSuccess;
}

}  // namespace

extern "C" {

la_status la_recurrent_bwd_ste_noalloc(const la_config* cfg, const void* q, const void* k,
                                       const void* v, const void* g, const void* beta,
                                       const float* S0, const float* ckpts, const float* dout,
                                       const float* dS_T, float* dq, float* dk, float* dv,
                                       float* dg, float* dbeta, float* dS0, void* stream) {
    return la::bwd_ste(cfg, q, k, v, g, beta, S0, ckpts, dout, dS_T, dq, dk, dv, dg, dbeta, dS0, nullptr,
                       kScratchBytes, scratch_on_current_device, stream);
}

size_t la_noalloc_workspace_limit(void) { return kScratchBytes; }

}  // extern "C"
