// hf_hybrid_step_noalloc: the hybrid step for callers that cannot allocate device memory
// (code under graph capture, tight serving loops, harnesses that forbid it).  Its
// transient data live in one file-scope device array instead of a caller workspace; every
// kernel is the one hf_hybrid_step launches, handed this array's address as its workspace.
//
// Each GPU holds its own copy of the array from the library's first use on it until the
// process ends.  Its host-side name is only a stand-in for the symbol, so the device
// address is looked up once per device with hipGetSymbolAddress and kept; host code uses
// that address only.  Calls on one GPU share the array: calls that overlap in time on one
// GPU (different streams, or threads) race on it.  Nothing in it needs a starting value,
// so nothing is cleared.
#include <mutex>

#include "hf_internal.h"

namespace {

constexpr size_t kScratchBytes = (size_t)32 << 20;   // 32 MiB per GPU
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void *g_ptr[kMaxDevices];   // device address of `scratch` per device, once looked up

// Device address of this device's copy of `scratch` (looked up on the first call per
// device, with that device current).
hipError_t scratch_for(int dev, void **out) {
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
        int cur = -1;
        hipError_t e = hipGetDevice(&cur);
        if (e != hipSuccess) return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess) e = e2;
        }
        if (e != hipSuccess) return e;
        g_ptr[dev] = p;
    }
    *out = g_ptr[dev];
    return hipSuccess;
}

}  // namespace

extern "C" hf_status hf_hybrid_step_noalloc(const hf_dims *d, const void *q, const void *k_cur, const void *v_cur,
                                            hf_kv_ring *ring, int32_t top_k, uint32_t flags, float *S, float *z,
                                            float eps, int32_t *idx, float *out, const hf_step_events *events,
                                            hipStream_t stream) {
    hf_status st = hf_step_validate(d, q, k_cur, v_cur, ring, top_k, flags, S, z, eps, idx, out);
    if (st != HF_OK) return st;
    const size_t need = hf_step_workspace_bytes(d);
    if (need > kScratchBytes)
        return hf_fail_unsupported("the step's transient data exceed the allocation-free entry point's 32 MiB",
                                   need, kScratchBytes);
    // the device that runs the work: the stream's (the current device for the null stream)
    int dev = -1;
    hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
    if (e == hipSuccess && (dev < 0 || dev >= kMaxDevices)) e = hipErrorInvalidDevice;
    void *ws = nullptr;
    if (e == hipSuccess) e = scratch_for(dev, &ws);
    if (e != hipSuccess) return hf_fail_hip(e, "allocation-free step scratch lookup");
    return hf_step_enqueue(d, q, k_cur, v_cur, ring, top_k, flags, S, z, eps, nullptr, idx, out, ws, events, stream);
}
