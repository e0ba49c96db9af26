// cpattn_ring_fwd_noalloc: the ring step with the library's own scratch, for
// callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid hipMalloc).
//
// The only scratch of the one-launch ring step is the pieces of query tiles cut
// between workgroups (fp32 outputs and LSEs, at most two slots per workgroup),
// whose size is fixed by the chip's workgroup slots, not by the problem:
// kRingScratchMax bytes (68,157,440, the d = 64 case) cover every shape with up
// to kRingMaxChunks chunks.  That array lives at file scope below; each GPU the
// library runs on holds its own copy until the process ends.
#include <hip/hip_runtime.h>

#include <mutex>

#include "cpattn.h"
#include "internal.h"

#define CPATTN_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

__device__ __align__(256) char scratch[cpattn::kRingScratchMax];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];  // device address of `scratch` on each device, once looked up

// The device that `stream` belongs to (the current device for the null stream).
hipError_t stream_device(hipStream_t stream, int* dev) {
    if (stream == nullptr) return hipGetDevice(dev);
    return hipStreamGetDevice(stream, dev);
}

// Device address of this device's `scratch`: looked up once per device, with
// that device current (the host-side name of the array is only a stand-in for
// it and is never passed to a kernel).
int scratch_on(int dev, void** out) {
    if (dev < 0 || dev >= kMaxDevices) return cpattn::report_hip_error(hipErrorInvalidDevice, "scratch device");
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_scratch[dev] == nullptr) {
        int cur = 0;
        hipError_t e = hipGetDevice(&cur);
        if (e != hipSuccess) return cpattn::report_hip_error(e, "hipGetDevice");
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return cpattn::report_hip_error(e, "hipSetDevice");
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess) e = e2;
        }
        if (e != hipSuccess) return cpattn::report_hip_error(e, "hipGetSymbolAddress(scratch)");
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return CPATTN_OK;
}

}  // namespace

CPATTN_EXPORT size_t cpattn_ring_fwd_noalloc_scratch_bytes(void) { return cpattn::kRingScratchMax; }

CPATTN_EXPORT int cpattn_ring_fwd_noalloc(const void* q, const void* k, const void* v, void* out, float* lse,
                                          int64_t B, int64_t H, int64_t Sq, int64_t Skv, int64_t d, float scale,
                                          int ring_degree, const int64_t* chunk_lens, int in_dtype, int out_dtype,
                                          void* stream) {
    int dev = 0;
    const hipError_t e = stream_device(static_cast<hipStream_t>(stream), &dev);
    if (e != hipSuccess) return cpattn::report_hip_error(e, "stream device");
    void* ws = nullptr;
    const int st = scratch_on(dev, &ws);
    if (st != CPATTN_OK) return st;
    return cpattn::ring_fwd_on_scratch(q, k, v, out, lse, B, H, Sq, Skv, d, scale, ring_degree, chunk_lens, ws,
                                       cpattn::kRingScratchMax, in_dtype, out_dtype, stream);
}
