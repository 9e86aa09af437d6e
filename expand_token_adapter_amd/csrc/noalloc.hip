// noalloc.hip -- lora_shrink_noalloc: lora_shrink whose workspace is a static
// device array of the library, for callers that cannot allocate device memory
// (code under graph capture, tight serving loops, harnesses that forbid it).
//
// `scratch` below is one file-scope device array per GPU; host code never
// uses its name as an address (on the host it is only a stand-in symbol).
// Its device address is looked up once per device with hipGetSymbolAddress,
// that device current, and kept in scratch_ptr_of[]; the kernels receive that
// pointer exactly as they receive a caller's workspace in lora_shrink.
#include <hip/hip_runtime.h>

#include <mutex>

#include "host_checks.h"
#include "lora_batch.h"

namespace lora {
int shrink_check(int dtype, const void* x, int64_t ldx, int32_t T, int32_t d_in, const lora_adapter* adapters,
                 int32_t num_adapters, int32_t r_max, const lora_segments& seg, const float* v, int64_t ldv);
int shrink_entry(int dtype, const void* x, int64_t ldx, int32_t T, int32_t d_in, const lora_adapter* adapters,
                 int32_t num_adapters, int32_t r_max, lora_segments seg, float* v, int64_t ldv, void* ws,
                 size_t ws_bytes, void* stream);
}

namespace {

static __device__ __align__(256) char scratch[LORA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr_of[kMaxDevices] = {};

// Device address of `scratch` on the device that runs `stream` (the current
// device for the null stream).  The first call on a device looks it up with
// that device current and keeps it; the caller's current device is restored.
int scratch_address(void* stream, void** out) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return LORA_ERR_HIP;
    int dev = cur;
    if (stream && hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev) != hipSuccess) return LORA_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return LORA_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_ptr_of[dev]) {
        if (dev != cur && hipSetDevice(dev) != hipSuccess) return LORA_ERR_HIP;
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (dev != cur && hipSetDevice(cur) != hipSuccess) return LORA_ERR_HIP;
        if (e != hipSuccess || !p) return LORA_ERR_HIP;
        scratch_ptr_of[dev] = p;
    }
    *out = scratch_ptr_of[dev];
    return LORA_OK;
}

}  // namespace

using lora::shrink_check;
using lora::shrink_entry;

extern "C" int lora_shrink_noalloc(int dtype, const void* x, int64_t ldx, int32_t T, int32_t d_in,
                                   const lora_adapter* adapters, int32_t num_adapters, int32_t r_max,
                                   lora_segments seg, float* v, int64_t ldv, void* stream) {
    // lora_shrink's checks, then the size against the static scratch, all
    // before anything touches the device
    int rc = shrink_check(dtype, x, ldx, T, d_in, adapters, num_adapters, r_max, seg, v, ldv);
    if (rc != LORA_OK || T == 0) return rc;
    if (lora_shrink_workspace_bytes(dtype, T, d_in, r_max) > (size_t)LORA_NOALLOC_SCRATCH_BYTES)
        return LORA_ERR_TOO_LARGE;
    void* ws = nullptr;
    rc = scratch_address(stream, &ws);
    if (rc != LORA_OK) return rc;
    return shrink_entry(dtype, x, ldx, T, d_in, adapters, num_adapters, r_max, seg, v, ldv, ws,
                        (size_t)LORA_NOALLOC_SCRATCH_BYTES, stream);
}
