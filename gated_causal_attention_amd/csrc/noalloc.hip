// noalloc.hip -- resolvent_forward_noalloc: the forward pass with its
// workspace in a fixed device array of this library instead of a buffer the
// caller provides, for callers that cannot allocate device memory.
//
// The array lives in the code object's zero-initialised data.  Each device
// holds its own copy at its own address from the first use of the library on
// that device until the process ends; host code reaches it only through the
// address hipGetSymbolAddress returns for the current device (the array's
// name in host code is a host-side stand-in, not a device address).
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "resolvent.h"

namespace {

constexpr size_t kScratchBytes = size_t(RESOLVENT_NOALLOC_SCRATCH_BYTES);
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex scratch_mutex;
std::atomic<void *> scratch_addr[kMaxDevices];

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept for later calls.
int32_t scratch_on_current_device(void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return RESOLVENT_DEVICE_ERROR;
    void *p = scratch_addr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(scratch_mutex);
        p = scratch_addr[dev].load(std::memory_order_relaxed);
        if (!p) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
                return RESOLVENT_DEVICE_ERROR;
            scratch_addr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return RESOLVENT_OK;
}

}  // namespace

extern "C" {

size_t resolvent_noalloc_scratch_bytes(void) { return kScratchBytes; }

int32_t resolvent_forward_noalloc(const void *q, const void *k, const float *u,
                                  const float *theta, const void *v, double beta, double qk,
                                  double g, int64_t B, int64_t H, int64_t n, int64_t d,
                                  int32_t qk_dtype, int32_t v_dtype, float *o_re, float *o_im,
                                  int32_t *status_dev, hipStream_t stream) {
    const size_t need = resolvent_workspace_bytes(B, H, n, d, qk_dtype, v_dtype);
    if (need == 0)  // empty, invalid or unsupported: rejected before any device work
        return resolvent_forward(q, k, u, theta, v, beta, qk, g, B, H, n, d, qk_dtype, v_dtype,
                                 o_re, o_im, nullptr, 0, status_dev, stream);
    if (need > kScratchBytes) return RESOLVENT_TOO_LARGE;
    void *ws = nullptr;
    const int32_t rc = scratch_on_current_device(&ws);
    if (rc != RESOLVENT_OK) return rc;
    return resolvent_forward(q, k, u, theta, v, beta, qk, g, B, H, n, d, qk_dtype, v_dtype, o_re,
                             o_im, ws, kScratchBytes, status_dev, stream);
}

}  // extern "C"
