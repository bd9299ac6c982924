// ssd_forward for callers that cannot allocate: the workspace is a
// file-scope device array of fixed size instead of an argument.
//
// Each GPU the library's code object is loaded on holds its own copy of the
// array until the process ends.  Host code never passes the array's name to
// a kernel (on the host that name is only a stand-in for the symbol): the
// first call on a device looks up the array's device address with
// hipGetSymbolAddress, with that device current, and keeps it per device;
// every call after that uses the kept address.  Nothing here or in
// ssd_forward allocates (no hipMalloc, hipFree or allocating library call).
#include <hip/hip_runtime.h>

#include <mutex>

#include "ssd.h"
#include "ssd_internal.h"

namespace {

constexpr size_t kScratchBytes = SSD_NOALLOC_WORKSPACE_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_scratch[kMaxDevices];  // device address of `scratch` on each GPU; null until looked up

}  // namespace

extern "C" ssd_status ssd_forward_noalloc(const ssd_dims *dims, const void *x, const void *dt,
                                          const float *A, const void *B, const void *C, const float *D,
                                          const float *init_state, void *y, float *final_state,
                                          void *stream) {
    // host-only checks first: a shape whose workspace does not fit is
    // rejected before any HIP call
    size_t need = 0;
    ssd_status st = ssd::forward_dims_check(dims, &need);
    if (st != SSD_OK) return st;
    if (need > kScratchBytes) return SSD_ERR_WORKSPACE;
    int dev = -1;
    if ((st = ssd::hip_error(hipGetDevice(&dev))) != SSD_OK) return st;
    if (dev < 0 || dev >= kMaxDevices) return SSD_ERR_UNSUPPORTED;
    void *ws = nullptr;
    {
        std::lock_guard<std::mutex> lock(g_mu);
        if (!g_scratch[dev]) {
            void *p = nullptr;
            if ((st = ssd::hip_error(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)))) != SSD_OK) return st;
            if (!p) return SSD_ERR_HIP;
            g_scratch[dev] = p;
        }
        ws = g_scratch[dev];
    }
    return ssd_forward(dims, x, dt, A, B, C, D, init_state, y, final_state, ws, kScratchBytes, stream);
}
