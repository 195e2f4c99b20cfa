// The library's one piece of device state: a fixed scratch area that stands in for the caller's
// workspace in dpsgd_step_noalloc, for callers that cannot allocate device memory (code under
// HIP graph capture, tight serving loops).  Each device the library runs on holds its own copy of
// the array from the code object's load until the process ends.  Host code never passes the
// array's name to a kernel (on the host it is only a stand-in for the symbol): its device address
// is looked up once per device with hipGetSymbolAddress, with that device current, and that
// address is what the kernels receive.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "internal.h"

namespace dpsgd {

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mutex;
}  // namespace

hipError_t scratch_pointer(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mutex);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (!p) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            if (!p) return hipErrorInvalidSymbol;
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return hipSuccess;
}

__global__ void k_status_copy(const uint32_t* status, uint32_t* out) {
    if (threadIdx.x == 0 && blockIdx.x == 0) *out = *status;
}

hipError_t launch_status_copy(const uint32_t* status, uint32_t* out, hipStream_t s) {
    hipLaunchKernelGGL(k_status_copy, dim3(1), dim3(64), 0, s, status, out);
    return hipGetLastError();
}

}  // namespace dpsgd
