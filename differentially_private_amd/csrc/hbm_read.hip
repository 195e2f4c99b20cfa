// Measurement aid: a plain streaming read of a device buffer, the reference for
// the fraction of HBM bandwidth that this part reaches with 16-byte loads (the
// vendor figure is the other reference).  The loads carry the non-temporal hint,
// as the kernels' single-use reads do (2 GiB: 7.1 TB/s with it, 6.4 without).
// 2048 workgroups of 256 threads stride over the buffer; each wavefront folds
// what it read into one XOR word, so the result is checkable and the loads cannot
// be dropped.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dpsgd {

constexpr int kHbmReadBlocks = 2048;   // kHbmReadBlocks * 4 wavefronts = the sink's words

typedef uint32_t hr_u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void k_hbm_read(const hr_u32x4* __restrict__ p, int64_t n16, uint32_t* sink) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    hr_u32x4 acc = {0u, 0u, 0u, 0u};
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
        acc ^= __builtin_nontemporal_load(p + i);
    uint32_t v = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v ^= __shfl_xor(v, o, 64);
    if ((threadIdx.x & 63) == 0) sink[blockIdx.x * 4 + (threadIdx.x >> 6)] = v;
}

hipError_t launch_hbm_read(const void* buf, int64_t bytes, uint32_t* sink, hipStream_t s) {
    hipLaunchKernelGGL(k_hbm_read, dim3(kHbmReadBlocks), dim3(256), 0, s,
                       static_cast<const hr_u32x4*>(buf), bytes / 16, sink);
    return hipGetLastError();
}

}  // namespace dpsgd
