// noise: out[e] += sigma * C * Z[e] for every coordinate of every layer, drawn
// once per logical step ("Privacy-Preserving Machine Learning", DP-SGD phase 4:
// N(0, sigma^2 C^2 I) added to the clipped sum).
//
// Z is a pure function of (seed, step, flat element index e): Philox4x32-10
// (Salmon, Moraes, Dror, Shaw, SC'11) with key (seed mod 2^32, seed div 2^32)
// and counter (b mod 2^32, b div 2^32, step mod 2^32, step div 2^32), b = e / 4,
// gives four words; words (0, 1) and (2, 3) each feed one Box-Muller transform
// (Box & Muller 1958) with u1 = ((w_even >> 8) + 1) 2^-24 in (0, 1] and
// u2 = (w_odd >> 8) 2^-24 in [0, 1): lanes 0/2 get r cos(2 pi u2), lanes 1/3
// r sin(2 pi u2), r = sqrt(-2 ln u1).  Both uniforms are exact in fp32.  One
// thread per four consecutive elements of a layer (one Philox block when the
// layer starts on a multiple of 4); the add is a coalesced read-modify-write.
// One launch covers every layer of a plan up to the kernel-argument limit (320 layers, 160 with
// the descent step), so a LoRA plan's noise is one pass over the flat index.
#include <algorithm>

#include "philox.h"

namespace dpsgd {

// Grid: x = 256-thread chunks of a piece (4 elements per thread), y = piece.
__global__ __launch_bounds__(256) void k_noise(NoiseArgs a) {
    if (a.status && *a.status) return;
    const int l = blockIdx.y;
    const int64_t off = a.base + a.off[l];
    const int64_t n_l = (int64_t)(a.off[l + 1] - a.off[l]);
    const int64_t x0 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
    if (x0 >= n_l) return;
    float* const out_l = a.ptr[l];
    float* const par_l = a.with_params ? a.ptr[a.n_pieces + l] : nullptr;
    float* o = out_l + x0;
    float* th = par_l ? par_l + x0 : nullptr;   // descent step target
    if (x0 + 4 <= n_l && (off & 3) == 0 && (n_l & 3) == 0 &&
        ((reinterpret_cast<uintptr_t>(out_l) | reinterpret_cast<uintptr_t>(par_l)) & 15u) == 0) {
        float z[4];
        gauss4((uint64_t)(off + x0) >> 2, a.step, a.seed, z);
        f32x4 v = *reinterpret_cast<f32x4*>(o);
        v[0] += a.scale * z[0];
        v[1] += a.scale * z[1];
        v[2] += a.scale * z[2];
        v[3] += a.scale * z[3];
        *reinterpret_cast<f32x4*>(o) = v;
        if (th) {
            f32x4 t = *reinterpret_cast<f32x4*>(th);
#pragma unroll
            for (int q = 0; q < 4; ++q) t[q] = fmaf(-a.descent, v[q], t[q]);
            *reinterpret_cast<f32x4*>(th) = t;
        }
        return;
    }
    for (int q = 0; q < 4 && x0 + q < n_l; ++q) {
        const uint64_t e = (uint64_t)(off + x0 + q);
        float z4[4];
        gauss4(e >> 2, a.step, a.seed, z4);
        const float v = o[q] + a.scale * z4[e & 3];
        o[q] = v;
        if (th) th[q] = fmaf(-a.descent, v, th[q]);
    }
}

__global__ __launch_bounds__(256) void k_philox_raw(uint64_t seed, uint64_t step, uint64_t first,
                                                    uint64_t n, uint32_t* out) {
    const uint64_t q = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (q >= n) return;
    const Philox4 w = philox4x32_10(first + q, step, seed);
    *reinterpret_cast<u32x4*>(out + 4 * q) = u32x4{w.x[0], w.x[1], w.x[2], w.x[3]};
}

hipError_t launch_noise(const NoiseArgs& a, hipStream_t s) {
    int64_t max_n = 0;
    for (int l = 0; l < a.n_pieces; ++l) max_n = std::max<int64_t>(max_n, (int64_t)(a.off[l + 1] - a.off[l]));
    if (max_n == 0) return hipSuccess;
    const dim3 grid((unsigned)((max_n + 1023) / 1024), a.n_pieces);
    hipLaunchKernelGGL(k_noise, grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_philox_raw(uint64_t seed, uint64_t step, uint64_t first_block, uint64_t n_blocks,
                             uint32_t* out, hipStream_t s) {
    if (n_blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(k_philox_raw, dim3((unsigned)((n_blocks + 255) / 256)), dim3(256), 0, s,
                       seed, step, first_block, n_blocks, out);
    return hipGetLastError();
}

}  // namespace dpsgd
