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
// thread per Philox block; the add is fused into a coalesced read-modify-write.
#include "device_common.h"
#include "internal.h"

namespace dpsgd {

struct Philox4 {
    uint32_t x[4];
};

__device__ __forceinline__ Philox4 philox4x32_10(uint64_t block, uint64_t step, uint64_t seed) {
    uint32_t x0 = (uint32_t)block, x1 = (uint32_t)(block >> 32);
    uint32_t x2 = (uint32_t)step, x3 = (uint32_t)(step >> 32);
    uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        const uint32_t lo0 = 0xD2511F53u * x0;
        const uint32_t hi0 = __umulhi(0xD2511F53u, x0);
        const uint32_t lo1 = 0xCD9E8D57u * x2;
        const uint32_t hi1 = __umulhi(0xCD9E8D57u, x2);
        const uint32_t y0 = hi1 ^ x1 ^ k0;
        const uint32_t y2 = hi0 ^ x3 ^ k1;
        x0 = y0;
        x1 = lo1;
        x2 = y2;
        x3 = lo0;
    }
    Philox4 o;
    o.x[0] = x0; o.x[1] = x1; o.x[2] = x2; o.x[3] = x3;
    return o;
}

__device__ __forceinline__ void box_muller(uint32_t we, uint32_t wo, float& z_even, float& z_odd) {
    const float u1 = (float)((we >> 8) + 1u) * 0x1.0p-24f;
    const float u2 = (float)(wo >> 8) * 0x1.0p-24f;
    const float r = sqrtf(-2.0f * logf(u1));
    float sn, cs;
    sincospif(2.0f * u2, &sn, &cs);
    z_even = r * cs;
    z_odd = r * sn;
}

__global__ __launch_bounds__(256) void k_noise(NoiseArgs a) {
    if (a.status && *a.status) return;
    const int64_t e_begin = a.off[0];
    const int64_t e_end = a.off[a.n_layers];
    const uint64_t b = (uint64_t)(e_begin >> 2) + (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t e0 = (int64_t)(b << 2);
    if (e0 >= e_end) return;
    const Philox4 w = philox4x32_10(b, a.step, a.seed);
    float z[4];
    box_muller(w.x[0], w.x[1], z[0], z[1]);
    box_muller(w.x[2], w.x[3], z[2], z[3]);

    const int64_t first = e0 < e_begin ? e_begin : e0;
    int lo = 0, hi = a.n_layers - 1;  // layer containing `first`
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (a.off[mid] <= first) lo = mid; else hi = mid - 1;
    }
    int l = lo;
    const int64_t rel0 = e0 - a.off[l];
    float* o = a.out[l];
    if (e0 >= e_begin && e0 + 4 <= a.off[l + 1] && (rel0 & 3) == 0 &&
        ((reinterpret_cast<uintptr_t>(o) & 15u) == 0)) {
        f32x4 v = *reinterpret_cast<f32x4*>(o + rel0);
        v[0] += a.scale * z[0];
        v[1] += a.scale * z[1];
        v[2] += a.scale * z[2];
        v[3] += a.scale * z[3];
        *reinterpret_cast<f32x4*>(o + rel0) = v;
        return;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int64_t e = e0 + q;
        if (e < e_begin || e >= e_end) continue;
        while (a.off[l + 1] <= e) ++l;
        float* p = a.out[l] + (e - a.off[l]);
        *p += a.scale * z[q];
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
    const int64_t e_begin = a.off[0], e_end = a.off[a.n_layers];
    if (e_end <= e_begin) return hipSuccess;
    const int64_t n_blocks = ((e_end - 1) >> 2) - (e_begin >> 2) + 1;
    hipLaunchKernelGGL(k_noise, dim3((unsigned)((n_blocks + 255) / 256)), dim3(256), 0, s, a);
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
