// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy
// as 1, 2, 3", SC'11) and the Box-Muller transform (Box & Muller 1958) as used
// by the noise of the DP-SGD step.  Block b of the stream for (seed, step) is
// Philox4x32-10 with key (seed mod 2^32, seed div 2^32) and counter
// (b mod 2^32, b div 2^32, step mod 2^32, step div 2^32); words (0, 1) and (2, 3)
// each give two normals.
#pragma once

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
        // each 32 x 32 -> 64-bit product as one 64-bit multiply, so that both halves come
        // from a single v_mad_u64_u32 rather than a mul_lo / mul_hi pair
        const uint64_t p0 = (uint64_t)0xD2511F53u * x0;
        const uint64_t p1 = (uint64_t)0xCD9E8D57u * x2;
        const uint32_t lo0 = (uint32_t)p0, hi0 = (uint32_t)(p0 >> 32);
        const uint32_t lo1 = (uint32_t)p1, hi1 = (uint32_t)(p1 >> 32);
        // three-input XORs as one v_bitop3_b32 each (truth table 0x96 = a ^ b ^ c)
        const uint32_t y0 = __builtin_amdgcn_bitop3_b32(hi1, x1, k0, 0x96);
        const uint32_t y2 = __builtin_amdgcn_bitop3_b32(hi0, x3, k1, 0x96);
        x0 = y0;
        x1 = lo1;
        x2 = y2;
        x3 = lo0;
    }
    Philox4 o;
    o.x[0] = x0; o.x[1] = x1; o.x[2] = x2; o.x[3] = x3;
    return o;
}

// r = sqrt(-2 ln u1) with -2 ln u1 = (-2 ln 2) log2 u1, and the angle 2 pi u2, from the hardware's
// log2 and its sine and cosine, which take their argument in revolutions (sin(2 pi x) for x): u1
// in [2^-24, 1] is never denormal and u2 in [0, 1) needs no range reduction.  Checked on every one
// of the 2^24 uniforms against float64: log2 within 1.2e-7 relative (next to u1 = 1 as well), sine
// and cosine within 2.1 * 2^-24 absolute, so |Z - Z_exact| stays within 5.3 * 2^-24 (1 + |Z|).
__device__ __forceinline__ void box_muller(uint32_t we, uint32_t wo, float& z_even, float& z_odd) {
    const float u1 = (float)((we >> 8) + 1u) * 0x1.0p-24f;
    const float u2 = (float)(wo >> 8) * 0x1.0p-24f;
    const float r = sqrtf(-1.38629436111989061883f * __builtin_amdgcn_logf(u1));
    z_even = r * __builtin_amdgcn_cosf(u2);
    z_odd = r * __builtin_amdgcn_sinf(u2);
}


// The four normals of Philox block b (flat elements 4b .. 4b + 3).
__device__ __forceinline__ void gauss4(uint64_t b, uint64_t step, uint64_t seed, float (&z)[4]) {
    const Philox4 w = philox4x32_10(b, step, seed);
    box_muller(w.x[0], w.x[1], z[0], z[1]);
    box_muller(w.x[2], w.x[3], z[2], z[3]);
}

}  // namespace dpsgd
