/*
 * Seeded synthetic input generator for the per-layer activations A[B,T,d_in]
 * and output gradients G[B,T,d_out] that the DP-SGD clip/sum/noise step
 * consumes.  It holds none of the method's arithmetic: it only turns
 * (seed, layer, tensor, record, token, column) into one input value.
 *
 * Both the host fill (gcc, for the CPU oracle) and the device fill (HIP, for
 * inputs too large to upload) include this file, so that the two produce the
 * same bytes.  Every step is integer arithmetic or a correctly rounded IEEE
 * double operation (+, *, /, sqrt) evaluated in a fixed order with FMA
 * contraction disabled, so host and device agree bit for bit.
 *
 * Value of element (record i, token t, column j) of one tensor:
 *   e      = (i*T + t)*d + j                      (global record index i)
 *   key    = mix64(mix64(seed) ^ (2*layer + tensor + 1) * PHI)
 *   u16[w] = 16-bit words of mix64(key + (3e+q)*PHI), q = 0..2  (12 words)
 *   z      = (sum_w u16[w] - 393210) / 65536        (Irwin-Hall sum of 12
 *            uniforms, centred: mean 0, variance 1 - 2^-32, exact in fp32)
 *   heavy records: z <- z / sqrt((h0^2 + h1^2 + h2^2) / 3), with h0..h2 three
 *            further Irwin-Hall draws from a second key (a Student-t draw with
 *            3 degrees of freedom built from approximately normal parts)
 *   value  = round_to_dtype(scale[i] * z)          (double -> fp32 RNE,
 *            then fp32 -> bf16 RNE for bf16 tensors)
 * mix64 is the splitmix64 output mixer (Steele, Lea, Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014; constants from Vigna's
 * public-domain splitmix64).
 */
#ifndef DPGEN_DG_H
#define DPGEN_DG_H

#include <stdint.h>

#ifdef __HIPCC__
#define DG_FN static inline __host__ __device__
#else
#define DG_FN static inline
#endif

#define DG_F32 0
#define DG_BF16 1

#define DG_PHI 0x9E3779B97F4A7C15ull
#define DG_HEAVY_SALT 0x5851F42D4C957F2Dull

DG_FN uint64_t dg_mix64(uint64_t x) {
    x ^= x >> 30;
    x *= 0xBF58476D1CE4E5B9ull;
    x ^= x >> 27;
    x *= 0x94D049BB133111EBull;
    x ^= x >> 31;
    return x;
}

DG_FN uint64_t dg_stream_key(uint64_t seed, uint32_t layer, uint32_t tensor) {
    return dg_mix64(dg_mix64(seed) ^ (((uint64_t)layer * 2u + tensor + 1u) * DG_PHI));
}

/* Centred Irwin-Hall draw number n of the stream `key`: an integer in
 * [-393210, 393210] divided by 2^16, so it is exact in both fp32 and fp64. */
DG_FN double dg_ih(uint64_t key, uint64_t n) {
    int64_t s = 0;
    for (int q = 0; q < 3; ++q) {
        uint64_t h = dg_mix64(key + (3u * n + (uint64_t)q) * DG_PHI);
        s += (int64_t)(h & 0xFFFFu) + (int64_t)((h >> 16) & 0xFFFFu) +
             (int64_t)((h >> 32) & 0xFFFFu) + (int64_t)(h >> 48);
    }
    return (double)(s - 393210) * (1.0 / 65536.0);
}

/* Unscaled standard draw for element e (heavy != 0: Student-t, 3 dof). */
DG_FN double dg_draw(uint64_t key, uint64_t e, int heavy) {
    double z = dg_ih(key, e);
    if (heavy) {
        uint64_t hk = dg_mix64(key ^ DG_HEAVY_SALT);
        double h0 = dg_ih(hk, 3u * e + 0u);
        double h1 = dg_ih(hk, 3u * e + 1u);
        double h2 = dg_ih(hk, 3u * e + 2u);
        double p0 = h0 * h0;
        double p1 = h1 * h1;
        double p2 = h2 * h2;
        double q = (p0 + p1) + p2;
        if (q == 0.0) return 0.0;
        double v = q / 3.0;
        z = z / __builtin_sqrt(v);
    }
    return z;
}

/* fp32 -> bf16 bits, round to nearest even (NaN kept quiet). */
DG_FN uint16_t dg_f32_to_bf16(float f) {
    union { float f; uint32_t u; } c;
    c.f = f;
    uint32_t u = c.u;
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

#endif
