// Device-side helpers shared by the kernels: MFMA operand types, bf16
// widening, and fixed-order wavefront reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dpsgd {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_bits_to_float(uint16_t b) {
    return __uint_as_float((uint32_t)b << 16);
}

// Sum over the 64 lanes of a wavefront; the butterfly order is fixed, so the
// result depends only on the lane values.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// v_mfma_f32_16x16x32_bf16: lane l supplies row (l % 16) of the A block and
// column (l % 16) of the B block, each with 8 consecutive k of group l / 16;
// the 16x16 fp32 result has column l % 16, rows 4 * (l / 16) + {0..3} in lane l.
__device__ __forceinline__ f32x4 mfma_bf16(const u32x4& a, const u32x4& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// v_mfma_f32_16x16x4_f32: lane l supplies A[l % 16][l / 16] and B[l / 16][l % 16];
// the result layout is the same as above.
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

}  // namespace dpsgd
