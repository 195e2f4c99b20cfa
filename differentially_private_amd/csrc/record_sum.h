// Record sums of per-record gradient blocks (the STORED clipped sum): products of
// two floats are exact in fp64, so accumulating c_i * P_i[e] in fp64 in a fixed
// order and rounding once leaves an error that does not grow with the record count.
#pragma once

#include "device_common.h"

namespace dpsgd {

// d[q] += c * v[q] in fp64
__device__ __forceinline__ void add_scaled(double (&d)[4], float c, f32x4 v) {
#pragma unroll
    for (int q = 0; q < 4; ++q) d[q] = fma((double)c, (double)v[q], d[q]);
}

}  // namespace dpsgd
