// Record sums of per-record gradient blocks (the STORED clipped sum): products of
// two floats are exact in fp64, so accumulating c_i * P_i[e] in fp64 in a fixed
// order and rounding once leaves an error that does not grow with the record count.
#pragma once

#include "device_common.h"
#include "internal.h"

namespace dpsgd {

// d[q] += c * v[q] in fp64
__device__ __forceinline__ void add_scaled(double (&d)[4], float c, f32x4 v) {
#pragma unroll
    for (int q = 0; q < 4; ++q) d[q] = fma((double)c, (double)v[q], d[q]);
}

// Flat index within the layer of the element that a stored block keeps at flat position x (the
// inverse of the order the norm kernel writes, see StoredMap).  For x a multiple of 4, the four
// positions x .. x + 3 hold the elements stored_logical(x) .. + 3.
__device__ __forceinline__ int64_t stored_logical(const StoredMap& m, int64_t x) {
    if (m.mode == 0) return x;
    const int64_t r = x / m.d_out, col = x - r * m.d_out;
    if (m.mode == 3) {
        if (col >= m.full) return x;
        const int s = (int)(col & 127);   // stored 64 q + 4 c + u holds 8 c + 4 q + u
        return x - s + (8 * ((s >> 2) & 15) + 4 * (s >> 6) + (s & 3));
    }
    if (r >= m.full) return x;
    const int s = (int)(r & 127);         // stored row 16 i + c holds row dcol(c, i)
    const int j = m.mode == 1 ? 8 * (s & 15) + (s >> 4) : 64 * (s >> 6) + 4 * (s & 15) + ((s >> 4) & 3);
    return x + (int64_t)(j - s) * m.d_out;
}

}  // namespace dpsgd
