// Poisson sampling of a step's records ("Privacy-Preserving Machine Learning", DP-SGD phase 1:
// each record is included independently with public probability q).  Record i draws word i mod 4
// of Philox4x32-10 block 2^63 + floor(i / 4) under key = seed and counter words 2-3 = step (the
// top bit of the block index keeps these words apart from the noise stream, whose blocks stay
// below 2^62) and is included iff that word < floor(q 2^32).
//
// Three launches and no atomics, so the index list is increasing and reproducible: each 256-
// thread workgroup draws 1024 records (one Philox block per thread), optionally writes the
// inclusion mask and stores its count; one workgroup scans the counts; each workgroup then
// redraws its records and writes their indices at its offset plus an in-workgroup prefix.
#include <algorithm>

#include "philox.h"

namespace dpsgd {

namespace {

constexpr int kThreads = 256;
constexpr int64_t kPerWG = 4 * kThreads;

__device__ __forceinline__ uint32_t draw4(uint64_t seed, uint64_t step, uint64_t thr, int64_t b, int64_t n) {
    uint32_t bits = 0;
    if (4 * b < n) {
        const Philox4 w = philox4x32_10((uint64_t)b | (1ull << 63), step, seed);
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (4 * b + k < n && (uint64_t)w.x[k] < thr) bits |= 1u << k;
    }
    return bits;
}

// inclusive prefix sum of v over the wavefront
__device__ __forceinline__ int wave_prefix(int v, int lane) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int u = __shfl_up(v, o, 64);
        if (lane >= o) v += u;
    }
    return v;
}

}  // namespace

__global__ __launch_bounds__(256) void k_sample_count(uint64_t seed, uint64_t step, uint64_t thr,
                                                      int64_t n, uint8_t* mask, int64_t* wg_count) {
    __shared__ int wsum[kThreads / 64];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int64_t b = (int64_t)blockIdx.x * kThreads + tid;
    const uint32_t bits = draw4(seed, step, thr, b, n);
    if (mask && 4 * b < n) {
        if (4 * b + 4 <= n) {
            const uint32_t m = (bits & 1u) | ((bits & 2u) << 7) | ((bits & 4u) << 14) | ((bits & 8u) << 21);
            *reinterpret_cast<uint32_t*>(mask + 4 * b) = m;   // mask is 4-byte aligned
        } else {
            for (int k = 0; 4 * b + k < n; ++k) mask[4 * b + k] = (uint8_t)((bits >> k) & 1u);
        }
    }
    const int total = wave_prefix(__popc(bits), lane);
    if (lane == 63) wsum[w] = total;
    __syncthreads();
    if (tid == 0) wg_count[blockIdx.x] = (int64_t)wsum[0] + wsum[1] + wsum[2] + wsum[3];
}

// exclusive scan of the workgroup counts (one workgroup of 1024 threads, 1024 counts at a time)
__global__ __launch_bounds__(1024) void k_sample_scan(const int64_t* wg_count, int64_t n_wg,
                                                      int64_t* wg_off, int64_t* total) {
    __shared__ int64_t part[1024 / 64];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    int64_t carry = 0;
    for (int64_t c0 = 0; c0 < n_wg; c0 += 1024) {
        const int64_t i = c0 + tid;
        const int64_t v = i < n_wg ? wg_count[i] : 0;
        int64_t x = v;   // inclusive wave scan (int64)
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int64_t u = __shfl_up(x, o, 64);
            if (lane >= o) x += u;
        }
        if (lane == 63) part[w] = x;
        __syncthreads();
        int64_t before = carry;
        for (int k = 0; k < w; ++k) before += part[k];
        if (i < n_wg) wg_off[i] = before + x - v;
        int64_t chunk = 0;
        for (int k = 0; k < 1024 / 64; ++k) chunk += part[k];
        __syncthreads();
        carry += chunk;
    }
    if (tid == 0) *total = carry;
}

__global__ __launch_bounds__(256) void k_sample_write(uint64_t seed, uint64_t step, uint64_t thr,
                                                      int64_t n, const int64_t* wg_off,
                                                      int64_t* indices) {
    __shared__ int wsum[kThreads / 64];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int64_t b = (int64_t)blockIdx.x * kThreads + tid;
    const uint32_t bits = draw4(seed, step, thr, b, n);
    const int c = __popc(bits);
    const int incl = wave_prefix(c, lane);
    if (lane == 63) wsum[w] = incl;
    __syncthreads();
    int64_t pos = wg_off[blockIdx.x] + incl - c;
    for (int k = 0; k < w; ++k) pos += wsum[k];
#pragma unroll
    for (int k = 0; k < 4; ++k)
        if ((bits >> k) & 1u) indices[pos++] = 4 * b + k;
}

int64_t sample_wgs(int64_t n) { return (n + kPerWG - 1) / kPerWG; }

hipError_t launch_poisson_sample(uint64_t seed, uint64_t step, uint64_t thr, int64_t n, uint8_t* mask,
                                 int64_t* indices, int64_t* count, int64_t* ws, hipStream_t s) {
    const int64_t nwg = sample_wgs(n);
    int64_t* wg_count = ws;
    int64_t* wg_off = ws + nwg;
    if (nwg > 0)
        hipLaunchKernelGGL(k_sample_count, dim3((unsigned)nwg), dim3(kThreads), 0, s, seed, step, thr,
                           n, mask, wg_count);
    hipLaunchKernelGGL(k_sample_scan, dim3(1), dim3(1024), 0, s, wg_count, nwg, wg_off, count);
    if (nwg > 0)
        hipLaunchKernelGGL(k_sample_write, dim3((unsigned)nwg), dim3(kThreads), 0, s, seed, step, thr,
                           n, wg_off, indices);
    return hipGetLastError();
}

}  // namespace dpsgd
