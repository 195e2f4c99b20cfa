// Poisson sampling of a step's records ("Privacy-Preserving Machine Learning", DP-SGD phase 1:
// each record is included independently with public probability q).  Record i draws word i mod 4
// of Philox4x32-10 block 2^63 + floor(i / 4) under key = seed and counter words 2-3 = step (the
// top bit of the block index keeps these words apart from the noise stream, whose blocks stay
// below 2^62) and is included iff that word < floor(q 2^32).
//
// Three launches and no atomics, so the index list is increasing and reproducible: each thread
// draws 32 records (eight Philox blocks), writes their bytes of the optional inclusion mask and their
// 32 inclusion bits to the workspace, and each 256-thread workgroup stores its count; one
// workgroup scans the counts (each thread a contiguous run of them, loaded eight at a time); each
// workgroup then reads its bits back and writes the included indices at its offset plus an
// in-workgroup prefix.  The Philox words are drawn once: the write pass reads 4 bytes per 32
// records instead of redrawing them.
#include <algorithm>

#include "philox.h"

namespace dpsgd {

namespace {

constexpr int kThreads = 256;
constexpr int kBlocksPerThread = 8;                     // Philox blocks of 4 records per thread
constexpr int64_t kPerThread = 4 * kBlocksPerThread;    // 32 records: bit k is record 32 g + k
constexpr int64_t kPerWG = kPerThread * kThreads;
constexpr int kScanThreads = 1024;

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

// draw4 for a block whose four records all exist, with the threshold as thr - 1 (thr >= 1): a
// word w is included iff w <= thr - 1, a 32-bit compare even for thr = 2^32 (q = 1)
__device__ __forceinline__ uint32_t draw4_full(uint64_t seed, uint64_t step, uint32_t thr_m1, int64_t b) {
    const Philox4 w = philox4x32_10((uint64_t)b | (1ull << 63), step, seed);
    uint32_t bits = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) bits |= (uint32_t)(w.x[k] <= thr_m1) << k;
    return bits;
}

// inclusive prefix sum of v over the wavefront
template <typename V>
__device__ __forceinline__ V wave_prefix(V v, int lane) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const V u = __shfl_up(v, o, 64);
        if (lane >= o) v += u;
    }
    return v;
}

// bytes 0/1 of four inclusion bits, as one little-endian word
__device__ __forceinline__ uint32_t mask_word(uint32_t b4) {
    return (b4 & 1u) | ((b4 & 2u) << 7) | ((b4 & 4u) << 14) | ((b4 & 8u) << 21);
}

}  // namespace

__global__ __launch_bounds__(kThreads) void k_sample_count(uint64_t seed, uint64_t step, uint64_t thr,
                                                           int64_t n, uint8_t* mask, uint32_t* bitsw,
                                                           int64_t* wg_count) {
    __shared__ int wsum[kThreads / 64];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int64_t g = (int64_t)blockIdx.x * kThreads + tid;
    const int64_t r0 = kPerThread * g;
    uint32_t bits = 0;
    if (thr != 0 && r0 + kPerThread <= n) {
        // all 32 records exist: no per-record bounds, 32-bit compares
        const uint32_t thr_m1 = (uint32_t)(thr - 1);
#pragma unroll
        for (int j = 0; j < kBlocksPerThread; ++j)
            bits |= draw4_full(seed, step, thr_m1, kBlocksPerThread * g + j) << (4 * j);
    } else {
#pragma unroll
        for (int j = 0; j < kBlocksPerThread; ++j)
            bits |= draw4(seed, step, thr, kBlocksPerThread * g + j, n) << (4 * j);
    }
    if (r0 < n) {
        bitsw[g] = bits;
        if (mask) {
            if (r0 + kPerThread <= n) {
#pragma unroll
                for (int j = 0; j < kBlocksPerThread; ++j)   // mask is 4-byte aligned
                    *reinterpret_cast<uint32_t*>(mask + r0 + 4 * j) = mask_word((bits >> (4 * j)) & 15u);
            } else {
                for (int k = 0; r0 + k < n; ++k) mask[r0 + k] = (uint8_t)((bits >> k) & 1u);
            }
        }
    }
    const int total = wave_prefix(__popc(bits), lane);
    if (lane == 63) wsum[w] = total;
    __syncthreads();
    if (tid == 0) wg_count[blockIdx.x] = (int64_t)wsum[0] + wsum[1] + wsum[2] + wsum[3];
}

// exclusive scan of the workgroup counts by one workgroup: thread t sums counts
// [t seg, (t + 1) seg), the sums are scanned across the workgroup, and each thread then writes the
// offsets of its run in order
__global__ __launch_bounds__(kScanThreads) void k_sample_scan(const int64_t* wg_count, int64_t n_wg,
                                                              int64_t* wg_off, int64_t* total) {
    __shared__ int64_t part[kScanThreads / 64];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int64_t seg = (n_wg + kScanThreads - 1) / kScanThreads;
    const int64_t lo = std::min<int64_t>(n_wg, tid * seg), hi = std::min<int64_t>(n_wg, lo + seg);
    int64_t sum = 0;
    int64_t i = lo;
    for (; i + 8 <= hi; i += 8) {   // eight independent loads in flight
        int64_t v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = wg_count[i + k];
#pragma unroll
        for (int k = 0; k < 8; ++k) sum += v[k];
    }
    for (; i < hi; ++i) sum += wg_count[i];
    const int64_t incl = wave_prefix(sum, lane);
    if (lane == 63) part[w] = incl;
    __syncthreads();
    int64_t off = incl - sum;
    for (int k = 0; k < w; ++k) off += part[k];
    for (i = lo; i + 8 <= hi; i += 8) {
        int64_t v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = wg_count[i + k];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            wg_off[i + k] = off;
            off += v[k];
        }
    }
    for (; i < hi; ++i) {
        const int64_t c = wg_count[i];
        wg_off[i] = off;
        off += c;
    }
    if (tid == kScanThreads - 1) *total = off;
}

__global__ __launch_bounds__(kThreads) void k_sample_write(int64_t n, const uint32_t* bitsw,
                                                           const int64_t* wg_off, int64_t* indices) {
    __shared__ int wsum[kThreads / 64];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int64_t g = (int64_t)blockIdx.x * kThreads + tid;
    const int64_t r0 = kPerThread * g;
    const uint32_t bits = r0 < n ? bitsw[g] : 0u;
    const int c = __popc(bits);
    const int incl = wave_prefix(c, lane);
    if (lane == 63) wsum[w] = incl;
    __syncthreads();
    int64_t pos = wg_off[blockIdx.x] + incl - c;
    for (int k = 0; k < w; ++k) pos += wsum[k];
    for (uint32_t m = bits; m; m &= m - 1) indices[pos++] = r0 + __builtin_ctz(m);
}

int64_t sample_wgs(int64_t n) { return (n + kPerWG - 1) / kPerWG; }

// workspace: wg_count[nwg], wg_off[nwg] (int64), then the inclusion bits (uint32 per 32 records)
int64_t sample_ws_bytes(int64_t n) {
    return 16 * sample_wgs(n) + 8 * (((n + kPerThread - 1) / kPerThread * 4 + 7) / 8);
}

hipError_t launch_poisson_sample(uint64_t seed, uint64_t step, uint64_t thr, int64_t n, uint8_t* mask,
                                 int64_t* indices, int64_t* count, int64_t* ws, hipStream_t s) {
    const int64_t nwg = sample_wgs(n);
    int64_t* wg_count = ws;
    int64_t* wg_off = ws + nwg;
    uint32_t* bitsw = reinterpret_cast<uint32_t*>(ws + 2 * nwg);
    if (nwg > 0)
        hipLaunchKernelGGL(k_sample_count, dim3((unsigned)nwg), dim3(kThreads), 0, s, seed, step, thr,
                           n, mask, bitsw, wg_count);
    hipLaunchKernelGGL(k_sample_scan, dim3(1), dim3(kScanThreads), 0, s, wg_count, nwg, wg_off, count);
    if (nwg > 0)
        hipLaunchKernelGGL(k_sample_write, dim3((unsigned)nwg), dim3(kThreads), 0, s, n, bitsw, wg_off,
                           indices);
    return hipGetLastError();
}

}  // namespace dpsgd
