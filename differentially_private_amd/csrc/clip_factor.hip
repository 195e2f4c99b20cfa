// clip_factor: one joint norm per record over all layers, then the clip factor
//   n_i = sqrt(sum of the record's partial squared norms),
//   c_i = 1 if n_i <= C (a zero gradient is left unchanged), else C / n_i
// ("Privacy-Preserving Machine Learning", DP-SGD phase 3; the DP-SGD exhibit
// card's g / max(1, ||g||/C) is the same factor).  One wavefront per record:
// the lanes stride over the record's partials in a fixed order and a fixed
// shuffle butterfly combines them (in fp64), so n_i and c_i depend only on the
// record's own partials.  Up to 64 records, a single workgroup also resolves the
// status word (nonfinite norm) without inter-block synchronisation; larger batches
// spread over many workgroups (k_clip_wide).
#include "device_common.h"
#include "internal.h"

namespace dpsgd {

__global__ __launch_bounds__(1024) void k_clip(ClipArgs a) {
    __shared__ uint32_t bad;
    if (threadIdx.x == 0) bad = 0u;
    __syncthreads();
    const int w = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int nw = blockDim.x >> 6;
    for (int64_t rec0 = w; rec0 < a.n_rec; rec0 += 4 * nw) {
        double s4[4];
        record_norm2_x4(a.parts, a.parts_stride, a.n_parts, rec0, nw, a.n_rec, lane, s4);
        // every lane holds the four sums; lane j < 4 finishes record rec0 + j nw
        const int64_t rec = rec0 + (int64_t)lane * nw;
        if (lane < 4 && rec < a.n_rec) {
            const double s = lane == 0 ? s4[0] : lane == 1 ? s4[1] : lane == 2 ? s4[2] : s4[3];
            double n, cf;
            if (clip_of_norm2(s, a.C, n, cf)) atomicOr(&bad, 1u);
            a.n_ws[rec] = (float)n;
            a.c_ws[rec] = (float)cf;
            if (a.n_user) a.n_user[rec] = (float)n;
            if (a.c_user) a.c_user[rec] = (float)cf;
        }
    }
    __syncthreads();
    if (threadIdx.x == 0) *a.status = a.accumulate ? (*a.status | bad) : bad;
}

// The same per-record arithmetic over many workgroups, for batches with more records than one
// workgroup covers in a pass: wavefront gw of TW handles records gw + j TW (j < 4), so every record's
// partials are reduced exactly as in k_clip and n_i, c_i are bitwise the same.  A workgroup that
// saw a nonfinite norm ORs the flag into the status word, which a preceding k_status_clear has
// zeroed unless the call accumulates.
__global__ __launch_bounds__(256) void k_clip_wide(ClipArgs a) {
    __shared__ uint32_t bad;
    if (threadIdx.x == 0) bad = 0u;
    __syncthreads();
    const int lane = threadIdx.x & 63;
    const int64_t tw = (int64_t)gridDim.x * (blockDim.x >> 6);
    const int64_t gw = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    for (int64_t rec0 = gw; rec0 < a.n_rec; rec0 += 4 * tw) {
        double s4[4];
        record_norm2_x4(a.parts, a.parts_stride, a.n_parts, rec0, tw, a.n_rec, lane, s4);
        const int64_t rec = rec0 + (int64_t)lane * tw;
        if (lane < 4 && rec < a.n_rec) {
            const double s = lane == 0 ? s4[0] : lane == 1 ? s4[1] : lane == 2 ? s4[2] : s4[3];
            double n, cf;
            if (clip_of_norm2(s, a.C, n, cf)) atomicOr(&bad, 1u);
            a.n_ws[rec] = (float)n;
            a.c_ws[rec] = (float)cf;
            if (a.n_user) a.n_user[rec] = (float)n;
            if (a.c_user) a.c_user[rec] = (float)cf;
        }
    }
    __syncthreads();
    if (threadIdx.x == 0 && bad) atomicOr(a.status, bad);
}

__global__ void k_status_clear(uint32_t* status) {
    if (threadIdx.x == 0 && blockIdx.x == 0) *status = 0u;
}

__global__ __launch_bounds__(256) void k_layer_norm2(LayerNormArgs a) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= a.n_rec * a.n_layers) return;
    const int l = (int)(idx / a.n_rec);
    const int64_t rec = idx - (int64_t)l * a.n_rec;
    const float* p = a.parts + rec * a.parts_stride + a.part_off[l];
    double s = 0.0;
    for (int k = 0; k < a.n_part[l]; ++k) s += (double)p[k];
    a.out[idx] = (float)(s < 0.0 ? 0.0 : s);   // a squared norm: a negative rounded sum is 0
}

// One workgroup of 16 wavefronts covers 64 records per pass; larger batches go over
// ceil(n_rec / 16) workgroups of 4 wavefronts, each wavefront with four records.
hipError_t launch_clip(const ClipArgs& a, hipStream_t s) {
    if (a.n_rec <= 64) {
        hipLaunchKernelGGL(k_clip, dim3(1), dim3(1024), 0, s, a);
        return hipGetLastError();
    }
    if (!a.accumulate) {
        hipLaunchKernelGGL(k_status_clear, dim3(1), dim3(64), 0, s, a.status);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int64_t wgs = (a.n_rec + 15) / 16;
    hipLaunchKernelGGL(k_clip_wide, dim3((unsigned)wgs), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_status_clear(uint32_t* status, hipStream_t s) {
    hipLaunchKernelGGL(k_status_clear, dim3(1), dim3(64), 0, s, status);
    return hipGetLastError();
}

hipError_t launch_layer_norm2(const LayerNormArgs& a, hipStream_t s) {
    const int64_t n = a.n_rec * a.n_layers;
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(k_layer_norm2, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace dpsgd
