// clipped_sum: S_l = sum_i c_i A_l[i]^T G_l[i] = A_l^T diag(c (x) 1_T) G_l
// ("Privacy-Preserving Machine Learning", DP-SGD phase 4, the sum of the
// clipped vectors; "Sensitivity Inflation ...", Eq. 3 F(D)).
//
// GEMM strategy: the tile engine of the direct path forms each record's block
// of A_i^T G_i with MFMA (fp32 accumulate) over its T tokens; the per-record
// scale c_i is applied to that fp32 block when it is folded into the running
// sum, so the bf16 operands are never rescaled and rounded.  Records are split
// into contiguous ranges (split-K over records); each range writes a partial
// block and a fixed-order reduction adds the partials, so the result is
// bitwise repeatable.
// STORED strategy: the direct norm pass already wrote every record's gradient
// block; the sum is sum_i c_i P_i over them in ascending record order.
// Both skip all work while the workspace status reports a nonfinite norm.
#include "record_sum.h"
#include "tile_direct.h"

namespace dpsgd {

// MB = 1: at least 3 wavefronts per SIMD (168 registers instead of 180-184, which allowed only
// two): the reads stream with more loads in flight (the 7B-shaped LoRA sum 46.9 -> 42.7 ms, the
// OPT-125M-shaped one 75.5 -> 67.8 us, bitwise equal); MB = 2 would spill at that bound.
template <int DT, int MB>
__global__ __launch_bounds__(128, MB == 1 ? 3 : 1) void k_sum_direct(DirectArgs args) {
    if (args.status && *args.status) return;
    const DirectLayer& L = args.L[blockIdx.z];
    const int w = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4, c = lane & 15;
    const int tile_y = blockIdx.x / L.wg_x;
    const int tile_x = (blockIdx.x - tile_y * L.wg_x) * args.wpb + w;
    if (tile_y >= L.tiles_y || tile_x >= L.tiles_x) return;
    const int n0 = tile_x * 128;
    const int m0 = tile_y * 16 * MB;
    const int64_t split = blockIdx.y;
    const int64_t r0 = split * args.rec_per_split;
    int64_t r1 = r0 + args.rec_per_split;
    if (r1 > args.n_rec) r1 = args.n_rec;

    f32x4 sum[MB][8];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int j = 0; j < 8; ++j) sum[mb][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int64_t rec = r0; rec < r1; ++rec) {
        f32x4 acc[MB][8];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[mb][j] = f32x4{0.f, 0.f, 0.f, 0.f};
        int64_t row0, len;
        record_rows(args.seg, rec, args.T, row0, len);
        direct_block<DT, MB>(L.X, L.Y, row0, len, L.dX, L.dY, n0, m0, L.vec_x != 0, g, c, acc);
        const float cf = args.clip[rec];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int j = 0; j < 8; ++j) sum[mb][j] += cf * acc[mb][j];
    }
    float* dst = L.P;
    bool add = args.accumulate != 0;
    if (L.split_stride) {
        dst += split * L.split_stride;
        add = false;
    }
    direct_store<DT, MB>(dst, L, n0, m0, g, c, sum, add);
}

// out[e] (+)= sum_k w_k src[k][e'], k ascending, accumulated in fp64 and rounded to fp32 once;
// w_k = clip[k] (STORED) or 1 (split partials); e' is the position where the blocks keep element
// e (a thread takes stored positions e' and writes e = stored_logical(e')).
template <bool WEIGHTED>
__global__ __launch_bounds__(256) void k_reduce(ReduceArgs a) {
    if (a.status && *a.status) return;
    const ReduceLayer& L = a.L[blockIdx.y];
    const int64_t e = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
    if (e >= L.n) return;
    const bool vec = (e + 4 <= L.n) && ((L.n & 3) == 0);
    if (vec) {
        double d[4] = {0.0, 0.0, 0.0, 0.0};
        int64_t k = 0;
        for (; k + 8 <= a.n_src; k += 8) {     // 8 independent loads in flight, ascending order
            f32x4 v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = load_stream(reinterpret_cast<const f32x4*>(L.src + (k + u) * L.n + e));
#pragma unroll
            for (int u = 0; u < 8; ++u) add_scaled(d, WEIGHTED ? a.clip[k + u] : 1.f, v[u]);
        }
        for (; k < a.n_src; ++k)
            add_scaled(d, WEIGHTED ? a.clip[k] : 1.f, load_stream(reinterpret_cast<const f32x4*>(L.src + k * L.n + e)));
        f32x4 s = {(float)d[0], (float)d[1], (float)d[2], (float)d[3]};
        f32x4* o = reinterpret_cast<f32x4*>(L.out + stored_logical(L.map, e));
        if (a.accumulate) s = *o + s;
        *o = s;
    } else {
        for (int64_t x = e; x < e + 4 && x < L.n; ++x) {
            double d = 0.0;
            for (int64_t k = 0; k < a.n_src; ++k)
                d = fma(WEIGHTED ? (double)a.clip[k] : 1.0, (double)L.src[k * L.n + x], d);
            const float s = (float)d;
            float* o = L.out + stored_logical(L.map, x);
            *o = a.accumulate ? *o + s : s;
        }
    }
}

hipError_t launch_sum_direct(const DirectArgs& a, int dtype, int mb, int n_splits, hipStream_t s) {
    int gx = 1;
    for (int l = 0; l < a.n_layers; ++l) {
        const int v = a.L[l].wg_x * a.L[l].tiles_y;
        if (v > gx) gx = v;
    }
    const dim3 grid(gx, n_splits, a.n_layers);
    if (dtype == kBF16) {
        if (mb == 1) hipLaunchKernelGGL((k_sum_direct<kBF16, 1>), grid, dim3(64 * a.wpb), 0, s, a);
        else hipLaunchKernelGGL((k_sum_direct<kBF16, 2>), grid, dim3(64 * a.wpb), 0, s, a);
    } else {
        if (mb == 1) hipLaunchKernelGGL((k_sum_direct<kF32, 1>), grid, dim3(64 * a.wpb), 0, s, a);
        else hipLaunchKernelGGL((k_sum_direct<kF32, 2>), grid, dim3(64 * a.wpb), 0, s, a);
    }
    return hipGetLastError();
}

hipError_t launch_reduce(const ReduceArgs& a, bool weighted, hipStream_t s) {
    const int64_t blocks = (a.max_n4 + 255) / 256;
    if (blocks == 0 || a.n_layers == 0) return hipSuccess;
    const dim3 grid((unsigned)blocks, a.n_layers);
    if (weighted) hipLaunchKernelGGL(k_reduce<true>, grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL(k_reduce<false>, grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace dpsgd
