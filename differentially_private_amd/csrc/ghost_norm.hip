// ghost_norm: per-record partial squared gradient norms of each layer, without
// forming the per-record gradient P_i = A_i^T G_i in memory ("Privacy-Preserving
// Machine Learning", DP-SGD phase 2: clipping factors before reduction, e.g. by
// ghost clipping).  Two paths, chosen per layer:
//  - direct (T^2 >= d_in * d_out): tiles of P_i formed in registers by MFMA over
//    the record's tokens, squared and summed (tile_direct.h); optionally the
//    tile is also written out for the STORED clipped-sum strategy;
//  - Gram (T^2 < d_in * d_out): ||A_i^T G_i||_F^2 = <A_i A_i^T, G_i G_i^T>_F =
//    sum_{t,s} (a_t . a_s)(g_t . g_s), with 64x64 blocks of both token Grams
//    formed by MFMA (rows of A and G are the MFMA reduction axis, so both
//    operands load straight from row-major memory) and reduced as a Hadamard
//    product; only the upper triangle of block pairs is visited, off-diagonal
//    pairs weighted by 2.
// Each wavefront writes one fp32 partial per (record, tile): the partials of a
// record depend only on that record's rows, so the norms are batch-invariant.
#include "tile_direct.h"

namespace dpsgd {

// fp32, MB = 1 (LoRA shapes): ask for at least 4 wavefronts per SIMD (the kernel
// then fits 5 without spilling), so that a whole LoRA workload's tiles are
// resident at once and no tail of late wavefronts is left.
template <int DT, int MB, bool STORE>
__global__ __launch_bounds__(128, (DT == kF32 && MB == 1) ? 4 : 1) void k_norm_direct(DirectArgs args) {
    const DirectLayer& L = args.L[blockIdx.z];
    const int w = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4, c = lane & 15;
    const int tile_y = blockIdx.x / L.wg_x;
    const int tile_x = (blockIdx.x - tile_y * L.wg_x) * args.wpb + w;
    if (tile_y >= L.tiles_y || tile_x >= L.tiles_x) return;
    const int n0 = tile_x * 128;
    const int m0 = tile_y * 16 * MB;
    const int64_t rec = blockIdx.y;

    f32x4 acc[MB][8];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[mb][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    direct_block<DT, MB>(L.X, L.Y, rec, args.T, L.dX, L.dY, n0, m0, L.vec_x != 0, g, c, acc);

    float s = 0.f;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) s += acc[mb][j][r] * acc[mb][j][r];
    s = wave_sum(s);
    if (lane == 0)
        args.parts[rec * args.parts_stride + L.part_off + tile_y * L.tiles_x + tile_x] = s;
    if (STORE) {
        float* dst = L.P + rec * (int64_t)L.dX * L.dY;
        direct_store<DT, MB>(dst, L, n0, m0, g, c, acc, false);
    }
}

// ---- Gram path ----

template <int DT>
__device__ __forceinline__ void gram_block(const void* M_, int64_t rec, int64_t T, int d, int t0,
                                           int s0, bool vec, int g, int c, f32x4 (&acc)[4][4]) {
    const bool diag = (t0 == s0);
    if (DT == kBF16) {
        const uint16_t* M = static_cast<const uint16_t*>(M_) + rec * T * d;
        for (int k0 = 0; k0 < d; k0 += 32) {
            const int k = k0 + 8 * g;
            const bool full = vec && (k + 8 <= d);
            u32x4 av[4], bv[4];
#pragma unroll
            for (int h = 0; h < 8; ++h) {
                if (diag && h >= 4) break;
                const int64_t t = (h < 4 ? t0 + 16 * h : s0 + 16 * (h - 4)) + c;
                u32x4 v;
                if (t < T && full) {
                    v = *reinterpret_cast<const u32x4*>(M + t * d + k);
                } else {
                    uint32_t wd[4] = {0u, 0u, 0u, 0u};
                    if (t < T) {
#pragma unroll
                        for (int u = 0; u < 8; ++u) {
                            const uint32_t e = (k + u < d) ? (uint32_t)M[t * d + k + u] : 0u;
                            wd[u >> 1] |= e << (16 * (u & 1));
                        }
                    }
                    v = u32x4{wd[0], wd[1], wd[2], wd[3]};
                }
                if (h < 4) av[h] = v; else bv[h - 4] = v;
            }
            if (diag) {
#pragma unroll
                for (int h = 0; h < 4; ++h) bv[h] = av[h];
            }
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = mfma_bf16(av[mi], bv[ni], acc[mi][ni]);
        }
    } else {
        const float* M = static_cast<const float*>(M_) + rec * T * d;
        for (int k0 = 0; k0 < d; k0 += 16) {
            const int k = k0 + 4 * g;
            const bool full = vec && (k + 4 <= d);
            f32x4 av[4], bv[4];
#pragma unroll
            for (int h = 0; h < 8; ++h) {
                if (diag && h >= 4) break;
                const int64_t t = (h < 4 ? t0 + 16 * h : s0 + 16 * (h - 4)) + c;
                f32x4 v = {0.f, 0.f, 0.f, 0.f};
                if (t < T && full) {
                    v = *reinterpret_cast<const f32x4*>(M + t * d + k);
                } else if (t < T) {
#pragma unroll
                    for (int u = 0; u < 4; ++u) v[u] = (k + u < d) ? M[t * d + k + u] : 0.f;
                }
                if (h < 4) av[h] = v; else bv[h - 4] = v;
            }
            if (diag) {
#pragma unroll
                for (int h = 0; h < 4; ++h) bv[h] = av[h];
            }
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                    for (int ni = 0; ni < 4; ++ni)
                        acc[mi][ni] = mfma_f32(av[mi][q], bv[ni][q], acc[mi][ni]);
        }
    }
}

template <int DT>
__global__ __launch_bounds__(256) void k_norm_gram(GramArgs args) {
    const GramLayer& L = args.L[blockIdx.z];
    const int w = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4, c = lane & 15;
    const int pair = blockIdx.x * 4 + w;
    if (pair >= args.n_pairs) return;
    int tb = 0, rem = pair;
    while (rem >= args.nb - tb) {
        rem -= args.nb - tb;
        ++tb;
    }
    const int sb = tb + rem;
    const int t0 = tb * 64, s0 = sb * 64;
    const int64_t rec = blockIdx.y;

    f32x4 ga[4][4], gg[4][4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) {
            ga[mi][ni] = f32x4{0.f, 0.f, 0.f, 0.f};
            gg[mi][ni] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    gram_block<DT>(L.A, rec, args.T, L.d_in, t0, s0, L.vec_a != 0, g, c, ga);
    gram_block<DT>(L.G, rec, args.T, L.d_out, t0, s0, L.vec_g != 0, g, c, gg);

    float s = 0.f;
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
#pragma unroll
            for (int r = 0; r < 4; ++r) s += ga[mi][ni][r] * gg[mi][ni][r];
    s = wave_sum(s);
    if (lane == 0)
        args.parts[rec * args.parts_stride + L.part_off + pair] = (tb == sb) ? s : 2.f * s;
}

hipError_t launch_norm_direct(const DirectArgs& a, int dtype, int mb, bool store, hipStream_t s) {
    int gx = 1;
    for (int l = 0; l < a.n_layers; ++l) {
        const int v = a.L[l].wg_x * a.L[l].tiles_y;
        if (v > gx) gx = v;
    }
    const dim3 grid(gx, (unsigned)a.n_rec, a.n_layers);
#define DPSGD_LAUNCH(DT, MB, ST) hipLaunchKernelGGL((k_norm_direct<DT, MB, ST>), grid, dim3(64 * a.wpb), 0, s, a)
    if (dtype == kBF16) {
        if (mb == 1) { if (store) DPSGD_LAUNCH(kBF16, 1, true); else DPSGD_LAUNCH(kBF16, 1, false); }
        else { if (store) DPSGD_LAUNCH(kBF16, 2, true); else DPSGD_LAUNCH(kBF16, 2, false); }
    } else {
        if (mb == 1) { if (store) DPSGD_LAUNCH(kF32, 1, true); else DPSGD_LAUNCH(kF32, 1, false); }
        else { if (store) DPSGD_LAUNCH(kF32, 2, true); else DPSGD_LAUNCH(kF32, 2, false); }
    }
#undef DPSGD_LAUNCH
    return hipGetLastError();
}

hipError_t launch_norm_gram(const GramArgs& a, int dtype, hipStream_t s) {
    const dim3 grid((a.n_pairs + 3) / 4, (unsigned)a.n_rec, a.n_layers);
    if (dtype == kBF16)
        hipLaunchKernelGGL(k_norm_gram<kBF16>, grid, dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL(k_norm_gram<kF32>, grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace dpsgd
