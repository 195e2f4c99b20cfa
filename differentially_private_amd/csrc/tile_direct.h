// Direct-path tile engine: for one record i, one wavefront forms the block
//   D[m][n] = sum_t Y_i[t][m0 + m] * X_i[t][n0 + n]      (m < 16*MB, n < 128)
// of the record's gradient P_i = A_i^T G_i (or its transpose) with MFMA, the
// reduction running over the record's T tokens.  The block never leaves
// registers: the norm path squares and sums it, the clipped-sum path scales it
// by c_i and accumulates it over records, the STORED strategy writes it out.
//
// Both operands live in memory as [T, d] rows (d contiguous) while MFMA wants
// each lane to hold consecutive reduction indices (tokens).  X, the operand
// with the wide rows, is read straight from HBM with 16-byte loads (8 bf16 or
// 4 fp32 columns of one token row per lane) and, for bf16, transposed inside
// the lane: a lane loads the same 8 columns of 8 token rows and repacks the
// 8x8 block so that each of its 8 column vectors holds 8 tokens; the lane then
// feeds 8 MFMAs, one per column, whose 16 lanes of a row group cover 128
// columns.  fp32 MFMA 16x16x4 takes one token per lane, so there the 16-byte
// load feeds 4 MFMAs directly.  Y (at most 16*MB columns) is small and cached,
// and is read element-wise.
#pragma once

#include "device_common.h"
#include "internal.h"

namespace dpsgd {

// ---- bf16: 32 tokens per step, lane (g, c) holds tokens t0 + 8g + (0..7) ----
template <int MB>
__device__ __forceinline__ void direct_block_bf16(const uint16_t* __restrict__ X,
                                                  const uint16_t* __restrict__ Y, int64_t T,
                                                  int dX, int dY, int n0, int m0, bool vec_x,
                                                  int g, int c, f32x4 (&acc)[MB][8]) {
    const int col = n0 + 8 * c;
    const bool full = vec_x && (col + 8 <= dX);
    for (int64_t t0 = 0; t0 < T; t0 += 32) {
        u32x4 raw[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int64_t t = t0 + 8 * g + q;
            if (t < T && full) {
                raw[q] = load_stream(reinterpret_cast<const u32x4*>(X + t * dX + col));
            } else {
                uint32_t w[4] = {0u, 0u, 0u, 0u};
                if (t < T) {
#pragma unroll
                    for (int u = 0; u < 8; ++u) {
                        const uint32_t v = (col + u < dX) ? (uint32_t)X[t * dX + col + u] : 0u;
                        w[u >> 1] |= v << (16 * (u & 1));
                    }
                }
                raw[q] = u32x4{w[0], w[1], w[2], w[3]};
            }
        }
        // 8x8 transpose inside the lane: bv[j] word p = (token 2p, token 2p+1) of column j
        u32x4 bv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const uint32_t lo = raw[2 * p][j >> 1];
                const uint32_t hi = raw[2 * p + 1][j >> 1];
                bv[j][p] = (j & 1) ? __builtin_amdgcn_perm(hi, lo, 0x07060302u)
                                   : __builtin_amdgcn_perm(hi, lo, 0x05040100u);
            }
        }
        u32x4 av[MB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const int m = m0 + 16 * mb + c;
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const int64_t t = t0 + 8 * g + 2 * p;
                const uint32_t lo = (m < dY && t < T) ? (uint32_t)Y[t * dY + m] : 0u;
                const uint32_t hi = (m < dY && t + 1 < T) ? (uint32_t)Y[(t + 1) * dY + m] : 0u;
                av[mb][p] = lo | (hi << 16);
            }
        }
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[mb][j] = mfma_bf16(av[mb], bv[j], acc[mb][j]);
    }
}

// ---- fp32: MFMA 16x16x4 takes one token per lane: lane (g, c) holds token 4s + g ----
// The token rows are processed in half-steps of 8: the loads of one half are in
// flight while the MFMAs of the other run.
template <int MB>
__device__ __forceinline__ void load_half_f32(const float* __restrict__ X, const float* __restrict__ Y,
                                              int64_t T, int dX, int dY, int m0, int g, int c,
                                              int64_t t0, const int (&cols)[2], const bool (&full)[2],
                                              f32x4 (&xv)[2][2], float (&yv)[2][MB]) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        const int64_t t = t0 + 4 * s + g;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            if (t < T && full[h]) {
                xv[s][h] = load_stream(reinterpret_cast<const f32x4*>(X + t * dX + cols[h]));
            } else {
                f32x4 v = {0.f, 0.f, 0.f, 0.f};
                if (t < T) {
#pragma unroll
                    for (int u = 0; u < 4; ++u)
                        v[u] = (cols[h] + u < dX) ? X[t * dX + cols[h] + u] : 0.f;
                }
                xv[s][h] = v;
            }
        }
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const int m = m0 + 16 * mb + c;
            yv[s][mb] = (t < T && m < dY) ? Y[t * dY + m] : 0.f;
        }
    }
}

template <int MB>
__device__ __forceinline__ void mfma_half_f32(const f32x4 (&xv)[2][2], const float (&yv)[2][MB],
                                              f32x4 (&acc)[MB][8]) {
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[mb][h * 4 + j] = mfma_f32(yv[s][mb], xv[s][h][j], acc[mb][h * 4 + j]);
}

template <int MB>
__device__ __forceinline__ void direct_block_f32(const float* __restrict__ X,
                                                      const float* __restrict__ Y, int64_t T,
                                                      int dX, int dY, int n0, int m0, bool vec_x,
                                                      int g, int c, f32x4 (&acc)[MB][8]) {
    int cols[2];
    bool full[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        cols[h] = n0 + 64 * h + 4 * c;
        full[h] = vec_x && (cols[h] + 4 <= dX);
    }
    f32x4 xa[2][2], xb[2][2];
    float ya[2][MB], yb[2][MB];
    load_half_f32<MB>(X, Y, T, dX, dY, m0, g, c, 0, cols, full, xa, ya);
    for (int64_t t0 = 0; t0 < T; t0 += 16) {
        if (t0 + 8 < T) load_half_f32<MB>(X, Y, T, dX, dY, m0, g, c, t0 + 8, cols, full, xb, yb);
        mfma_half_f32<MB>(xa, ya, acc);
        if (t0 + 8 >= T) break;
        if (t0 + 16 < T) load_half_f32<MB>(X, Y, T, dX, dY, m0, g, c, t0 + 16, cols, full, xa, ya);
        mfma_half_f32<MB>(xb, yb, acc);
    }
}

// X column of accumulator `idx` for lane column c (see the two block routines).
template <int DT>
__device__ __forceinline__ int direct_col(int n0, int c, int idx) {
    if (DT == kBF16) return n0 + 8 * c + idx;
    return n0 + 64 * (idx >> 2) + 4 * c + (idx & 3);
}

// The record's block over its T token rows starting at row0.
template <int DT, int MB>
__device__ __forceinline__ void direct_block(const void* X, const void* Y, int64_t row0, int64_t T,
                                             int dX, int dY, int n0, int m0, bool vec_x, int g,
                                             int c, f32x4 (&acc)[MB][8]) {
    if (DT == kBF16) {
        direct_block_bf16<MB>(static_cast<const uint16_t*>(X) + row0 * dX,
                              static_cast<const uint16_t*>(Y) + row0 * dY, T, dX, dY, n0, m0,
                              vec_x, g, c, acc);
    } else {
        direct_block_f32<MB>(static_cast<const float*>(X) + row0 * dX,
                             static_cast<const float*>(Y) + row0 * dY, T, dX, dY, n0, m0, vec_x,
                             g, c, acc);
    }
}

// Write (or add) the block into a [d_in, d_out] row-major fp32 matrix `dst`.
// Element (m, n) of the block is row m0 + m of Y's columns and column n of X's.
// STORED (per-record gradient blocks in the workspace): the X indices of a whole tile are kept in
// store order when stored_permuted(d_out) (see StoredMap).
template <int DT, int MB, bool STREAM = false, bool STORED = false>
__device__ __forceinline__ void direct_store(float* __restrict__ dst, const DirectLayer& L, int n0,
                                             int m0, int g, int c, const f32x4 (&acc)[MB][8],
                                             bool add) {
    const int64_t d_out = L.d_out;
    const bool perm = STORED && stored_permuted(d_out) && n0 + 128 <= L.dX;
    if (L.x_is_in) {
        // dst[x_col * d_out + y_row]: the 4 rows r of a lane are consecutive y_row
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const int mr = m0 + 16 * mb + 4 * g;
#pragma unroll
            for (int idx = 0; idx < 8; ++idx) {
                const int n = direct_col<DT>(n0, c, idx);
                if (n >= L.dX) continue;
                float* p = dst + (int64_t)(perm ? n0 + 16 * idx + c : n) * d_out + mr;
                if (mr + 4 <= L.dY && (reinterpret_cast<uintptr_t>(p) & 15u) == 0) {
                    f32x4 v = acc[mb][idx];
                    if (add) v += *reinterpret_cast<f32x4*>(p);
                    if constexpr (STREAM) store_stream(v, reinterpret_cast<f32x4*>(p));
                    else *reinterpret_cast<f32x4*>(p) = v;
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (mr + r < L.dY) p[r] = (add ? p[r] : 0.f) + acc[mb][idx][r];
                }
            }
        }
    } else {
        // dst[y_row * d_out + x_col]: groups of 4 accumulators have consecutive x_col
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m0 + 16 * mb + 4 * g + r;
                if (m >= L.dY) continue;
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const int n = direct_col<DT>(n0, c, 4 * q);
                    float* p = dst + (int64_t)m * d_out + (perm ? n0 + 64 * q + 4 * c : n);
                    const f32x4 v0 = {acc[mb][4 * q][r], acc[mb][4 * q + 1][r],
                                      acc[mb][4 * q + 2][r], acc[mb][4 * q + 3][r]};
                    if (n + 4 <= L.dX && (reinterpret_cast<uintptr_t>(p) & 15u) == 0) {
                        f32x4 v = v0;
                        if (add) v += *reinterpret_cast<f32x4*>(p);
                        if constexpr (STREAM) store_stream(v, reinterpret_cast<f32x4*>(p));
                        else *reinterpret_cast<f32x4*>(p) = v;
                    } else {
#pragma unroll
                        for (int u = 0; u < 4; ++u)
                            if (n + u < L.dX) p[u] = (add ? p[u] : 0.f) + v0[u];
                    }
                }
            }
        }
    }
}

}  // namespace dpsgd
