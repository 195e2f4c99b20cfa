// clipped_sum for dense layers (both d_in and d_out wide), bf16 inputs:
//   S = A^T diag(c (x) 1_T) G = sum_i c_i A_i^T G_i
// ("Privacy-Preserving Machine Learning", DP-SGD phase 4; "Sensitivity
// Inflation ...", Eq. 3), an MFMA GEMM with M = d_in, N = d_out and the
// reduction over the n_records * T token rows.
//
// Workgroup tile 256 (d_in) x 128 (d_out), 4 wavefronts of 128 x 64 (32 MFMAs
// per k-step each), two workgroups per CU, k-step 32 tokens (one
// v_mfma_f32_16x16x32_bf16 deep).  Both
// operands are stored with the reduction axis (tokens) as rows, so each k-step is
// staged through LDS transposed: a thread loads an 8 token x 8 column block
// (16-byte loads), transposes it in registers and writes 8 column vectors of 8
// tokens, so the MFMA operands are single 16-byte LDS reads.  Pitch 48 elements
// (96 bytes): measured on gfx950, the 16-lane operand reads then take 4 cycles
// (conflict-free; 8 at 80/112/144 bytes) and the staging writes 16.  Global loads
// run two k-steps ahead of the MFMAs (a register ring of two slots, the loop
// unrolled by two so that each slot stays in fixed registers: 244 VGPRs, no
// scratch), LDS is double-buffered with one barrier per k-step, and the second
// workgroup on the CU computes while the first waits.
//
// The per-record factor is applied to the fp32 accumulator, never to the bf16
// operands: with acc holding sum_{j<=i} (c_j / c_i) P_j during record i, the
// switch to record i+1 multiplies acc by c_i / c_{i+1}, and the end multiplies
// by the last factor (Horner form of sum_i c_i P_i).  |acc| stays below
// n_records * max(max_i n_i, C), far from fp32 overflow for finite fp32 norms.
#include <algorithm>

#include "device_common.h"
#include "internal.h"

namespace dpsgd {

namespace {

constexpr int kTM = 256;      // d_in columns per workgroup
constexpr int kTN = 128;      // d_out columns per workgroup
constexpr int kTK = 32;       // tokens per k-step
constexpr int kPitch = 48;    // LDS row pitch in bf16 elements (96 bytes)
constexpr int kDepth = 2;     // k-steps of global loads in flight ahead of the MFMAs

// Staging: thread b < 128 stages 8x8 block b of A's k-step tile (256 columns), thread
// 128 <= b < 192 block b - 128 of G's (128 columns): tokens 8 * (blk % 4) + (0..7), columns
// 8 * (blk / 4) + (0..7).  Threads 192..255 only compute.
struct Loader {
    int t8, col8;
};

__device__ __forceinline__ void load_step(const uint16_t* __restrict__ M, int64_t T, int d,
                                          int64_t rec, int ks, int col0, bool vec,
                                          const Loader& ld, u32x4 (&r)[8]) {
    const int col = col0 + 8 * ld.col8;
    const bool full = vec && (col + 8 <= d);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const int64_t t = (int64_t)ks * kTK + 8 * ld.t8 + q;
        const uint16_t* row = M + (rec * T + t) * (int64_t)d;
        if (t < T && full) {
            r[q] = *reinterpret_cast<const u32x4*>(row + col);
        } else {
            uint32_t w[4] = {0u, 0u, 0u, 0u};
            if (t < T) {
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const uint32_t v = (col + u < d) ? (uint32_t)row[col + u] : 0u;
                    w[u >> 1] |= v << (16 * (u & 1));
                }
            }
            r[q] = u32x4{w[0], w[1], w[2], w[3]};
        }
    }
}

// In-register 8x8 transpose: column j's 8 tokens become one 16-byte vector, written at
// Xs[8 * col8 + j][8 * t8].
__device__ __forceinline__ void store_step(uint16_t* Xs, const Loader& ld, const u32x4 (&r)[8]) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
        u32x4 v;
#pragma unroll
        for (int p = 0; p < 4; ++p) v[p] = __builtin_amdgcn_perm(r[2 * p + 1][j >> 1], r[2 * p][j >> 1], sel);
        *reinterpret_cast<u32x4*>(Xs + (8 * ld.col8 + j) * kPitch + 8 * ld.t8) = v;
    }
}

}  // namespace

__global__ __launch_bounds__(256, 2) void k_sum_dense_bf16(DenseSumArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t lds_a[2][kTM * kPitch];
    __shared__ __attribute__((aligned(16))) uint16_t lds_g[2][kTN * kPitch];
    if (a.status && *a.status) return;

    const DenseSumLayer& L = a.L[blockIdx.z];
    // XCD-aware order: workgroup ids go round-robin over the 8 XCDs; consecutive logical
    // tiles (same row band of d_in) are gathered on one XCD so that its L2 reuses them.
    const int n_tiles = L.tiles_m * L.tiles_n;
    int tile = blockIdx.x;
    if (n_tiles % 8 == 0) tile = (blockIdx.x % 8) * (n_tiles / 8) + blockIdx.x / 8;
    if (tile >= n_tiles) return;
    const int tm = tile / L.tiles_n, tn = tile % L.tiles_n;
    const int m0 = tm * kTM, n0 = tn * kTN;

    const int tid = threadIdx.x;
    const int w = tid >> 6, lane = tid & 63;
    const int g = lane >> 4, c = lane & 15;
    const int wm = w & 1, wn = w >> 1;          // wave tile: rows wm*128.., cols wn*64..
    const bool loads = tid < 192;
    const bool is_a = tid < 128;
    Loader ld;
    {
        const int b = is_a ? tid : tid - 128;
        ld.t8 = b & 3;
        ld.col8 = b >> 2;
    }
    const uint16_t* src = static_cast<const uint16_t*>(is_a ? L.A : L.G);
    const int d = is_a ? L.d_in : L.d_out;
    const int col0 = is_a ? m0 : n0;
    const bool vec = is_a ? L.vec_a : L.vec_g;
    uint16_t* stage[2] = {is_a ? lds_a[0] : lds_g[0], is_a ? lds_a[1] : lds_g[1]};

    const int64_t split = blockIdx.y;
    const int64_t r0 = split * a.rec_per_split;
    int64_t r1 = r0 + a.rec_per_split;
    if (r1 > a.n_rec) r1 = a.n_rec;
    const int nks = (int)((a.T + kTK - 1) / kTK);
    const int64_t total = (r1 - r0) * nks;

    f32x4 acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    float c_cur = 1.f;
    if (total > 0) {
        constexpr int D = kDepth;
        u32x4 ring[D][8];
        // (record, k-step) of the next load and of the step being multiplied
        int64_t lrec = r0, crec = r0;
        int lks = 0, cks = 0;
        auto advance = [nks](int64_t& rec, int& ks) {
            if (++ks == nks) {
                ks = 0;
                ++rec;
            }
        };
        // prologue: steps 0 .. D-1 in flight, step 0 staged into LDS buffer 0
#pragma unroll
        for (int k = 0; k < D; ++k) {
            if (loads && k < total) load_step(src, a.T, d, lrec, lks, col0, vec, ld, ring[k]);
            advance(lrec, lks);
        }
        if (loads) store_step(stage[0], ld, ring[0]);
        __syncthreads();

        c_cur = a.clip[r0];
        // one k-step: refill the slot step s came from with step s + D, multiply step s
        // out of LDS, stage step s + 1 (slot `next`) into the other LDS buffer.  The loop
        // below is unrolled by D so that every ring slot is a fixed register set.
        auto kstep = [&](int64_t s, u32x4 (&mine)[8], const u32x4 (&next)[8]) {
            const int buf = (int)(s & 1);
            if (loads && s + D < total) load_step(src, a.T, d, lrec, lks, col0, vec, ld, mine);
            advance(lrec, lks);
            // record boundary: rescale the accumulator to the new record's factor
            if (cks == 0 && s > 0) {
                const float c_new = a.clip[crec];
                const float f = c_cur / c_new;
#pragma unroll
                for (int i = 0; i < 8; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j) acc[i][j] *= f;
                c_cur = c_new;
            }
            advance(crec, cks);
            const uint16_t* As = lds_a[buf];
            const uint16_t* Gs = lds_g[buf];
            u32x4 bv[4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                bv[j] = *reinterpret_cast<const u32x4*>(Gs + (wn * 64 + 16 * j + c) * kPitch + 8 * g);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const u32x4 av = *reinterpret_cast<const u32x4*>(As + (wm * 128 + 16 * i + c) * kPitch + 8 * g);
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = mfma_bf16(av, bv[j], acc[i][j]);
            }
            if (loads && s + 1 < total) store_step(stage[buf ^ 1], ld, next);
            __syncthreads();
        };
        for (int64_t s = 0; s < total; s += D) {
#pragma unroll
            for (int k = 0; k < D; ++k)
                if (s + k < total) kstep(s + k, ring[k], ring[(k + 1) % D]);
        }
    }

    // epilogue: S = c_last * acc; lane (g, c) holds rows 4g + r, column c of each 16x16 block
    float* dst = L.out;
    bool add = a.accumulate != 0;
    if (L.split_stride) {
        dst = L.split + split * L.split_stride;
        add = false;
    }
    const int64_t d_out = L.d_out;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = m0 + wm * 128 + 16 * i + 4 * g + r;
            if (row >= L.d_in) continue;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int col = n0 + wn * 64 + 16 * j + c;
                if (col >= L.d_out) continue;
                float* p = dst + (int64_t)row * d_out + col;
                *p = (add ? *p : 0.f) + c_cur * acc[i][j][r];
            }
        }
    }
}

hipError_t launch_sum_dense(const DenseSumArgs& a, int n_splits, hipStream_t s) {
    int gx = 1;
    for (int l = 0; l < a.n_layers; ++l) gx = std::max(gx, a.L[l].tiles_m * a.L[l].tiles_n);
    hipLaunchKernelGGL(k_sum_dense_bf16, dim3(gx, n_splits, a.n_layers), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace dpsgd
