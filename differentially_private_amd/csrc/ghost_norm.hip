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
#include <algorithm>
#include <type_traits>

#include "tile_direct.h"

namespace dpsgd {

// fp32, MB = 1 (LoRA shapes): ask for at least 4 wavefronts per SIMD (the kernel
// then fits 5 without spilling), so that a whole LoRA workload's tiles are
// resident at once and no tail of late wavefronts is left.  STORE: 0 = norms only, 1 = the
// gradient blocks written too (non-temporal stores, whole tiles in store order).
template <int DT, int MB, int STORE>
__global__ __launch_bounds__(128, (DT == kF32 && MB == 1) ? 4 : 1) void k_norm_direct(DirectArgs args) {
    const DirectLayer& L = args.L[blockIdx.z];
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // scalar: the tile origin is uniform
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

    int64_t row0, len;
    record_rows(args.seg, rec, args.T, row0, len);
    direct_block<DT, MB>(L.X, L.Y, row0, len, L.dX, L.dY, n0, m0, L.vec_x != 0, g, c, acc);

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
        direct_store<DT, MB, true, true>(dst, L, n0, m0, g, c, acc, false);
    }
}

// ---- Gram path ----

template <int DT>
__device__ __forceinline__ void gram_block(const void* M_, int64_t row0, int64_t T, int d, int t0,
                                           int s0, bool vec, int g, int c, f32x4 (&acc)[4][4]) {
    const bool diag = (t0 == s0);
    if (DT == kBF16) {
        const uint16_t* M = static_cast<const uint16_t*>(M_) + row0 * d;
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
        const float* M = static_cast<const float*>(M_) + row0 * d;
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
    int64_t row0, len;
    record_rows(args.seg, rec, args.T, row0, len);
    gram_block<DT>(L.A, row0, len, L.d_in, t0, s0, L.vec_a != 0, g, c, ga);
    gram_block<DT>(L.G, row0, len, L.d_out, t0, s0, L.vec_g != 0, g, c, gg);

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

// ---- Gram path, bf16 inputs with 16-byte aligned rows and d_in, d_out multiples of 32 ----
//
// One workgroup (4 waves) per (record, layer, 128-token block pair I <= J).  Wave (wm, wn) owns
// the 64 x 64 sub-pair (2I + wm, 2J + wn) of the 64-token block grid and writes the partial of
// that sub-pair to the same slot k_norm_gram uses: the Gram blocks of A and of G over all
// features, then the sum of their Hadamard product, doubled off the diagonal.  In a diagonal
// workgroup wave (1, 0) holds the mirror image of wave (0, 1)'s sub-pair and writes nothing.
//
// Features stream in steps of 64 through one copy pipeline, first A's d_in features, then G's
// d_out: per step the 128 I rows and 128 J rows (16 blocks of 16 rows, 32 KB) are copied by
// global_load_lds_dwordx4 with the non-temporal policy into 2 LDS stages, one step ahead, one
// barrier per step.  Each copy instruction moves 8 rows x 128 bytes, whole lines (64-byte pieces
// of long rows stream at about 70% of the rate of whole lines).  Stage layout: 16-row block b at
// 2 KB * b, rows 0-7 in its first KB and 8-15 in its second, 128 bytes per row, logical 16-byte
// chunk j of row r at chunk j ^ row_swz(r), so that the 16 rows of an MFMA operand read (lane
// 16 g + c: row c, chunk 4 q + g for the q-th 32 features of the step) fall on 16 distinct
// 16-byte bank slots; the copies write LDS linearly by lane, so the swizzle is applied to the
// source chunk, inside the same line.  A width that is an odd multiple of 32 ends with a half
// step.  Token rows past T are copied from row T - 1 and left out of the Hadamard sum.
constexpr int kGramB = 128;                   // tokens per block
constexpr int kGramK = 32;                    // feature granularity of the Gram copy kernels
constexpr int kGramCK = 64;                   // features per step
constexpr int kGramStages = 2;
constexpr int kGramStage = 2 * kGramB * kGramCK * 2;   // 32 KB: I rows, then J rows

__device__ __forceinline__ int row_swz(int r) { return (r >> 1) & 7; }

// a step of NQ 32-feature halves (2, or 1 for a half step)
template <int N>
using Subs = std::integral_constant<int, N>;

__global__ __launch_bounds__(256, 2) void k_norm_gram_copy(GramArgs args) {
    __shared__ __attribute__((aligned(16))) uint16_t lds[kGramStages * kGramStage / 2];
    const GramLayer& L = args.L[blockIdx.z];
    const int nb = (int)((args.T + kGramB - 1) / kGramB);
    const int np = nb * (nb + 1) / 2;
    // workgroup -> (record, pair): workgroup ids go round-robin over the 8 XCDs and the pairs
    // of one record get ids equal mod 8, so they share an XCD's L2
    const int x = blockIdx.x;
    const int q8 = x >> 3;
    const int pair = q8 % np;
    const int64_t rec = 8 * (int64_t)(q8 / np) + (x & 7);
    if (rec >= args.n_rec) return;
    int I = 0, rem = pair;
    while (rem >= nb - I) {
        rem -= nb - I;
        ++I;
    }
    const int J = I + rem;

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;   // w: scalar
    const int g = lane >> 4, c = lane & 15;
    const int wm = w & 1, wn = w >> 1;
    const int64_t T = args.T;
    const int tb = 2 * I + wm, sb = 2 * J + wn;          // 64-token sub-blocks of this wave
    const bool mirror = (I == J) && wm > wn;
    const bool active = !mirror && tb < args.nb && sb < args.nb;

    // copies: half-blocks 0..15 are I rows 8 h .., 16..31 J rows 8 (h - 16) ..; wave w issues
    // half-blocks 8 w .. 8 w + 7 (half-block h is 16-row block h / 2, rows 8 (h % 2) ..); lane L
    // fetches physical chunk L % 8 of row L / 8 of the half-block, i.e. logical chunk
    // (L % 8) ^ row_swz(8 (h % 2) + L / 8), the row clamped to T - 1
    uint32_t offa[8], offg[8];   // byte offsets from the record's row 0 at the step's features
    uint32_t hi4[2];             // what a half step takes off (logical chunk j -> j & 3)
#pragma unroll
    for (int e = 0; e < 2; ++e) hi4[e] = 16u * (uint32_t)((((lane & 7) ^ row_swz(8 * e + (lane >> 3)))) & 4);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int h = 8 * w + k;
        const int jl = (lane & 7) ^ row_swz(8 * (h & 1) + (lane >> 3));
        int64_t t = (h < 16 ? (int64_t)I * kGramB + 8 * h : (int64_t)J * kGramB + 8 * (h - 16)) + (lane >> 3);
        if (t > T - 1) t = T - 1;
        offa[k] = (uint32_t)((t * L.d_in + 8 * jl) * 2);
        offg[k] = (uint32_t)((t * L.d_out + 8 * jl) * 2);
    }
    const int nA = (L.d_in + kGramCK - 1) / kGramCK, nG = (L.d_out + kGramCK - 1) / kGramCK;
    const bool halfA = L.d_in % kGramCK != 0, halfG = L.d_out % kGramCK != 0;
    const int total = nA + nG;
    const char* recA = static_cast<const char*>(L.A) + rec * T * L.d_in * 2;
    const char* recG = static_cast<const char*>(L.G) + rec * T * L.d_out * 2;
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_addr(lds));
    auto issue = [&](int s, int st) {
        const uint32_t dst = lds0 + (uint32_t)(st * kGramStage + 8 * w * 1024);
        if (s < nA) {
            const char* base = recA + (int64_t)s * kGramCK * 2;
            const bool half = halfA && s == nA - 1;
#pragma unroll
            for (int k = 0; k < 8; ++k) copy16_nt(base, offa[k] - (half ? hi4[k & 1] : 0u), dst + k * 1024);
        } else {
            const char* base = recG + (int64_t)(s - nA) * kGramCK * 2;
            const bool half = halfG && s == total - 1;
#pragma unroll
            for (int k = 0; k < 8; ++k) copy16_nt(base, offg[k] - (half ? hi4[k & 1] : 0u), dst + k * 1024);
        }
    };
    // operand offsets (elements, within a 16-row block) of this lane's row c, logical chunk
    // 4 q + g, for the two 32-feature halves q of a step
    int lofs[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) lofs[q] = 512 * (c >> 3) + 64 * (c & 7) + 8 * ((4 * q + g) ^ row_swz(c));

    f32x4 ga[4][4], gg[4][4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) {
            ga[mi][ni] = f32x4{0.f, 0.f, 0.f, 0.f};
            gg[mi][ni] = f32x4{0.f, 0.f, 0.f, 0.f};
        }

    auto step = [&](const uint16_t* S, f32x4 (&acc)[4][4], auto subs) {
        constexpr int NQ = decltype(subs)::value;
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            u32x4 av[4], bv[4];
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
                av[mi] = *reinterpret_cast<const u32x4*>(S + (4 * wm + mi) * 1024 + lofs[q]);
#pragma unroll
            for (int ni = 0; ni < 4; ++ni)
                bv[ni] = *reinterpret_cast<const u32x4*>(S + (8 + 4 * wn + ni) * 1024 + lofs[q]);
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = mfma_bf16(av[mi], bv[ni], acc[mi][ni]);
        }
    };
    if (total > 0) issue(0, 0);
    int s = 0;
    // publish step s (this wave's copies done, the next step's may stay in flight); the barrier
    // also retires step s - 1, whose stage the copies of step s + 1 reuse
    auto begin = [&]() -> const uint16_t* {
        if (s + 1 < total) {
            __syncthreads();   // step s - 1's stage is free
            issue(s + 1, (s + 1) & 1);
            asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
        } else {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }
        __syncthreads();
        return lds + (s & 1) * (kGramStage / 2);
    };
    // one loop per phase and kind of step, so that each loop touches one accumulator set
    for (const int e = nA - (halfA ? 1 : 0); s < e; ++s) {
        const uint16_t* S = begin();
        if (active) step(S, ga, Subs<2>{});
    }
    if (halfA) {
        const uint16_t* S = begin();
        if (active) step(S, ga, Subs<1>{});
        ++s;
    }
    for (const int e = total - (halfG ? 1 : 0); s < e; ++s) {
        const uint16_t* S = begin();
        if (active) step(S, gg, Subs<2>{});
    }
    if (halfG) {
        const uint16_t* S = begin();
        if (active) step(S, gg, Subs<1>{});
        ++s;
    }

    // Hadamard sum over this wave's valid entries: lane (g, c) holds rows 4g + r, column c of
    // each 16 x 16 block
    float sum = 0.f;
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t t = (int64_t)64 * tb + 16 * mi + 4 * g + r;
                const int64_t u = (int64_t)64 * sb + 16 * ni + c;
                const float v = ga[mi][ni][r] * gg[mi][ni][r];
                sum += (t < T && u < T) ? v : 0.f;
            }
    sum = wave_sum(sum);
    if (active && lane == 0) {
        const int nb64 = args.nb;
        const int p64 = tb * nb64 - tb * (tb - 1) / 2 + (sb - tb);
        args.parts[rec * args.parts_stride + L.part_off + p64] = (tb == sb) ? sum : 2.f * sum;
    }
}

// ---- Gram path, one workgroup per (record, layer) when T <= 256 ----
//
// Same inputs as k_norm_gram_copy (bf16, 16-byte aligned rows, d_in and d_out multiples
// of 32), with the nb (nb + 1) / 2 upper-triangle pairs of 64-token blocks of one
// (record, layer) in a single workgroup, so each token row is copied into LDS once per
// feature step rather than once per block pair it belongs to.  A feature step is 64 features,
// one whole 128-byte line of every token row: each copy instruction moves 8 rows x 128 bytes,
// so no line is fetched from HBM in two halves at different times (64-byte pieces of 8 KB rows,
// the 32-feature steps of the pair kernel, stream at about 70% of the rate of whole lines), and
// the copies take the non-temporal policy, since every byte is read once.  The last step of A
// or G is a half step when the width is an odd multiple of 32.
// Wavefronts:
//  - one per off-diagonal pair (tb < sb): the full 64 x 64 Gram blocks of A and G,
//    formed exactly as a k_norm_gram_copy wavefront forms them;
//  - one per two diagonal blocks: only the 10 upper-triangle 16 x 16 tiles of each
//    64 x 64 diagonal block (the Gram is symmetric), the strictly upper ones doubled in
//    the Hadamard sum.
// For nb = 4 that is 6 + 2 = 8 wavefronts, two per SIMD.  Each wavefront issues the
// same number of 1 KB copies per step (half-blocks w * per + j mod 8 nb; a half-block may be
// copied twice, with the same bytes to the same place), so one vmcnt value describes every
// wavefront's copies in flight.  Partials go to the slots k_norm_gram uses.
//
// Stage layout: 16-row block b at 2 KB * b, its rows 0-7 in the first KB and 8-15 in the
// second, 128 bytes per row; logical 16-byte chunk j of row r (8 features) sits at chunk
// j ^ row_swz(r).  An MFMA operand read (lane 16 g + c: row c, chunk 4 q + g for the q-th 32
// features of the step) then puts the 16 rows of each 16-lane group on 16 distinct 16-byte
// bank slots (rows of one parity differ in r >> 1).  The copies write LDS linearly by lane,
// so the swizzle is applied to the source chunk, inside the same 128-byte line.
constexpr int kGramRecMaxNb = 4;                 // T <= 256
constexpr int kGramRecWaves = 8;                 // for nb = 4
constexpr int kGramRecK = 64;                    // features per step
constexpr int kGramRecMaxLds = 144 * 1024;
constexpr int kGramRecMaxStages = 8;
// a pair of steps per barrier needs both copied before the previous pair's barrier retires
// its stages: 4 stages or more (nb = 4: 4; nb = 3: 6; nb <= 2: 8)
static_assert(kGramRecMaxLds / (8 * kGramRecMaxNb * 1024) >= 4, "stages");

// s_waitcnt vmcnt(n) for a run-time n in [0, 63]
__device__ __forceinline__ void wait_vm(int n) {
    switch (n) {
#define DPSGD_VM(k) case k: asm volatile("s_waitcnt vmcnt(" #k ")" ::: "memory"); break;
        DPSGD_VM(1) DPSGD_VM(2) DPSGD_VM(3) DPSGD_VM(4) DPSGD_VM(5) DPSGD_VM(6) DPSGD_VM(7)
        DPSGD_VM(8) DPSGD_VM(9) DPSGD_VM(10) DPSGD_VM(11) DPSGD_VM(12) DPSGD_VM(13) DPSGD_VM(14)
        DPSGD_VM(15) DPSGD_VM(16) DPSGD_VM(17) DPSGD_VM(18) DPSGD_VM(19) DPSGD_VM(20) DPSGD_VM(21)
        DPSGD_VM(22) DPSGD_VM(23) DPSGD_VM(24) DPSGD_VM(25) DPSGD_VM(26) DPSGD_VM(27) DPSGD_VM(28)
        DPSGD_VM(29) DPSGD_VM(30) DPSGD_VM(31) DPSGD_VM(32) DPSGD_VM(33) DPSGD_VM(34) DPSGD_VM(35)
        DPSGD_VM(36) DPSGD_VM(37) DPSGD_VM(38) DPSGD_VM(39) DPSGD_VM(40) DPSGD_VM(41) DPSGD_VM(42)
        DPSGD_VM(43) DPSGD_VM(44) DPSGD_VM(45) DPSGD_VM(46) DPSGD_VM(47) DPSGD_VM(48) DPSGD_VM(49)
        DPSGD_VM(50) DPSGD_VM(51) DPSGD_VM(52) DPSGD_VM(53) DPSGD_VM(54) DPSGD_VM(55) DPSGD_VM(56)
        DPSGD_VM(57) DPSGD_VM(58) DPSGD_VM(59) DPSGD_VM(60) DPSGD_VM(61) DPSGD_VM(62) DPSGD_VM(63)
#undef DPSGD_VM
        default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    }
}

// upper-triangle 16 x 16 tile (mi <= ni) of a 64 x 64 diagonal block -> 0..9
__host__ __device__ constexpr int tri_tile(int mi, int ni) { return mi * 4 - mi * (mi - 1) / 2 + (ni - mi); }

__global__ __launch_bounds__(64 * kGramRecWaves) void k_norm_gram_rec(GramArgs args, int n_stages) {
    extern __shared__ __attribute__((aligned(16))) uint16_t lds_rec[];
    const GramLayer& L = args.L[blockIdx.y];
    const int64_t rec = blockIdx.x;
    const int64_t T = args.T;
    const int nb = args.nb;                 // 64-token blocks (1..4)
    const int n_off = nb * (nb - 1) / 2;    // off-diagonal pairs: waves 0 .. n_off - 1
    const int n8 = 8 * nb;                  // 8-row half-blocks per stage (rows past T repeat row T - 1)
    const int stage_elems = n8 * 512;       // 1 KB per half-block
    const int nw = (int)(blockDim.x >> 6);  // n_off + ceil(nb / 2)
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int g = lane >> 4, c = lane & 15;
    const bool off_wave = w < n_off;
    // off-diagonal wave: pair (tb, sb), tb < sb, in row-major order; diagonal wave: blocks
    // d0 = 2 (w - n_off) and d0 + 1 (if < nb)
    int tb = 0, sb = 0;
    if (off_wave) {
        int rem = w;
        while (rem >= nb - 1 - tb) {
            rem -= nb - 1 - tb;
            ++tb;
        }
        sb = tb + 1 + rem;
    }
    const int d0 = 2 * (w - n_off);
    const bool has_d1 = !off_wave && d0 + 1 < nb;

    // copies: wave w issues half-blocks h = (w * per + j) mod n8, j < per; lane L fetches
    // physical chunk L % 8 of row 8 (h % 2) + L / 8 of block h / 2 (token row clamped to T - 1),
    // i.e. logical chunk (L % 8) ^ row_swz(row); a half step reads chunk (logical & 3) instead,
    // inside the row, and those LDS chunks are never read.
    const int per = (n8 + nw - 1) / nw;     // 4 .. 8
    // Half-block h of a step holds token rows 8 h .. 8 h + 7 (rows 8 e .. 8 e + 7 of 16-row block
    // h / 2, e = h % 2); this lane copies row 8 h + lane / 8 (clamped to T - 1), logical chunk
    // (lane % 8) ^ row_swz(8 e + lane / 8).  A wave's j-th copy has parity e = (w per + j) % 2 (8 nb
    // is even), so the lane's part of the source offset is one of two values per tensor, indexed
    // by j % 2; the rows' part, 16 h d bytes, goes into the scalar base.
    const int tlast = (int)T - 1;           // T <= 256 here
    int hs[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) hs[j] = (w * per + j) % n8;
    int jls[2];
    uint32_t vA[2], vG[2], hi4[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const int par = (w * per + e) & 1;
        jls[e] = (lane & 7) ^ row_swz(8 * par + (lane >> 3));
        vA[e] = (uint32_t)(lane >> 3) * (uint32_t)L.d_in * 2u + 16u * (uint32_t)jls[e];
        vG[e] = (uint32_t)(lane >> 3) * (uint32_t)L.d_out * 2u + 16u * (uint32_t)jls[e];
        hi4[e] = 16u * (uint32_t)(jls[e] & 4);   // a half step reads logical chunk j & 3
    }
    const int nA = (L.d_in + kGramRecK - 1) / kGramRecK, nG = (L.d_out + kGramRecK - 1) / kGramRecK;
    const bool halfA = L.d_in % kGramRecK != 0, halfG = L.d_out % kGramRecK != 0;
    const int total = nA + nG;
    const char* recA = static_cast<const char*>(L.A) + rec * T * L.d_in * 2;
    const char* recG = static_cast<const char*>(L.G) + rec * T * L.d_out * 2;
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_addr(lds_rec));
    auto issue = [&](int s, int st) {
        const uint32_t dst = lds0 + (uint32_t)(st * stage_elems * 2);
        const bool a_step = s < nA;
        const char* base = a_step ? recA + (int64_t)s * kGramRecK * 2 : recG + (int64_t)(s - nA) * kGramRecK * 2;
        const bool half = a_step ? (halfA && s == nA - 1) : (halfG && s == total - 1);
        const uint32_t d = (uint32_t)(a_step ? L.d_in : L.d_out);
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (j < per) {
                const int h = hs[j];
                if (8 * h + 7 <= tlast) {
                    const uint32_t off = (a_step ? vA[j & 1] : vG[j & 1]) - (half ? hi4[j & 1] : 0u);
                    copy16_nt(base + (int64_t)h * 16 * d, off, dst + (uint32_t)h * 1024u);
                } else {
                    const int t = min(8 * h + (lane >> 3), tlast);
                    const int jl = half ? (jls[j & 1] & 3) : jls[j & 1];
                    copy16_nt(base, (uint32_t)t * d * 2u + 16u * (uint32_t)jl, dst + (uint32_t)h * 1024u);
                }
            }
    };
    // operand offsets (elements, within a 16-row block) of this lane's row c, logical chunk
    // 4 q + g, for the two 32-feature halves q of a step
    int lofs[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) lofs[q] = 512 * (c >> 3) + 64 * (c & 7) + 8 * ((4 * q + g) ^ row_swz(c));

    // The copy pipeline: feature steps in pairs per barrier (one at the end of a phase), the A
    // steps then the G steps, so that the second step's LDS reads overlap the first's MFMAs and
    // the wavefronts meet half as often (189 against 201 us per launch on workload 4 with one
    // step per barrier).  At a group's barrier its steps are copied and every earlier step is
    // retired, and the freed stages are refilled with the next steps to copy.  Each role runs
    // its own copy of the loop so that its accumulators live only there; both pass the same
    // barriers.
    const int n = n_stages;
    auto pipeline = [&](auto&& step_a, auto&& step_g) {
        int next = min(n, total);   // next step to copy
        for (int k = 0; k < next; ++k) issue(k, k);
        int s = 0;
        // steps s .. s + m - 1 published by one barrier, which also retires the steps before s
        auto begin = [&](int m) {
            wait_vm(per * (next - s - m));
            __syncthreads();
            const int lim = min(total, s + n);
            for (; next < lim; ++next) issue(next, next % n);
        };
        auto S = [&](int k) { return lds_rec + (k % n) * stage_elems; };
        // one loop per phase and kind of step, so that each loop touches one accumulator set
        for (const int e = nA - (halfA ? 1 : 0); s + 1 < e; s += 2) {
            begin(2);
            step_a(S(s), Subs<2>{});
            step_a(S(s + 1), Subs<2>{});
        }
        if (s < nA - (halfA ? 1 : 0)) begin(1), step_a(S(s), Subs<2>{}), ++s;
        if (halfA) begin(1), step_a(S(s), Subs<1>{}), ++s;
        for (const int e = total - (halfG ? 1 : 0); s + 1 < e; s += 2) {
            begin(2);
            step_g(S(s), Subs<2>{});
            step_g(S(s + 1), Subs<2>{});
        }
        if (s < total - (halfG ? 1 : 0)) begin(1), step_g(S(s), Subs<2>{}), ++s;
        if (halfG) begin(1), step_g(S(s), Subs<1>{}), ++s;
    };
    float* parts = args.parts + rec * args.parts_stride + L.part_off;

    // Hadamard sums below: lane (g, c) holds rows 4g + r, column c of each 16 x 16 tile
    if (off_wave) {
        f32x4 ga[16], gg[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            ga[i] = f32x4{0.f, 0.f, 0.f, 0.f};
            gg[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        auto step = [&](const uint16_t* S, f32x4 (&acc)[16], auto subs) {
            constexpr int NQ = decltype(subs)::value;
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                u32x4 av[4], bv[4];
#pragma unroll
                for (int mi = 0; mi < 4; ++mi)
                    av[mi] = *reinterpret_cast<const u32x4*>(S + (4 * tb + mi) * 1024 + lofs[q]);
#pragma unroll
                for (int ni = 0; ni < 4; ++ni)
                    bv[ni] = *reinterpret_cast<const u32x4*>(S + (4 * sb + ni) * 1024 + lofs[q]);
#pragma unroll
                for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                    for (int ni = 0; ni < 4; ++ni)
                        acc[4 * mi + ni] = mfma_bf16(av[mi], bv[ni], acc[4 * mi + ni]);
                // the next half's operand reads follow these MFMAs (and overlap their execution)
                if (q + 1 < NQ) __builtin_amdgcn_sched_barrier(0);
            }
        };
        pipeline([&](const uint16_t* S, auto subs) { step(S, ga, subs); },
                 [&](const uint16_t* S, auto subs) { step(S, gg, subs); });
        float sum = 0.f;
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
            for (int ni = 0; ni < 4; ++ni)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int64_t t = (int64_t)64 * tb + 16 * mi + 4 * g + r;
                    const int64_t u = (int64_t)64 * sb + 16 * ni + c;
                    const float v = ga[4 * mi + ni][r] * gg[4 * mi + ni][r];
                    sum += (t < T && u < T) ? v : 0.f;
                }
        sum = wave_sum(sum);
        if (lane == 0) parts[tb * nb - tb * (tb - 1) / 2 + (sb - tb)] = 2.f * sum;
    } else {
        // tiles 0..9 of block d0, 10..19 of block d1 = min(d0 + 1, nb - 1) (computed, and
        // dropped, when d0 is the last block: no branch between the loads and the MFMAs)
        const int d1 = has_d1 ? d0 + 1 : d0;
        f32x4 da[20], dg[20];
#pragma unroll
        for (int i = 0; i < 20; ++i) {
            da[i] = f32x4{0.f, 0.f, 0.f, 0.f};
            dg[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        auto step = [&](const uint16_t* S, f32x4 (&acc)[20], auto subs) {
            constexpr int NQ = decltype(subs)::value;
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                u32x4 av[2][4];
#pragma unroll
                for (int mi = 0; mi < 4; ++mi) {
                    av[0][mi] = *reinterpret_cast<const u32x4*>(S + (4 * d0 + mi) * 1024 + lofs[q]);
                    av[1][mi] = *reinterpret_cast<const u32x4*>(S + (4 * d1 + mi) * 1024 + lofs[q]);
                }
#pragma unroll
                for (int e = 0; e < 2; ++e)
#pragma unroll
                    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                        for (int ni = mi; ni < 4; ++ni) {
                            const int k = 10 * e + tri_tile(mi, ni);
                            acc[k] = mfma_bf16(av[e][mi], av[e][ni], acc[k]);
                        }
                if (q + 1 < NQ) __builtin_amdgcn_sched_barrier(0);
            }
        };
        pipeline([&](const uint16_t* S, auto subs) { step(S, da, subs); },
                 [&](const uint16_t* S, auto subs) { step(S, dg, subs); });
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            if (e == 1 && !has_d1) break;
            const int d = d0 + e;
            float sum = 0.f;
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                for (int ni = mi; ni < 4; ++ni) {
                    const int q = 10 * e + tri_tile(mi, ni);
                    float part = 0.f;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int64_t t = (int64_t)64 * d + 16 * mi + 4 * g + r;
                        const int64_t u = (int64_t)64 * d + 16 * ni + c;
                        const float v = da[q][r] * dg[q][r];
                        part += (t < T && u < T) ? v : 0.f;
                    }
                    sum += (mi == ni) ? part : 2.f * part;
                }
            sum = wave_sum(sum);
            if (lane == 0) parts[d * nb - d * (d - 1) / 2] = sum;
        }
    }
}

hipError_t launch_norm_direct(const DirectArgs& a, int dtype, int mb, int store, hipStream_t s) {
    int gx = 1;
    for (int l = 0; l < a.n_layers; ++l) {
        const int v = a.L[l].wg_x * a.L[l].tiles_y;
        if (v > gx) gx = v;
    }
    const dim3 grid(gx, (unsigned)a.n_rec, a.n_layers);
#define DPSGD_LAUNCH(DT, MB, ST) hipLaunchKernelGGL((k_norm_direct<DT, MB, ST>), grid, dim3(64 * a.wpb), 0, s, a)
#define DPSGD_LAUNCH_ST(DT, MB)                          \
    do {                                                 \
        if (store) DPSGD_LAUNCH(DT, MB, 1);              \
        else DPSGD_LAUNCH(DT, MB, 0);                    \
    } while (0)
    if (dtype == kBF16) {
        if (mb == 1) DPSGD_LAUNCH_ST(kBF16, 1);
        else DPSGD_LAUNCH_ST(kBF16, 2);
    } else {
        if (mb == 1) DPSGD_LAUNCH_ST(kF32, 1);
        else DPSGD_LAUNCH_ST(kF32, 2);
    }
#undef DPSGD_LAUNCH_ST
#undef DPSGD_LAUNCH
    return hipGetLastError();
}

hipError_t launch_norm_gram(const GramArgs& a, int dtype, hipStream_t s) {
    // the copy kernel: bf16, rows 16-byte aligned, whole k-steps of features, and byte offsets
    // within a record below 2^31
    bool copy = dtype == kBF16 && a.n_rec > 0 && !a.seg;
    for (int l = 0; l < a.n_layers; ++l) {
        const GramLayer& d = a.L[l];
        copy = copy && d.vec_a && d.vec_g && d.d_in % kGramK == 0 && d.d_out % kGramK == 0 &&
               a.T * (int64_t)std::max(d.d_in, d.d_out) * 2 < ((int64_t)1 << 31);
    }
    if (copy && a.nb <= kGramRecMaxNb) {
        const int n_stages = std::min(kGramRecMaxStages, kGramRecMaxLds / (8 * a.nb * 1024));
        const size_t lds = (size_t)n_stages * 8 * a.nb * 1024;
        const int nw = a.nb * (a.nb - 1) / 2 + (a.nb + 1) / 2;
        hipLaunchKernelGGL(k_norm_gram_rec, dim3((unsigned)a.n_rec, a.n_layers), dim3(64 * nw), lds, s, a,
                           n_stages);
        return hipGetLastError();
    }
    if (copy) {
        const int64_t nb = (a.T + kGramB - 1) / kGramB;
        const int64_t gx = nb * (nb + 1) / 2 * 8 * ((a.n_rec + 7) / 8);
        hipLaunchKernelGGL(k_norm_gram_copy, dim3((unsigned)gx, 1, a.n_layers), dim3(256), 0, s, a);
        return hipGetLastError();
    }
    const dim3 grid((a.n_pairs + 3) / 4, (unsigned)a.n_rec, a.n_layers);
    if (dtype == kBF16)
        hipLaunchKernelGGL(k_norm_gram<kBF16>, grid, dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL(k_norm_gram<kF32>, grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace dpsgd
