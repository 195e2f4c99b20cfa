// clipped_sum for dense layers (both d_in and d_out wide), bf16 inputs:
//   S = A^T diag(c (x) 1_T) G = sum_i c_i A_i^T G_i
// ("Privacy-Preserving Machine Learning", DP-SGD phase 4; "Sensitivity
// Inflation ...", Eq. 3), an MFMA GEMM with M = d_in, N = d_out and the
// reduction over the n_records * T token rows.
//
// Wave tiles are 128 (d_in) x 64 (d_out), 32 v_mfma_f32_16x16x32_bf16 per k-step
// of 32 tokens.  Both operands are stored with the reduction axis (tokens) as
// rows, so the MFMA operands (8 consecutive tokens of one column per lane) are a
// transpose of what memory holds.  Two kernels:
//
// k_sum_dense_dma (T a multiple of 32, rows 16-byte aligned): 256 x 256 workgroup
// tiles (8 waves, one workgroup per CU).  Each k-step tile is copied token-major
// into LDS by global_load_lds_dwordx4 (no registers, no VALU), three LDS stages
// with copies two k-steps ahead and one barrier per k-step, and the operands
// come out of LDS through ds_read_b64_tr_b16: within each 16-lane
// group, result lane i element e is element i % 4 of what lane 4e + i / 4 read,
// so lane 4e + p points at columns 4p..4p+3 of token row e and two such reads give
// one MFMA operand.  The 16-byte chunk c of token row r sits at chunk c ^ swz(r),
// which spreads each half-wave's transposed reads over all banks.
//
// k_sum_dense_bf16 (any T, any alignment): 256 x 128 workgroup tiles (4 waves, two
// workgroups per CU); each k-step is loaded into registers as
// 8 token x 8 column blocks (16-byte loads, zero-filled past T and d), transposed
// in registers and written as column vectors (pitch 96 bytes: the 16-lane operand
// reads are conflict-free, the staging writes take 16 cycles), two k-steps of
// loads in flight in a two-slot register ring (loop unrolled by two so each slot
// stays in fixed registers), LDS double-buffered.
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


constexpr int kCopyTN = 256;     // d_out columns per workgroup of the copy kernel
constexpr int kCopyStages = 5;   // its LDS stages: all 160 KB (5% fewer cycles per k-step than 3)

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Physical 16-byte chunk of logical chunk c in token row r of a staged k-step is c ^ swz(r):
// the transposed reads of one half-wave (token rows 8g + 4h + 0..3 for g in {0, 1}, two chunks
// each) then fall on 16 distinct chunk slots of the 256-byte bank space.
__device__ __forceinline__ int swz(int r) { return 2 * ((r & 3) | (((r >> 3) & 1) << 2)); }

__device__ __forceinline__ u32x2 tr_read(const uint16_t* l) {
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(l));
    return __builtin_bit_cast(u32x2, v);
}

// Clip factors of records base .. base + 63, one per lane (1 past the end), so that a record
// boundary inside the k-loop reads its factor with v_readlane instead of a vector load whose
// wait would also drain the operand loads in flight.
struct ClipWindow {
    int64_t base;
    float v;
    __device__ __forceinline__ void load(const float* clip, int64_t b, int64_t end, int lane) {
        base = b;
        v = (b + lane < end) ? clip[b + lane] : 1.f;
        asm volatile("" ::"v"(v));   // consume the load here: no wait at the join after a reload
    }
    __device__ __forceinline__ float get(const float* clip, int64_t rec, int64_t end, int lane) {
        if (rec - base >= 64) load(clip, rec, end, lane);
        return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), (int)(rec - base)));
    }
};

// Writes scale * acc for a wave tile of 128 x 16 NB at (m0 + 128 wm, n0 + 16 NB wn); lane (g, c)
// holds rows 4g + r, column c of each 16 x 16 block.
template <int NB>
__device__ __forceinline__ void store_tile(const DenseSumLayer& L, int accumulate, int64_t split,
                                           int m0, int n0, int wm, int wn, int g, int c,
                                           float scale, const f32x4 (&acc)[8][NB]) {
    float* dst = L.out;
    bool add = accumulate != 0;
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
            for (int j = 0; j < NB; ++j) {
                const int col = n0 + wn * 16 * NB + 16 * j + c;
                if (col >= L.d_out) continue;
                float* p = dst + (int64_t)row * d_out + col;
                *p = (add ? *p : 0.f) + scale * acc[i][j][r];
            }
        }
    }
}

// Writes scale * acc for a wave tile of 128 (d_in) x 16 NB (d_out) at (m0 + 128 wm, n0 + 16 NB wn)
// from accumulators of mfma(G block, A block): lane (g, c) holds d_in row 16 i + c and the d_out
// columns 16 jb + 4 g .. + 3 of each 16 x 16 block, so a lane writes 16 contiguous bytes (when the
// rows allow it; otherwise element by element, with the same arithmetic).
template <int NB>
__device__ __forceinline__ void store_tile_rows(const DenseSumLayer& L, int accumulate, int64_t split,
                                                int m0, int n0, int wm, int wn, int g, int c,
                                                float scale, const f32x4 (&acc)[8][NB]) {
    float* dst = L.out;
    bool add = accumulate != 0;
    if (L.split_stride) {
        dst = L.split + split * L.split_stride;
        add = false;
    }
    const int64_t d_out = L.d_out;
    const bool vec = d_out % 4 == 0 && (reinterpret_cast<uintptr_t>(dst) & 15) == 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int row = m0 + wm * 128 + 16 * i + c;
        if (row >= L.d_in) continue;
#pragma unroll
        for (int jb = 0; jb < NB; ++jb) {
            const int col = n0 + wn * 16 * NB + 16 * jb + 4 * g;
            float* p = dst + (int64_t)row * d_out + col;
            f32x4 v = scale * acc[i][jb];
            if (vec && col + 4 <= d_out) {
                if (add) v += *reinterpret_cast<const f32x4*>(p);
                *reinterpret_cast<f32x4*>(p) = v;
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (col + r < d_out) p[r] = (add ? p[r] : 0.f) + v[r];
            }
        }
    }
}

}  // namespace

// 256 x 256 workgroup tiles, 8 wavefronts of 128 x 64, 5 LDS stages of 32 KB (copies run four
// k-steps ahead), one workgroup per CU.  The MFMA takes the G block as its first operand, so a
// lane's accumulators are four consecutive output columns of one row (16-byte stores).
__global__ __launch_bounds__(512, 1) void k_sum_dense_dma(DenseSumArgs a) {
    constexpr int TN = kCopyTN;                     // d_out columns per workgroup
    constexpr int WN = 64;                          // d_out columns per wave
    constexpr int NS = kCopyStages;
    constexpr int W = 2 * TN / WN;                  // wavefronts
    constexpr int NB = WN / 16;                     // 16-column G blocks per wave
    constexpr int kStageElems = (kTM + TN) * kTK;   // A rows (256 columns), then G rows (TN)
    constexpr int kGOff = kTM * kTK;
    constexpr int CA = 16 / W;                      // A copies per wave per k-step
    constexpr int CG = (TN / 16) / W;               // G copies per wave per k-step
    constexpr int kRowsG = 1024 / (TN * 2);         // token rows per G copy
    __shared__ __attribute__((aligned(16))) uint16_t lds[NS * kStageElems];
    if (a.status && *a.status) return;

    const DenseSumLayer& L = a.L[blockIdx.z];
    const int d_in = L.d_in, d_out = L.d_out;
    int tm, tn;
    if (!tile_of((d_in + kTM - 1) / kTM, (d_out + TN - 1) / TN, TN == 128 ? 8 : 4, tm, tn)) return;
    const int m0 = tm * kTM, n0 = tn * TN;
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;   // w: scalar
    const int g = lane >> 4, j = lane & 15;
    const int wm = w & 1, wn = w >> 1;          // wave tile: d_in cols wm*128.., d_out cols wn*WN..

    // Copies per k-step: 16 of A (token rows 2n, 2n + 1 of the 256-column band) and TN / 16 of G
    // (kRowsG token rows each), 64 lanes x 16 bytes each, landing linearly at LDS stage + 1 KB * n;
    // wave w issues A copies CA w .. CA w + CA - 1 and G copies CG w .. CG w + CG - 1.  A lane whose
    // chunk lies past d reads column 0 of its row instead: those LDS columns only feed output
    // columns past d, which are never stored.
    uint32_t offa[CA], offg[CG];   // byte offsets from the k-step's first token row
#pragma unroll
    for (int q = 0; q < CA; ++q) {
        const int row = 2 * (CA * w + q) + (lane >> 5);
        const int col = m0 + 8 * ((lane & 31) ^ swz(row));
        offa[q] = (uint32_t)(row * d_in + (col < d_in ? col : 0)) * 2u;
    }
#pragma unroll
    for (int q = 0; q < CG; ++q) {
        const int row = kRowsG * (CG * w + q) + lane / (64 / kRowsG);
        const int col = n0 + 8 * ((lane % (64 / kRowsG)) ^ swz(row));
        offg[q] = (uint32_t)(row * d_out + (col < d_out ? col : 0)) * 2u;
    }

    // Transposed operand reads: lane (g, j) points at token row 8g + 4h + j / 4 (h = 0; h = 1 is
    // 4 rows further), columns 16 blk + 4 (j % 4) .. + 3 of the wave's band, i.e. chunk
    // c = 16 wm + 2 blk + (j % 4) / 2 (A) or (WN / 8) wn + 2 blk + (j % 4) / 2 (G), stored at c ^ sw.
    const int sw = 2 * ((j >> 2) | ((g & 1) << 2));    // swz() of those rows
    const int row0 = 8 * g + (j >> 2);
    int oa[8], og[NB];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        oa[i] = row0 * kTM + 8 * ((16 * wm + 2 * i + ((j & 3) >> 1)) ^ sw) + 4 * (j & 1);
#pragma unroll
    for (int jb = 0; jb < NB; ++jb)
        og[jb] = kGOff + row0 * TN + 8 * (((WN / 8) * wn + 2 * jb + ((j & 3) >> 1)) ^ sw) + 4 * (j & 1);

    const int64_t split = blockIdx.y;
    const int64_t r0 = split * a.rec_per_split;
    int64_t r1 = r0 + a.rec_per_split;
    if (r1 > a.n_rec) r1 = a.n_rec;
    const int nks = (int)(a.T / kTK);
    const int64_t total = (r1 - r0) * nks;
    // k-step s covers flat token rows r0 * T + 32 s .. + 31 (T is a multiple of 32)
    const char* baseA = static_cast<const char*>(L.A) + (r0 * a.T) * (int64_t)d_in * 2;
    const char* baseG = static_cast<const char*>(L.G) + (r0 * a.T) * (int64_t)d_out * 2;
    const int64_t strideA = (int64_t)kTK * d_in * 2, strideG = (int64_t)kTK * d_out * 2;
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_addr(lds));
    auto issue = [&](int64_t s, int st) {
        const char* pa = baseA + s * strideA;
        const char* pg = baseG + s * strideG;
        const uint32_t dst = lds0 + (uint32_t)(st * kStageElems) * 2u;
#pragma unroll
        for (int q = 0; q < CA; ++q) copy16(pa, offa[q], dst + (uint32_t)(CA * w + q) * 1024u);
#pragma unroll
        for (int q = 0; q < CG; ++q)
            copy16(pg, offg[q], dst + (uint32_t)(kGOff * 2 + (CG * w + q) * 1024));
    };

    f32x4 acc[8][NB];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int jb = 0; jb < NB; ++jb) acc[i][jb] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Wait until this wave's copies of step t are done, given that steps up to `last` have been
    // issued (later ones may stay in flight); the barrier then publishes every wave's copies.
    static_assert(NS >= 2 && NS <= 5, "stages");
    auto wait_step = [&](int64_t t, int64_t last) {
        wait_copies<CA + CG>(last - t);
        __syncthreads();
    };

    float c_cur = 1.f;
    if (total > 0) {
        ClipWindow cw;
        cw.load(a.clip, r0, r1, lane);
        c_cur = cw.get(a.clip, r0, r1, lane);
#pragma unroll
        for (int k = 0; k < NS - 1; ++k)
            if (k < total) issue(k, k);
        int64_t crec = r0;
        int cks = 0;
        int st = 0, stn = NS - 1;     // stages of steps s and s + NS - 1
        for (int64_t s = 0; s < total; ++s) {
            // publish step s; the barrier also retires step s - 1, whose stage the copies of step
            // s + NS - 1 reuse
            wait_step(s, min<int64_t>(s + NS - 2, total - 1));
            if (s + NS - 1 < total) issue(s + NS - 1, stn);
            // record boundary: rescale the accumulator to the new record's factor
            if (cks == 0 && s > 0) {
                const float c_new = cw.get(a.clip, crec, r1, lane);
                const float f = c_cur / c_new;
#pragma unroll
                for (int i = 0; i < 8; ++i)
#pragma unroll
                    for (int jb = 0; jb < NB; ++jb) acc[i][jb] *= f;
                c_cur = c_new;
            }
            if (++cks == nks) {
                cks = 0;
                ++crec;
            }
            const uint16_t* S = lds + st * kStageElems;
            u32x4 bv[NB];
#pragma unroll
            for (int jb = 0; jb < NB; ++jb) {
                const u32x2 lo = tr_read(S + og[jb]);
                const u32x2 hi = tr_read(S + og[jb] + 4 * TN);
                bv[jb] = u32x4{lo[0], lo[1], hi[0], hi[1]};
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const u32x2 lo = tr_read(S + oa[i]);
                const u32x2 hi = tr_read(S + oa[i] + 4 * kTM);
                const u32x4 av = u32x4{lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
                for (int jb = 0; jb < NB; ++jb) acc[i][jb] = mfma_bf16(bv[jb], av, acc[i][jb]);
            }
            st = st == NS - 1 ? 0 : st + 1;
            stn = stn == NS - 1 ? 0 : stn + 1;
        }
    }
    store_tile_rows(L, a.accumulate, split, m0, n0, wm, wn, g, j, c_cur, acc);
}

__global__ __launch_bounds__(256, 2) void k_sum_dense_bf16(DenseSumArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t lds_a[2][kTM * kPitch];
    __shared__ __attribute__((aligned(16))) uint16_t lds_g[2][kTN * kPitch];
    if (a.status && *a.status) return;

    const DenseSumLayer& L = a.L[blockIdx.z];
    int tm, tn;
    if (!tile_of(L.tiles_m, L.tiles_n, 8, tm, tn)) return;
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
        ClipWindow cw;
        cw.load(a.clip, r0, r1, tid & 63);
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

        c_cur = cw.get(a.clip, r0, r1, tid & 63);
        // one k-step: refill the slot step s came from with step s + D, multiply step s
        // out of LDS, stage step s + 1 (slot `next`) into the other LDS buffer.  The loop
        // below is unrolled by D so that every ring slot is a fixed register set.
        auto kstep = [&](int64_t s, u32x4 (&mine)[8], const u32x4 (&next)[8]) {
            const int buf = (int)(s & 1);
            if (loads && s + D < total) load_step(src, a.T, d, lrec, lks, col0, vec, ld, mine);
            advance(lrec, lks);
            // record boundary: rescale the accumulator to the new record's factor
            if (cks == 0 && s > 0) {
                const float c_new = cw.get(a.clip, crec, r1, tid & 63);
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

    store_tile(L, a.accumulate, split, m0, n0, wm, wn, g, c, c_cur, acc);
}

hipError_t launch_sum_dense(const DenseSumArgs& a, int n_splits, hipStream_t s) {
    int gx = 1;
    // the copy kernel needs whole k-steps per record and 16-byte aligned rows (and byte offsets
    // of 32 token rows that fit 32 bits)
    bool copy = a.T % kTK == 0;
    for (int l = 0; l < a.n_layers; ++l) {
        const DenseSumLayer& d = a.L[l];
        gx = std::max(gx, d.tiles_m * d.tiles_n);
        copy = copy && d.vec_a && d.vec_g && d.d_in <= (1 << 24) && d.d_out <= (1 << 24);
    }
    if (copy) {
        int gxc = 1;
        for (int l = 0; l < a.n_layers; ++l)
            gxc = std::max(gxc, ((a.L[l].d_in + kTM - 1) / kTM) * ((a.L[l].d_out + kCopyTN - 1) / kCopyTN));
        hipLaunchKernelGGL(k_sum_dense_dma, dim3(gxc, n_splits, a.n_layers), dim3(2 * kCopyTN), 0, s, a);
    }
    else
        hipLaunchKernelGGL(k_sum_dense_bf16, dim3(gx, n_splits, a.n_layers), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace dpsgd
