// Record-owned LLM.int8 forward of one frozen linear layer ("Sensitivity Inflation from
// Cross-Record Precision Routing in Private Quantized Fine-Tuning", Sec. 4.2, Eq. 6 and
// Algorithm 1; the LLM.int8 decomposition as its Sec. 2 describes it).
//
// Three launches per layer:
//   k_i8_scan   per row: its owner record and the row scale s_i = max |a| over the entries below
//               tau; per block of a record's rows: the OR of the per-entry tests |a| >= tau
//               (the first level of a segmented reduction; masks are bit sets of K bits);
//   k_i8_quant  per block: the record's outlier set O_r (OR of its blocks' masks), then the
//               codes round(127 a / s_i) of the block's rows, zero in O_r's columns;
//   k_i8_gemm   Y = fp16(dq16 + corr16): the exact integer product of the codes with the INT8
//               weight on MFMA (v_mfma_i32_16x16x64_i8), dequantised in the epilogue, plus the
//               FP16 correction of each row over its own record's outlier columns only.
// Row-wise weight quantisation (k_i8_weight) runs once per frozen weight.
//
// Rounding (identical IEEE fp32 operations on both sides of every parity test): codes are
// rint(fl(127 a) / s) with a correctly rounded division (fl(127 a) is exact), code 0 where s = 0;
// dq16 = fp16(fl(fl(float(acc) * fl(s_i / 127)) * fl(s_W / 127))); the dequantised weight is
// fp16(fl(float(code) * fl(s_W / 127))); the correction sums the exact products a * w in fp32
// in ascending column order and rounds once to fp16; the two fp16 halves are added and rounded.
//
// The GEMM tile takes the union of the outlier columns of the records its rows belong to, but
// every row multiplies only the columns in its own record's set (the others contribute exact
// zeros, which leave an fp32 sum unchanged), so another record's outliers never change a row's
// arithmetic.
#include <algorithm>

#include "device_common.h"
#include "internal.h"
#include "int8.h"

namespace dpsgd {

namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float h2f(uint32_t bits) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
}

__device__ __forceinline__ uint16_t f2h(float x) {   // round to nearest even
    return __builtin_bit_cast(uint16_t, (_Float16)x);
}

// fp16 of an fp32 result that must be rounded to fp32 first.  Without the empty asm the compiler
// merges the producing multiply or FMA and the conversion into one mixed-precision FMA
// (v_fma_mixlo_f16) that rounds the exact result to fp16 once; that differs from the two
// roundings whenever the fp32 value lands on an fp16 tie (the contraction flags do not stop it).
__device__ __forceinline__ uint16_t f2h_rounded(float x) {
    asm volatile("" : "+v"(x));
    return f2h(x);
}

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// The same rounding as f2h_rounded, as an fp16 value.
__device__ __forceinline__ _Float16 f16_rounded(float x) {
    asm volatile("" : "+v"(x));
    return (_Float16)x;
}

__device__ __forceinline__ float div_rn(float x, float y) { return __fdiv_rn(x, y); }

__device__ __forceinline__ int code_of(float a, float s) {
    return s == 0.f ? 0 : (int)rintf(div_rn(127.f * a, s));
}

// Fast form of code_of for a row of scale s, given r127 = fl(127 fl(1 / s)) with the hardware
// reciprocal (good to 1 ulp; r127 = 0 when s = 0): q0 = fl(a r127) is within 2^-22 |q| of the
// exact quotient q = 127 a / s, so for |q0| < 128 within 2^-15 + 2^-17 of the correctly rounded
// quotient d.  Where q0 is more than 2^-13 away from every half-integer, rint(q0) = rint(d) =
// code_of(a, s); code_fast reports the other elements (rare; always for NaN or infinity), which
// take code_of itself.
__device__ __forceinline__ float code_fast(float a, float r127, bool& exact) {
    const float q0 = a * r127;
    const float k = rintf(q0);
    exact = fabsf(q0) < 128.f && fabsf(q0 - k) < 0.5f - 0x1p-13f;
    return k;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

}  // namespace

// Row blocks: record r owns max(1, ceil(len / 16)) blocks of up to 16 of its rows, numbered from
// boff[r]; a workgroup takes one block, one row per wavefront.
constexpr int kScanRows = 16;

struct RowBlock {
    int64_t r, row0;
    int nrows;
};

__device__ __forceinline__ bool row_block(const I8Args& a, RowBlock& rb) {
    const int64_t* boff = a.offsets + a.n_rec + 1;
    const int64_t blk = blockIdx.x;
    if (blk >= boff[a.n_rec]) return false;
    int64_t lo = 0, hi = a.n_rec - 1;        // the record whose blocks include blk
    while (lo < hi) {
        const int64_t mid = (lo + hi + 1) >> 1;
        if (boff[mid] <= blk) lo = mid;
        else hi = mid - 1;
    }
    rb.r = lo;
    rb.row0 = a.offsets[lo] + kScanRows * (blk - boff[lo]);
    const int64_t row_end = std::min<int64_t>(a.offsets[lo + 1], a.n);
    rb.nrows = (int)std::max<int64_t>(0, std::min<int64_t>(kScanRows, row_end - rb.row0));
    return true;
}

// The routing kernels run one row of a block per wavefront (sixteen wavefronts per workgroup, so
// that four are resident per SIMD), and a lane loads CPL 16-byte chunks of its row together: all
// of a wavefront's loads for up to RPW rows x CPL chunks (a whole row of up to 3072 columns) are
// issued before any is used.
constexpr int kRouteWaves = 16;
constexpr int kRouteThreads = 64 * kRouteWaves;
constexpr int RPW = kScanRows / kRouteWaves;
constexpr int CPL = 6;

// Per block: each row's owner and scale s_i = max |a| over the entries below tau, and the block's
// partial outlier mask (the OR of its rows' per-entry tests |a| >= tau, taken in LDS) written
// whole with plain stores, so nothing needs clearing between calls.
__global__ __launch_bounds__(kRouteThreads) void k_i8_scan(I8Args a) {
    __shared__ uint32_t wm[kI8MaxKW];
    RowBlock rb;
    if (!row_block(a, rb)) return;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int KW = (int)a.KW;
    const bool on = a.tau_on != 0;
    const float tau = a.tau;
    float mx[RPW];
#pragma unroll
    for (int j = 0; j < RPW; ++j) mx[j] = 0.f;
    // a record without rows has one block with no rows (row0 may be n): no loads at all then;
    // otherwise masked-off loads read the block's first row, which exists
    const bool vec = rb.nrows > 0 && a.a_vec;
    const int64_t nch = a.K / 8;
    u32x4 v[RPW][CPL];
    auto load = [&](int64_t c0) {
#pragma unroll
        for (int j = 0; j < RPW; ++j)
#pragma unroll
            for (int b = 0; b < CPL; ++b) {
                const int rr = w + kRouteWaves * j;
                const int64_t c = c0 + 64 * b;
                const bool ok = rr < rb.nrows && c < nch;
                const uint16_t* x = a.A + (rb.row0 + (ok ? rr : 0)) * a.K + 8 * (ok ? c : 0);
                v[j][b] = ok ? *reinterpret_cast<const u32x4*>(x) : u32x4{0u, 0u, 0u, 0u};
            }
    };
    if (vec) load(lane);
    for (int t = tid; t < KW; t += kRouteThreads) wm[t] = 0u;
    __syncthreads();
    if (vec) {
        for (int64_t c0 = lane; c0 < nch; c0 += 64 * CPL) {
            if (c0 != lane) load(c0);
#pragma unroll
            for (int j = 0; j < RPW; ++j)
#pragma unroll
                for (int b = 0; b < CPL; ++b) {
                    const int64_t c = c0 + 64 * b;
                    uint32_t bits = 0;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float f = fabsf(h2f(v[j][b][e >> 1] >> (16 * (e & 1))));
                        const bool o = on && f >= tau;
                        bits |= (uint32_t)o << e;
                        mx[j] = o ? mx[j] : fmaxf(mx[j], f);
                    }
                    if (bits) atomicOr(wm + (8 * c) / 32, bits << ((8 * c) % 32));
                }
        }
    } else {
        for (int j = 0; j < RPW; ++j) {
            const int rr = w + kRouteWaves * j;
            if (rr >= rb.nrows) break;
            const uint16_t* x = a.A + (rb.row0 + rr) * a.K;
            for (int64_t k = lane; k < a.K; k += 64) {
                const float f = fabsf(h2f(x[k]));
                if (on && f >= tau) atomicOr(wm + k / 32, 1u << (k % 32));
                else mx[j] = fmaxf(mx[j], f);
            }
        }
    }
#pragma unroll
    for (int j = 0; j < RPW; ++j) {
        const int rr = w + kRouteWaves * j;
        const float m = wave_max(mx[j]);
        if (lane == 0 && rr < rb.nrows) {
            a.s[rb.row0 + rr] = m;
            a.own[rb.row0 + rr] = (int32_t)rb.r;
        }
    }
    __syncthreads();
    uint32_t* pm = a.pmask + (int64_t)blockIdx.x * KW;
    for (int t = tid; t < KW; t += kRouteThreads) pm[t] = wm[t];
}

// Per block: the record's outlier set O_r = OR of its blocks' partial masks (in LDS; the record's
// first block also writes it out for the GEMM), then the codes of the block's rows in Q (pitch
// Kp bytes, zero past K): round(127 a / s_i), zero in O_r's columns.
__global__ __launch_bounds__(kRouteThreads) void k_i8_quant(I8Args a) {
    __shared__ uint32_t om[kI8MaxKW];
    RowBlock rb;
    if (!row_block(a, rb)) return;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int KW = (int)a.KW;
    const int64_t* boff = a.offsets + a.n_rec + 1;
    float sj[RPW], rj[RPW];
#pragma unroll
    for (int j = 0; j < RPW; ++j) {
        const int rr = w + kRouteWaves * j;
        sj[j] = rr < rb.nrows ? a.s[rb.row0 + rr] : 0.f;
        rj[j] = sj[j] == 0.f ? 0.f : 127.f * __builtin_amdgcn_rcpf(sj[j]);
    }
    const bool vec = rb.nrows > 0 && a.a_vec;
    const int64_t nch = a.K / 8, npc = a.Kp / 8;
    // the block's activations for (up to) RPW rows x CPL chunks per lane, loaded before the mask
    // reduction so that the two latencies overlap; a block without rows loads nothing
    u32x4 v[RPW][CPL];
    auto load = [&](int64_t c0) {
#pragma unroll
        for (int j = 0; j < RPW; ++j)
#pragma unroll
            for (int b = 0; b < CPL; ++b) {
                const int rr = w + kRouteWaves * j;
                const int64_t c = c0 + 64 * b;
                const bool ok = rr < rb.nrows && c < nch;
                const uint16_t* x = a.A + (rb.row0 + (ok ? rr : 0)) * a.K + 8 * (ok ? c : 0);
                v[j][b] = ok ? *reinterpret_cast<const u32x4*>(x) : u32x4{0u, 0u, 0u, 0u};
            }
    };
    if (vec) load(lane);
    for (int t = tid; t < KW; t += kRouteThreads) om[t] = 0u;
    __syncthreads();
    // thread t ORs word t % KW of blocks t / KW, t / KW + NT / KW, ... of the record
    const int64_t b0 = boff[rb.r], nb = boff[rb.r + 1] - b0;
    const uint32_t* pr = a.pmask + b0 * KW;
    {
        const int wd = tid % KW, bs = kRouteThreads / KW;
        uint32_t m = 0;
        if (tid < bs * KW)
            for (int64_t b = tid / KW; b < nb; b += bs) m |= pr[b * KW + wd];
        if (m) atomicOr(om + wd, m);
    }
    __syncthreads();
    if ((int64_t)blockIdx.x == b0)
        for (int t = tid; t < KW; t += kRouteThreads) a.omask[rb.r * KW + t] = om[t];
    if (vec) {
        for (int64_t c0 = lane; c0 < npc; c0 += 64 * CPL) {
            if (c0 != lane) load(c0);
#pragma unroll
            for (int j = 0; j < RPW; ++j)
#pragma unroll
                for (int b = 0; b < CPL; ++b) {
                    const int rr = w + kRouteWaves * j;
                    const int64_t c = c0 + 64 * b;
                    if (rr >= rb.nrows || c >= npc) continue;
                    uint32_t lo = 0, hi = 0;
                    if (c < nch) {
                        const uint32_t m = om[(8 * c) / 32] >> ((8 * c) % 32);
                        float k[8];
                        bool all_exact = true;
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            bool ex;
                            k[e] = code_fast(h2f(v[j][b][e >> 1] >> (16 * (e & 1))), rj[j], ex);
                            all_exact = all_exact && ex;
                        }
                        if (!all_exact) {
#pragma unroll
                            for (int e = 0; e < 8; ++e) {
                                const float f = h2f(v[j][b][e >> 1] >> (16 * (e & 1)));
                                bool ex;
                                code_fast(f, rj[j], ex);
                                if (!ex) k[e] = (float)code_of(f, sj[j]);
                            }
                        }
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const int code = ((m >> e) & 1u) ? 0 : (int)k[e];
                            const uint32_t bb = (uint32_t)(code & 0xFF) << (8 * (e & 3));
                            if (e < 4) lo |= bb;
                            else hi |= bb;
                        }
                    }
                    *reinterpret_cast<uint2*>(a.Q + (rb.row0 + rr) * a.Kp + 8 * c) = make_uint2(lo, hi);
                }
        }
    } else {
        for (int j = 0; j < RPW; ++j) {
            const int rr = w + kRouteWaves * j;
            if (rr >= rb.nrows) break;
            const int64_t row = rb.row0 + rr;
            const uint16_t* x = a.A + row * a.K;
            int8_t* q = a.Q + row * a.Kp;
            for (int64_t k = lane; k < a.Kp; k += 64) {
                int code = 0;
                if (k < a.K && !((om[k / 32] >> (k % 32)) & 1u)) code = code_of(h2f(x[k]), sj[j]);
                q[k] = (int8_t)code;
            }
        }
    }
}

// One wavefront per output feature: s_W = max |w|, codes round(127 w / s_W) (pitch Kp).
__global__ __launch_bounds__(256) void k_i8_weight(const uint16_t* __restrict__ W, int64_t N,
                                                   int64_t K, int64_t Kp, int8_t* __restrict__ Wq,
                                                   float* __restrict__ sW) {
    const int lane = threadIdx.x & 63;
    const int64_t o = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (o >= N) return;
    const uint16_t* w = W + o * K;
    float mx = 0.f;
    for (int64_t j = lane; j < K; j += 64) mx = fmaxf(mx, fabsf(h2f(w[j])));
    mx = wave_max(mx);
    int8_t* q = Wq + o * Kp;
    for (int64_t j = lane; j < Kp; j += 64) q[j] = (int8_t)(j < K ? code_of(h2f(w[j]), mx) : 0);
    if (lane == 0) sW[o] = mx;
}

namespace {

constexpr int kStages = 3;
constexpr int kUC = 16;           // union columns staged per correction chunk
constexpr int kRS = kUC + 4;      // row stride (floats) of the staged residual

// Byte offset of 16-byte chunk c (0..3) of row r inside a staged k-step (rows of 64 bytes):
// the chunk index is XOR-ed with bits 2-3 of the row, so the 16 rows read by one MFMA operand
// load spread over all 64 LDS banks.
__device__ __forceinline__ uint32_t stage_off(int r, int c) {
    return (uint32_t)(r * 64 + 16 * (c ^ ((r >> 2) & 3)));
}

}  // namespace

// Workgroup tile: BI = 16 FI WI rows (i) x BO = 16 FO WO output features (o); WI x WO
// wavefronts of (16 FI) x (16 FO).  MFMA operand a = weight rows (o), b = code rows (i): lane l
// of a 16x16 result holds row i = l % 16 and the four features 4 (l / 16) .. + 3, so the fp16
// output is written 8 bytes per lane.
//
// The correction's operands (the tile's union of record outlier columns, each row's own bits,
// the residual activations and the dequantised weight columns) are staged into their own LDS
// region while the first k-steps' copies are in flight, so their gathers overlap the copy
// latency instead of following the MFMA loop.  Unions wider than kUC columns are restaged chunk
// by chunk after the loop.
template <int FI, int FO, int WI, int WO>
__global__ __launch_bounds__(64 * WI * WO, 1) void k_i8_gemm(I8Args a) {
    constexpr int NW = WI * WO, NT = 64 * NW;
    constexpr int BI = 16 * FI * WI, BO = 16 * FO * WO;
    constexpr int STAGE = (BI + BO) * 64;
    constexpr int CQ = BI / 16 / NW, CW = BO / 16 / NW;   // copies per wave per k-step
    static_assert(CQ * 16 * NW == BI && CW * 16 * NW == BO, "copy split");
    constexpr int EPI = (BI + BI + BO + kI8MaxKW + kUC + 16 + BI) * 4 + (BI * kRS + kUC * BO) * 4;
    __shared__ __attribute__((aligned(16))) char lds[kStages * STAGE + EPI];

    const int64_t n = a.n, N = a.N;
    int ti, to;
    if (!tile_of((int)((n + BI - 1) / BI), (int)((N + BO - 1) / BO), 4, ti, to)) return;
    const int64_t i0 = (int64_t)ti * BI, o0 = (int64_t)to * BO;
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int wi = w % WI, wo = w / WI;
    const int l16 = lane & 15, g = lane >> 4;

    // copies: copy q of a k-step moves rows 16 q .. 16 q + 15 of the code tile (or the weight
    // tile), 64 bytes each; lane L lands at 16 L, i.e. row 16 q + L / 4, stored chunk L % 4,
    // which holds logical chunk (L % 4) ^ ((L / 16) % 4).  Rows past the end re-read the last row.
    uint32_t offq[CQ], offw[CW];
#pragma unroll
    for (int q = 0; q < CQ; ++q) {
        const int64_t r = std::min<int64_t>(i0 + 16 * (CQ * w + q) + (lane >> 2), n - 1);
        offq[q] = (uint32_t)(r * a.Kp + 16 * ((lane & 3) ^ (g & 3)));
    }
#pragma unroll
    for (int q = 0; q < CW; ++q) {
        const int64_t r = std::min<int64_t>(o0 + 16 * (CW * w + q) + (lane >> 2), N - 1);
        offw[q] = (uint32_t)(r * a.Kp + 16 * ((lane & 3) ^ (g & 3)));
    }
    // operand reads: lane l reads row l % 16 of a 16-row block, logical chunk l / 16
    const uint32_t rd_w = (uint32_t)(BI * 64) + stage_off(16 * FO * wo + l16, g);
    const uint32_t rd_q = stage_off(16 * FI * wi + l16, g);

    const char* baseq = reinterpret_cast<const char*>(a.Q);
    const char* basew = reinterpret_cast<const char*>(a.Wq);
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_addr(lds));
    auto issue = [&](int64_t s, int st) {
        const char* pq = baseq + 64 * s;
        const char* pw = basew + 64 * s;
        const uint32_t dst = lds0 + (uint32_t)(st * STAGE);
#pragma unroll
        for (int q = 0; q < CQ; ++q) copy16(pq, offq[q], dst + (uint32_t)(CQ * w + q) * 1024u);
#pragma unroll
        for (int q = 0; q < CW; ++q)
            copy16(pw, offw[q], dst + (uint32_t)(BI * 64 + (CW * w + q) * 1024));
    };

    const int64_t total = a.Kp / 64;
#pragma unroll
    for (int k = 0; k < kStages - 1; ++k)
        if (k < total) issue(k, k);

    // ---- correction operands, staged while those copies are in flight
    char* E = lds + kStages * STAGE;
    int* own_t = reinterpret_cast<int*>(E);            // owner record of each tile row (-1 past n)
    float* sat = reinterpret_cast<float*>(own_t + BI);  // fl(s_i / 127)
    float* sbt = sat + BI;                              // fl(s_W / 127)
    uint32_t* tmask = reinterpret_cast<uint32_t*>(sbt + BO);   // union of the rows' record sets
    int* cols = reinterpret_cast<int*>(tmask + kI8MaxKW);      // columns of the staged chunk
    int* wsum = cols + kUC;                                    // scan scratch (NW + 1)
    uint32_t* rbits = reinterpret_cast<uint32_t*>(wsum + 16);  // per tile row: chunk bits
    float* Rt = reinterpret_cast<float*>(rbits + BI);          // [BI][kRS] residual a or 0
    float* Wt = Rt + BI * kRS;                                 // [kUC][BO] dequantised weight
    for (int t = tid; t < BI; t += NT) {
        const int64_t r = i0 + t;
        const int32_t ow = r < n ? a.own[r] : -1;
        own_t[t] = r < n ? (ow >= 0 && ow < a.n_rec ? ow : 0) : -1;
        sat[t] = r < n ? div_rn(a.s[r], 127.f) : 0.f;
    }
    for (int t = tid; t < BO; t += NT) {
        const int64_t o = o0 + t;
        sbt[t] = o < N ? div_rn(a.sW[o], 127.f) : 0.f;
    }
    __syncthreads();
    const int rows_valid = (int)std::min<int64_t>(BI, n - i0);
    const int r_lo = own_t[0], r_hi = own_t[rows_valid - 1];
    const int KW = (int)a.KW;
    for (int wd = tid; wd < KW; wd += NT) {
        uint32_t m = 0;
        for (int r = r_lo; r <= r_hi; ++r) m |= a.omask[(int64_t)r * KW + wd];
        tmask[wd] = m;
    }
    __syncthreads();
    // rank of each thread's first union column: thread t owns words [t WPT, t WPT + WPT)
    constexpr int WPT = (kI8MaxKW + NT - 1) / NT;
    int mine = 0;
#pragma unroll
    for (int k = 0; k < WPT; ++k) {
        const int wd = tid * WPT + k;
        if (wd < KW) mine += __popc(tmask[wd]);
    }
    int incl = mine;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int u = __shfl_up(incl, o, 64);
        if (lane >= o) incl += u;
    }
    if (lane == 63) wsum[w] = incl;
    __syncthreads();
    int base = incl - mine, nu = 0;
    for (int k = 0; k < NW; ++k) {
        if (k < w) base += wsum[k];
        nu += wsum[k];
    }
    const int n_chunks = (nu + kUC - 1) / kUC;

    // stage union columns c0 .. c0 + kUC - 1: Rt[i][u] = a (row i's own outlier column) or 0,
    // Wt[u][o] = the dequantised weight
    auto stage = [&](int c0) {
        const int nuc = std::min(kUC, nu - c0);
        __syncthreads();   // the previous chunk's staged values are consumed
        int rank = base;
        for (int k = 0; k < WPT; ++k) {
            const int wd = tid * WPT + k;
            if (wd >= KW) break;
            uint32_t m = tmask[wd];
            while (m) {
                const int b = __builtin_ctz(m);
                m &= m - 1;
                if (rank >= c0 && rank < c0 + kUC) cols[rank - c0] = 32 * wd + b;
                ++rank;
            }
        }
        for (int t = tid; t < BI; t += NT) rbits[t] = 0u;
        __syncthreads();
        // rbits[il] bit u: chunk column u is in the outlier set of tile row il's record
        for (int t = tid; t < rows_valid * nuc; t += NT) {
            const int il = t / nuc, u = t - il * nuc;
            const int col = cols[u];
            if ((a.omask[(int64_t)own_t[il] * KW + col / 32] >> (col % 32)) & 1u)
                atomicOr(&rbits[il], 1u << u);
        }
        __syncthreads();
        // residual pairs (row, u) and weight pairs (u, feature) for u < nuc4 (nuc rounded up to 4;
        // the padding is zero on both sides, so the correction loop runs in whole groups of four
        // and a zero product leaves the fp32 sum unchanged): loads from clamped in-bounds addresses,
        // masked afterwards, four per thread issued back to back
        const int nuc4 = (nuc + 3) & ~3;
        const int nr = BI * nuc4;
        for (int t0 = tid; t0 < nr; t0 += 4 * NT) {
            float v[4];
            int at[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int t = t0 + k * NT;
                const bool ok = t < nr;
                const int il = ok ? t / nuc4 : 0;
                const int u = ok ? t - il * nuc4 : 0;
                const bool live = ok && u < nuc && ((rbits[il] >> u) & 1u);
                const uint16_t raw = a.A[(i0 + (live ? il : 0)) * a.K + (live ? cols[u] : 0)];
                v[k] = live ? h2f(raw) : 0.f;
                at[k] = ok ? il * kRS + u : -1;
            }
#pragma unroll
            for (int k = 0; k < 4; ++k)
                if (at[k] >= 0) Rt[at[k]] = v[k];
        }
        const int nw = nuc4 * BO;
        for (int t0 = tid; t0 < nw; t0 += 4 * NT) {
            float v[4];
            int at[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int t = t0 + k * NT;
                const bool ok = t < nw;
                const int u = ok ? t / BO : 0, ol = t % BO;
                const bool live = ok && u < nuc && o0 + ol < N;
                const int64_t o = std::min<int64_t>(o0 + ol, N - 1);
                const int8_t raw = a.Wq[o * a.Kp + (live ? cols[u] : 0)];
                v[k] = live ? h2f(f2h_rounded((float)raw * sbt[ol])) : 0.f;
                at[k] = ok ? u * BO + ol : -1;
            }
#pragma unroll
            for (int k = 0; k < 4; ++k)
                if (at[k] >= 0) Wt[at[k]] = v[k];
        }
        __syncthreads();
    };
    if (n_chunks == 1) stage(0);

    // ---- main loop: the exact integer product
    i32x4 acc[FO][FI];
#pragma unroll
    for (int f = 0; f < FO; ++f)
#pragma unroll
        for (int e = 0; e < FI; ++e) acc[f][e] = i32x4{0, 0, 0, 0};
    int st = 0, stn = kStages - 1;
    for (int64_t s = 0; s < total; ++s) {
        // this wave's copies of step s are done once at most the later issued steps are in
        // flight; the barrier publishes all waves' copies and retires step s - 1's stage
        wait_copies<CQ + CW>(std::min<int64_t>(s + kStages - 2, total - 1) - s);
        __syncthreads();
        if (s + kStages - 1 < total) issue(s + kStages - 1, stn);
        const char* S = lds + st * STAGE;
        i32x4 bq[FI];
#pragma unroll
        for (int e = 0; e < FI; ++e) bq[e] = *reinterpret_cast<const i32x4*>(S + rd_q + e * 1024);
#pragma unroll
        for (int f = 0; f < FO; ++f) {
            const i32x4 aw = *reinterpret_cast<const i32x4*>(S + rd_w + f * 1024);
#pragma unroll
            for (int e = 0; e < FI; ++e)
                acc[f][e] = __builtin_amdgcn_mfma_i32_16x16x64_i8(aw, bq[e], acc[f][e], 0, 0, 0);
        }
        st = st == kStages - 1 ? 0 : st + 1;
        stn = stn == kStages - 1 ? 0 : stn + 1;
    }

    // ---- epilogue, one 16-row group at a time: correction (fp32, ascending columns), then
    // Y = fp16(dq16 + corr16) with dq16 = fp16(fl(fl(float(acc) * fl(s_i/127)) * fl(s_W/127)))
    f4 sbv[FO];   // fl(s_W/127) of the lane's four features in each 16-feature block
#pragma unroll
    for (int f = 0; f < FO; ++f) sbv[f] = *reinterpret_cast<const f4*>(sbt + 16 * FO * wo + 16 * f + 4 * g);
    const bool interior = a.y_vec && i0 + BI <= n && o0 + BO <= N;   // uniform per workgroup
#pragma unroll
    for (int e = 0; e < FI; ++e) {
        const int il = 16 * FI * wi + 16 * e + l16;
        f4 corr[FO];
#pragma unroll
        for (int f = 0; f < FO; ++f) corr[f] = f4{0.f, 0.f, 0.f, 0.f};
        for (int ch = 0; ch < n_chunks; ++ch) {
            if (n_chunks > 1) stage(ch * kUC);
            const int nuc4 = (std::min(kUC, nu - ch * kUC) + 3) & ~3;
            const float* rrow = Rt + il * kRS;
            for (int u = 0; u < nuc4; u += 4) {
                const f4 rv = *reinterpret_cast<const f4*>(rrow + u);
#pragma unroll
                for (int uu = 0; uu < 4; ++uu)
#pragma unroll
                    for (int f = 0; f < FO; ++f) {
                        const f4 wv = *reinterpret_cast<const f4*>(
                            Wt + (u + uu) * BO + 16 * FO * wo + 16 * f + 4 * g);
#pragma unroll
                        for (int r = 0; r < 4; ++r) corr[f][r] = fmaf(rv[uu], wv[r], corr[f][r]);
                    }
            }
        }
        const int64_t i = i0 + il;
        const float sa = sat[il];
#pragma unroll
        for (int f = 0; f < FO; ++f) {
            const int64_t ob = o0 + 16 * FO * wo + 16 * f + 4 * g;
            // the two fp16 halves are added in fp16, two outputs per instruction: rounding the fp32
            // sum of two fp16 values to fp16 gives the correctly rounded fp16 sum (fp32 carries
            // 24 >= 2 x 11 + 2 significand bits), so this is fp16(float(dq16) + float(corr16))
            uint32_t yw[2];
#pragma unroll
            for (int r = 0; r < 4; r += 2) {
                f16x2 dq, co;
                dq[0] = f16_rounded(((float)acc[f][e][r] * sa) * sbv[f][r]);
                dq[1] = f16_rounded(((float)acc[f][e][r + 1] * sa) * sbv[f][r + 1]);
                co[0] = f16_rounded(corr[f][r]);
                co[1] = f16_rounded(corr[f][r + 1]);
                yw[r / 2] = __builtin_bit_cast(uint32_t, dq + co);
            }
            const uint16_t y[4] = {(uint16_t)yw[0], (uint16_t)(yw[0] >> 16), (uint16_t)yw[1],
                                   (uint16_t)(yw[1] >> 16)};
            uint16_t* dst = a.Y + i * N + ob;
            const uint2 packed = make_uint2(yw[0], yw[1]);
            if (interior) {
                *reinterpret_cast<uint2*>(dst) = packed;
            } else if (i < n) {
                if (a.y_vec && ob + 4 <= N) {
                    *reinterpret_cast<uint2*>(dst) = packed;
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (ob + r < N) dst[r] = y[r];
                }
            }
        }
    }
}

namespace {

template <int FI, int FO, int WI, int WO>
void launch_gemm(const I8Args& a, hipStream_t s) {
    constexpr int BI = 16 * FI * WI, BO = 16 * FO * WO;
    const int64_t tiles = ((a.n + BI - 1) / BI) * ((a.N + BO - 1) / BO);
    hipLaunchKernelGGL((k_i8_gemm<FI, FO, WI, WO>), dim3((unsigned)tiles), dim3(64 * WI * WO), 0, s, a);
}

}  // namespace

int64_t i8_tiles(int64_t n, int64_t N, int big) {
    const int64_t b = big ? 256 : 128;
    return ((n + b - 1) / b) * ((N + b - 1) / b);
}

int64_t i8_scan_blocks(int64_t n, int64_t n_rec) { return (n + kScanRows - 1) / kScanRows + n_rec; }

hipError_t launch_i8_route(const I8Args& a, hipStream_t s) {
    if (a.n_rec > 0) {
        const dim3 g((unsigned)i8_scan_blocks(a.n, a.n_rec));
        hipLaunchKernelGGL(k_i8_scan, g, dim3(kRouteThreads), 0, s, a);
        hipLaunchKernelGGL(k_i8_quant, g, dim3(kRouteThreads), 0, s, a);
    }
    return hipGetLastError();
}

hipError_t launch_i8_gemm(const I8Args& a, int big, hipStream_t s) {
    if (a.n > 0 && a.N > 0) {
        if (big) launch_gemm<4, 8, 4, 2>(a, s);
        else launch_gemm<4, 4, 2, 2>(a, s);
    }
    return hipGetLastError();
}

hipError_t launch_i8_weight(const uint16_t* W, int64_t N, int64_t K, int64_t Kp, int8_t* Wq,
                            float* sW, hipStream_t s) {
    if (N > 0) hipLaunchKernelGGL(k_i8_weight, dim3((unsigned)((N + 3) / 4)), dim3(256), 0, s, W, N, K, Kp, Wq, sW);
    return hipGetLastError();
}

}  // namespace dpsgd
