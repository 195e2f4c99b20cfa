// Device-side helpers shared by the kernels: MFMA operand types, bf16
// widening, and fixed-order wavefront reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dpsgd {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// x if keep, else +0.  An integer AND instead of a select, so that the compiler
// keeps the load that produced x unconditional (a select lets it sink the load
// into a branch followed by an immediate wait, which serialises a batch of loads).
__device__ __forceinline__ float keep_or_zero(float x, bool keep) {
    return __uint_as_float(__float_as_uint(x) & (keep ? 0xFFFFFFFFu : 0u));
}

__device__ __forceinline__ float bf16_bits_to_float(uint16_t b) {
    return __uint_as_float((uint32_t)b << 16);
}

// Sum over the 64 lanes of a wavefront; the butterfly order is fixed, so the
// result depends only on the lane values.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// v from lane (lane ^ k) for the patterns one DPP move reaches inside a row of 16
// lanes (CTRL: 0xB1 quad_perm 1,0,3,2 = k 1; 0x4E quad_perm 2,3,0,1 = k 2; 0x1B
// quad_perm 3,2,1,0 = k 3; 0x141 row_half_mirror = k 7; 0x128 row_ror 8 = k 8).
template <int CTRL>
__device__ __forceinline__ double dpp_d(double v) {
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)b, CTRL, 0xF, 0xF, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(b >> 32), CTRL, 0xF, 0xF, false);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// The same butterfly as wave_sum (partner lane ^ 32, ^ 16, ..., ^ 1, each step
// v + partner) in fp64; the steps inside a row of 16 lanes move the partner's value
// with DPP instead of an LDS permute.  The moves are exact, so the result is the one
// the all-shuffle butterfly gives.
__device__ __forceinline__ double wave_sum_d(double v) {
    v += __shfl_xor(v, 32, 64);
    v += __shfl_xor(v, 16, 64);
    v += dpp_d<0x128>(v);                // lane ^ 8
    v += dpp_d<0x141>(dpp_d<0x1B>(v));   // lane ^ 4 = (lane ^ 3) ^ 7
    v += dpp_d<0x4E>(v);                 // lane ^ 2
    v += dpp_d<0xB1>(v);                 // lane ^ 1
    return v;
}

// One batch of partials for up to four records (record rec0 + j * rec_step holds its
// partials at parts + rec * stride, n_parts of them): lane values k0, k0 + 64, ...,
// k0 + 448.  A partial past the end, or a record >= n_rec, reads an in-bounds
// address and yields +0, so the loads are unconditional and issue back to back.
__device__ __forceinline__ void record_parts_load_x4(const float* __restrict__ parts, int64_t stride,
                                                     int64_t n_parts, int64_t rec0, int64_t rec_step,
                                                     int64_t n_rec, int64_t k0, float (&v)[4][8]) {
    const float* p[4];
    bool ok[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t rec = rec0 + j * rec_step;
        ok[j] = rec < n_rec;
        p[j] = parts + (ok[j] ? rec : 0) * stride;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        const int64_t k = k0 + 64 * u;
        const int64_t kc = k < n_parts ? k : n_parts - 1;
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j][u] = keep_or_zero(p[j][kc], ok[j] && k < n_parts);
    }
}

// Squared norms of up to four records from their partials, the first batch (k0 =
// lane) already loaded into v0 by record_parts_load_x4: every lane sums its
// partials lane, lane + 64, ... in ascending order in fp64 (the +0 of a partial
// past the end changes no sum of squares), then a fixed butterfly combines the
// lanes.  The per-record order depends only on n_parts, never on which or how many
// records are reduced together, so every caller gets bitwise the same value for a
// record.  Records >= n_rec are skipped (their result is 0).
__device__ __forceinline__ void record_norm2_x4_from(const float (&v0)[4][8],
                                                     const float* __restrict__ parts, int64_t stride,
                                                     int64_t n_parts, int64_t rec0, int64_t rec_step,
                                                     int64_t n_rec, int lane, double (&out)[4]) {
    double s[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int j = 0; j < 4; ++j) s[j] += (double)v0[j][u];
    for (int64_t k0 = lane + 64 * 8; k0 < n_parts; k0 += 64 * 8) {
        float v[4][8];
        record_parts_load_x4(parts, stride, n_parts, rec0, rec_step, n_rec, k0, v);
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
            for (int j = 0; j < 4; ++j) s[j] += (double)v[j][u];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) out[j] = wave_sum_d(s[j]);
}

__device__ __forceinline__ void record_norm2_x4(const float* __restrict__ parts, int64_t stride,
                                                int64_t n_parts, int64_t rec0, int64_t rec_step,
                                                int64_t n_rec, int lane, double (&out)[4]) {
    float v0[4][8];
    record_parts_load_x4(parts, stride, n_parts, rec0, rec_step, n_rec, lane, v0);
    record_norm2_x4_from(v0, parts, stride, n_parts, rec0, rec_step, n_rec, lane, out);
}

// Norm and clip factor of one record from the sum s of its partial squared norms
// ("Privacy-Preserving Machine Learning", DP-SGD phase 3: n = ||g||, c = min(1, C/n), a
// zero gradient left unchanged).  s is a sum of squares, but the Gram path's partials of
// off-diagonal token blocks are signed, and for a record whose token contributions nearly
// cancel their rounded sum can fall below zero: a negative s is taken as 0 (n = 0, c = 1).
// A NaN s stays NaN in n and c.  Returns true when s, or n or c as stored in fp32, is not
// finite (the caller raises the nonfinite status).
__device__ __forceinline__ bool clip_of_norm2(double s, double C, double& n, double& c) {
    const double s0 = s < 0.0 ? 0.0 : s + 0.0;   // + 0.0 turns a -0 into +0
    n = sqrt(s0);
    c = (n <= C) ? 1.0 : C / n;
    return !isfinite(s) || !isfinite((float)n) || !isfinite((float)c);
}

// LDS byte address of a pointer into a __shared__ array
// Loads of data that is read once, and stores of data that is not read again soon: the
// non-temporal hint keeps such lines from displacing reused ones in the caches.  Streaming reads
// on this part also run faster with it (2 GiB of 16-byte loads: 7.1 against 6.4 TB/s).
template <typename V>
__device__ __forceinline__ V load_stream(const V* p) { return __builtin_nontemporal_load(p); }
template <typename V>
__device__ __forceinline__ void store_stream(const V& v, V* p) { __builtin_nontemporal_store(v, p); }

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(size_t)(const __attribute__((address_space(3))) void*)p;
}

// global_load_lds_dwordx4: 16 bytes per lane from base + voff into LDS at lds + 16 * lane.
// Written out so that the compiler does not track it as an LDS store: it would otherwise wait
// for every copy in flight (vmcnt(0)) before each LDS read and barrier, since it cannot tell
// the stages of a multi-stage pipeline apart.  Callers await completion explicitly (vmcnt)
// before the barrier that publishes a stage; base and lds must be wave-uniform.
__device__ __forceinline__ void copy16(const char* base, uint32_t voff, uint32_t lds) {
    asm volatile(
        "s_mov_b32 m0, %2\n\t"
        "global_load_lds_dwordx4 %0, %1"
        :
        : "v"(voff), "s"(base), "s"(lds)
        : "memory", "m0");
}

// copy16 with the non-temporal (streaming) cache policy, for bytes that are read once
__device__ __forceinline__ void copy16_nt(const char* base, uint32_t voff, uint32_t lds) {
    asm volatile(
        "s_mov_b32 m0, %2\n\t"
        "global_load_lds_dwordx4 %0, %1 nt"
        :
        : "v"(voff), "s"(base), "s"(lds)
        : "memory", "m0");
}

// s_waitcnt vmcnt(min(later, 3) * PER): wait until at most the `later` most recently issued
// k-steps of PER copies each are still in flight (copies complete in issue order).
template <int PER>
__device__ __forceinline__ void wait_copies(int64_t later) {
    static_assert(3 * PER <= 63, "vmcnt range");
    if (later >= 3)
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(3 * PER) : "memory");
    else if (later == 2)
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * PER) : "memory");
    else if (later == 1)
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(PER) : "memory");
    else
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Tile of this workgroup among tiles_m x tiles_n.  Workgroup ids go round-robin over the 8 XCDs
// (ids x, x + 8, ... run on XCD x); those get consecutive logical ids, and logical ids walk groups
// of group_m tile rows column by column, so the workgroups resident on one XCD cover a compact
// block of tiles and share their A and G column bands through that XCD's L2.
__device__ __forceinline__ bool tile_of(int tiles_m, int tiles_n, int group_m, int& tm, int& tn) {
    const int n_tiles = tiles_m * tiles_n;
    int t = blockIdx.x;
    if (t >= n_tiles) return false;
    if (n_tiles % 8 == 0) t = (t % 8) * (n_tiles / 8) + t / 8;
    const int group = t / (group_m * tiles_n);
    const int first_m = group * group_m;
    const int gm = min(tiles_m - first_m, group_m);
    const int r = t - group * group_m * tiles_n;
    tm = first_m + r % gm;
    tn = r / gm;
    return true;
}

// First token row and token count of record `rec`: fixed-length records (seg null) own rows
// [rec T, rec T + T); variable-length records own rows [seg[rec], seg[rec + 1]).
__device__ __forceinline__ void record_rows(const int64_t* seg, int64_t rec, int64_t T,
                                            int64_t& row0, int64_t& len) {
    if (seg) {
        row0 = seg[rec];
        len = seg[rec + 1] - row0;
    } else {
        row0 = rec * T;
        len = T;
    }
}

// v_mfma_f32_16x16x32_bf16: lane l supplies row (l % 16) of the A block and
// column (l % 16) of the B block, each with 8 consecutive k of group l / 16;
// the 16x16 fp32 result has column l % 16, rows 4 * (l / 16) + {0..3} in lane l.
__device__ __forceinline__ f32x4 mfma_bf16(const u32x4& a, const u32x4& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// v_mfma_f32_16x16x4_f32: lane l supplies A[l % 16][l / 16] and B[l / 16][l % 16];
// the result layout is the same as above.
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

}  // namespace dpsgd
