// Fused tail of the step for plans whose layers all keep their per-record
// gradient blocks (the STORED clipped-sum strategy): in one launch over the
// flat parameter index e,
//   out[e] (+)= sum_i c_i P_i[e] + sigma * C * Z[e]
// (the record sum accumulated in fp64 in ascending i and rounded to fp32 once)
// ("Privacy-Preserving Machine Learning", DP-SGD phases 3-4: clip each record,
// sum, add N(0, sigma^2 C^2 I) once), optionally followed by the descent step
// params[e] -= lr / L * out[e] (phase 5).  When the partials are few, every block
// first recomputes all clip factors itself with exactly the arithmetic of the
// clip_factor kernel (one wavefront per record, lanes striding the record's
// partials in a fixed order, fp64 butterfly), so the factors are bitwise the
// ones clip_factor would produce and no separate launch is needed; block 0
// publishes n_i, c_i and the status word.  Otherwise the factors come from a
// preceding clip_factor launch.  A nonfinite norm skips every write to out.
#include <algorithm>
#include <atomic>

#include "philox.h"
#include "record_sum.h"

namespace dpsgd {

constexpr int kFinalBatch = 16;  // records whose blocks a thread loads before the clip prologue
constexpr int kFinalMaxThreads = 512;

// Grid: x = chunks of a layer (4 elements per thread, 64 * nw threads, nw chosen by
// the host so that the grid is about one workgroup per compute unit), y = layer of
// the launch.  A thread reads the blocks at stored positions x .. x + 3 of layer l, which
// hold its elements xl .. xl + 3 (xl = stored_logical(x)), flat indices off_l + xl.  VEC: every layer of the
// launch has n_l and off_l multiples of 4 and 16-byte aligned blocks (checked on the
// host), so the gradient loads are unconditional 16-byte loads (a thread past the end
// of its layer loads the layer's last four elements and stores nothing).  Loads
// complete in issue order and the compiler counts them exactly only when no branch
// decides whether they are issued, so this is what lets the clip prologue wait for
// its own loads alone while the gradient blocks are still in flight.
template <bool CLIP_INSIDE, bool VEC>
__global__ __launch_bounds__(kFinalMaxThreads) void k_finalize(FinalizeArgs a) {
    __shared__ float cs[kFinalMaxRecords];
    __shared__ uint32_t bad;
    const int tid = threadIdx.x;
    const int w = tid >> 6, lane = tid & 63;
    const int nw = (int)(blockDim.x >> 6);
    const int l = blockIdx.y;
    const int64_t off = a.off[l];
    const int64_t n_l = a.off[l + 1] - off;
    const int64_t x0 = ((int64_t)blockIdx.x * blockDim.x + tid) * 4;
    const bool active = x0 < n_l;
    const int64_t xl = active ? stored_logical(a.map[l], x0) : x0;   // the elements' own index
    float* th = a.params[l];   // descent step target, or null
    const bool vec = VEC ? active
                         : active && x0 + 4 <= n_l && (n_l & 3) == 0 && (off & 3) == 0 &&
                               ((reinterpret_cast<uintptr_t>(a.out[l]) |
                                 reinterpret_cast<uintptr_t>(a.src[l]) |
                                 reinterpret_cast<uintptr_t>(th)) & 15u) == 0;

    // 1) what the clip factors depend on, issued first: the status word and the first
    //    batch of partials of this wave's first four records (w, w + nw, w + 2 nw, w + 3 nw)
    const uint32_t status0 = *a.status;
    float pv[4][8];
    if (CLIP_INSIDE) record_parts_load_x4(a.parts, a.parts_stride, a.n_parts, w, nw, a.n_rec, lane, pv);

    // 2) the first batch of this thread's gradient-block loads, independent of the factors
    const float* src = a.src[l] + (VEC && !active ? n_l - 4 : x0);
    f32x4 v[kFinalBatch];
    const int64_t nb0 = a.n_rec < kFinalBatch ? a.n_rec : kFinalBatch;
    if (VEC || vec) {
#pragma unroll
        for (int u = 0; u < kFinalBatch; ++u)   // unconditional: rows past n_rec repeat the last
            v[u] = load_stream(reinterpret_cast<const f32x4*>(src + (u < nb0 ? u : nb0 - 1) * n_l));
    }

    // 3) this thread's normals (Philox + Box-Muller), computed while the loads are in flight
    float z[4] = {0.f, 0.f, 0.f, 0.f};
    if (a.noise && vec) gauss4((uint64_t)(off + xl) >> 2, a.step, a.seed, z);

    // 4) clip factors
    const float* cf = a.clip;
    bool skip;
    if (CLIP_INSIDE) {
        const uint32_t old = a.accumulate ? status0 : 0u;
        if (tid == 0) bad = 0u;
        __syncthreads();
        for (int64_t rec0 = w; rec0 < a.n_rec; rec0 += 4 * nw) {
            double s4[4];
            if (rec0 == w)
                record_norm2_x4_from(pv, a.parts, a.parts_stride, a.n_parts, rec0, nw, a.n_rec, lane, s4);
            else
                record_norm2_x4(a.parts, a.parts_stride, a.n_parts, rec0, nw, a.n_rec, lane, s4);
            // every lane holds the four sums; lane j < 4 finishes record rec0 + j nw
            const int64_t rec = rec0 + (int64_t)lane * nw;
            if (lane < 4 && rec < a.n_rec) {
                const double s = lane == 0 ? s4[0] : lane == 1 ? s4[1] : lane == 2 ? s4[2] : s4[3];
                double n, c;
                if (clip_of_norm2(s, a.C, n, c)) atomicOr(&bad, 1u);
                cs[rec] = (float)c;
                if (blockIdx.x == 0 && l == 0) {
                    a.n_ws[rec] = (float)n;
                    a.c_ws[rec] = (float)c;
                    if (a.n_user) a.n_user[rec] = (float)n;
                    if (a.c_user) a.c_user[rec] = (float)c;
                }
            }
        }
        __syncthreads();
        if (blockIdx.x == 0 && l == 0 && tid == 0) *a.status = old | bad;
        skip = (old | bad) != 0u;
        cf = cs;
    } else {
        skip = status0 != 0u;
    }
    if (skip || !active) return;

    // 4) out (+)= sum_i c_i P_i (ascending i, accumulated in fp64 and rounded once) + sigma C Z
    if (vec) {
        double d[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
        for (int u = 0; u < kFinalBatch; ++u) add_scaled(d, keep_or_zero(cf[u < nb0 ? u : 0], u < nb0), v[u]);
        for (int64_t i = kFinalBatch; i < a.n_rec; i += 8) {   // further records, 8 loads at a time
            f32x4 w8[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int64_t r = i + u < a.n_rec ? i + u : a.n_rec - 1;
                w8[u] = load_stream(reinterpret_cast<const f32x4*>(src + r * n_l));
            }
#pragma unroll
            for (int u = 0; u < 8; ++u)
                add_scaled(d, keep_or_zero(cf[i + u < a.n_rec ? i + u : 0], i + u < a.n_rec), w8[u]);
        }
        f32x4 s = {(float)d[0], (float)d[1], (float)d[2], (float)d[3]};
        f32x4* o = reinterpret_cast<f32x4*>(a.out[l] + xl);
        if (a.accumulate) s = *o + s;
        s[0] += a.scale * z[0];
        s[1] += a.scale * z[1];
        s[2] += a.scale * z[2];
        s[3] += a.scale * z[3];
        *o = s;
        if (th) {
            f32x4* tp = reinterpret_cast<f32x4*>(th + xl);
            f32x4 t = *tp;
#pragma unroll
            for (int q = 0; q < 4; ++q) t[q] = fmaf(-a.descent, s[q], t[q]);
            *tp = t;
        }
        return;
    }
    for (int q = 0; q < 4; ++q) {
        const int64_t xs = x0 + q;             // stored position
        if (xs >= n_l) break;
        const int64_t x = stored_logical(a.map[l], xs);
        const uint64_t e = (uint64_t)(off + x);
        float z = 0.f;
        if (a.noise) {
            float z4[4];
            gauss4(e >> 2, a.step, a.seed, z4);
            z = z4[e & 3];
        }
        double d = 0.0;
        for (int64_t i = 0; i < a.n_rec; ++i) d = fma((double)cf[i], (double)a.src[l][i * n_l + xs], d);
        float s = (float)d;
        float* o = a.out[l] + x;
        if (a.accumulate) s = *o + s;
        const float v = s + a.scale * z;
        *o = v;
        if (th) th[x] = fmaf(-a.descent, v, th[x]);
    }
}

// compute units of the current device (cached per device)
static int64_t compute_units() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

hipError_t launch_finalize(const FinalizeArgs& a, bool clip_inside, hipStream_t s) {
    int64_t max_n = 0;
    bool vec = true;
    for (int l = 0; l < a.n_layers; ++l) {
        const int64_t n_l = a.off[l + 1] - a.off[l];
        max_n = std::max<int64_t>(max_n, n_l);
        const uintptr_t ptrs = reinterpret_cast<uintptr_t>(a.out[l]) | reinterpret_cast<uintptr_t>(a.src[l]) |
                               reinterpret_cast<uintptr_t>(a.params[l]);
        if (n_l < 4 || (n_l & 3) != 0 || (a.off[l] & 3) != 0 || (ptrs & 15u) != 0) vec = false;
    }
    if (max_n == 0) return hipSuccess;
    // about one workgroup per compute unit: chunks per layer so that the layers fill the
    // chip, wavefronts per workgroup so that the chunks cover a layer
    const int64_t n_cu = compute_units();
    const int64_t max_f4 = (max_n + 3) / 4;
    const int64_t per_layer = std::max<int64_t>(1, n_cu / a.n_layers);
    const int64_t nw = std::min<int64_t>(kFinalMaxThreads / 64, (max_f4 + 64 * per_layer - 1) / (64 * per_layer));
    const int64_t threads = 64 * nw;
    const dim3 grid((unsigned)((max_f4 + threads - 1) / threads), a.n_layers);
    if (clip_inside && vec) hipLaunchKernelGGL((k_finalize<true, true>), grid, dim3((unsigned)threads), 0, s, a);
    else if (clip_inside) hipLaunchKernelGGL((k_finalize<true, false>), grid, dim3((unsigned)threads), 0, s, a);
    else if (vec) hipLaunchKernelGGL((k_finalize<false, true>), grid, dim3((unsigned)threads), 0, s, a);
    else hipLaunchKernelGGL((k_finalize<false, false>), grid, dim3((unsigned)threads), 0, s, a);
    return hipGetLastError();
}

}  // namespace dpsgd
