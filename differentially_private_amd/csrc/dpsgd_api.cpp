// Host side of the C ABI in include/dpsgd.h: plan construction (path choice per
// layer, workspace layout), argument validation (every argument error is
// returned before anything is enqueued), and launch sequencing of the kernels.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "../../include/dpsgd.h"
#include "internal.h"
#include "int8.h"

using namespace dpsgd;

namespace {

thread_local std::string g_last_error;

int fail(int code, const std::string& msg) {
    g_last_error = msg;
    return code;
}

int hip_fail(hipError_t e, const char* where) {
    g_last_error = std::string(where) + ": " + hipGetErrorString(e);
    return DPSGD_ERR_HIP;
}

constexpr int64_t kAlign = 256;
int64_t align_up(int64_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool mul_ok(int64_t a, int64_t b, int64_t* out) {
    __int128 p = (__int128)a * (__int128)b;
    if (p > (__int128)INT64_MAX / 4) return false;  // leave room for byte sizes
    *out = (int64_t)p;
    return true;
}

struct Tiles {
    int x_is_in;
    int64_t dX, dY;
    int mb;
    int tiles_x, tiles_y, wg_x;
};

Tiles direct_tiles(int64_t d_in, int64_t d_out) {
    Tiles t;
    t.x_is_in = d_in >= d_out ? 1 : 0;
    t.dX = t.x_is_in ? d_in : d_out;
    t.dY = t.x_is_in ? d_out : d_in;
    t.mb = t.dY <= 16 ? 1 : 2;
    t.tiles_x = (int)((t.dX + 127) / 128);
    t.tiles_y = (int)((t.dY + 16 * t.mb - 1) / (16 * t.mb));
    t.wg_x = (t.tiles_x + 3) / 4;
    return t;
}

}  // namespace

struct LayerPlan {
    int64_t d_in, d_out, n_params, param_off;
    int path;      // DPSGD_PATH_GRAM / DPSGD_PATH_DIRECT
    int sum_mode;  // DPSGD_SUM_GEMM / DPSGD_SUM_STORED
    Tiles tiles;   // direct decomposition (norm on the direct path, and the GEMM sum)
    int nb, n_pairs;
    int64_t n_parts, part_off;
    int64_t stored_off;  // bytes into ws (STORED)
    StoredMap smap;      // order of the STORED blocks, written by the norm kernel
    int64_t split_off;   // bytes into ws (GEMM with splits)
    bool dense;          // GEMM sum on the dense MFMA kernels (bf16, both dimensions > 16)
};

namespace {

// Order of a layer's STORED gradient blocks (StoredMap): the norm kernel keeps whole 128-wide X
// tiles in store order when stored_permuted(d_out), the natural order otherwise.
StoredMap stored_map(int dtype, const LayerPlan& lp) {
    StoredMap m{0, 0, lp.d_out};
    if (lp.sum_mode != DPSGD_SUM_STORED || !stored_permuted(lp.d_out)) return m;
    if (lp.tiles.x_is_in) m.mode = dtype == DPSGD_DTYPE_BF16 ? 1 : 2;
    else if (dtype == DPSGD_DTYPE_BF16) m.mode = 3;
    m.full = (int32_t)(lp.tiles.dX / 128 * 128);
    return m;
}

}  // namespace

struct dpsgd_plan {
    std::vector<LayerPlan> layers;
    int dtype;
    int64_t B, T;
    int64_t parts_total;
    int64_t n_params;
    int n_splits_max;        // tile-engine GEMM sums
    int n_splits_dense_max;  // dense GEMM sums
    bool segments;           // variable-length records (DPSGD_PLAN_SEGMENTS)
    int64_t status_off, parts_off, n_off, c_off, seg_off;
    int64_t ws_bytes;
};

namespace {

int elem_size(int dtype) { return dtype == DPSGD_DTYPE_F32 ? 4 : 2; }

bool ptr_aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

float* ws_f(void* ws, int64_t off) { return reinterpret_cast<float*>(static_cast<char*>(ws) + off); }
uint32_t* ws_status(void* ws, const dpsgd_plan* p) {
    return reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + p->status_off);
}
// the segment table of a segment plan's workspace (null for fixed-length records)
const int64_t* ws_seg(const void* ws, const dpsgd_plan* p) {
    return p->segments ? reinterpret_cast<const int64_t*>(static_cast<const char*>(ws) + p->seg_off)
                       : nullptr;
}

int check_plan(const dpsgd_plan* p) {
    if (!p) return fail(DPSGD_ERR_INVALID_ARG, "plan is NULL");
    return DPSGD_OK;
}

int check_ws(const void* ws) {
    if (!ws) return fail(DPSGD_ERR_INVALID_ARG, "workspace is NULL");
    if (reinterpret_cast<uintptr_t>(ws) % kAlign) return fail(DPSGD_ERR_INVALID_ARG, "workspace is not 256-byte aligned");
    return DPSGD_OK;
}

int check_records(const dpsgd_plan* p, int64_t n) {
    if (n < 0 || n > p->B)
        return fail(DPSGD_ERR_INVALID_ARG, "n_records outside [0, max_records]");
    return DPSGD_OK;
}

int check_range(const dpsgd_plan* p, int32_t l0, int32_t l1) {
    if (l0 < 0 || l1 > (int32_t)p->layers.size() || l0 > l1)
        return fail(DPSGD_ERR_INVALID_ARG, "layer range outside [0, n_layers]");
    return DPSGD_OK;
}

int check_c_sigma(double C, double sigma, bool need_sigma) {
    if (!std::isfinite(C) || !(C > 0.0)) return fail(DPSGD_ERR_INVALID_ARG, "C must be finite and > 0");
    if (need_sigma && (!std::isfinite(sigma) || sigma < 0.0))
        return fail(DPSGD_ERR_INVALID_ARG, "sigma must be finite and >= 0");
    return DPSGD_OK;
}

// ---- phase implementations (arguments already validated) ----

// Layers per launch when `count` layers go out in launches of at most `cap`: as few launches as
// the cap allows, with their layer counts as equal as possible (so that every launch of a phase
// moves about the same bytes and a per-launch average describes each of them).
int balanced_chunk(int count, int cap) {
    if (count <= 0) return cap;
    const int launches = (count + cap - 1) / cap;
    return (count + launches - 1) / launches;
}

// Waves per workgroup for a launch group: 2 when every layer's column-tile count
// is even, else 1, so that no workgroup carries idle waves (measured on the
// LoRA workloads: small workgroups stream best; 4-8 waves per workgroup were
// 5-18% slower).
void set_wpb(DirectArgs& a) {
    int wpb = 2;
    for (int l = 0; l < a.n_layers; ++l)
        if (a.L[l].tiles_x % 2) wpb = 1;
    a.wpb = wpb;
    for (int l = 0; l < a.n_layers; ++l) a.L[l].wg_x = (a.L[l].tiles_x + wpb - 1) / wpb;
}

// STORED gradient blocks leave the norm kernel by non-temporal stores, each whole tile in store
// order so that every instruction writes whole lines: against plain stores, the norm launch of a
// 43-layer slice of the 7B-shaped LoRA batch (2.9 GB of blocks) ran 9.30 against 9.66 ms, the OPT-125M-shaped step (19 MB)
// 61.8 against 63.4 us and the 1024-hidden LoRA step (403 MB per physical batch) 17.95 against
// 17.98 ms.  (Before the store order, a non-temporal store wrote half lines, and plain stores were
// the faster choice below 1 GiB of blocks.)

int do_norms(const dpsgd_plan* p, int64_t n_rec, int l0, int l1, const void* const* A,
             const void* const* G, void* ws, hipStream_t s) {
    if (n_rec == 0 || l0 == l1) return DPSGD_OK;
    float* parts = ws_f(ws, p->parts_off);
    const int es = elem_size(p->dtype);
    // direct layers, grouped by (MB, store); Gram layers in their own launches
    for (int mb = 1; mb <= 2; ++mb) {
        for (int store = 0; store <= 1; ++store) {
            auto in_group = [&](const LayerPlan& lp) {
                return lp.path == DPSGD_PATH_DIRECT && lp.tiles.mb == mb &&
                       (lp.sum_mode == DPSGD_SUM_STORED) == (store == 1);
            };
            int count = 0;
            for (int l = l0; l < l1; ++l) count += in_group(p->layers[l]) ? 1 : 0;
            const int per = balanced_chunk(count, kMaxLaunchLayers);
            DirectArgs a;
            std::memset(&a, 0, sizeof(a));
            a.T = p->T;
            a.n_rec = n_rec;
            a.parts_stride = p->parts_total;
            a.parts = parts;
            a.seg = ws_seg(ws, p);
            for (int l = l0; l < l1; ++l) {
                const LayerPlan& lp = p->layers[l];
                if (!in_group(lp)) continue;
                DirectLayer& d = a.L[a.n_layers];
                const void* a_ptr = A[l - l0];
                const void* g_ptr = G[l - l0];
                d.X = lp.tiles.x_is_in ? a_ptr : g_ptr;
                d.Y = lp.tiles.x_is_in ? g_ptr : a_ptr;
                d.P = store ? ws_f(ws, lp.stored_off) : nullptr;
                d.dX = (int32_t)lp.tiles.dX;
                d.dY = (int32_t)lp.tiles.dY;
                d.x_is_in = lp.tiles.x_is_in;
                d.tiles_x = lp.tiles.tiles_x;
                d.tiles_y = lp.tiles.tiles_y;
                d.wg_x = lp.tiles.wg_x;
                d.part_off = (int32_t)lp.part_off;
                d.vec_x = ptr_aligned16(d.X) && ((lp.tiles.dX * es) % 16 == 0);
                d.d_out = lp.d_out;
                d.split_stride = 0;
                if (++a.n_layers == per) {
                    set_wpb(a);
                    hipError_t e = launch_norm_direct(a, p->dtype, mb, store, s);
                    if (e != hipSuccess) return hip_fail(e, "ghost_norm (direct) launch");
                    a.n_layers = 0;
                }
            }
            if (a.n_layers) {
                set_wpb(a);
                hipError_t e = launch_norm_direct(a, p->dtype, mb, store, s);
                if (e != hipSuccess) return hip_fail(e, "ghost_norm (direct) launch");
            }
        }
    }
    // Gram layers: grouped by identical block counts (all share T, so one group)
    GramArgs g;
    std::memset(&g, 0, sizeof(g));
    g.T = p->T;
    g.seg = ws_seg(ws, p);
    g.n_rec = n_rec;
    g.parts_stride = p->parts_total;
    g.parts = parts;
    g.nb = (int32_t)((p->T + 63) / 64);
    g.n_pairs = g.nb * (g.nb + 1) / 2;
    for (int l = l0; l < l1; ++l) {
        const LayerPlan& lp = p->layers[l];
        if (lp.path != DPSGD_PATH_GRAM) continue;
        GramLayer& d = g.L[g.n_layers];
        d.A = A[l - l0];
        d.G = G[l - l0];
        d.d_in = (int32_t)lp.d_in;
        d.d_out = (int32_t)lp.d_out;
        d.part_off = (int32_t)lp.part_off;
        d.vec_a = ptr_aligned16(d.A) && ((lp.d_in * es) % 16 == 0);
        d.vec_g = ptr_aligned16(d.G) && ((lp.d_out * es) % 16 == 0);
        if (++g.n_layers == kMaxLaunchLayers) {
            hipError_t e = launch_norm_gram(g, p->dtype, s);
            if (e != hipSuccess) return hip_fail(e, "ghost_norm (Gram) launch");
            g.n_layers = 0;
        }
    }
    if (g.n_layers) {
        hipError_t e = launch_norm_gram(g, p->dtype, s);
        if (e != hipSuccess) return hip_fail(e, "ghost_norm (Gram) launch");
    }
    return DPSGD_OK;
}

int do_clip(const dpsgd_plan* p, int64_t n_rec, double C, uint32_t flags, void* ws,
            float* n_user, float* c_user, hipStream_t s) {
    ClipArgs a;
    std::memset(&a, 0, sizeof(a));
    a.parts = ws_f(ws, p->parts_off);
    a.parts_stride = p->parts_total;
    a.n_parts = p->parts_total;
    a.n_rec = n_rec;
    a.C = C;
    a.n_ws = ws_f(ws, p->n_off);
    a.c_ws = ws_f(ws, p->c_off);
    a.n_user = n_user;
    a.c_user = c_user;
    a.status = ws_status(ws, p);
    a.accumulate = (flags & DPSGD_ACCUMULATE) ? 1 : 0;
    hipError_t e = launch_clip(a, s);
    if (e != hipSuccess) return hip_fail(e, "clip_factor launch");
    return DPSGD_OK;
}

int do_sum(const dpsgd_plan* p, int64_t n_rec, int l0, int l1, const void* const* A,
           const void* const* G, const float* clip, float* const* out, uint32_t flags, void* ws,
           hipStream_t s) {
    if (l0 == l1) return DPSGD_OK;
    const bool acc = (flags & DPSGD_ACCUMULATE) != 0;
    const uint32_t* status = ws_status(ws, p);
    if (!clip) clip = ws_f(ws, p->c_off);
    const int es = elem_size(p->dtype);

    // split count for this call
    int ns = 1;
    int64_t rps = n_rec;
    if (n_rec > 0) {
        ns = (int)std::min<int64_t>(p->n_splits_max, n_rec);
        rps = (n_rec + ns - 1) / ns;
        ns = (int)((n_rec + rps - 1) / rps);
    }

    // 1) STORED layers (and every layer when n_rec == 0): weighted reduce over records
    {
        ReduceArgs r;
        std::memset(&r, 0, sizeof(r));
        r.accumulate = acc;
        r.n_src = n_rec;
        r.clip = clip;
        r.status = status;
        auto flush = [&]() -> int {
            if (!r.n_layers) return DPSGD_OK;
            hipError_t e = launch_reduce(r, true, s);
            if (e != hipSuccess) return hip_fail(e, "clipped_sum (stored) launch");
            r.n_layers = 0;
            r.max_n4 = 0;
            return DPSGD_OK;
        };
        for (int l = l0; l < l1; ++l) {
            const LayerPlan& lp = p->layers[l];
            if (n_rec > 0 && lp.sum_mode != DPSGD_SUM_STORED) continue;
            ReduceLayer& d = r.L[r.n_layers];
            d.src = (lp.sum_mode == DPSGD_SUM_STORED) ? ws_f(ws, lp.stored_off) : nullptr;
            d.out = out[l - l0];
            d.n = lp.n_params;
            d.map = lp.smap;
            r.max_n4 = std::max<int64_t>(r.max_n4, (lp.n_params + 3) / 4);
            if (++r.n_layers == kMaxLaunchLayers) {
                int rc = flush();
                if (rc) return rc;
            }
        }
        int rc = flush();
        if (rc) return rc;
    }
    if (n_rec == 0) return DPSGD_OK;

    // 2) dense GEMM layers (bf16): MFMA GEMM kernels, split over records
    {
        int nsd = (int)std::min<int64_t>(p->n_splits_dense_max, n_rec);
        const int64_t rpsd = (n_rec + nsd - 1) / nsd;
        nsd = (int)((n_rec + rpsd - 1) / rpsd);
        DenseSumArgs a;
        std::memset(&a, 0, sizeof(a));
        a.accumulate = acc;
        a.T = p->T;
        a.n_rec = n_rec;
        a.rec_per_split = rpsd;
        a.clip = clip;
        a.status = status;
        ReduceArgs r;
        std::memset(&r, 0, sizeof(r));
        r.accumulate = acc;
        r.n_src = nsd;
        r.status = status;
        auto flush = [&]() -> int {
            if (!a.n_layers) return DPSGD_OK;
            hipError_t e = launch_sum_dense(a, nsd, s);
            if (e != hipSuccess) return hip_fail(e, "clipped_sum (dense) launch");
            if (nsd > 1) {
                e = launch_reduce(r, false, s);
                if (e != hipSuccess) return hip_fail(e, "clipped_sum (split reduce) launch");
            }
            a.n_layers = 0;
            r.n_layers = 0;
            r.max_n4 = 0;
            return DPSGD_OK;
        };
        for (int l = l0; l < l1; ++l) {
            const LayerPlan& lp = p->layers[l];
            if (lp.sum_mode != DPSGD_SUM_GEMM || !lp.dense) continue;
            DenseSumLayer& d = a.L[a.n_layers];
            d.A = A[l - l0];
            d.G = G[l - l0];
            d.d_in = (int32_t)lp.d_in;
            d.d_out = (int32_t)lp.d_out;
            d.tiles_m = (int32_t)((lp.d_in + 255) / 256);
            d.tiles_n = (int32_t)((lp.d_out + 127) / 128);
            d.vec_a = ptr_aligned16(d.A) && ((lp.d_in * es) % 16 == 0);
            d.vec_g = ptr_aligned16(d.G) && ((lp.d_out * es) % 16 == 0);
            if (nsd > 1) {
                d.split = ws_f(ws, lp.split_off);
                d.split_stride = lp.n_params;
                d.out = nullptr;
                ReduceLayer& rl = r.L[r.n_layers++];
                rl.src = d.split;
                rl.out = out[l - l0];
                rl.n = lp.n_params;
                r.max_n4 = std::max<int64_t>(r.max_n4, (lp.n_params + 3) / 4);
            } else {
                d.out = out[l - l0];
                d.split = nullptr;
                d.split_stride = 0;
            }
            if (++a.n_layers == kDenseMaxLayers) {
                int rc = flush();
                if (rc) return rc;
            }
        }
        int rc = flush();
        if (rc) return rc;
    }

    // 3) other GEMM layers: tile-engine sum, split over records, then a fixed-order reduce
    for (int mb = 1; mb <= 2; ++mb) {
        DirectArgs a;
        std::memset(&a, 0, sizeof(a));
        a.T = p->T;
        a.seg = ws_seg(ws, p);
        a.n_rec = n_rec;
        a.clip = clip;
        a.rec_per_split = rps;
        a.status = status;
        a.accumulate = acc;
        ReduceArgs r;
        std::memset(&r, 0, sizeof(r));
        r.accumulate = acc;
        r.n_src = ns;
        r.status = status;
        auto flush = [&]() -> int {
            if (!a.n_layers) return DPSGD_OK;
            set_wpb(a);
            hipError_t e = launch_sum_direct(a, p->dtype, mb, ns, s);
            if (e != hipSuccess) return hip_fail(e, "clipped_sum (GEMM) launch");
            if (ns > 1) {
                e = launch_reduce(r, false, s);
                if (e != hipSuccess) return hip_fail(e, "clipped_sum (split reduce) launch");
            }
            a.n_layers = 0;
            r.n_layers = 0;
            r.max_n4 = 0;
            return DPSGD_OK;
        };
        int count = 0;
        for (int l = l0; l < l1; ++l) {
            const LayerPlan& lp = p->layers[l];
            count += (lp.sum_mode == DPSGD_SUM_GEMM && !lp.dense && lp.tiles.mb == mb) ? 1 : 0;
        }
        const int per = balanced_chunk(count, kMaxLaunchLayers);
        for (int l = l0; l < l1; ++l) {
            const LayerPlan& lp = p->layers[l];
            if (lp.sum_mode != DPSGD_SUM_GEMM || lp.dense || lp.tiles.mb != mb) continue;
            DirectLayer& d = a.L[a.n_layers];
            const void* a_ptr = A[l - l0];
            const void* g_ptr = G[l - l0];
            d.X = lp.tiles.x_is_in ? a_ptr : g_ptr;
            d.Y = lp.tiles.x_is_in ? g_ptr : a_ptr;
            d.dX = (int32_t)lp.tiles.dX;
            d.dY = (int32_t)lp.tiles.dY;
            d.x_is_in = lp.tiles.x_is_in;
            d.tiles_x = lp.tiles.tiles_x;
            d.tiles_y = lp.tiles.tiles_y;
            d.wg_x = lp.tiles.wg_x;
            d.vec_x = ptr_aligned16(d.X) && ((lp.tiles.dX * es) % 16 == 0);
            d.d_out = lp.d_out;
            if (ns > 1) {
                d.P = ws_f(ws, lp.split_off);
                d.split_stride = lp.n_params;
                ReduceLayer& rl = r.L[r.n_layers++];
                rl.src = d.P;
                rl.out = out[l - l0];
                rl.n = lp.n_params;
                r.max_n4 = std::max<int64_t>(r.max_n4, (lp.n_params + 3) / 4);
            } else {
                d.P = out[l - l0];
                d.split_stride = 0;
            }
            if (++a.n_layers == per) {
                int rc = flush();
                if (rc) return rc;
            }
        }
        int rc = flush();
        if (rc) return rc;
    }
    return DPSGD_OK;
}

// params (or null): the descent step params_l -= descent * out_l after the noise.  The layers are
// cut into pieces of at most kNoisePieceMax elements and go out in as few launches as the
// kernel-argument limit allows (one for every plan of this library's workloads), each launch's
// pieces spanning less than 2^32 elements.
int do_noise(const dpsgd_plan* p, float* const* out, float* const* params, double descent, double C,
             double sigma, uint64_t seed, uint64_t step, const void* ws, hipStream_t s) {
    struct Piece { float* out; float* par; int64_t off, n; };
    std::vector<Piece> pieces;
    for (size_t l = 0; l < p->layers.size(); ++l) {
        const LayerPlan& lp = p->layers[l];
        for (int64_t x = 0; x < lp.n_params; x += kNoisePieceMax) {
            const int64_t n = std::min<int64_t>(kNoisePieceMax, lp.n_params - x);
            pieces.push_back({out[l] + x, params ? params[l] + x : nullptr, lp.param_off + x, n});
        }
    }
    const int cap = params ? kNoiseMaxPiecesDescent : kNoiseMaxPieces;
    const int per = balanced_chunk((int)pieces.size(), cap);
    NoiseArgs a;
    size_t k = 0;
    while (k < pieces.size()) {
        std::memset(&a, 0, sizeof(a));
        a.base = pieces[k].off;
        a.seed = seed;
        a.step = step;
        a.scale = (float)(sigma * C);
        a.descent = (float)descent;
        a.status = ws ? reinterpret_cast<const uint32_t*>(static_cast<const char*>(ws) + p->status_off) : nullptr;
        a.with_params = params ? 1 : 0;
        int n = 0;
        while (k + n < pieces.size() && n < per &&
               pieces[k + n].off + pieces[k + n].n - a.base <= (int64_t)UINT32_MAX) {
            a.off[n] = (uint32_t)(pieces[k + n].off - a.base);
            ++n;
        }
        a.n_pieces = n;
        a.off[n] = (uint32_t)(pieces[k + n - 1].off + pieces[k + n - 1].n - a.base);
        for (int q = 0; q < n; ++q) {
            a.ptr[q] = pieces[k + q].out;
            if (params) a.ptr[n + q] = pieces[k + q].par;
        }
        hipError_t e = launch_noise(a, s);
        if (e != hipSuccess) return hip_fail(e, "noise launch");
        k += n;
    }
    return DPSGD_OK;
}

// Fused tail for plans whose layers all keep their gradient blocks: clip (inside
// the kernel when the partials are few, else a clip_factor launch first), the
// weighted sum and, unless NO_NOISE, the noise in one pass per layer group.
int do_finalize(const dpsgd_plan* p, int64_t n_rec, double C, double sigma, uint64_t seed,
                uint64_t step, uint32_t flags, void* ws, float* const* out, float* n_user,
                float* c_user, float* const* params, double descent, hipStream_t s) {
    const bool inside = n_rec <= kFinalMaxRecords && n_rec * p->parts_total <= kFinalMaxClipWork;
    if (!inside)
        if (int rc = do_clip(p, n_rec, C, flags, ws, n_user, c_user, s)) return rc;
    const int L = (int)p->layers.size();
    const int per = balanced_chunk(L, kFinalMaxLayers);
    FinalizeArgs a;
    for (int l0 = 0; l0 < L; l0 += per) {
        const int l1 = std::min(L, l0 + per);
        std::memset(&a, 0, sizeof(a));
        a.n_layers = l1 - l0;
        a.accumulate = (flags & DPSGD_ACCUMULATE) ? 1 : 0;
        a.noise = (flags & DPSGD_NO_NOISE) ? 0 : 1;
        a.n_rec = n_rec;
        a.seed = seed;
        a.step = step;
        a.scale = a.noise ? (float)(sigma * C) : 0.f;
        a.parts = ws_f(ws, p->parts_off);
        a.parts_stride = p->parts_total;
        a.n_parts = p->parts_total;
        a.C = C;
        a.n_ws = ws_f(ws, p->n_off);
        a.c_ws = ws_f(ws, p->c_off);
        a.n_user = n_user;
        a.c_user = c_user;
        a.status = ws_status(ws, p);
        a.clip = ws_f(ws, p->c_off);
        a.descent = (float)descent;
        for (int l = l0; l < l1; ++l) {
            a.out[l - l0] = out[l];
            a.params[l - l0] = params ? params[l] : nullptr;
            a.src[l - l0] = ws_f(ws, p->layers[l].stored_off);
            a.off[l - l0] = p->layers[l].param_off;
            a.map[l - l0] = p->layers[l].smap;
        }
        a.off[l1 - l0] = p->layers[l1 - 1].param_off + p->layers[l1 - 1].n_params;
        hipError_t e = launch_finalize(a, inside, s);
        if (e != hipSuccess) return hip_fail(e, "finalize launch");
    }
    return DPSGD_OK;
}

bool all_stored(const dpsgd_plan* p) {
    for (const LayerPlan& lp : p->layers)
        if (lp.sum_mode != DPSGD_SUM_STORED) return false;
    return true;
}

}  // namespace

// Host plan of the record-owned INT8 forward: capacities and the workspace layout.
struct I8PlanImpl {
    int64_t max_rows, max_records, max_k, kp, kw;
    int64_t off_offsets, off_own, off_s, off_omask, off_pmask, off_q, ws_bytes;
};

int64_t i8_pitch(int64_t k) { return (k + 63) / 64 * 64; }


namespace dpsgd {
hipError_t launch_hbm_read(const void* buf, int64_t bytes, uint32_t* sink, hipStream_t s);
}

extern "C" {

int dpsgd_plan_create(const dpsgd_plan_desc* d, dpsgd_plan** out, size_t* ws_bytes) {
    if (!d || !out || !ws_bytes) return fail(DPSGD_ERR_INVALID_ARG, "null argument");
    *out = nullptr;
    if (d->n_layers < 1 || !d->layers) return fail(DPSGD_ERR_INVALID_ARG, "n_layers < 1 or layers NULL");
    if (d->dtype != DPSGD_DTYPE_F32 && d->dtype != DPSGD_DTYPE_BF16)
        return fail(DPSGD_ERR_UNSUPPORTED, "dtype must be DPSGD_DTYPE_F32 or DPSGD_DTYPE_BF16");
    if (d->path_policy < DPSGD_PATH_AUTO || d->path_policy > DPSGD_PATH_DIRECT)
        return fail(DPSGD_ERR_UNSUPPORTED, "unknown path_policy");
    if (d->sum_policy < DPSGD_SUM_AUTO || d->sum_policy > DPSGD_SUM_STORED)
        return fail(DPSGD_ERR_UNSUPPORTED, "unknown sum_policy");
    if (d->max_records < 1 || d->max_records > 65535)
        return fail(DPSGD_ERR_INVALID_ARG, "max_records must be in [1, 65535]");
    if (d->tokens < 1) return fail(DPSGD_ERR_INVALID_ARG, "tokens (T) must be >= 1");
    if (d->flags & ~DPSGD_PLAN_SEGMENTS) return fail(DPSGD_ERR_INVALID_ARG, "unknown plan flags");
    const int es = elem_size(d->dtype);

    dpsgd_plan* p = new (std::nothrow) dpsgd_plan();
    if (!p) return fail(DPSGD_ERR_INVALID_ARG, "out of host memory");
    p->dtype = d->dtype;
    p->B = d->max_records;
    p->T = d->tokens;
    p->segments = (d->flags & DPSGD_PLAN_SEGMENTS) != 0;
    int64_t param_off = 0, part_off = 0;
    for (int l = 0; l < d->n_layers; ++l) {
        const int64_t di = d->layers[l].d_in, dd = d->layers[l].d_out;
        if (di < 1 || dd < 1 || di > (1 << 30) || dd > (1 << 30)) {
            delete p;
            return fail(DPSGD_ERR_INVALID_ARG, "layer dimensions must be in [1, 2^30]");
        }
        int64_t np_, rows, in_bytes, tmp;
        if (!mul_ok(di, dd, &np_) || !mul_ok(p->B, p->T, &rows) || !mul_ok(rows, di + dd, &tmp) ||
            !mul_ok(tmp, es, &in_bytes) || !mul_ok(np_, p->B * 4, &tmp)) {
            delete p;
            return fail(DPSGD_ERR_INVALID_ARG, "sizes overflow");
        }
        LayerPlan lp;
        std::memset(&lp, 0, sizeof(lp));
        lp.d_in = di;
        lp.d_out = dd;
        lp.n_params = np_;
        lp.param_off = param_off;
        param_off += np_;
        if (d->path_policy == DPSGD_PATH_AUTO) {
            const __int128 t2 = (__int128)p->T * p->T;
            lp.path = t2 < (__int128)di * dd ? DPSGD_PATH_GRAM : DPSGD_PATH_DIRECT;
        } else {
            lp.path = d->path_policy;
        }
        lp.tiles = direct_tiles(di, dd);
        if (lp.path == DPSGD_PATH_GRAM) {
            lp.nb = (int)((p->T + 63) / 64);
            lp.n_pairs = lp.nb * (lp.nb + 1) / 2;
            lp.n_parts = lp.n_pairs;
            lp.sum_mode = DPSGD_SUM_GEMM;
        } else {
            lp.n_parts = (int64_t)lp.tiles.tiles_x * lp.tiles.tiles_y;
            if (d->sum_policy == DPSGD_SUM_AUTO) {
                // keep the per-record gradient blocks when writing + re-reading them (8 bytes
                // per parameter) moves fewer bytes than re-reading the record's A and G rows
                const __int128 stored = (__int128)8 * np_;
                const __int128 reread = (__int128)p->T * (di + dd) * es;
                lp.sum_mode = stored < reread ? DPSGD_SUM_STORED : DPSGD_SUM_GEMM;
            } else {
                lp.sum_mode = d->sum_policy;
            }
        }
        lp.part_off = part_off;
        part_off += lp.n_parts;
        p->layers.push_back(lp);
    }
    p->parts_total = part_off;
    p->n_params = param_off;
    if (p->parts_total > INT32_MAX) {
        delete p;
        return fail(DPSGD_ERR_INVALID_ARG, "too many norm partials");
    }

    // split counts of the GEMM clipped sums: ~16384 wavefronts per launch for the tile
    // engine, >= 256 workgroups of 256 x 256 tiles (one per CU) for the dense kernels
    int64_t waves_mb[3] = {0, 0, 0}, layers_mb[3] = {0, 0, 0}, dense_wgs = 0;
    for (LayerPlan& lp : p->layers) {
        if (lp.sum_mode != DPSGD_SUM_GEMM) continue;
        // (segment plans keep every GEMM sum on the tile engine, which walks each record's rows)
        lp.dense = p->dtype == DPSGD_DTYPE_BF16 && lp.tiles.mb == 2 && !p->segments;
        if (lp.dense) {
            dense_wgs += ((lp.d_in + 255) / 256) * ((lp.d_out + 255) / 256);
        } else {
            waves_mb[lp.tiles.mb] += (int64_t)lp.tiles.tiles_x * lp.tiles.tiles_y;
            ++layers_mb[lp.tiles.mb];
        }
    }
    // the tile-engine sums go out in launches of at most kMaxLaunchLayers layers of one MB, so the
    // wavefronts that matter are those of one launch: the smallest launch sets the split count (the
    // 7B-shaped LoRA plan's 256 layers go out as six launches of ~1,370 wavefronts: 13 splits;
    // measured there 52.8 / 49.5 / 47.9 / 47.0 / 48.9 ms for 1 / 4 / 7 / 13 / 25 splits, the last
    // paying for its partials in the reduce)
    int64_t waves = 0;
    for (int mb = 1; mb <= 2; ++mb) {
        if (!layers_mb[mb]) continue;
        const int64_t launches = (layers_mb[mb] + kMaxLaunchLayers - 1) / kMaxLaunchLayers;
        const int64_t per = std::max<int64_t>(1, waves_mb[mb] / launches);
        waves = waves ? std::min(waves, per) : per;
    }
    auto splits_for = [&](int64_t units, int64_t target) -> int {
        if (units <= 0) return 1;
        return (int)std::min<int64_t>(std::min<int64_t>(p->B, 64),
                                      std::max<int64_t>(1, (target + units - 1) / units));
    };
    const int ns = splits_for(waves, 16384);
    const int nsd = splits_for(dense_wgs, 256);
    p->n_splits_max = ns;
    p->n_splits_dense_max = nsd;

    // workspace layout (every region 256-byte aligned; a total past 2^62 bytes is refused)
    int64_t off = 0;
    bool fits = true;
    auto region = [&](int64_t count, int64_t elem) -> int64_t {
        const int64_t at = off;
        int64_t bytes = 0;
        if (!mul_ok(count, elem, &bytes) || bytes > ((int64_t)1 << 62) - off) fits = false;
        else off = align_up(off + bytes);
        return at;
    };
    p->status_off = region(1, kAlign);
    p->parts_off = region(p->B * p->parts_total, 4);
    p->n_off = region(p->B, 4);
    p->c_off = region(p->B, 4);
    p->seg_off = region(p->segments ? p->B + 1 : 0, 8);
    for (LayerPlan& lp : p->layers) {
        lp.smap = stored_map(p->dtype, lp);
        if (lp.sum_mode == DPSGD_SUM_STORED)
            lp.stored_off = region(p->B, lp.n_params * 4);
        else if ((lp.dense ? nsd : ns) > 1)
            lp.split_off = region(lp.dense ? nsd : ns, lp.n_params * 4);
    }
    if (!fits) {
        delete p;
        return fail(DPSGD_ERR_INVALID_ARG, "workspace size overflows");
    }
    p->ws_bytes = off;
    *ws_bytes = (size_t)off;
    *out = p;
    return DPSGD_OK;
}

void dpsgd_plan_destroy(dpsgd_plan* p) { delete p; }

int dpsgd_plan_layer_info(const dpsgd_plan* p, int32_t layer, int32_t* path, int32_t* sum_mode) {
    if (int rc = check_plan(p)) return rc;
    if (layer < 0 || layer >= (int32_t)p->layers.size()) return fail(DPSGD_ERR_INVALID_ARG, "layer out of range");
    if (path) *path = p->layers[layer].path;
    if (sum_mode) *sum_mode = p->layers[layer].sum_mode;
    return DPSGD_OK;
}

int64_t dpsgd_plan_num_params(const dpsgd_plan* p) { return p ? p->n_params : -1; }

int dpsgd_ws_init(const dpsgd_plan* p, void* ws, void* stream) {
    if (int rc = check_plan(p)) return rc;
    if (int rc = check_ws(ws)) return rc;
    hipError_t e = launch_status_clear(ws_status(ws, p), (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "status clear launch");
    return DPSGD_OK;
}

int dpsgd_ws_segments(const dpsgd_plan* p, void* ws, const int64_t* offsets, int64_t n_records,
                      void* stream) {
    if (int rc = check_plan(p)) return rc;
    if (!p->segments) return fail(DPSGD_ERR_INVALID_ARG, "the plan was not created with DPSGD_PLAN_SEGMENTS");
    if (int rc = check_ws(ws)) return rc;
    if (int rc = check_records(p, n_records)) return rc;
    if (!offsets) return fail(DPSGD_ERR_INVALID_ARG, "offsets is NULL");
    if (offsets[0] != 0) return fail(DPSGD_ERR_INVALID_ARG, "offsets[0] must be 0");
    for (int64_t r = 0; r < n_records; ++r) {
        const int64_t len = offsets[r + 1] - offsets[r];
        if (offsets[r + 1] < offsets[r] || len < 0 || len > p->T)
            return fail(DPSGD_ERR_INVALID_ARG, "segment lengths must be in [0, tokens] (non-decreasing offsets)");
    }
    hipError_t e = hipMemcpyAsync(static_cast<char*>(ws) + p->seg_off, offsets,
                                  (size_t)(n_records + 1) * sizeof(int64_t), hipMemcpyHostToDevice,
                                  (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "segment offsets copy");
    return DPSGD_OK;
}

int dpsgd_norms(const dpsgd_plan* p, int64_t n_rec, int32_t l0, int32_t l1, const void* const* A,
                const void* const* G, void* ws, void* stream) {
    if (int rc = check_plan(p)) return rc;
    if (int rc = check_records(p, n_rec)) return rc;
    if (int rc = check_range(p, l0, l1)) return rc;
    if (int rc = check_ws(ws)) return rc;
    if (l1 > l0 && (!A || !G)) return fail(DPSGD_ERR_INVALID_ARG, "A or G array is NULL");
    for (int l = l0; l < l1 && n_rec > 0; ++l)
        if (!A[l - l0] || !G[l - l0]) return fail(DPSGD_ERR_INVALID_ARG, "null A or G pointer");
    return do_norms(p, n_rec, l0, l1, A, G, ws, (hipStream_t)stream);
}

int dpsgd_clip(const dpsgd_plan* p, int64_t n_rec, double C, uint32_t flags, void* ws,
               float* norms_out, float* clip_out, void* stream) {
    if (int rc = check_plan(p)) return rc;
    if (int rc = check_records(p, n_rec)) return rc;
    if (int rc = check_c_sigma(C, 0.0, false)) return rc;
    if (int rc = check_ws(ws)) return rc;
    if (flags & ~(DPSGD_ACCUMULATE | DPSGD_NO_NOISE)) return fail(DPSGD_ERR_INVALID_ARG, "unknown flags");
    return do_clip(p, n_rec, C, flags, ws, norms_out, clip_out, (hipStream_t)stream);
}

int dpsgd_clipped_sum(const dpsgd_plan* p, int64_t n_rec, int32_t l0, int32_t l1,
                      const void* const* A, const void* const* G, const float* clip,
                      float* const* out, uint32_t flags, void* ws, void* stream) {
    if (int rc = check_plan(p)) return rc;
    if (int rc = check_records(p, n_rec)) return rc;
    if (int rc = check_range(p, l0, l1)) return rc;
    if (int rc = check_ws(ws)) return rc;
    if (flags & ~(DPSGD_ACCUMULATE | DPSGD_NO_NOISE)) return fail(DPSGD_ERR_INVALID_ARG, "unknown flags");
    if (l1 > l0 && !out) return fail(DPSGD_ERR_INVALID_ARG, "out array is NULL");
    for (int l = l0; l < l1; ++l) {
        if (!out[l - l0]) return fail(DPSGD_ERR_INVALID_ARG, "null out pointer");
        if (n_rec > 0 && p->layers[l].sum_mode == DPSGD_SUM_GEMM &&
            (!A || !G || !A[l - l0] || !G[l - l0]))
            return fail(DPSGD_ERR_INVALID_ARG, "null A or G pointer for a GEMM-sum layer");
    }
    return do_sum(p, n_rec, l0, l1, A, G, clip, out, flags, ws, (hipStream_t)stream);
}

int dpsgd_noise(const dpsgd_plan* p, float* const* out, double C, double sigma, uint64_t seed,
                uint64_t step, const void* ws, void* stream) {
    if (int rc = check_plan(p)) return rc;
    if (int rc = check_c_sigma(C, sigma, true)) return rc;
    if (ws && reinterpret_cast<uintptr_t>(ws) % kAlign) return fail(DPSGD_ERR_INVALID_ARG, "workspace is not 256-byte aligned");
    if (!out) return fail(DPSGD_ERR_INVALID_ARG, "out array is NULL");
    for (size_t l = 0; l < p->layers.size(); ++l)
        if (!out[l]) return fail(DPSGD_ERR_INVALID_ARG, "null out pointer");
    return do_noise(p, out, nullptr, 0.0, C, sigma, seed, step, ws, (hipStream_t)stream);
}

namespace {

// the descent step's arguments: one parameter buffer per layer, finite learning rate, finite
// normaliser > 0
int check_descent(const dpsgd_plan* p, float* const* params, double lr, double normalizer) {
    if (!params) return fail(DPSGD_ERR_INVALID_ARG, "params array is NULL");
    for (size_t l = 0; l < p->layers.size(); ++l)
        if (!params[l]) return fail(DPSGD_ERR_INVALID_ARG, "null params pointer");
    if (!std::isfinite(lr)) return fail(DPSGD_ERR_INVALID_ARG, "learning rate is not finite");
    if (!(normalizer > 0.0) || !std::isfinite(normalizer))
        return fail(DPSGD_ERR_INVALID_ARG, "normalizer must be finite and > 0");
    if (!std::isfinite((float)(lr / normalizer)))
        return fail(DPSGD_ERR_INVALID_ARG, "lr / normalizer overflows float32");
    return DPSGD_OK;
}

}  // namespace

int dpsgd_noise_descent(const dpsgd_plan* p, float* const* out, float* const* params, double C,
                        double sigma, uint64_t seed, uint64_t step, double lr, double normalizer,
                        const void* ws, void* stream) {
    if (int rc = check_plan(p)) return rc;
    if (int rc = check_c_sigma(C, sigma, true)) return rc;
    if (ws && reinterpret_cast<uintptr_t>(ws) % kAlign) return fail(DPSGD_ERR_INVALID_ARG, "workspace is not 256-byte aligned");
    if (!out) return fail(DPSGD_ERR_INVALID_ARG, "out array is NULL");
    for (size_t l = 0; l < p->layers.size(); ++l)
        if (!out[l]) return fail(DPSGD_ERR_INVALID_ARG, "null out pointer");
    if (int rc = check_descent(p, params, lr, normalizer)) return rc;
    return do_noise(p, out, params, lr / normalizer, C, sigma, seed, step, ws, (hipStream_t)stream);
}

namespace {

// every host-side check of dpsgd_step's arguments (plan and args non-null)
int check_step_args(const dpsgd_plan* p, const dpsgd_step_args* a) {
    if (int rc = check_records(p, a->n_records)) return rc;
    if (int rc = check_c_sigma(a->C, a->sigma, true)) return rc;
    if (int rc = check_ws(a->ws)) return rc;
    if (a->flags & ~(DPSGD_ACCUMULATE | DPSGD_NO_NOISE | DPSGD_DESCENT)) return fail(DPSGD_ERR_INVALID_ARG, "unknown flags");
    const bool descend = (a->flags & DPSGD_DESCENT) != 0;
    if (descend && (a->flags & DPSGD_NO_NOISE))
        return fail(DPSGD_ERR_INVALID_ARG, "DPSGD_DESCENT releases the sum: it needs the noise phase");
    if (descend)
        if (int rc = check_descent(p, a->params, a->lr, a->normalizer)) return rc;
    const int L = (int)p->layers.size();
    if (!a->out) return fail(DPSGD_ERR_INVALID_ARG, "out array is NULL");
    if (a->n_records > 0 && (!a->A || !a->G)) return fail(DPSGD_ERR_INVALID_ARG, "A or G array is NULL");
    for (int l = 0; l < L; ++l) {
        if (!a->out[l]) return fail(DPSGD_ERR_INVALID_ARG, "null out pointer");
        if (a->n_records > 0 && (!a->A[l] || !a->G[l])) return fail(DPSGD_ERR_INVALID_ARG, "null A or G pointer");
    }
    return DPSGD_OK;
}

// the step's launches (arguments already checked)
int run_step(const dpsgd_plan* p, const dpsgd_step_args* a, hipStream_t s) {
    const bool descend = (a->flags & DPSGD_DESCENT) != 0;
    float* const* params = descend ? a->params : nullptr;
    const double descent = descend ? a->lr / a->normalizer : 0.0;
    const int L = (int)p->layers.size();
    if (int rc = do_norms(p, a->n_records, 0, L, a->A, a->G, a->ws, s)) return rc;
    if (a->n_records > 0 && all_stored(p))
        return do_finalize(p, a->n_records, a->C, a->sigma, a->seed, a->step, a->flags, a->ws,
                           a->out, a->norms_out, a->clip_out, params, descent, s);
    if (int rc = do_clip(p, a->n_records, a->C, a->flags, a->ws, a->norms_out, a->clip_out, s)) return rc;
    if (int rc = do_sum(p, a->n_records, 0, L, a->A, a->G, nullptr, a->out, a->flags, a->ws, s)) return rc;
    if (!(a->flags & DPSGD_NO_NOISE))
        if (int rc = do_noise(p, a->out, params, descent, a->C, a->sigma, a->seed, a->step, a->ws, s)) return rc;
    return DPSGD_OK;
}

}  // namespace

int dpsgd_step(const dpsgd_plan* p, const dpsgd_step_args* a, void* stream) {
    if (int rc = check_plan(p)) return rc;
    if (!a) return fail(DPSGD_ERR_INVALID_ARG, "args is NULL");
    if (int rc = check_step_args(p, a)) return rc;
    return run_step(p, a, (hipStream_t)stream);
}

int dpsgd_step_noalloc(const dpsgd_plan* p, const dpsgd_step_args* a, uint32_t* status_out, void* stream) {
    if (int rc = check_plan(p)) return rc;
    if (!a) return fail(DPSGD_ERR_INVALID_ARG, "args is NULL");
    if (a->ws) return fail(DPSGD_ERR_INVALID_ARG, "dpsgd_step_noalloc uses the library's scratch: args->ws must be NULL");
    if (p->segments)
        return fail(DPSGD_ERR_INVALID_ARG, "segment plans need their offsets in a caller workspace (dpsgd_ws_segments)");
    if (p->ws_bytes > kScratchBytes)
        return fail(DPSGD_ERR_INVALID_ARG, "the plan's workspace (" + std::to_string(p->ws_bytes) +
                                               " bytes) exceeds the library's scratch of " +
                                               std::to_string(kScratchBytes) + " bytes");
    if (status_out && reinterpret_cast<uintptr_t>(status_out) % 4)
        return fail(DPSGD_ERR_INVALID_ARG, "status_out must be 4-byte aligned");
    // the same host checks as dpsgd_step, on a copy of the arguments that names a placeholder
    // workspace, so that every argument error is returned before the scratch is looked up
    dpsgd_step_args b = *a;
    b.ws = reinterpret_cast<void*>(kAlign);
    if (int rc = check_step_args(p, &b)) return rc;
    void* scratch = nullptr;
    hipError_t e = scratch_pointer(&scratch);
    if (e != hipSuccess) return hip_fail(e, "scratch address lookup");
    b.ws = scratch;
    hipStream_t s = (hipStream_t)stream;
    if (int rc = run_step(p, &b, s)) return rc;
    if (status_out) {
        e = launch_status_copy(ws_status(scratch, p), status_out, s);
        if (e != hipSuccess) return hip_fail(e, "status copy launch");
    }
    return DPSGD_OK;
}

int dpsgd_status(const dpsgd_plan* p, const void* ws, void* stream) {
    if (int rc = check_plan(p)) return rc;
    if (int rc = check_ws(ws)) return rc;
    uint32_t v = 0;
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = hipMemcpyAsync(&v, static_cast<const char*>(ws) + p->status_off, 4, hipMemcpyDeviceToHost, s);
    if (e != hipSuccess) return hip_fail(e, "status copy");
    e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "stream synchronize");
    return v ? DPSGD_ERR_NONFINITE : DPSGD_OK;
}

int dpsgd_layer_norm2(const dpsgd_plan* p, int64_t n_rec, int32_t l0, int32_t l1, const void* ws,
                      float* out, void* stream) {
    if (int rc = check_plan(p)) return rc;
    if (int rc = check_records(p, n_rec)) return rc;
    if (int rc = check_range(p, l0, l1)) return rc;
    if (int rc = check_ws(ws)) return rc;
    if (!out) return fail(DPSGD_ERR_INVALID_ARG, "out is NULL");
    for (int b = l0; b < l1; b += kMaxLaunchLayers) {
        const int e_ = std::min(l1, b + kMaxLaunchLayers);
        LayerNormArgs a;
        std::memset(&a, 0, sizeof(a));
        a.parts = reinterpret_cast<const float*>(static_cast<const char*>(ws) + p->parts_off);
        a.parts_stride = p->parts_total;
        a.n_rec = n_rec;
        a.n_layers = e_ - b;
        for (int l = b; l < e_; ++l) {
            a.part_off[l - b] = (int32_t)p->layers[l].part_off;
            a.n_part[l - b] = (int32_t)p->layers[l].n_parts;
        }
        a.out = out + (int64_t)(b - l0) * n_rec;
        hipError_t e = launch_layer_norm2(a, (hipStream_t)stream);
        if (e != hipSuccess) return hip_fail(e, "layer norm launch");
    }
    return DPSGD_OK;
}

int dpsgd_hbm_read(const void* buf, int64_t bytes, uint32_t* sink, void* stream) {
    if (!buf || !sink) return fail(DPSGD_ERR_INVALID_ARG, "buf or sink is NULL");
    if (bytes <= 0 || bytes % 16 != 0) return fail(DPSGD_ERR_INVALID_ARG, "bytes must be a positive multiple of 16");
    if (!ptr_aligned16(buf)) return fail(DPSGD_ERR_INVALID_ARG, "buf must be 16-byte aligned");
    hipError_t e = dpsgd::launch_hbm_read(buf, bytes, sink, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "hbm_read launch");
    return DPSGD_OK;
}

int dpsgd_philox_raw(uint64_t seed, uint64_t step, uint64_t first_block, uint64_t n_blocks,
                     uint32_t* dev_out, void* stream) {
    if (n_blocks > 0 && !dev_out) return fail(DPSGD_ERR_INVALID_ARG, "dev_out is NULL");
    if (n_blocks > (1ull << 40)) return fail(DPSGD_ERR_INVALID_ARG, "n_blocks too large");
    if (first_block + n_blocks < first_block) return fail(DPSGD_ERR_INVALID_ARG, "block range wraps");
    hipError_t e = launch_philox_raw(seed, step, first_block, n_blocks, dev_out, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "philox launch");
    return DPSGD_OK;
}

int64_t dpsgd_poisson_ws_bytes(int64_t population) {
    if (population < 0) return -1;
    return std::max<int64_t>(16, sample_ws_bytes(population));
}

int dpsgd_poisson_sample(uint64_t seed, uint64_t step, double q, int64_t population, uint8_t* mask,
                         int64_t* indices, int64_t* count, void* ws, void* stream) {
    if (!(q >= 0.0 && q <= 1.0)) return fail(DPSGD_ERR_INVALID_ARG, "q must be in [0, 1]");
    if (population < 0 || population > ((int64_t)1 << 36))
        return fail(DPSGD_ERR_INVALID_ARG, "population must be in [0, 2^36]");
    if (!count) return fail(DPSGD_ERR_INVALID_ARG, "count is NULL");
    if (population > 0 && (!indices || !ws)) return fail(DPSGD_ERR_INVALID_ARG, "indices or ws is NULL");
    if (reinterpret_cast<uintptr_t>(ws) % 8) return fail(DPSGD_ERR_INVALID_ARG, "ws is not 8-byte aligned");
    if (reinterpret_cast<uintptr_t>(mask) % 4) return fail(DPSGD_ERR_INVALID_ARG, "mask is not 4-byte aligned");
    const uint64_t thr = (uint64_t)std::floor(q * 4294967296.0);
    hipError_t e = launch_poisson_sample(seed, step, thr, population, mask, indices, count,
                                         static_cast<int64_t*>(ws), (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "poisson sample launch");
    return DPSGD_OK;
}

int dpsgd_rdp_sampled_gaussian(double q, double sigma, const double* orders, int32_t n_orders,
                               double* rdp_out) {
    if (!(q >= 0.0 && q <= 1.0)) return fail(DPSGD_ERR_INVALID_ARG, "q must be in [0, 1]");
    if (!(sigma > 0.0) || !std::isfinite(sigma)) return fail(DPSGD_ERR_INVALID_ARG, "sigma must be finite and > 0");
    if (n_orders < 1 || !orders || !rdp_out) return fail(DPSGD_ERR_INVALID_ARG, "orders or rdp_out missing");
    for (int k = 0; k < n_orders; ++k)
        if (!(orders[k] > 1.0) || !std::isfinite(orders[k]))
            return fail(DPSGD_ERR_INVALID_ARG, "orders must be finite and > 1");
    for (int k = 0; k < n_orders; ++k) rdp_out[k] = rdp_sampled_gaussian(q, sigma, orders[k]);
    return DPSGD_OK;
}

int dpsgd_rdp_to_epsilon(const double* orders, const double* rdp, int32_t n_orders, double delta,
                         int32_t tight, double* eps_out, double* order_out) {
    if (!(delta > 0.0 && delta < 1.0)) return fail(DPSGD_ERR_INVALID_ARG, "delta must be in (0, 1)");
    if (n_orders < 1 || !orders || !rdp || !eps_out) return fail(DPSGD_ERR_INVALID_ARG, "orders, rdp or eps_out missing");
    for (int k = 0; k < n_orders; ++k) {
        if (!(orders[k] > 1.0) || !std::isfinite(orders[k]))
            return fail(DPSGD_ERR_INVALID_ARG, "orders must be finite and > 1");
        if (!(rdp[k] >= 0.0)) return fail(DPSGD_ERR_INVALID_ARG, "rdp values must be >= 0");
    }
    *eps_out = rdp_epsilon(orders, rdp, n_orders, delta, tight != 0, order_out);
    return DPSGD_OK;
}

int dpsgd_gaussian_pair_delta(double eps, double mu, double* delta_out) {
    if (!(eps >= 0.0) || !std::isfinite(eps)) return fail(DPSGD_ERR_INVALID_ARG, "eps must be finite and >= 0");
    if (!(mu > 0.0) || !std::isfinite(mu)) return fail(DPSGD_ERR_INVALID_ARG, "mu must be finite and > 0");
    if (!delta_out) return fail(DPSGD_ERR_INVALID_ARG, "delta_out is NULL");
    *delta_out = gaussian_pair_delta(eps, mu);
    return DPSGD_OK;
}

int dpsgd_gaussian_pair_epsilon(double delta, double mu, double* eps_out) {
    if (!(delta > 0.0 && delta < 1.0)) return fail(DPSGD_ERR_INVALID_ARG, "delta must be in (0, 1)");
    if (!(mu > 0.0) || !std::isfinite(mu)) return fail(DPSGD_ERR_INVALID_ARG, "mu must be finite and > 0");
    if (!eps_out) return fail(DPSGD_ERR_INVALID_ARG, "eps_out is NULL");
    *eps_out = gaussian_pair_epsilon(delta, mu);
    return DPSGD_OK;
}

// ---------------------------------------------------------------- record-owned INT8 forward

struct dpsgd_i8_plan : I8PlanImpl {};

int64_t dpsgd_i8_pitch(int64_t k) { return k >= 1 && k <= kI8MaxKW * 32 ? i8_pitch(k) : 0; }

int dpsgd_i8_plan_create(int64_t max_rows, int64_t max_records, int64_t max_k, dpsgd_i8_plan** out,
                         size_t* ws_bytes) {
    if (!out || !ws_bytes) return fail(DPSGD_ERR_INVALID_ARG, "out or ws_bytes is NULL");
    *out = nullptr;
    if (max_rows < 0 || max_records < 1 || max_k < 1 || max_k > kI8MaxKW * 32)
        return fail(DPSGD_ERR_INVALID_ARG, "need max_rows >= 0, max_records >= 1, 1 <= max_k <= 32768");
    const int64_t kp = i8_pitch(max_k), kw = (max_k + 31) / 32;
    if (max_rows * kp >= ((int64_t)1 << 31))
        return fail(DPSGD_ERR_INVALID_ARG, "max_rows * pitch(max_k) must be below 2^31 bytes");
    if (max_records > ((int64_t)1 << 31) / kw)
        return fail(DPSGD_ERR_INVALID_ARG, "max_records too large");
    dpsgd_i8_plan* p = new (std::nothrow) dpsgd_i8_plan();
    if (!p) return fail(DPSGD_ERR_INVALID_ARG, "out of host memory");
    p->max_rows = max_rows;
    p->max_records = max_records;
    p->max_k = max_k;
    p->kp = kp;
    p->kw = kw;
    int64_t off = 0;
    p->off_offsets = off;
    off = align_up(off + 2 * (max_records + 1) * 8);
    p->off_own = off;
    off = align_up(off + max_rows * 4);
    p->off_s = off;
    off = align_up(off + max_rows * 4);
    p->off_omask = off;
    off = align_up(off + max_records * kw * 4);
    p->off_pmask = off;
    off = align_up(off + i8_scan_blocks(max_rows, max_records) * kw * 4);
    p->off_q = off;
    off = align_up(off + max_rows * kp);
    p->ws_bytes = off;
    *out = p;
    *ws_bytes = (size_t)off;
    return DPSGD_OK;
}

void dpsgd_i8_plan_destroy(dpsgd_i8_plan* p) { delete p; }

int dpsgd_i8_set_records(const dpsgd_i8_plan* p, void* ws, const int64_t* offsets, int64_t n_records,
                         void* stream) {
    if (!p) return fail(DPSGD_ERR_INVALID_ARG, "plan is NULL");
    if (!ws || reinterpret_cast<uintptr_t>(ws) % 256) return fail(DPSGD_ERR_INVALID_ARG, "ws is NULL or not 256-byte aligned");
    if (n_records < 1 || n_records > p->max_records) return fail(DPSGD_ERR_INVALID_ARG, "n_records must be in [1, max_records]");
    if (!offsets) return fail(DPSGD_ERR_INVALID_ARG, "offsets is NULL");
    if (offsets[0] != 0) return fail(DPSGD_ERR_INVALID_ARG, "offsets[0] must be 0");
    for (int64_t r = 0; r < n_records; ++r)
        if (offsets[r + 1] < offsets[r]) return fail(DPSGD_ERR_INVALID_ARG, "offsets must be non-decreasing");
    if (offsets[n_records] > p->max_rows) return fail(DPSGD_ERR_INVALID_ARG, "offsets[n_records] exceeds max_rows");
    // row offsets, then the scan's block offsets (max(1, ceil(len / 16)) blocks per record)
    std::vector<int64_t> h(2 * (size_t)(n_records + 1));
    for (int64_t r = 0; r <= n_records; ++r) h[r] = offsets[r];
    int64_t b = 0;
    for (int64_t r = 0; r < n_records; ++r) {
        h[n_records + 1 + r] = b;
        b += std::max<int64_t>(1, (offsets[r + 1] - offsets[r] + 15) / 16);
    }
    h[2 * n_records + 1] = b;
    char* w = static_cast<char*>(ws);
    hipError_t e = hipMemcpyAsync(w + p->off_offsets, h.data(), h.size() * sizeof(int64_t),
                                  hipMemcpyHostToDevice, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "record offsets copy");
    return DPSGD_OK;
}

int dpsgd_i8_quantize_weight(const uint16_t* w, int64_t n_out, int64_t k, int8_t* wq, float* w_scale,
                             void* stream) {
    if (k < 1 || k > kI8MaxKW * 32) return fail(DPSGD_ERR_INVALID_ARG, "k must be in [1, 32768]");
    if (n_out < 0) return fail(DPSGD_ERR_INVALID_ARG, "n_out must be >= 0");
    if (n_out > 0 && (!w || !wq || !w_scale)) return fail(DPSGD_ERR_INVALID_ARG, "null pointer");
    hipError_t e = launch_i8_weight(w, n_out, k, i8_pitch(k), wq, w_scale, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "weight quantisation launch");
    return DPSGD_OK;
}

namespace {

int i8_args(const dpsgd_i8_plan* p, void* ws, int64_t n_rows, int64_t n_records, int64_t k,
            I8Args& a) {
    if (!p) return fail(DPSGD_ERR_INVALID_ARG, "plan is NULL");
    if (!ws || reinterpret_cast<uintptr_t>(ws) % 256) return fail(DPSGD_ERR_INVALID_ARG, "ws is NULL or not 256-byte aligned");
    if (n_rows < 0 || n_rows > p->max_rows) return fail(DPSGD_ERR_INVALID_ARG, "n_rows must be in [0, max_rows]");
    if (n_records < 1 || n_records > p->max_records) return fail(DPSGD_ERR_INVALID_ARG, "n_records must be in [1, max_records]");
    if (k < 1 || k > p->max_k) return fail(DPSGD_ERR_INVALID_ARG, "k must be in [1, max_k]");
    char* w = static_cast<char*>(ws);
    a = I8Args{};
    a.n = n_rows;
    a.K = k;
    a.Kp = i8_pitch(k);
    a.KW = (k + 31) / 32;
    a.n_rec = n_records;
    a.offsets = reinterpret_cast<const int64_t*>(w + p->off_offsets);
    a.own = reinterpret_cast<int32_t*>(w + p->off_own);
    a.s = reinterpret_cast<float*>(w + p->off_s);
    a.omask = reinterpret_cast<uint32_t*>(w + p->off_omask);
    a.pmask = reinterpret_cast<uint32_t*>(w + p->off_pmask);
    a.Q = reinterpret_cast<int8_t*>(w + p->off_q);
    return DPSGD_OK;
}

}  // namespace

namespace {

int i8_check_a(const I8Args& a, const uint16_t* a_in, float tau) {
    if (std::isnan(tau)) return fail(DPSGD_ERR_INVALID_ARG, "tau is NaN");
    if (a.n > 0 && !a_in) return fail(DPSGD_ERR_INVALID_ARG, "a is NULL");
    return DPSGD_OK;
}

int i8_check_w(I8Args& a, const int8_t* wq, const float* w_scale, int64_t n_out, uint16_t* y) {
    if (n_out < 0) return fail(DPSGD_ERR_INVALID_ARG, "n_out must be >= 0");
    if (n_out * a.Kp >= ((int64_t)1 << 31)) return fail(DPSGD_ERR_INVALID_ARG, "n_out * pitch(k) must be below 2^31 bytes");
    if (n_out > 0 && (!wq || !w_scale)) return fail(DPSGD_ERR_INVALID_ARG, "wq or w_scale is NULL");
    if (a.n > 0 && n_out > 0 && !y) return fail(DPSGD_ERR_INVALID_ARG, "y is NULL");
    if (reinterpret_cast<uintptr_t>(wq) % 16) return fail(DPSGD_ERR_INVALID_ARG, "wq must be 16-byte aligned");
    a.Wq = wq;
    a.sW = w_scale;
    a.N = n_out;
    a.Y = y;
    a.y_vec = (n_out % 4 == 0 && reinterpret_cast<uintptr_t>(y) % 8 == 0) ? 1 : 0;
    return DPSGD_OK;
}

void i8_set_a(I8Args& a, const uint16_t* a_in, float tau) {
    a.A = a_in;
    a.tau = tau;
    a.tau_on = (tau > 0.f && !std::isinf(tau)) ? 1 : 0;
    a.a_vec = (a.K % 8 == 0 && reinterpret_cast<uintptr_t>(a_in) % 16 == 0) ? 1 : 0;
}

}  // namespace

int dpsgd_i8_route(const dpsgd_i8_plan* p, void* ws, int64_t n_rows, int64_t n_records,
                   const uint16_t* a_in, int64_t k, float tau, void* stream) {
    I8Args a;
    if (int rc = i8_args(p, ws, n_rows, n_records, k, a)) return rc;
    if (int rc = i8_check_a(a, a_in, tau)) return rc;
    i8_set_a(a, a_in, tau);
    hipError_t e = launch_i8_route(a, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "int8 routing launch");
    return DPSGD_OK;
}

int dpsgd_i8_matmul(const dpsgd_i8_plan* p, void* ws, int64_t n_rows, int64_t n_records,
                    const uint16_t* a_in, int64_t k, const int8_t* wq, const float* w_scale,
                    int64_t n_out, uint16_t* y, void* stream) {
    I8Args a;
    if (int rc = i8_args(p, ws, n_rows, n_records, k, a)) return rc;
    if (int rc = i8_check_a(a, a_in, 6.0f)) return rc;
    if (int rc = i8_check_w(a, wq, w_scale, n_out, y)) return rc;
    i8_set_a(a, a_in, 6.0f);
    hipError_t e = launch_i8_gemm(a, i8_tiles(n_rows, n_out, 1) >= 128 ? 1 : 0, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "int8 gemm launch");
    return DPSGD_OK;
}

int dpsgd_i8_forward(const dpsgd_i8_plan* p, void* ws, int64_t n_rows, int64_t n_records,
                     const uint16_t* a_in, int64_t k, const int8_t* wq, const float* w_scale,
                     int64_t n_out, float tau, uint16_t* y, void* stream) {
    I8Args a;
    if (int rc = i8_args(p, ws, n_rows, n_records, k, a)) return rc;
    if (int rc = i8_check_a(a, a_in, tau)) return rc;
    if (int rc = i8_check_w(a, wq, w_scale, n_out, y)) return rc;
    i8_set_a(a, a_in, tau);
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = launch_i8_route(a, s);
    if (e != hipSuccess) return hip_fail(e, "int8 routing launch");
    e = launch_i8_gemm(a, i8_tiles(n_rows, n_out, 1) >= 128 ? 1 : 0, s);
    if (e != hipSuccess) return hip_fail(e, "int8 gemm launch");
    return DPSGD_OK;
}

int dpsgd_i8_intermediates(const dpsgd_i8_plan* p, const void* ws, int64_t n_rows, int64_t n_records,
                           int64_t k, int8_t* q, float* row_scale, uint32_t* outlier_mask,
                           int32_t* owner, void* stream) {
    I8Args a;
    if (int rc = i8_args(p, const_cast<void*>(ws), n_rows, n_records, k, a)) return rc;
    hipStream_t s = (hipStream_t)stream;
    struct Part { void* dst; const void* src; int64_t bytes; } parts[] = {
        {q, a.Q, n_rows * a.Kp},
        {row_scale, a.s, n_rows * 4},
        {outlier_mask, a.omask, n_records * a.KW * 4},
        {owner, a.own, n_rows * 4},
    };
    for (const Part& pt : parts) {
        if (!pt.dst || pt.bytes == 0) continue;
        hipError_t e = hipMemcpyAsync(pt.dst, pt.src, (size_t)pt.bytes, hipMemcpyDeviceToDevice, s);
        if (e != hipSuccess) return hip_fail(e, "intermediates copy");
    }
    return DPSGD_OK;
}


const char* dpsgd_error_string(int code) {
    switch (code) {
        case DPSGD_OK: return "ok";
        case DPSGD_ERR_INVALID_ARG: return "invalid argument";
        case DPSGD_ERR_UNSUPPORTED: return "unsupported dtype or policy";
        case DPSGD_ERR_NONFINITE: return "nonfinite per-record norm: clipped sum and noise skipped";
        case DPSGD_ERR_HIP: return "HIP runtime error";
        default: return "unknown status code";
    }
}

const char* dpsgd_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
