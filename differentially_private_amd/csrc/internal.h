// Internal interface between the host API (dpsgd_api.cpp) and the kernel
// translation units.  Kernel-argument structs are passed by value, so every
// per-layer pointer travels in the kernarg segment (no device-side tables).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dpsgd {

constexpr int kMaxLaunchLayers = 48;  // per-launch layer descriptors (kernarg <= 4 KB)

enum Dtype : int32_t { kF32 = 0, kBF16 = 1 };

// Tile decomposition of one layer on the direct path.  X is the operand whose
// columns are streamed 128 at a time (the larger of d_in / d_out), Y the other
// one, whose columns form 16*MB-row MFMA blocks.
struct DirectLayer {
    const void* X;      // [n_rec, T, dX]
    const void* Y;      // [n_rec, T, dY]
    float* P;           // NORM+STORE: per-record gradient blocks [rec][d_in*d_out]; SUM: destination
    int32_t dX, dY;
    int32_t x_is_in;    // 1: X = A (d_in), Y = G (d_out); 0: X = G, Y = A
    int32_t tiles_x;    // ceil(dX / 128)
    int32_t tiles_y;    // ceil(dY / (16*MB))
    int32_t wg_x;       // ceil(tiles_x / waves per workgroup)
    int32_t part_off;   // first norm partial of this layer
    int32_t vec_x;      // X rows are 16-byte aligned (vector loads allowed)
    int64_t d_out;      // for output addressing
    int64_t split_stride;  // SUM: floats between split partial blocks (0 = write `P` directly)
};

struct DirectArgs {
    DirectLayer L[kMaxLaunchLayers];
    int32_t n_layers;
    int32_t accumulate;        // SUM with direct write: out += tile
    int32_t wpb;               // wavefronts per workgroup (1..8), one column tile each
    int32_t pad;
    int64_t T;
    int64_t n_rec;
    int64_t parts_stride;      // partials per record (record-major partial array)
    float* parts;
    const float* clip;         // SUM: per-record factors
    int64_t rec_per_split;     // SUM
    const uint32_t* status;    // SUM: skip while nonzero
    const int64_t* seg;        // variable-length records: rows [seg[r], seg[r + 1]) (null: r T ..)
};

struct GramLayer {
    const void* A;     // [n_rec, T, d_in]
    const void* G;     // [n_rec, T, d_out]
    int32_t d_in, d_out;
    int32_t part_off;
    int32_t vec_a, vec_g;
    int32_t pad;
};

struct GramArgs {
    GramLayer L[kMaxLaunchLayers];
    int32_t n_layers;
    int32_t nb;        // 64-row blocks of T
    int32_t n_pairs;   // nb (nb + 1) / 2 upper-triangle block pairs
    int32_t pad;
    int64_t T;
    int64_t n_rec;
    int64_t parts_stride;
    float* parts;
    const int64_t* seg;        // variable-length records: rows [seg[r], seg[r + 1]) (null: r T ..)
};

struct ClipArgs {
    const float* parts;
    int64_t parts_stride;
    int64_t n_parts;
    int64_t n_rec;
    double C;
    float* n_ws;
    float* c_ws;
    float* n_user;
    float* c_user;
    uint32_t* status;
    int32_t accumulate;
};

// Order of a STORED layer's per-record gradient block in the workspace.  When d_out is a
// multiple of 4 (stored_permuted), the norm kernel keeps the 128 X indices of every whole X tile
// (n0 + 128 <= dX) in the order in which its store instructions produce them, so that each
// instruction writes consecutive addresses instead of sixteen pieces spread over the tile (on the
// 7B-shaped LoRA batch, 2.9 GB of blocks per norm launch by non-temporal stores, the HBM writes
// counted went from 1.35 to 1.00 times the blocks' bytes and the launch from 8.40 to 8.08 ms): X index
// n0 + dcol(c, i) of lane column c and accumulator i, where the tile engine keeps it, sits at
// n0 + 16 i + c (X along d_in: whole rows of d_out move) or, for bf16 tiles with X along d_out, the
// 4-column chunk n0 + dcol(c, 4q) sits at n0 + 64 q + 4 c (fp32 tiles already write those chunks
// in order).  The last, partial X tile keeps the natural order.  Readers map each stored flat
// position back to the element's index with stored_logical().
__host__ __device__ inline bool stored_permuted(int64_t d_out) { return d_out % 4 == 0; }

struct StoredMap {
    int32_t mode;   // 0 natural; 1 rows, bf16 tiles; 2 rows, fp32 tiles; 3 4-column chunks, bf16 tiles
    int32_t full;   // X indices inside whole 128-wide tiles (a multiple of 128)
    int64_t d_out;
};

struct ReduceLayer {
    const float* src;   // SPLIT: [n_splits][n]; STORED: [n_rec][n]
    float* out;         // [n]
    int64_t n;          // elements (d_in * d_out)
    StoredMap map;      // order of STORED blocks (mode 0 for split partials)
};

struct ReduceArgs {
    ReduceLayer L[kMaxLaunchLayers];
    int32_t n_layers;
    int32_t accumulate;
    int64_t n_src;       // splits or records
    const float* clip;   // STORED: weights per record; SPLIT: null
    const uint32_t* status;
    int64_t max_n4;      // max over layers of ceil(n / 4)
};

// One noise launch covers up to kNoiseMaxPieces pieces of layers (a layer of more than
// kNoisePieceMax elements is cut into pieces of that size), each with its out pointer and, for the
// descent step, its parameter pointer, so that a whole LoRA plan goes out in one launch.
constexpr int kNoiseMaxPieces = 320;                     // without the descent step
constexpr int kNoiseMaxPiecesDescent = 160;              // with it (two pointers per piece)
constexpr int64_t kNoisePieceMax = (int64_t)1 << 30;     // elements per piece (a multiple of 4)
struct NoiseArgs {
    int64_t base;                      // flat index of the launch's first element
    uint64_t seed, step;
    const uint32_t* status;
    float scale;                       // sigma * C
    float descent;                     // lr / normalizer (with params)
    int32_t n_pieces;
    int32_t with_params;               // ptr[n_pieces + k]: parameters of piece k
    uint32_t off[kNoiseMaxPieces + 1]; // flat offsets relative to base, off[0] = 0
    float* ptr[kNoiseMaxPieces];       // out pointers of the pieces, then (with_params) theirs
};
static_assert(sizeof(NoiseArgs) <= 4096, "kernel arguments of the noise launch exceed 4 KB");

constexpr int kFinalMaxLayers = 48;
constexpr int kFinalMaxRecords = 1024;      // records whose factors a block recomputes itself
constexpr int64_t kFinalMaxClipWork = 65536;  // records x partials a block reduces itself

// Fused tail of a step whose layers all keep their per-record gradient blocks:
// clip factors (recomputed per block from the partials, or read), the weighted
// sum over records and the noise, in one pass over the flat parameter index.
struct FinalizeArgs {
    float* out[kFinalMaxLayers];
    const float* src[kFinalMaxLayers];     // stored gradient blocks [max_records][n_l]
    int64_t off[kFinalMaxLayers + 1];      // flat offsets of the launch's layers
    int32_t n_layers;
    int32_t accumulate;
    int32_t noise;
    int32_t pad;
    int64_t n_rec;
    uint64_t seed, step;
    float scale;                           // sigma * C
    // clip factors computed inside (first variant) ...
    const float* parts;
    int64_t parts_stride;
    int64_t n_parts;
    double C;
    float* n_ws;
    float* c_ws;
    float* n_user;
    float* c_user;
    uint32_t* status;
    // ... or read (second variant)
    const float* clip;
    // descent step after the noise: params[l] -= descent * out[l] (null: none)
    float* params[kFinalMaxLayers];
    float descent;
    StoredMap map[kFinalMaxLayers];        // order of each layer's stored blocks
};

constexpr int kDenseMaxLayers = 32;

// Dense clipped sum (bf16, both dimensions wide): 256 x 128 output tiles.
struct DenseSumLayer {
    const void* A;       // [n_rec, T, d_in]
    const void* G;       // [n_rec, T, d_out]
    float* out;          // [d_in, d_out] (used when split_stride == 0)
    float* split;        // [n_splits][d_in * d_out] split partials
    int32_t d_in, d_out;
    int32_t tiles_m, tiles_n;
    int32_t vec_a, vec_g;
    int64_t split_stride;
};

struct DenseSumArgs {
    DenseSumLayer L[kDenseMaxLayers];
    int32_t n_layers;
    int32_t accumulate;
    int64_t T;
    int64_t n_rec;
    int64_t rec_per_split;
    const float* clip;
    const uint32_t* status;
};

struct LayerNormArgs {
    const float* parts;
    int64_t parts_stride;
    int64_t n_rec;
    int32_t n_layers;
    int32_t pad;
    int32_t part_off[kMaxLaunchLayers];
    int32_t n_part[kMaxLaunchLayers];
    float* out;
};

static_assert(sizeof(DirectArgs) <= 4096 && sizeof(GramArgs) <= 4096 && sizeof(ReduceArgs) <= 4096 &&
                  sizeof(FinalizeArgs) <= 4096 && sizeof(DenseSumArgs) <= 4096 &&
                  sizeof(LayerNormArgs) <= 4096,
              "kernel arguments travel by value and must stay under 4 KB");

// Size of the fixed device scratch that dpsgd_step_noalloc uses in place of a caller workspace.
constexpr int64_t kScratchBytes = (int64_t)64 << 20;

// ---- launchers (return hipError_t of the launch) ----
hipError_t launch_norm_direct(const DirectArgs& a, int dtype, int mb, int store, hipStream_t s);  // store: write the blocks
hipError_t launch_norm_gram(const GramArgs& a, int dtype, hipStream_t s);
hipError_t launch_clip(const ClipArgs& a, hipStream_t s);
hipError_t launch_sum_direct(const DirectArgs& a, int dtype, int mb, int n_splits, hipStream_t s);
hipError_t launch_reduce(const ReduceArgs& a, bool weighted, hipStream_t s);
hipError_t launch_noise(const NoiseArgs& a, hipStream_t s);
hipError_t launch_philox_raw(uint64_t seed, uint64_t step, uint64_t first_block, uint64_t n_blocks,
                             uint32_t* out, hipStream_t s);
hipError_t launch_layer_norm2(const LayerNormArgs& a, hipStream_t s);
hipError_t launch_status_clear(uint32_t* status, hipStream_t s);
hipError_t launch_finalize(const FinalizeArgs& a, bool clip_inside, hipStream_t s);
hipError_t launch_sum_dense(const DenseSumArgs& a, int n_splits, hipStream_t s);
// device address of this device's scratch (looked up once per device)
hipError_t scratch_pointer(void** out);
hipError_t launch_status_copy(const uint32_t* status, uint32_t* out, hipStream_t s);

// privacy accounting (host)
double rdp_sampled_gaussian(double q, double sigma, double alpha);
double rdp_epsilon(const double* orders, const double* rdp, int n, double delta, bool tight,
                   double* best_order);
double gaussian_pair_delta(double eps, double mu);
double gaussian_pair_epsilon(double delta, double mu);

// Poisson sampler: ws holds 2 * sample_wgs(n) int64 and the inclusion bits, sample_ws_bytes(n) in all
int64_t sample_wgs(int64_t n);
int64_t sample_ws_bytes(int64_t n);
hipError_t launch_poisson_sample(uint64_t seed, uint64_t step, uint64_t thr, int64_t n, uint8_t* mask,
                                 int64_t* indices, int64_t* count, int64_t* ws, hipStream_t s);

}  // namespace dpsgd
