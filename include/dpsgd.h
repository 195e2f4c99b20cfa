/*
 * dpsgd.h -- C ABI of the DP-SGD private-gradient step on one AMD Instinct
 * MI355X (gfx950) GPU.
 *
 * The step (Abadi et al. DP-SGD, restated in "Privacy-Preserving Machine
 * Learning", section "Differentially private stochastic gradient descent",
 * phases 2-4, and in "Sensitivity Inflation from Cross-Record Precision
 * Routing in Private Quantized Fine-Tuning", Sec. 2, Eqs. 2-3):
 *
 *   for each record i of the batch and each trainable linear layer l, with the
 *   layer's input activations A_l[i] (T x d_in) and output gradients
 *   G_l[i] (T x d_out), the record's gradient is P_{i,l} = A_l[i]^T G_l[i]
 *   (d_in x d_out, summed over the record's T tokens);
 *   n_i   = || (P_{i,1}, ..., P_{i,L}) ||_2        one norm over all layers
 *   c_i   = 1 if n_i <= C (also n_i = 0), else C / n_i
 *   S_l   = sum_i c_i P_{i,l}                     the clipped sum
 *   S~_l  = S_l + sigma * C * Z_l,  Z ~ N(0, I)    noise once per logical step
 *
 * n_i is computed without forming P_{i,l} ("ghost" norms): through the Gram
 * identity sum_{t,s} (a_t . a_s)(g_t . g_s) when T^2 < d_in * d_out, else from
 * tiles of P_{i,l} that never leave registers.  Z comes from Philox4x32-10
 * (Salmon et al., SC'11) keyed by the 64-bit seed, counter = (flat element
 * index / 4, step), and the Box-Muller transform; the library never divides
 * by the batch size (that belongs to the optimizer step, phase 5).
 *
 * Conventions for every entry point:
 *  - Device pointers point to memory on the current HIP device; `stream` is a
 *    hipStream_t (NULL = the default stream).  All launches are asynchronous on
 *    `stream` unless stated otherwise.
 *  - Host pointer arrays (A, G, out) are read during the call only.
 *  - The caller owns every buffer (inputs, outputs, workspace).  The library
 *    allocates no device memory and keeps no device state.
 *  - Argument errors are detected on the host before any launch and returned
 *    as DPSGD_ERR_INVALID_ARG / DPSGD_ERR_UNSUPPORTED; nothing is enqueued then.
 *    No C++ exception crosses this interface.  dpsgd_last_error() gives a
 *    thread-local text for the last failure.
 *  - Records: A_l is [n_records, T, d_in] and G_l is [n_records, T, d_out],
 *    row-major, contiguous, in the plan's dtype.  A record owns its T rows in
 *    every layer; padding tokens are zero rows of G.  Any loss normaliser is
 *    already folded into G.
 *  - Outputs out_l are [d_in, d_out] row-major float32 (the transpose of the
 *    gradient of a weight stored d_out x d_in).
 */
#ifndef DPSGD_H
#define DPSGD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---- */
#define DPSGD_OK 0
#define DPSGD_ERR_INVALID_ARG (-1) /* bad pointer, size, C, sigma, layer range, flags */
#define DPSGD_ERR_UNSUPPORTED (-2) /* dtype or policy value not supported */
#define DPSGD_ERR_NONFINITE (-3)   /* a record's norm was NaN/Inf: sums and noise were skipped */
#define DPSGD_ERR_HIP (-4)         /* the HIP runtime reported an error (see dpsgd_last_error) */

/* ---- element types of A and G ---- */
#define DPSGD_DTYPE_F32 0
#define DPSGD_DTYPE_BF16 1

/* ---- per-layer norm path ---- */
#define DPSGD_PATH_AUTO 0   /* Gram iff T^2 < d_in * d_out (a tie takes the direct path) */
#define DPSGD_PATH_GRAM 1   /* force the Gram identity for every layer */
#define DPSGD_PATH_DIRECT 2 /* force per-record gradient tiles for every layer */

/* ---- clipped-sum strategy ---- */
#define DPSGD_SUM_AUTO 0   /* STORED where it moves fewer HBM bytes, else GEMM */
#define DPSGD_SUM_GEMM 1   /* S = A^T diag(c) G, re-reading A and G */
#define DPSGD_SUM_STORED 2 /* direct-path layers keep each record's gradient block in the
                              workspace during dpsgd_norms; the sum reads it back (Gram-path
                              layers fall back to GEMM) */

/* ---- flags ---- */
#define DPSGD_ACCUMULATE 1u /* add into out (and OR into the status) instead of overwriting */
#define DPSGD_NO_NOISE 2u   /* dpsgd_step: skip the noise phase */
#define DPSGD_DESCENT 4u    /* dpsgd_step: after the noise, the descent step on args->params */

/* Plan flag: records are variable-length segments of token rows, e.g. users
 * whose records' rows are concatenated ("Privacy-Preserving Machine Learning",
 * user-level clipping: a user's vector is the sum of its records' gradients,
 * A_u^T G_u over the concatenated rows, clipped as one).  Record r owns rows
 * [off[r], off[r + 1]) of A_l [rows, d_in] and G_l [rows, d_out]; `tokens` is
 * the longest segment; the offsets are set per workspace by dpsgd_ws_segments.
 * Such plans run the register kernels (no dense copy kernels). */
#define DPSGD_PLAN_SEGMENTS 1u

typedef struct dpsgd_layer_shape {
    int64_t d_in;
    int64_t d_out;
} dpsgd_layer_shape;

typedef struct dpsgd_plan_desc {
    int32_t n_layers;                /* >= 1 */
    const dpsgd_layer_shape* layers; /* n_layers shapes, in plan order (also the noise order) */
    int32_t dtype;                   /* DPSGD_DTYPE_*: one type for all A and G */
    int64_t max_records;             /* largest n_records of any call (>= 1) */
    int64_t tokens;                  /* T, tokens per record (>= 1) */
    int32_t path_policy;             /* DPSGD_PATH_* */
    int32_t sum_policy;              /* DPSGD_SUM_* */
    uint32_t flags;                  /* DPSGD_PLAN_SEGMENTS or 0 */
} dpsgd_plan_desc;

typedef struct dpsgd_plan dpsgd_plan; /* immutable host object */

typedef struct dpsgd_step_args {
    int64_t n_records;     /* 0 <= n_records <= max_records (0: empty batch, noise only) */
    const void* const* A;  /* n_layers device pointers, A_l [n_records, T, d_in] (segment plans: [rows, d_in]) */
    const void* const* G;  /* n_layers device pointers, G_l [n_records, T, d_out] (segment plans: [rows, d_out]) */
    float* const* out;     /* n_layers device pointers, out_l [d_in, d_out] float32 */
    void* ws;              /* device workspace of dpsgd_plan_create's ws_bytes (256-B aligned) */
    double C;              /* clipping bound, finite and > 0 */
    double sigma;          /* noise multiplier, finite and >= 0 */
    uint64_t seed;         /* Philox key */
    uint64_t step;         /* Philox counter words 2-3 (e.g. the logical step index) */
    uint32_t flags;        /* DPSGD_ACCUMULATE | DPSGD_NO_NOISE | DPSGD_DESCENT */
    float* norms_out;      /* optional device [n_records]: n_i */
    float* clip_out;       /* optional device [n_records]: c_i */
    /* DPSGD_DESCENT only (ignored otherwise): */
    float* const* params;  /* n_layers device pointers, theta_l [d_in, d_out] float32, updated in place */
    double lr;             /* learning rate eta, finite */
    double normalizer;     /* the fixed public normaliser L, finite and > 0 */
} dpsgd_step_args;

/* Build a plan: validate shapes, choose the path of every layer and lay out
 * the workspace.  Host only (no device call).  The plan describes the records
 * and layers of the clipped sum F(D) = sum_r clip(g_r) of "Sensitivity Inflation
 * from Cross-Record Precision Routing in Private Quantized Fine-Tuning", Sec. 2
 * Eqs. 2-3: every record's gradient g_r over all the plan's layers, one norm
 * per record ("Differential Privacy: DP-SGD, Privacy Budgets, and LLMs", the
 * combined norm of the concatenated per-example gradient).  *ws_bytes receives the size of
 * the device workspace every call with this plan needs.  Returns
 * DPSGD_ERR_INVALID_ARG for a null pointer, n_layers < 1, a dimension < 1,
 * max_records < 1, T < 1, or sizes whose products overflow 64 bits;
 * DPSGD_ERR_UNSUPPORTED for an unknown dtype or policy. */
int dpsgd_plan_create(const dpsgd_plan_desc* desc, dpsgd_plan** out, size_t* ws_bytes);

/* Free a plan (NULL is ignored). */
void dpsgd_plan_destroy(dpsgd_plan* plan);

/* Path (DPSGD_PATH_GRAM / _DIRECT) and sum strategy (DPSGD_SUM_GEMM / _STORED)
 * chosen for `layer`.  Host only. */
int dpsgd_plan_layer_info(const dpsgd_plan* plan, int32_t layer, int32_t* path, int32_t* sum_mode);

/* Total trainable parameters sum_l d_in * d_out (the flat noise index space). */
int64_t dpsgd_plan_num_params(const dpsgd_plan* plan);

/* Segment plans only: set the token-row offsets of the next n_records records
 * in `ws` (host array `offsets` of n_records + 1 entries: offsets[0] = 0,
 * non-decreasing, each segment at most the plan's `tokens` rows; copied
 * stream-ordered: pageable host memory is staged before the call returns and
 * may be reused at once, pinned host memory must stay unchanged until the
 * stream has passed the copy).  The following
 * dpsgd_norms / dpsgd_clipped_sum / dpsgd_step calls on this workspace must
 * use the same n_records.  Empty segments are allowed (norm 0, factor 1). */
int dpsgd_ws_segments(const dpsgd_plan* plan, void* ws, const int64_t* offsets, int64_t n_records,
                      void* stream);

/* Clear the workspace status word (a fill kernel, no memset node).  Needed only
 * before a dpsgd_noise with a workspace that no dpsgd_clip has touched yet. */
int dpsgd_ws_init(const dpsgd_plan* plan, void* ws, void* stream);

/* Phase 1 ("Privacy-Preserving Machine Learning", DP-SGD phase 2, computed
 * without per-record gradient tensors): per-record partial squared norms of
 * layers [l0, l1) into the workspace.  A and G hold (l1 - l0) device pointers,
 * entry k for layer l0 + k.  For layers whose sum strategy is STORED, each
 * record's gradient block is also written to the workspace.  Calls over
 * disjoint layer ranges may be issued in any order before dpsgd_clip
 * (layer-chunk streaming). */
int dpsgd_norms(const dpsgd_plan* plan, int64_t n_records, int32_t l0, int32_t l1,
                const void* const* A, const void* const* G, void* ws, void* stream);

/* Phase 2 (DP-SGD phase 3, g * min(1, C/||g||)): n_i and c_i from the partials
 * of all layers (fixed summation order: record i's results do not depend on the
 * other records, their number or i's position).  n_i^2 is the sum of the
 * partials, taken as 0 when rounding makes it negative (Gram-path records whose
 * token contributions nearly cancel), so n_i >= 0 and c_i is in (0, 1].  Sets
 * the status word to NONFINITE if some n_i^2, n_i or c_i is NaN/Inf (ORs into
 * it with DPSGD_ACCUMULATE).
 * norms_out / clip_out are optional device arrays of n_records floats. */
int dpsgd_clip(const dpsgd_plan* plan, int64_t n_records, double C, uint32_t flags, void* ws,
               float* norms_out, float* clip_out, void* stream);

/* Phase 3 (DP-SGD phase 4, sum of the clipped gradients; Eq. 3 F(D)): for
 * layers [l0, l1), out_l = sum_i c_i A_l[i]^T G_l[i] (or out_l += ... with
 * DPSGD_ACCUMULATE).  `clip` is a device array of n_records factors, or NULL
 * to use the factors of the last dpsgd_clip in `ws`.  For STORED layers the
 * gradient blocks written by the last dpsgd_norms are used and A_l/G_l may be
 * NULL.  Skipped on device (out untouched) while the status is NONFINITE. */
int dpsgd_clipped_sum(const dpsgd_plan* plan, int64_t n_records, int32_t l0, int32_t l1,
                      const void* const* A, const void* const* G, const float* clip,
                      float* const* out, uint32_t flags, void* ws, void* stream);

/* Phase 4 (DP-SGD phase 4, N(0, sigma^2 C^2 I) added once): out_l[e] +=
 * sigma * C * Z[off_l + e] over all layers (off_l = parameters of the layers
 * before l).  Z is a pure function of (seed, step, flat index).  ws may be NULL
 * (no status check); else the launch is skipped on device while the status is
 * NONFINITE. */
int dpsgd_noise(const dpsgd_plan* plan, float* const* out, double C, double sigma, uint64_t seed,
                uint64_t step, const void* ws, void* stream);

/* Phases 4-5 ("Privacy-Preserving Machine Learning", DP-SGD phases 4 and 5:
 * the noise, then the descent step theta <- theta - eta * g~ / L with L the
 * fixed public normaliser), in one pass over the flat parameter index:
 * out_l[e] += sigma * C * Z[off_l + e] as dpsgd_noise does, then
 * params_l[e] -= (lr / normalizer) * out_l[e] (fp32, lr / normalizer rounded
 * to fp32).  out keeps the noised sum.  params: one device pointer per layer,
 * [d_in, d_out] float32, overlapping no out buffer.  For virtual batching after
 * the last physical batch.  Skipped on device (out and params untouched) while
 * the status is NONFINITE (ws given). */
int dpsgd_noise_descent(const dpsgd_plan* plan, float* const* out, float* const* params, double C,
                        double sigma, uint64_t seed, uint64_t step, double lr, double normalizer,
                        const void* ws, void* stream);

/* The whole step: dpsgd_norms(all layers) -> dpsgd_clip -> dpsgd_clipped_sum
 * (all layers) -> dpsgd_noise unless DPSGD_NO_NOISE (dpsgd_noise_descent with
 * DPSGD_DESCENT).  DPSGD_DESCENT with DPSGD_NO_NOISE is an INVALID_ARG: the
 * update releases the sum, which must carry the noise.  Virtual batching: call
 * with DPSGD_NO_NOISE for every physical batch, DPSGD_ACCUMULATE for all but
 * the first, then dpsgd_noise (or dpsgd_noise_descent) once. */
int dpsgd_step(const dpsgd_plan* plan, const dpsgd_step_args* args, void* stream);

/* dpsgd_step for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same launches as dpsgd_step, with the workspace taken from a scratch area of
 * 64 MiB (67,108,864 bytes) that the library holds on each device it runs on
 * from the code object's load until the process ends.  args->ws must be NULL.
 * Returns DPSGD_ERR_INVALID_ARG, before any launch, for a plan whose ws_bytes
 * exceed 64 MiB or that was created with DPSGD_PLAN_SEGMENTS, and for every
 * argument error dpsgd_step reports.  status_out (optional device uint32,
 * 4-byte aligned) receives the step's status word after the step (0, or nonzero
 * when a norm was NaN/Inf and the sum and noise were skipped), written by a
 * one-thread kernel on `stream`.  Calls no allocating routine.  Every call on a
 * device shares that device's scratch and leaves its contents (partials,
 * factors, gradient blocks, status) for the next call: calls that overlap on one
 * device (other streams or threads) race.  With DPSGD_ACCUMULATE the status is
 * OR-ed with the previous call's, as in a virtual batch on one workspace; a call
 * without it resets the status. */
int dpsgd_step_noalloc(const dpsgd_plan* plan, const dpsgd_step_args* args, uint32_t* status_out,
                       void* stream);

/* Poisson sampling of a step's records ("Privacy-Preserving Machine Learning",
 * DP-SGD phase 1: each of `population` records included independently with
 * public probability q, 0 <= q <= 1).  Record i draws word i mod 4 of
 * Philox4x32-10 block 2^63 + floor(i / 4) (key = seed, counter words 2-3 =
 * step; the top bit keeps these words apart from the noise stream) and is
 * included iff that word < floor(q * 2^32).  Device outputs: `indices` (room
 * for `population` int64; the included records in increasing order), `count`
 * (one int64), optional `mask` (population bytes, 0/1, 4-byte aligned).  `ws`:
 * device scratch of dpsgd_poisson_ws_bytes(population) bytes, 8-byte aligned
 * (may be NULL when population is 0).  population <= 2^36. */
int64_t dpsgd_poisson_ws_bytes(int64_t population);
int dpsgd_poisson_sample(uint64_t seed, uint64_t step, double q, int64_t population, uint8_t* mask,
                         int64_t* indices, int64_t* count, void* ws, void* stream);

/* Privacy accounting, host only ("Privacy-Preserving Machine Learning",
 * section on privacy accounting: RDP bounds add over steps and convert to
 * (epsilon, delta)).  dpsgd_rdp_sampled_gaussian: per-step Renyi DP at each
 * order (> 1) of the Poisson-subsampled Gaussian mechanism, sampling
 * probability q in [0, 1], noise multiplier sigma > 0 (multiply by the number
 * of steps to compose; alpha / (2 sigma^2) at q = 1).  dpsgd_rdp_to_epsilon:
 * epsilon at delta in (0, 1), minimised over the orders, with the conservative
 * conversion rdp + log(1/delta) / (alpha - 1) (tight = 0) or the tighter
 * rdp + log((alpha - 1) / alpha) - (log delta + log alpha) / (alpha - 1)
 * (tight = 1); order_out (optional) receives the minimising order.
 * dpsgd_gaussian_pair_delta / _epsilon: Eq. 5 of "Sensitivity Inflation from
 * Cross-Record Precision Routing in Private Quantized Fine-Tuning" (Sec. 3.2),
 * delta(eps) = Phi(mu/2 - eps/mu) - e^eps Phi(-mu/2 - eps/mu) for a one-step
 * Gaussian release with mu = Delta / (sigma C) > 0, and its inverse. */
int dpsgd_rdp_sampled_gaussian(double q, double sigma, const double* orders, int32_t n_orders,
                               double* rdp_out);
int dpsgd_rdp_to_epsilon(const double* orders, const double* rdp, int32_t n_orders, double delta,
                         int32_t tight, double* eps_out, double* order_out);
int dpsgd_gaussian_pair_delta(double eps, double mu, double* delta_out);
int dpsgd_gaussian_pair_epsilon(double delta, double mu, double* eps_out);

/* ---- Record-owned LLM.int8 forward of a frozen linear layer ----
 * ("Sensitivity Inflation from Cross-Record Precision Routing in Private
 * Quantized Fine-Tuning", Sec. 4.2, Eq. 6 and Algorithm 1; LLM.int8 as its
 * Sec. 2 describes it.)  The upstream producer of a layer's activations on a
 * quantised frozen backbone.  For n activation rows A (fp16, n x k, row-major,
 * contiguous) owned by records (record r owns rows [offsets[r], offsets[r+1])):
 *   M_ij = |A_ij| >= tau;  O_r = columns where a row of record r has M true;
 *   s_i  = max |A_ij| over the entries with M_ij false (0 if none);
 *   Q_ij = round(127 A_ij / s_i), ties to even, 0 if j in O_owner(i) or s_i = 0;
 *   Y_i  = fp16(dq16 + corr16), where
 *     dq16   = fp16(fl(fl(float(Q_i . Wq_o) * fl(s_i/127)) * fl(s_W,o/127))),
 *     corr16 = fp16(sum over j in O_owner(i), ascending, in fp32, of
 *              A_ij * What_oj), What_oj = fp16(fl(float(Wq_oj) * fl(s_W,o/127))).
 * Every row multiplies only its own record's outlier columns, so a record's
 * output does not depend on the other records of the physical batch.  Batched
 * LLM.int8 (one outlier set for all rows) is the case of a single record
 * spanning all rows.  tau <= 0 or +inf: no outlier path (threshold zero).
 * Non-finite activations give unspecified (but in-bounds) results.
 *
 * Weights: Wq is [n_out, pitch(k)] int8 (row-wise codes, zero past k) with one
 * scale s_W per output feature (the row's max |w|), as written by
 * dpsgd_i8_quantize_weight.  Y is [n, n_out] fp16, row-major.  The plan is a
 * host object with the capacities; its workspace (device, 256-byte aligned,
 * dpsgd_i8_plan_create's ws_bytes) holds the record offsets, owners, row
 * scales, outlier masks and codes of the current batch.  Argument errors are
 * returned before any launch. */
typedef struct dpsgd_i8_plan dpsgd_i8_plan;

/* Bytes per INT8 code row: k rounded up to a multiple of 64 (0 unless
 * 1 <= k <= 32768). */
int64_t dpsgd_i8_pitch(int64_t k);

/* Capacities: at most max_rows activation rows (max_rows * pitch(max_k)
 * < 2^31), max_records >= 1 records, 1 <= max_k <= 32768 columns. */
int dpsgd_i8_plan_create(int64_t max_rows, int64_t max_records, int64_t max_k, dpsgd_i8_plan** out,
                         size_t* ws_bytes);
void dpsgd_i8_plan_destroy(dpsgd_i8_plan* plan);

/* Row-wise quantisation of a frozen fp16 weight W [n_out, k] (device, row-major):
 * w_scale[o] = max_j |W_oj| (float32), wq[o][j] = round(127 W_oj / w_scale[o])
 * (ties to even, 0 where the scale is 0; zero for j in [k, pitch(k))).
 * wq: device, n_out x pitch(k) bytes, 16-byte aligned. */
int dpsgd_i8_quantize_weight(const uint16_t* w, int64_t n_out, int64_t k, int8_t* wq, float* w_scale,
                             void* stream);

/* Record offsets of the current physical batch (host array of n_records + 1
 * entries: offsets[0] = 0, non-decreasing, offsets[n_records] <= max_rows;
 * empty records allowed), copied stream-ordered into `ws` (the host array may
 * be reused on return).  Every following dpsgd_i8_forward on this workspace
 * must pass n_rows = offsets[n_records] and the same n_records. */
int dpsgd_i8_set_records(const dpsgd_i8_plan* plan, void* ws, const int64_t* offsets, int64_t n_records,
                         void* stream);

/* Y = record-owned INT8 forward of the n_rows x k activations `a` (device fp16)
 * through (wq, w_scale) (n_out output features).  tau: the outlier threshold
 * (6 in LLM.int8's default; NaN is rejected).  Four launches; the workspace
 * keeps this call's intermediates until the next call. */
int dpsgd_i8_forward(const dpsgd_i8_plan* plan, void* ws, int64_t n_rows, int64_t n_records,
                     const uint16_t* a, int64_t k, const int8_t* wq, const float* w_scale,
                     int64_t n_out, float tau, uint16_t* y, void* stream);

/* The two halves of dpsgd_i8_forward, for callers that time or overlap them:
 * dpsgd_i8_route runs Algorithm 1's steps 1-6 (masks, owners, row scales,
 * codes) into the workspace; dpsgd_i8_matmul runs step 7 (the INT8 product,
 * dequantisation and the per-record FP16 correction) and must follow a route
 * of the same activations (same a, k, n_rows, n_records) on this workspace. */
int dpsgd_i8_route(const dpsgd_i8_plan* plan, void* ws, int64_t n_rows, int64_t n_records,
                   const uint16_t* a, int64_t k, float tau, void* stream);
int dpsgd_i8_matmul(const dpsgd_i8_plan* plan, void* ws, int64_t n_rows, int64_t n_records,
                    const uint16_t* a, int64_t k, const int8_t* wq, const float* w_scale,
                    int64_t n_out, uint16_t* y, void* stream);

/* Copies of the last forward's intermediates (device destinations, each
 * optional): q [n_rows, pitch(k)] int8 codes, row_scale [n_rows] float32,
 * outlier_mask [n_records, ceil(k/32)] uint32 (bit j % 32 of word j / 32 set
 * iff column j is in O_r), owner [n_rows] int32. */
int dpsgd_i8_intermediates(const dpsgd_i8_plan* plan, const void* ws, int64_t n_rows, int64_t n_records,
                           int64_t k, int8_t* q, float* row_scale, uint32_t* outlier_mask,
                           int32_t* owner, void* stream);

/* Synchronise `stream` and read the status word: DPSGD_OK or
 * DPSGD_ERR_NONFINITE (or DPSGD_ERR_HIP).  A record whose norm is not finite
 * cannot be clipped to the bound ("Privacy-Preserving Machine Learning": its
 * clip_vector_l2 example refuses non-finite coordinates and a norm that
 * overflows); the kernels skip the sum and the noise and report it here. */
int dpsgd_status(const dpsgd_plan* plan, const void* ws, void* stream);

/* Per-layer squared norms of layers [l0, l1) from the partials of the last
 * dpsgd_norms: out[(l - l0) * n_records + i] = ||P_{i,l}||_F^2 (device).  On the
 * Gram path the partials of off-diagonal token blocks are signed; a negative
 * rounded sum is reported as 0. */
int dpsgd_layer_norm2(const dpsgd_plan* plan, int64_t n_records, int32_t l0, int32_t l1,
                      const void* ws, float* out, void* stream);

/* Raw Philox4x32-10 words of blocks first_block .. first_block + n_blocks - 1
 * for key = seed and counter = (block, step): 4 * n_blocks uint32 at dev_out.
 * The words behind the noise N(0, sigma^2 C^2 I) of DP-SGD phase 4
 * ("Privacy-Preserving Machine Learning"); the pages fix no generator (the
 * sensitivity paper's release audit, Sec. 6.5, uses the framework's own), so the
 * stream is Philox4x32-10 (Salmon et al., SC'11), exported for bit-exact
 * comparison with an independent implementation. */
int dpsgd_philox_raw(uint64_t seed, uint64_t step, uint64_t first_block, uint64_t n_blocks,
                     uint32_t* dev_out, void* stream);

/* Measurement aid (not a step of the method): a plain streaming read of `bytes`
 * bytes at device pointer `buf` (16-byte aligned, bytes a positive multiple of
 * 16), the reference for the HBM bandwidth that 16-byte loads with the
 * non-temporal hint (as the library's single-use reads are) reach on this device.  Writes DPSGD_HBM_READ_SINK_WORDS words to device pointer `sink`
 * (caller-owned): the XOR of all of them equals the XOR of every 32-bit word of
 * the buffer.  Asynchronous on `stream`; argument errors are returned before any
 * launch. */
#define DPSGD_HBM_READ_SINK_WORDS 8192
int dpsgd_hbm_read(const void* buf, int64_t bytes, uint32_t* sink, void* stream);

/* Static text for a status code. */
const char* dpsgd_error_string(int code);

/* Thread-local text describing the last failed call on this thread. */
const char* dpsgd_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DPSGD_H */
