/*
 * CPU oracle of the DP-SGD private-gradient step, in double precision.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call this file:
 * only the tests, the smoke check and the bench's CPU-baseline leg use it.  It
 * shares no code with the GPU library (its own loops, Philox and Box-Muller).
 *
 * What it computes, written out as the plain definitions of the method
 * (Abadi et al. DP-SGD as restated on the pages):
 *  - per-record gradient of a linear layer y = x W, W in R^{d_in x d_out}, with
 *    a loss summed over the record's T tokens:  P_i = A_i^T G_i  (materialised;
 *    "Privacy-Preserving Machine Learning", DP-SGD phase 2; "Sensitivity
 *    Inflation from Cross-Record Precision Routing...", Sec. 2 Eq. 2 g_r);
 *  - one L2 norm per record over all layers jointly (the concatenated gradient
 *    vector; "Differential Privacy: DP-SGD, Privacy Budgets, and LLMs",
 *    from-scratch implementation);
 *  - clip factor c_i = min(1, C/n_i), with a zero gradient left unchanged
 *    ("Privacy-Preserving Machine Learning", DP-SGD phase 3 and its
 *    clip_vector_l2 example; equivalently g / max(1, ||g||/C) of the DP-SGD
 *    exhibit card);
 *  - clipped sum S = sum_i c_i P_i in ascending record order (phase 4; Eq. 3 F(D));
 *  - Gaussian noise N(0, sigma^2 C^2 I) added once to the sum (phase 4), drawn
 *    from Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers:
 *    As Easy as 1, 2, 3", SC'11) keyed by the seed with counter
 *    (element block, step), turned into normals by the Box-Muller transform
 *    (Box & Muller 1958).
 *
 * Inputs are the same bytes the GPU consumes: fp32 values or bf16 bit
 * patterns, widened exactly to double.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_F32 0
#define ORC_BF16 1
#define ORC_F64 2 /* exact decimal pins only; the GPU consumes fp32 or bf16 */

static double orc_elem(const void* p, int dtype, int64_t idx) {
    if (dtype == ORC_F32) return (double)((const float*)p)[idx];
    if (dtype == ORC_F64) return ((const double*)p)[idx];
    union { uint32_t u; float f; } c;
    c.u = (uint32_t)((const uint16_t*)p)[idx] << 16;
    return (double)c.f;
}

/* Per-record gradient of one layer: P[j*d_out + k] = sum_t A_i[t][j] * G_i[t][k].
 * A_i is [T, d_in], G_i is [T, d_out] (row-major).  P is overwritten. */
void orc_record_grad(int dtype, const void* A_i, const void* G_i, int64_t T, int64_t d_in,
                     int64_t d_out, double* P) {
    memset(P, 0, sizeof(double) * (size_t)(d_in * d_out));
    double* g = (double*)malloc(sizeof(double) * (size_t)d_out);
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t k = 0; k < d_out; ++k) g[k] = orc_elem(G_i, dtype, t * d_out + k);
        for (int64_t j = 0; j < d_in; ++j) {
            double a = orc_elem(A_i, dtype, t * d_in + j);
            double* row = P + j * d_out;
            for (int64_t k = 0; k < d_out; ++k) row[k] += a * g[k];
        }
    }
    free(g);
}

static size_t orc_esize(int dtype) { return dtype == ORC_F64 ? 8 : (dtype == ORC_F32 ? 4 : 2); }
static int orc_dtype_ok(int dtype) { return dtype == ORC_F32 || dtype == ORC_BF16 || dtype == ORC_F64; }

/* Row j of one record's gradient: row[k] = sum_t A_i[t][j] * G_i[t][k]. */
static void orc_grad_row(int dtype, const void* A_i, const void* G_i, int64_t T, int64_t d_in,
                         int64_t d_out, int64_t j, double* row) {
    for (int64_t k = 0; k < d_out; ++k) row[k] = 0.0;
    for (int64_t t = 0; t < T; ++t) {
        const double a = orc_elem(A_i, dtype, t * d_in + j);
        for (int64_t k = 0; k < d_out; ++k) row[k] += a * orc_elem(G_i, dtype, t * d_out + k);
    }
}

/* Squared Frobenius norm of every record's gradient of one layer:
 * norm2[i] = sum_{j,k} P_i[j,k]^2, for records i = 0..B-1 of A [B,T,d_in], G [B,T,d_out].
 * Every row of every P_i is materialised (rows in parallel); each row's sum of squares is
 * kept and the rows are added in ascending order. */
int orc_layer_norm2(int dtype, const void* A, const void* G, int64_t B, int64_t T, int64_t d_in,
                    int64_t d_out, double* norm2) {
    if (!orc_dtype_ok(dtype)) return -1;
    const size_t es = orc_esize(dtype);
    double* rowsq = (double*)malloc(sizeof(double) * (size_t)(B * d_in));
#pragma omp parallel
    {
        double* row = (double*)malloc(sizeof(double) * (size_t)d_out);
#pragma omp for schedule(dynamic, 4)
        for (int64_t task = 0; task < B * d_in; ++task) {
            const int64_t i = task / d_in, j = task % d_in;
            const char* Ai = (const char*)A + (size_t)(i * T * d_in) * es;
            const char* Gi = (const char*)G + (size_t)(i * T * d_out) * es;
            orc_grad_row(dtype, Ai, Gi, T, d_in, d_out, j, row);
            double s = 0.0;
            for (int64_t k = 0; k < d_out; ++k) s += row[k] * row[k];
            rowsq[task] = s;
        }
        free(row);
    }
    for (int64_t i = 0; i < B; ++i) {
        double s = 0.0;
        for (int64_t j = 0; j < d_in; ++j) s += rowsq[i * d_in + j];
        norm2[i] = s;
    }
    free(rowsq);
    return 0;
}

/* Clip factor of one record from its joint squared norm: n = sqrt(norm2);
 * c = 1 when n <= C (this covers n = 0, a zero gradient stays unchanged), else C / n. */
double orc_clip_factor(double norm2, double C) {
    double n = sqrt(norm2);
    if (n <= C) return 1.0;
    return C / n;
}

void orc_clip(const double* norm2, int64_t B, double C, double* n_out, double* c_out) {
    for (int64_t i = 0; i < B; ++i) {
        if (n_out) n_out[i] = sqrt(norm2[i]);
        c_out[i] = orc_clip_factor(norm2[i], C);
    }
}

/* S[j*d_out + k] += sum_i c[i] * P_i[j,k], records in ascending order.
 * Rows j in parallel; each row of each record's gradient is materialised, scaled by the
 * record's clip factor and added, so every entry sums its records in the order i = 0..B-1. */
int orc_layer_clipped_sum(int dtype, const void* A, const void* G, int64_t B, int64_t T,
                          int64_t d_in, int64_t d_out, const double* c, double* S) {
    if (!orc_dtype_ok(dtype)) return -1;
    const size_t es = orc_esize(dtype);
#pragma omp parallel
    {
        double* row = (double*)malloc(sizeof(double) * (size_t)d_out);
#pragma omp for schedule(dynamic, 4)
        for (int64_t j = 0; j < d_in; ++j) {
            for (int64_t i = 0; i < B; ++i) {
                const char* Ai = (const char*)A + (size_t)(i * T * d_in) * es;
                const char* Gi = (const char*)G + (size_t)(i * T * d_out) * es;
                orc_grad_row(dtype, Ai, Gi, T, d_in, d_out, j, row);
                for (int64_t k = 0; k < d_out; ++k) S[j * d_out + k] += c[i] * row[k];
            }
        }
        free(row);
    }
    return 0;
}

/* ---------------- Philox4x32-10 (SC'11) ---------------- */

/* One Philox4x32 round on counter x with round key k: two 32x32->64 products of
 * the multipliers with words 0 and 2; the high halves are xored with the other
 * two words and the key, and the words are permuted. */
static void orc_philox_round(uint32_t x[4], const uint32_t k[2]) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * x[0];
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * x[2];
    const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    const uint32_t y0 = hi1 ^ x[1] ^ k[0];
    const uint32_t y1 = lo1;
    const uint32_t y2 = hi0 ^ x[3] ^ k[1];
    const uint32_t y3 = lo0;
    x[0] = y0; x[1] = y1; x[2] = y2; x[3] = y3;
}

/* Ten rounds; the key is advanced by the two Weyl increments between rounds. */
void orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
    uint32_t x[4] = {ctr[0], ctr[1], ctr[2], ctr[3]};
    uint32_t k[2] = {key[0], key[1]};
    for (int r = 0; r < 10; ++r) {
        if (r > 0) {
            k[0] += 0x9E3779B9u;
            k[1] += 0xBB67AE85u;
        }
        orc_philox_round(x, k);
    }
    out[0] = x[0]; out[1] = x[1]; out[2] = x[2]; out[3] = x[3];
}

/* Words of blocks first_block .. first_block+n_blocks-1 for (seed, step):
 * key = (seed mod 2^32, seed div 2^32), counter = (b mod 2^32, b div 2^32,
 * step mod 2^32, step div 2^32).  out holds 4*n_blocks words. */
void orc_philox_words(uint64_t seed, uint64_t step, uint64_t first_block, uint64_t n_blocks,
                      uint32_t* out) {
    const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
#pragma omp parallel for schedule(static)
    for (int64_t q = 0; q < (int64_t)n_blocks; ++q) {
        const uint64_t b = first_block + (uint64_t)q;
        const uint32_t ctr[4] = {(uint32_t)b, (uint32_t)(b >> 32), (uint32_t)step,
                                 (uint32_t)(step >> 32)};
        orc_philox4x32_10(ctr, key, out + 4 * q);
    }
}

/* Standard normals Z[e] for flat element indices e = first_e .. first_e+n-1.
 * Element e uses block e/4; lanes (0,1) share the pair (w0,w1), lanes (2,3) the
 * pair (w2,w3).  u1 = ((w_even >> 8) + 1) / 2^24 in (0,1], u2 = (w_odd >> 8) / 2^24
 * in [0,1); r = sqrt(-2 ln u1); even lane r cos(2 pi u2), odd lane r sin(2 pi u2). */
void orc_gauss(uint64_t seed, uint64_t step, uint64_t first_e, int64_t n, double* z) {
    const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    const double two_pi = 6.283185307179586476925286766559;
#pragma omp parallel for schedule(static)
    for (int64_t q = 0; q < n; ++q) {
        const uint64_t e = first_e + (uint64_t)q;
        const uint64_t b = e >> 2;
        const int lane = (int)(e & 3u);
        const uint32_t ctr[4] = {(uint32_t)b, (uint32_t)(b >> 32), (uint32_t)step,
                                 (uint32_t)(step >> 32)};
        uint32_t w[4];
        orc_philox4x32_10(ctr, key, w);
        const int pair = lane >> 1;
        const double u1 = ((double)(w[2 * pair] >> 8) + 1.0) * (1.0 / 16777216.0);
        const double u2 = (double)(w[2 * pair + 1] >> 8) * (1.0 / 16777216.0);
        const double r = sqrt(-2.0 * log(u1));
        z[q] = (lane & 1) ? r * sin(two_pi * u2) : r * cos(two_pi * u2);
    }
}

/* Noised sum: S[q] += (sigma * C) * Z[first_e + q]. */
void orc_add_noise(double* S, int64_t n, uint64_t first_e, double sigma, double C, uint64_t seed,
                   uint64_t step) {
    double* z = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    orc_gauss(seed, step, first_e, n, z);
    const double s = sigma * C;
    for (int64_t q = 0; q < n; ++q) S[q] += s * z[q];
    free(z);
}

/* Threads the oracle's parallel loops use (for reporting). */
int orc_num_threads(void) { return omp_get_max_threads(); }

/* Threads for the oracle's later parallel loops (for a single-thread timing). */
void orc_set_num_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }
