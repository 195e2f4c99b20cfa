/* Runs the oracle's functions on small inputs of every element type it reads, for a build with
 * AddressSanitizer and UndefinedBehaviorSanitizer (the run fails on any report).  Values are
 * checked against the closed forms they must meet, so the run also exercises the arithmetic. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

void orc_record_grad(int dtype, const void* A_i, const void* G_i, int64_t T, int64_t d_in, int64_t d_out,
                     double* P);
int orc_layer_norm2(int dtype, const void* A, const void* G, int64_t B, int64_t T, int64_t d_in,
                    int64_t d_out, double* norm2);
double orc_clip_factor(double norm2, double C);
void orc_clip(const double* norm2, int64_t B, double C, double* n_out, double* c_out);
int orc_layer_clipped_sum(int dtype, const void* A, const void* G, int64_t B, int64_t T, int64_t d_in,
                          int64_t d_out, const double* c, double* S);
void orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]);
void orc_philox_words(uint64_t seed, uint64_t step, uint64_t first_block, uint64_t n_blocks, uint32_t* out);
void orc_gauss(uint64_t seed, uint64_t step, uint64_t first_e, int64_t n, double* z);
void orc_add_noise(double* S, int64_t n, uint64_t first_e, double sigma, double C, uint64_t seed,
                   uint64_t step);

static int fails = 0;
#define CHECK(c) do { if (!(c)) { printf("FAIL %s:%d %s\n", __FILE__, __LINE__, #c); ++fails; } } while (0)

static uint16_t to_bf16(float f) { uint32_t u; memcpy(&u, &f, 4); return (uint16_t)(u >> 16); }

int main(void) {
    enum { B = 3, T = 5, DI = 7, DO = 4 };
    float A[B * T * DI], G[B * T * DO];
    uint16_t Ab[B * T * DI], Gb[B * T * DO];
    double Ad[B * T * DI], Gd[B * T * DO];
    for (int i = 0; i < B * T * DI; ++i) { A[i] = (float)((i * 7) % 5 - 2); Ab[i] = to_bf16(A[i]); Ad[i] = A[i]; }
    for (int i = 0; i < B * T * DO; ++i) { G[i] = (float)((i * 3) % 7 - 3); Gb[i] = to_bf16(G[i]); Gd[i] = G[i]; }
    const void* As[3] = {A, Ab, Ad};
    const void* Gs[3] = {G, Gb, Gd};
    double ref[B];
    for (int dt = 0; dt < 3; ++dt) {
        double n2[B], P[DI * DO];
        CHECK(orc_layer_norm2(dt, As[dt], Gs[dt], B, T, DI, DO, n2) == 0);
        for (int i = 0; i < B; ++i) {
            const size_t es = dt == 0 ? 4 : dt == 1 ? 2 : 8;
            orc_record_grad(dt, (const char*)As[dt] + (size_t)i * T * DI * es,
                            (const char*)Gs[dt] + (size_t)i * T * DO * es, T, DI, DO, P);
            double s = 0.0;
            for (int k = 0; k < DI * DO; ++k) s += P[k] * P[k];
            CHECK(s == n2[i]);                    /* integer inputs: exact */
            if (dt == 0) ref[i] = n2[i]; else CHECK(n2[i] == ref[i]);
        }
        double n[B], c[B], S[DI * DO];
        orc_clip(n2, B, 4.0, n, c);
        for (int i = 0; i < B; ++i) CHECK(c[i] > 0.0 && c[i] <= 1.0 && c[i] * n[i] <= 4.0 * (1 + 1e-15));
        memset(S, 0, sizeof S);
        CHECK(orc_layer_clipped_sum(dt, As[dt], Gs[dt], B, T, DI, DO, c, S) == 0);
    }
    CHECK(orc_layer_norm2(9, A, G, B, T, DI, DO, ref) != 0);   /* unknown type refused */
    CHECK(orc_clip_factor(0.0, 1.0) == 1.0 && orc_clip_factor(4.0, 1.0) == 0.5);
    uint32_t ctr[4] = {0, 0, 0, 0}, key[2] = {0, 0}, out[4], words[4 * 9];
    orc_philox4x32_10(ctr, key, out);
    orc_philox_words(0, 0, 0, 9, words);
    CHECK(memcmp(out, words, sizeof out) == 0);
    double z[37], S2[37];
    orc_gauss(5, 2, 3, 37, z);
    for (int i = 0; i < 37; ++i) { CHECK(isfinite(z[i]) && fabs(z[i]) < 6.0); S2[i] = 1.0; }
    orc_add_noise(S2, 37, 3, 2.0, 0.5, 5, 2);
    for (int i = 0; i < 37; ++i) CHECK(S2[i] == 1.0 + 1.0 * z[i]);
    printf(fails ? "FAILED\n" : "OK\n");
    return fails ? 1 : 0;
}
