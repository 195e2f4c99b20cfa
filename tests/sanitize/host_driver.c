/* Drives the host side of the C ABI (plan construction and layout, argument validation, the
 * accountant, the INT8 plan) for a build with AddressSanitizer and UndefinedBehaviorSanitizer.
 * Nothing here reaches a launch: every compute call is given an argument error, so it returns
 * before touching the device (there is none on the machine this runs on). */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "dpsgd.h"

static int fails = 0;
#define CHECK(c) do { if (!(c)) { printf("FAIL %s:%d %s (%s)\n", __FILE__, __LINE__, #c, dpsgd_last_error()); ++fails; } } while (0)

static int make(dpsgd_layer_shape* L, int n, int dtype, int64_t B, int64_t T, int path, int sum,
                uint32_t flags, dpsgd_plan** p, size_t* ws) {
    dpsgd_plan_desc d;
    memset(&d, 0, sizeof d);
    d.n_layers = n; d.layers = L; d.dtype = dtype; d.max_records = B; d.tokens = T;
    d.path_policy = path; d.sum_policy = sum; d.flags = flags;
    return dpsgd_plan_create(&d, p, ws);
}

int main(void) {
    dpsgd_layer_shape lora[4] = {{768, 8}, {8, 768}, {4096, 16}, {16, 4096}};
    dpsgd_layer_shape dense[2] = {{4096, 4096}, {320, 272}};
    dpsgd_layer_shape bad[1] = {{0, 5}};
    dpsgd_layer_shape huge[1] = {{(int64_t)1 << 30, (int64_t)1 << 30}};
    dpsgd_plan* p = NULL;
    size_t ws = 0;
    int32_t path, sm;
    for (int dt = 0; dt < 2; ++dt)
        for (int pol = 0; pol < 3; ++pol)
            for (int sum = 0; sum < 3; ++sum) {
                CHECK(make(lora, 4, dt, 17, 129, pol, sum, 0, &p, &ws) == DPSGD_OK && ws > 0);
                for (int l = 0; l < 4; ++l) CHECK(dpsgd_plan_layer_info(p, l, &path, &sm) == DPSGD_OK);
                CHECK(dpsgd_plan_layer_info(p, 4, &path, &sm) == DPSGD_ERR_INVALID_ARG);
                CHECK(dpsgd_plan_num_params(p) == 768 * 8 * 2 + 4096 * 16 * 2);
                dpsgd_plan_destroy(p);
                CHECK(make(dense, 2, dt, 64, 256, pol, sum, dt == 0 ? DPSGD_PLAN_SEGMENTS : 0, &p, &ws) == DPSGD_OK);
                dpsgd_plan_destroy(p);
            }
    CHECK(make(bad, 1, 0, 4, 4, 0, 0, 0, &p, &ws) == DPSGD_ERR_INVALID_ARG && p == NULL);
    CHECK(make(huge, 1, 1, 65535, 1 << 20, 0, 0, 0, &p, &ws) == DPSGD_ERR_INVALID_ARG);
    CHECK(make(lora, 4, 7, 4, 4, 0, 0, 0, &p, &ws) == DPSGD_ERR_UNSUPPORTED);
    CHECK(make(lora, 4, 0, 0, 4, 0, 0, 0, &p, &ws) == DPSGD_ERR_INVALID_ARG);
    CHECK(make(lora, 4, 0, 4, 4, 0, 0, 8, &p, &ws) == DPSGD_ERR_INVALID_ARG);
    CHECK(dpsgd_plan_create(NULL, &p, &ws) == DPSGD_ERR_INVALID_ARG);
    dpsgd_plan_destroy(NULL);

    /* argument errors of the compute entry points, all returned before any launch */
    CHECK(make(lora, 4, 1, 8, 64, 0, 0, 0, &p, &ws) == DPSGD_OK);
    char fake_ws_storage[512];
    void* fake_ws = (void*)(((uintptr_t)fake_ws_storage + 255) & ~(uintptr_t)255);
    const void* ptrs[4] = {fake_ws, fake_ws, fake_ws, fake_ws};
    float* outs[4] = {(float*)fake_ws, (float*)fake_ws, (float*)fake_ws, NULL};
    dpsgd_step_args a;
    memset(&a, 0, sizeof a);
    a.n_records = 8; a.A = ptrs; a.G = ptrs; a.out = outs; a.ws = fake_ws; a.C = 1.0; a.sigma = 1.0;
    CHECK(dpsgd_step(p, &a, NULL) == DPSGD_ERR_INVALID_ARG);            /* a null out pointer */
    a.C = -1.0;
    CHECK(dpsgd_step(p, &a, NULL) == DPSGD_ERR_INVALID_ARG);
    a.C = 1.0; a.sigma = NAN;
    CHECK(dpsgd_step(p, &a, NULL) == DPSGD_ERR_INVALID_ARG);
    a.sigma = 1.0; a.n_records = 9;
    CHECK(dpsgd_step(p, &a, NULL) == DPSGD_ERR_INVALID_ARG);
    a.n_records = 8; a.flags = DPSGD_DESCENT | DPSGD_NO_NOISE;
    CHECK(dpsgd_step(p, &a, NULL) == DPSGD_ERR_INVALID_ARG);
    a.flags = 0; a.ws = (char*)fake_ws + 8;
    CHECK(dpsgd_step(p, &a, NULL) == DPSGD_ERR_INVALID_ARG);
    CHECK(dpsgd_step_noalloc(p, &a, NULL, NULL) == DPSGD_ERR_INVALID_ARG);  /* ws must be NULL */
    CHECK(dpsgd_norms(p, 8, 2, 1, ptrs, ptrs, fake_ws, NULL) == DPSGD_ERR_INVALID_ARG);
    CHECK(dpsgd_clip(p, 8, 0.0, 0, fake_ws, NULL, NULL, NULL) == DPSGD_ERR_INVALID_ARG);
    CHECK(dpsgd_clipped_sum(p, 8, 0, 4, ptrs, ptrs, NULL, outs, 0, fake_ws, NULL) == DPSGD_ERR_INVALID_ARG);
    CHECK(dpsgd_noise(p, outs, 1.0, 1.0, 0, 0, NULL, NULL) == DPSGD_ERR_INVALID_ARG);
    CHECK(dpsgd_layer_norm2(p, 8, 0, 5, fake_ws, (float*)fake_ws, NULL) == DPSGD_ERR_INVALID_ARG);
    int64_t offs[3] = {0, 70, 80};
    CHECK(dpsgd_ws_segments(p, fake_ws, offs, 2, NULL) == DPSGD_ERR_INVALID_ARG);   /* not a segment plan */
    dpsgd_plan_destroy(p);
    CHECK(make(lora, 2, 0, 4, 64, 0, 0, DPSGD_PLAN_SEGMENTS, &p, &ws) == DPSGD_OK);
    CHECK(dpsgd_ws_segments(p, fake_ws, offs, 2, NULL) == DPSGD_ERR_INVALID_ARG);   /* 70 rows > 64 */
    CHECK(dpsgd_step_noalloc(p, &a, NULL, NULL) == DPSGD_ERR_INVALID_ARG);
    dpsgd_plan_destroy(p);
    CHECK(dpsgd_philox_raw(0, 0, 0, 4, NULL, NULL) == DPSGD_ERR_INVALID_ARG);
    CHECK(dpsgd_hbm_read(fake_ws, 17, (uint32_t*)fake_ws, NULL) == DPSGD_ERR_INVALID_ARG);

    /* accountant: host only */
    double orders[5] = {1.5, 2.0, 8.0, 32.0, 64.0}, rdp[5], eps, ord;
    CHECK(dpsgd_rdp_sampled_gaussian(0.01, 1.0, orders, 5, rdp) == DPSGD_OK);
    for (int i = 0; i < 5; ++i) rdp[i] *= 300;
    CHECK(dpsgd_rdp_to_epsilon(orders, rdp, 5, 1e-5, 1, &eps, &ord) == DPSGD_OK && eps > 0 && isfinite(eps));
    CHECK(dpsgd_rdp_sampled_gaussian(1.5, 1.0, orders, 5, rdp) == DPSGD_ERR_INVALID_ARG);
    double dl;
    CHECK(dpsgd_gaussian_pair_delta(1.0, 1.0, &dl) == DPSGD_OK && dl > 0 && dl < 1);
    CHECK(dpsgd_gaussian_pair_epsilon(dl, 1.0, &eps) == DPSGD_OK && fabs(eps - 1.0) < 1e-6);

    /* INT8 plan */
    dpsgd_i8_plan* ip = NULL;
    CHECK(dpsgd_i8_pitch(100) == 128 && dpsgd_i8_pitch(0) == 0 && dpsgd_i8_pitch(40000) == 0);
    CHECK(dpsgd_i8_plan_create(4096, 16, 3072, &ip, &ws) == DPSGD_OK && ws > 0);
    CHECK(dpsgd_i8_set_records(ip, fake_ws, offs, 2, NULL) == DPSGD_OK || 1);   /* copy may fail: no device */
    int64_t bad_offs[3] = {0, 90, 80};
    CHECK(dpsgd_i8_set_records(ip, fake_ws, bad_offs, 2, NULL) == DPSGD_ERR_INVALID_ARG);
    CHECK(dpsgd_i8_forward(ip, fake_ws, 80, 2, NULL, 768, NULL, NULL, 768, 6.0f, NULL, NULL) == DPSGD_ERR_INVALID_ARG);
    dpsgd_i8_plan_destroy(ip);
    CHECK(dpsgd_i8_plan_create(4096, 0, 3072, &ip, &ws) == DPSGD_ERR_INVALID_ARG);

    for (int c = -6; c <= 1; ++c) CHECK(dpsgd_error_string(c) != NULL);
    printf(fails ? "FAILED\n" : "OK\n");
    return fails ? 1 : 0;
}
