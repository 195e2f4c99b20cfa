/*
 * Host fill of one synthetic input tensor (see dg.h for the value recipe).
 * Built with gcc -O2 -ffp-contract=off -fopenmp; used by the tests, the bench
 * setup and the CPU oracle's inputs.  Holds none of the DP-SGD arithmetic.
 */
#include <stddef.h>
#include <stdint.h>
#include "dg.h"

/* Fill records [first_record, first_record + n_rec) of a tensor [*, T, d].
 * scale[r], heavy[r] describe record first_record + r.  out is float* (DG_F32)
 * or uint16_t* bf16 bits (DG_BF16), n_rec*T*d elements, record-major. */
int dg_fill_host(uint64_t seed, uint32_t layer, uint32_t tensor, int32_t dtype,
                 int64_t first_record, int64_t n_rec, int64_t T, int64_t d,
                 const double* scale, const uint8_t* heavy, void* out) {
    if (n_rec < 0 || T <= 0 || d <= 0 || first_record < 0) return -1;
    if (dtype != DG_F32 && dtype != DG_BF16) return -1;
    const uint64_t key = dg_stream_key(seed, layer, tensor);
    const int64_t per_rec = T * d;
    for (int64_t r = 0; r < n_rec; ++r) {
        const double s = scale[r];
        const int h = heavy ? heavy[r] : 0;
        const uint64_t base = (uint64_t)(first_record + r) * (uint64_t)per_rec;
#pragma omp parallel for schedule(static)
        for (int64_t x = 0; x < per_rec; ++x) {
            double v = s * dg_draw(key, base + (uint64_t)x, h);
            float f = (float)v;
            if (dtype == DG_F32)
                ((float*)out)[r * per_rec + x] = f;
            else
                ((uint16_t*)out)[r * per_rec + x] = dg_f32_to_bf16(f);
        }
    }
    return 0;
}

/* Gather single elements: out_vals[k] = value of (rec[k], tok[k], col[k]),
 * stored as float (the exact fp32 or bf16 value widened to float). */
int dg_gather_host(uint64_t seed, uint32_t layer, uint32_t tensor, int32_t dtype,
                   int64_t T, int64_t d, int64_t n, const int64_t* rec, const int64_t* tok,
                   const int64_t* col, const double* rec_scale, const uint8_t* rec_heavy,
                   float* out_vals) {
    if (dtype != DG_F32 && dtype != DG_BF16) return -1;
    const uint64_t key = dg_stream_key(seed, layer, tensor);
#pragma omp parallel for schedule(static)
    for (int64_t k = 0; k < n; ++k) {
        uint64_t e = ((uint64_t)rec[k] * (uint64_t)T + (uint64_t)tok[k]) * (uint64_t)d + (uint64_t)col[k];
        double v = rec_scale[k] * dg_draw(key, e, rec_heavy ? rec_heavy[k] : 0);
        float f = (float)v;
        if (dtype == DG_BF16) {
            union { float f; uint32_t u; } c;
            c.u = (uint32_t)dg_f32_to_bf16(f) << 16;
            f = c.f;
        }
        out_vals[k] = f;
    }
    return 0;
}
