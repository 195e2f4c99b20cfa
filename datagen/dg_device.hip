// Device fill of one synthetic input tensor, bit-identical to dg_fill_host
// (see dg.h for the recipe).  Used to fill inputs directly in HBM when the
// tensors are too large to generate on the host and upload.  Built with
// -ffp-contract=off so that the double arithmetic matches the host build.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include "dg.h"

__global__ void __launch_bounds__(256) dg_fill_kernel(uint64_t key, int32_t dtype, uint64_t first_e,
                                                      int64_t n_rec, int64_t per_rec,
                                                      const double* __restrict__ scale,
                                                      const uint8_t* __restrict__ heavy,
                                                      void* __restrict__ out) {
    const int64_t total = n_rec * per_rec;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x * 2;
    for (int64_t x = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 2; x < total; x += stride) {
        // two consecutive elements per thread (a 4-byte bf16 pair or two floats)
        float f[2];
        for (int u = 0; u < 2; ++u) {
            int64_t xe = x + u;
            if (xe < total) {
                int64_t r = xe / per_rec;
                double v = scale[r] * dg_draw(key, first_e + (uint64_t)xe, heavy ? heavy[r] : 0);
                f[u] = (float)v;
            } else {
                f[u] = 0.0f;
            }
        }
        if (dtype == DG_F32) {
            float* o = (float*)out;
            o[x] = f[0];
            if (x + 1 < total) o[x + 1] = f[1];
        } else {
            uint16_t* o = (uint16_t*)out;
            o[x] = dg_f32_to_bf16(f[0]);
            if (x + 1 < total) o[x + 1] = dg_f32_to_bf16(f[1]);
        }
    }
}

// Fill records [first_record, first_record + n_rec) of a [*, T, d] tensor into
// device memory `out` (record-major).  scale / heavy are device arrays of
// n_rec entries (heavy may be null).  Asynchronous on `stream`.
extern "C" int dg_fill_device(uint64_t seed, uint32_t layer, uint32_t tensor, int32_t dtype,
                              int64_t first_record, int64_t n_rec, int64_t T, int64_t d,
                              const double* scale, const uint8_t* heavy, void* out, void* stream) {
    if (n_rec < 0 || T <= 0 || d <= 0 || first_record < 0 || !scale || !out) return -1;
    if (dtype != DG_F32 && dtype != DG_BF16) return -1;
    if (n_rec == 0) return 0;
    const int64_t per_rec = T * d;
    const int64_t total = n_rec * per_rec;
    int64_t blocks = (total / 2 + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    if (blocks < 1) blocks = 1;
    uint64_t key = dg_stream_key(seed, layer, tensor);
    hipLaunchKernelGGL(dg_fill_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, key,
                       dtype, (uint64_t)first_record * (uint64_t)per_rec, n_rec, per_rec, scale, heavy,
                       out);
    return hipGetLastError() == hipSuccess ? 0 : -2;
}
