// Host/device interface of the record-owned LLM.int8 forward (kernels in int8_forward.hip,
// entry points in dpsgd_api.cpp).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dpsgd {

// Record-owned LLM.int8 forward of one frozen layer.  Rows of A (fp16, n x K, row stride K)
// belong to records by offsets[0..n_rec]; own, s, omask and Q live in the workspace.
constexpr int kI8MaxKW = 1024;     // outlier-mask words per record: K <= 32768
struct I8Args {
    const uint16_t* A;
    int64_t n, K, Kp, KW, n_rec;   // rows, columns, code pitch (K rounded up to 64), K / 32 words
    const int64_t* offsets;        // [n_rec + 1] record row offsets, then [n_rec + 1] scan
                                   // block offsets (record r: max(1, ceil(len / 16)) blocks)
    uint32_t* pmask;               // [scan blocks][KW] per-block partial outlier masks
    int32_t* own;                  // [n] owner record of each row
    float* s;                      // [n] row scales
    uint32_t* omask;               // [n_rec][KW] per-record outlier columns
    int8_t* Q;                     // [n][Kp] activation codes
    const int8_t* Wq;              // [N][Kp] weight codes
    const float* sW;               // [N] weight scales
    int64_t N;
    uint16_t* Y;                   // [n][N] fp16 output
    float tau;
    int32_t tau_on;                // 0: no outlier path
    int32_t a_vec;                 // K % 8 == 0 and A 16-byte aligned
    int32_t y_vec;                 // N % 4 == 0 and Y 8-byte aligned
};
int64_t i8_tiles(int64_t n, int64_t N, int big);
int64_t i8_scan_blocks(int64_t n, int64_t n_rec);   // upper bound of sum max(1, ceil(len / 16))
hipError_t launch_i8_route(const I8Args& a, hipStream_t s);
hipError_t launch_i8_gemm(const I8Args& a, int big, hipStream_t s);
hipError_t launch_i8_weight(const uint16_t* W, int64_t N, int64_t K, int64_t Kp, int8_t* Wq,
                            float* sW, hipStream_t s);

}  // namespace dpsgd
