// gemm_pairs.h -- arguments of one scaled-GEMM launch and the launchers of
// the four operand-format pairs (one translation unit each).
#ifndef FP8Q_GEMM_PAIRS_H
#define FP8Q_GEMM_PAIRS_H

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp8q_launch.h"

namespace fp8q {

struct GemmArgs {
    const uint8_t *A, *B;
    const float *sA, *sB;
    int64_t M, N, K;
    int mode;                   // 0 per-tensor, 1 1x128 x 128x128, 2 1x128 x 1x128, 3 MXFP8
    void *C;
    int out_kind;               // 0 bf16, 1 fp32, 2 E4M3FN codes, 3 E5M2 codes
    const float *bias;          // [N] fp32 or null
    int act;                    // 0 none, 1 ReLU, 2 GELU
    const float *out_scale_inv; // FP8 output: its dequant scale
    float *amax_out;            // or null
    GridScratch *gs;
    hipStream_t stream;
    int cus; // compute units of the device (tile-wave accounting)
};

hipError_t launch_gemm_e4m3_e4m3(const GemmArgs &a);
hipError_t launch_gemm_e5m2_e4m3(const GemmArgs &a);
hipError_t launch_gemm_e4m3_e5m2(const GemmArgs &a);
hipError_t launch_gemm_e5m2_e5m2(const GemmArgs &a);

} // namespace fp8q

#endif // FP8Q_GEMM_PAIRS_H
