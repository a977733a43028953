// gemm.hip -- dispatch of a scaled-GEMM launch to the translation unit of its
// operand-format pair (the kernels are in gemm_kernels.h).
#include "fp8q_device.h"
#include "gemm_pairs.h"

namespace fp8q {

hipError_t launch_gemm(const uint8_t *A, int fa, const float *sA, const uint8_t *B, int fb, const float *sB, int64_t M,
                       int64_t N, int64_t K, int mode, void *C, int out_kind, const float *bias, int act,
                       const float *out_scale_inv, float *amax_out, GridScratch *gs, hipStream_t s)
{
    // compute units of the current device, read once per device
    static int cu_count[64] = {0};
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < 64) {
        if (cu_count[dev] == 0) {
            int v = 0;
            if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess) cu_count[dev] = v;
        }
        cus = cu_count[dev];
    }
    const GemmArgs a{A, B, sA, sB, M, N, K, mode, C, out_kind, bias, act, out_scale_inv, amax_out, gs, s, cus};
    if (fa == kE4M3 && fb == kE4M3) return launch_gemm_e4m3_e4m3(a);
    if (fa == kE5M2 && fb == kE4M3) return launch_gemm_e5m2_e4m3(a);
    if (fa == kE4M3 && fb == kE5M2) return launch_gemm_e4m3_e5m2(a);
    return launch_gemm_e5m2_e5m2(a);
}

} // namespace fp8q
