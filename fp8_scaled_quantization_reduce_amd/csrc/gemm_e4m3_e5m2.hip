// gemm_e4m3_e5m2.hip -- the scaled-GEMM kernels with E4M3FN codes in A and E5M2
// codes in B (every scaling mode, output kind and epilogue).
#include "gemm_kernels.h"

namespace fp8q {

hipError_t launch_gemm_e4m3_e5m2(const GemmArgs &a) { return launch_gemm_pair<kE4M3, kE5M2>(a); }

} // namespace fp8q
