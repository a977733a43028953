// gemm_e4m3_e4m3.hip -- the scaled-GEMM kernels with E4M3FN codes in A and E4M3FN
// codes in B (every scaling mode, output kind and epilogue).
#include "gemm_kernels.h"

namespace fp8q {

hipError_t launch_gemm_e4m3_e4m3(const GemmArgs &a) { return launch_gemm_pair<kE4M3, kE4M3>(a); }

} // namespace fp8q
