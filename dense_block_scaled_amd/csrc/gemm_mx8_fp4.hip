// gemm_mx8_fp4.hip -- 8-bit MX GEMM kernels with an E2M1 operand (FP8 x FP4) or FP6 operands
// (instantiations of the kernel template in gemm_kernel.h; one translation
// unit per group of formats so that the library builds in parallel)
#include "gemm_kernel.h"

namespace dbs {

hipError_t launch_gemm_mx8_fp4(int shape, const Params &p, int grid, hipStream_t stream)
{
    return by_shape(shape, [&](auto s) { return launch_fp8_fp4<decltype(s)>(p, grid, stream); });
}
}  // namespace dbs
