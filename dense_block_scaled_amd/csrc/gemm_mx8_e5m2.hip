// gemm_mx8_e5m2.hip -- MXFP8 GEMM kernels with E5M2 on either side
// (instantiations of the kernel template in gemm_kernel.h; one translation
// unit per group of formats so that the library builds in parallel)
#include "gemm_kernel.h"

namespace dbs {

hipError_t launch_gemm_mx8_e5m2(int shape, const Params &p, int grid, hipStream_t stream)
{
    return by_shape(shape, [&](auto s) { return launch_fmt<kMXFP8, decltype(s), true>(p, grid, stream); });
}
}  // namespace dbs
