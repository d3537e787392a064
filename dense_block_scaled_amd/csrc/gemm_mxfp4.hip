// gemm_mxfp4.hip -- MXFP4 GEMM kernels
// (instantiations of the kernel template in gemm_kernel.h; one translation
// unit per group of formats so that the library builds in parallel)
#include "gemm_kernel.h"

namespace dbs {

hipError_t launch_gemm_mxfp4(int shape, const Params &p, int grid, hipStream_t stream)
{
    return by_shape(shape, [&](auto s) { return launch_fmt<kMXFP4, decltype(s)>(p, grid, stream); });
}
}  // namespace dbs
