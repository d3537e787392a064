// gemm_nvfp4.hip -- NVFP4 GEMM kernels: decoded into LDS, and the raw-staged kernels
// (instantiations of the kernel template in gemm_kernel.h; one translation
// unit per group of formats so that the library builds in parallel)
#include "gemm_kernel.h"

namespace dbs {

hipError_t launch_gemm_nvfp4(int shape, const Params &p, int grid, hipStream_t stream)
{
    return by_shape(shape, [&](auto s) { return launch_fmt<kNVFP4, decltype(s)>(p, grid, stream); });
}

hipError_t launch_gemm_nvfp4_raw(int shape, const Params &p, int grid, hipStream_t stream)
{
    return by_shape(shape, [&](auto s) { return launch_nvfp4_raw<decltype(s)>(p, grid, stream); });
}
}  // namespace dbs
