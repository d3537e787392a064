// gemm.hip -- the kernel launcher the C ABI calls: picks the translation unit
// of the format (gemm_bf16.hip, gemm_mxfp8.hip, gemm_mx8_e5m2.hip,
// gemm_mx8_fp4.hip, gemm_mxfp4.hip, gemm_nvfp4.hip, gemm_mxfp6.hip,
// gemm_bf16_ea.hip); the kernels and their
// design notes are in gemm_kernel.h.
#include "gemm_kernel.h"

namespace dbs {

hipError_t launch_gemm(int fmt, int shape, const Params &p, int grid, hipStream_t stream)
{
    switch (fmt) {
    case kBF16: return launch_gemm_bf16(shape, p, grid, stream);
    case kMXFP8: return launch_gemm_mxfp8(shape, p, grid, stream);
    case kMXFP4: return launch_gemm_mxfp4(shape, p, grid, stream);
    case kNVFP4: return launch_gemm_nvfp4(shape, p, grid, stream);
    case kNVFP4R: return launch_gemm_nvfp4_raw(shape, p, grid, stream);
    case kMXFP6: return shape == kShapeSquare ? launch_gemm_mxfp6(p, grid, stream) : hipErrorInvalidValue;
    case kBF16EA:
    case kBF16EL:
        return shape == kShapeSquare ? launch_gemm_bf16_ea(p, fmt == kBF16EA, grid, stream) : hipErrorNotSupported;
    default: return hipErrorInvalidValue;
    }
}

}  // namespace dbs
