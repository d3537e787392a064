// launch.h -- internal interface between the C ABI (dbs.cpp) and the gfx950
// kernels (gemm.hip, quant.hip).  Not installed; callers use include/dbs.h.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace dbs {

// kNVFP4R: NVFP4 staged raw (the E2M1 bytes as MXFP4 stages them, the E4M3
// scales as MX scales) and decoded in registers -- the path for MN-major
// NVFP4 operands; internal, chosen by the launcher.  kMXFP6: FP6 elements on
// both sides at the MFMA's FP6 rate (gemm_mxfp6.hip; ec holds the two FP6
// codes).
enum Format : int { kBF16 = 0, kMXFP8 = 1, kMXFP4 = 2, kNVFP4 = 3, kNVFP4R = 4, kMXFP6 = 5, kBF16EA = 6, kBF16EL = 7 };

constexpr int kMaxGroups = 64;

// Everything a kernel needs, passed by value.  Sizes were validated on the
// host: every per-tile byte offset fits in 31 bits.
struct Params {
    const uint8_t *A;     // M x lda bytes (K x ldam if MN-major)
    const uint8_t *B;     // N x lda bytes (K x ldbm if MN-major)
    const uint8_t *sA;    // M x sld scale bytes (null for bf16)
    const uint8_t *sB;    // N x sld scale bytes
    uint16_t *D;          // M x N bf16
    int M, N, K;
    int lda;              // bytes per operand row (K * element bits / 8)
    int sld;              // scale bytes per row (K / block size), 0 for bf16
    int nk;               // number of K stages (set by the launcher for the kernel it picks)
    int tiles_m, tiles_n;
    int group_m;          // tile rows per raster group
    int vec_store;        // 1 if D rows allow 8-byte stores (N % 4 == 0)
    int vec16;            // 1 if D rows allow 16-byte stores (N % 8 == 0, D 16-byte aligned)
    int scales_aligned;   // 1 if every scale row starts on a 4-byte boundary
    int lay;              // bit 0: A stored MN-major (K x M), bit 1: B stored MN-major (K x N)
    int ldam, ldbm;       // MN-major A / B: bytes per K-row (M or N elements)
    int ec;               // 8-bit MX element codes: A in bits 0..2, B in 3..5 (0 = E4M3, 1 = E5M2)
    int cv;               // 8-bit MX GEMM with E2M1 operands: bit 0 A, bit 1 B (widened to E4M3)
    int ldc;              // bytes per row of such an E2M1 operand (K / 2)
    float alpha;          // applied to the fp32 accumulator before rounding
    // Grouped GEMM (ngroups > 0): group g owns rows goff[g] .. goff[g+1]-1 of A
    // and D, the g-th N x K block of B (and of sB) and output tiles
    // gtiles[g] .. gtiles[g+1]-1 (tiles_m = gtiles[ngroups], tiles_n = 1);
    // its results are scaled by galpha[g] instead of alpha.
    int ngroups;
    int goff[kMaxGroups + 1];
    int gtiles[kMaxGroups + 1];
    float galpha[kMaxGroups];

    int blk6;             // FP6 kernel: operand rows stored stage-blocked (see gemm_mxfp6.hip), rows
                          // padded to a multiple of 8
};

// Output tile shapes (rows of A x rows of B per tile).  Square tiles are the
// default; skinny tiles serve problems whose square tiles would leave CUs idle.
enum Shape : int { kShapeSquare = 0, kShapeSkinny = 1 };
constexpr int kSquareTM = 256, kSquareTN = 256;
constexpr int kSkinnyTM = 256, kSkinnyTN = 64;

hipError_t launch_gemm(int fmt, int shape, const Params &p, int grid, hipStream_t stream);
// The native FP6 kernel's conditions beyond FP6 on both sides: K-major, K a
// multiple of 128 (whole stages), scale rows on 4-byte boundaries, 256 x 256
// tiles.
constexpr int kFp6StageK = 128;

// Quantisers (quant.hip): n elements of a row-major array whose rows are whole
// blocks (n a multiple of 32 for MX, 16 for NVFP4, 8 for bf16); x, codes and
// out 16-byte aligned.  NVFP4 uses *t as the tensor-amax accumulator and
// leaves the tensor scale there.
hipError_t launch_quant_mx(int elem, const float *x, int64_t n, uint8_t *codes, uint8_t *scales, int cus,
                           hipStream_t stream);
hipError_t launch_quant_nvfp4(const float *x, int64_t n, uint8_t *codes, uint8_t *scales, float *t, int cus,
                              hipStream_t stream);
// NVFP4 operand of n elements (packed E2M1 codes, E4M3 scales per 16; n a
// multiple of 32, codes and out 16-byte aligned) -> MXFP8 (E4M3 codes, E8M0
// scales per 32) for the FP8-rate NVFP4 GEMM.
hipError_t launch_requant_nvfp4_mx8(const uint8_t *codes, const uint8_t *scales, int64_t n, uint8_t *out,
                                    uint8_t *out_scales, int cus, hipStream_t stream);
// NVFP4 operand of rows x K elements (K-major) -> MXFP6 E2M3 (packed codes,
// E8M0 scales per 32, row-major) for the FP4-rate NVFP4 GEMM; out 8-byte
// aligned.  blocked: codes in the FP6 kernel's stage-blocked layout (K a
// multiple of 128), rows padded to a multiple of 8 with zero codes.
hipError_t launch_requant_nvfp4_e2m3(const uint8_t *codes, const uint8_t *scales, int64_t rows, int64_t K,
                                     bool blocked, uint8_t *out, uint8_t *out_scales, int cus, hipStream_t stream);
hipError_t launch_quant_bf16(const float *x, int64_t n, uint16_t *out, int cus, hipStream_t stream);

// The FP8-rate NVFP4 GEMM behind both of its entry points (dbs.cpp): host
// validation of the arguments (a dbs_status, with the error text recorded),
// its workspace size, and the requantisation into `workspace` plus the GEMM.
int nvfp4_fp8_check(const void *A, const uint8_t *sA, const void *B, const uint8_t *sB, const void *D, int64_t M,
                    int64_t N, int64_t K, int la, int lb);
int64_t nvfp4_fp8_workspace_bytes(int64_t M, int64_t N, int64_t K);
int nvfp4_fp8_run(const void *A, const uint8_t *sA, float tA, const void *B, const uint8_t *sB, float tB, void *D,
                  int64_t M, int64_t N, int64_t K, void *workspace, size_t workspace_bytes, hipStream_t stream);
// Records the text dbs_last_error() returns on this thread.
void set_error(const char *msg);

}  // namespace dbs
