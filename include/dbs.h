/*
 * dbs.h -- C ABI of the MI355X (gfx950) block-scaled GEMM library libdbs.so
 *
 *     D = bf16( alpha * (sA (.) A) . (sB (.) B)^T )      fp32 accumulation
 *
 * A is M x K, B is N x K (both K-major: K is the contiguous dimension), D is
 * M x N row-major bf16.  "(.)" applies one scale per block of consecutive K
 * elements of a row.  The operation is the A-times-B-transposed GEMM that the
 * "ThunderKittens Now on NVIDIA Vera Rubin NVL72" post builds on (mma_ABt,
 * section on the new Vera Rubin features, item 1); block scales are separate
 * tensors loaded next to their operand tiles ("ThunderKittens 2.0", sections
 * 1.2 and 2.1).  Formats (bit layouts per the OCP Microscaling v1.0 spec):
 *
 *   gemm_bf16   BF16 elements, no scales, alpha = 1
 *   gemm_mx     E4M3 or E2M1 elements, one E8M0 scale per 32 K elements, alpha = 1
 *   gemm_nvfp4  E2M1 elements, one E4M3 scale per 16 K elements, alpha = tA * tB
 *
 * Memory (all pointers are DEVICE pointers; dense, no leading dimensions):
 *   A   : M rows of K elements.  bf16: 2 bytes/element; E4M3: 1 byte; E2M1:
 *         two elements per byte, element 2j in bits [3:0], 2j+1 in bits [7:4].
 *   B   : N rows, same encoding as A.
 *   sA  : M rows of K/bs scale codes (1 byte each), row-major; bs = 32 (MX),
 *         16 (NVFP4).  sB likewise with N rows.
 *   D   : M x N bf16, row-major, fully overwritten.  Must not alias inputs.
 *   tA, tB : host fp32 values (NVFP4 per-tensor scales).
 *
 * Ownership and threading: the caller owns every buffer.  A call validates its
 * arguments on the host, then enqueues exactly one kernel on `stream` and
 * returns without synchronising; faults inside the kernel surface at the
 * caller's next synchronisation of that stream.  The library allocates no
 * device memory and keeps only a per-device cache of the CU count, so calls
 * from several host threads are safe.
 *
 * Errors: DBS_EINVAL is returned before any device work for a null pointer,
 * M, N or K <= 0, a K the format cannot take (see each entry point), a base
 * pointer of A or B not 16-byte aligned, or sizes beyond the documented
 * limits.  DBS_EUNSUPPORTED marks valid requests not implemented here (the
 * MN-major layouts).  DBS_EHIP means the HIP runtime reported an error (no
 * device, launch failure); dbs_last_error() then holds its text.
 */
#ifndef DBS_H
#define DBS_H

#include <stdint.h>

#if defined(__HIPCC__) || defined(__HIP_PLATFORM_AMD__)
#include <hip/hip_runtime_api.h>
#else
typedef struct ihipStream_t *hipStream_t;
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DBS_OK = 0,
    DBS_EINVAL = 1,
    DBS_EUNSUPPORTED = 2,
    DBS_EHIP = 3
} dbs_status;

/* Per-operand layout.  K_MAJOR: A is M x K, B is N x K with K contiguous.
 * MN_MAJOR (A stored K x M, B stored K x N) is reserved: DBS_EUNSUPPORTED. */
typedef enum {
    DBS_K_MAJOR = 0,
    DBS_MN_MAJOR = 1
} dbs_layout;

/* MX element formats; the values equal gfx950's f8f6f4 MFMA format codes. */
typedef enum {
    DBS_E4M3 = 0,
    DBS_E2M1 = 4
} dbs_mx_elem;

/*
 * BF16 GEMM.  A, B: bf16 (uint16 bit patterns).  K must be a multiple of 8
 * and at most 2^21.  M and N at most 2^25 (for every entry point).
 */
dbs_status gemm_bf16(const void *A, const void *B, void *D,
                     int64_t M, int64_t N, int64_t K,
                     dbs_layout la, dbs_layout lb, hipStream_t stream);

/*
 * MX GEMM (MXFP8 for elem = DBS_E4M3, MXFP4 for elem = DBS_E2M1): elements of
 * A and B in `elem`, E8M0 scales sA (M x K/32), sB (N x K/32).  Both operands
 * use the same element format.  K must be a multiple of 32, at most 2^22.
 */
dbs_status gemm_mx(dbs_mx_elem elem,
                   const void *A, const uint8_t *sA,
                   const void *B, const uint8_t *sB, void *D,
                   int64_t M, int64_t N, int64_t K,
                   dbs_layout la, dbs_layout lb, hipStream_t stream);

/*
 * NVFP4 GEMM: packed E2M1 elements, E4M3 block scales sA (M x K/16) and sB
 * (N x K/16), per-tensor fp32 scales tA, tB; D = bf16(tA*tB * sum).  The
 * format fixes K to a multiple of 16; this implementation needs a multiple
 * of 32 (DBS_EUNSUPPORTED otherwise), at most 2^22.
 */
dbs_status gemm_nvfp4(const void *A, const uint8_t *sA, float tA,
                      const void *B, const uint8_t *sB, float tB, void *D,
                      int64_t M, int64_t N, int64_t K,
                      dbs_layout la, dbs_layout lb, hipStream_t stream);

/* Static text for a status code. */
const char *dbs_status_str(dbs_status st);

/* Text of the last error recorded on the calling host thread ("" if none). */
const char *dbs_last_error(void);

/* Library ABI version (major * 100 + minor). */
int dbs_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DBS_H */
