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
 *   gemm_mx     E4M3, E5M2, E2M3, E3M2 or E2M1 elements, one E8M0 scale per 32 K elements, alpha = 1
 *   gemm_nvfp4  E2M1 elements, one E4M3 scale per 16 K elements, alpha = tA * tB
 *
 * Memory (all pointers are DEVICE pointers; dense, no leading dimensions):
 *   A   : M rows of K elements (K-major, the default).  bf16: 2 bytes/element;
 *         E4M3: 1 byte; E2M1: two elements per byte, element 2j in bits [3:0],
 *         2j+1 in bits [7:4].  MN-major (la = DBS_MN_MAJOR): K rows of M
 *         elements, i.e. A^T stored K-major, E2M1 pairs then packing
 *         consecutive M of one K-row (element (k, 2i) in bits [3:0]).
 *   B   : N rows, same encoding as A (MN-major: K rows of N elements).
 *   sA  : M rows of K/bs scale codes (1 byte each), row-major; bs = 32 (MX),
 *         16 (NVFP4).  sB likewise with N rows.
 *   D   : M x N bf16, row-major, fully overwritten.  Must not alias inputs.
 *   tA, tB : host fp32 values (NVFP4 per-tensor scales).
 *
 * Ownership and threading: the caller owns every buffer.  A call validates its
 * arguments on the host, then enqueues its kernels on `stream` (one for a
 * GEMM; gemm_nvfp4_fp8, gemm_nvfp4_fp6 and the quantisers name theirs below) and
 * returns without synchronising; faults inside the kernel surface at the
 * caller's next synchronisation of that stream.  The library allocates no
 * device memory and keeps only a per-device cache of the CU count (and, for
 * gemm_nvfp4_fp8_noalloc, its static workspace array and that array's
 * address per device), so calls from several host threads are safe, except
 * overlapping gemm_nvfp4_fp8_noalloc calls on one GPU (see there).
 *
 * Errors: DBS_EINVAL is returned before any device work for a null pointer,
 * M, N or K <= 0, a K the format cannot take (see each entry point), a base
 * pointer of A or B not 16-byte aligned, or sizes beyond the documented
 * limits.  DBS_EUNSUPPORTED marks valid requests not implemented here (see
 * dbs_layout and gemm_nvfp4).  DBS_EHIP means the HIP runtime reported an
 * error (no device, launch failure); dbs_last_error() then holds its text.
 */
#ifndef DBS_H
#define DBS_H

#include <stddef.h>
#include <stdint.h>

/* the HIP runtime's stream handle (hip_runtime_api.h declares the same type;
 * repeating an identical typedef is valid C11 and C++) */
typedef struct ihipStream_t *hipStream_t;

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
 * MN_MAJOR: A stored K x M, B stored K x N (M or N contiguous); the kernels
 * stage such tiles as K-rows and read MFMA fragments out of them with the
 * gfx950 transposed LDS reads, the role the "Dissecting ThunderKittens"
 * write-up gives to layout-aware tile loads (register tiles).  Taken by
 * gemm_bf16, gemm_mx and gemm_nvfp4, for A and B independently, when each
 * MN-major operand's K-rows are whole 16-byte chunks (M or N times the
 * element bits a multiple of 128) and it stays below 2 GiB; DBS_EUNSUPPORTED
 * otherwise, and for the grouped GEMMs (K-major only).  FP4 elements of an
 * MN-major operand pack two consecutive M (or N) per byte, low nibble first.
 * Block scales keep their K-major layout (rows x K/block) either way. */
typedef enum {
    DBS_K_MAJOR = 0,
    DBS_MN_MAJOR = 1
} dbs_layout;

/* MX element formats; the values equal gfx950's f8f6f4 MFMA format codes.
 * E5M2 (OCP MX v1.0: bias 15, two mantissa bits, infinities and NaNs) is the
 * other 8-bit element of the OCP format; E2M3 (bias 1, max 7.5) and E3M2
 * (bias 3, max 28) are its FP6 elements, neither with infinities or NaNs;
 * the pages name E4M3 and E2M1.  FP6 rows pack four elements into three
 * bytes: element j of a row at bits 6j .. 6j+5 of the row's bytes read as
 * one little-endian bit string. */
typedef enum {
    DBS_E4M3 = 0,
    DBS_E5M2 = 1,
    DBS_E2M3 = 2,
    DBS_E3M2 = 3,
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
 * The BF16 GEMM of gemm_bf16 (K-major A and B) on a kernel with decoupled A
 * and B rings, each of two slots: 256 x 256 tiles on one wave per SIMD
 * (128 x 128 each, accumulators in AGPRs).  early_release_a = 1 runs the
 * schedule that the "ThunderKittens Now on NVIDIA Vera Rubin NVL72" post
 * lists among its new features (item 5), where the loader refills A's slot
 * as soon as every consumer has read it: every wave first copies a stage's A
 * fragments into registers, the waves meet, and the next-but-one A stage is
 * loaded into the slot while the stage's MFMAs run.  early_release_a = 0
 * hands A's slot back at the stage's end, as B's (the comparison).  Same
 * inputs, outputs, limits and errors as gemm_bf16, plus: K must exceed 64
 * (DBS_EUNSUPPORTED otherwise); early_release_a other than 0 or 1 is
 * DBS_EINVAL.  The result is bit for bit that of gemm_bf16 (the same fp32
 * accumulation order).  Opt-in: gemm_bf16's own kernel (two waves per SIMD)
 * is the faster one on the shapes measured.
 */
dbs_status gemm_bf16_decoupled(const void *A, const void *B, void *D,
                               int64_t M, int64_t N, int64_t K, int early_release_a, hipStream_t stream);

/*
 * MX GEMM (MXFP8 for elem = DBS_E4M3 or DBS_E5M2, MXFP6 for DBS_E2M3 or
 * DBS_E3M2, MXFP4 for elem = DBS_E2M1): elements of A and B in `elem`, E8M0
 * scales sA (M x K/32), sB (N x K/32).  K must be a multiple of 32, at most
 * 2^22.  MXFP6 is K-major only and runs as gemm_mx_mixed runs it.
 */
dbs_status gemm_mx(dbs_mx_elem elem,
                   const void *A, const uint8_t *sA,
                   const void *B, const uint8_t *sB, void *D,
                   int64_t M, int64_t N, int64_t K,
                   dbs_layout la, dbs_layout lb, hipStream_t stream);

/*
 * MX GEMM with an element format per operand: A's elements in elem_a, B's in
 * elem_b, otherwise as gemm_mx (gemm_mx(e, ...) is gemm_mx_mixed(e, e, ...)).
 * Every pairing of E4M3, E5M2 and E2M1 is taken, and FP6 (E2M3, E3M2) with
 * E4M3, E5M2 or FP6, K-major only: an FP6 operand is widened on its way into
 * LDS to the 8-bit format that holds its values exactly (E2M3 -> E4M3, E3M2 ->
 * E5M2) and multiplied at the 8-bit rate.  FP6 with E2M1 returns
 * DBS_EUNSUPPORTED.  gfx950's scaled MFMA
 * takes a format code per operand, so 8-bit pairs run at the 8-bit rate on
 * MXFP8's staging.  An E2M1 operand beside an 8-bit one (FP8 x FP4) goes to
 * the MFMA as packed E2M1 (its format code) when K is a multiple of 256, and
 * is otherwise widened to E4M3 on its way into LDS -- exactly, every E2M1
 * value being an E4M3 value, with its E8M0 scales unchanged; both run at the
 * 8-bit rate.
 * Every pair takes either layout per operand, except that an FP8 x FP4 pair
 * with an MN-major operand needs K a multiple of 256 (DBS_EUNSUPPORTED
 * otherwise); an MN-major E2M1 operand then needs M (or N) a multiple of 32.
 */
dbs_status gemm_mx_mixed(dbs_mx_elem elem_a, dbs_mx_elem elem_b,
                         const void *A, const uint8_t *sA,
                         const void *B, const uint8_t *sB, void *D,
                         int64_t M, int64_t N, int64_t K,
                         dbs_layout la, dbs_layout lb, hipStream_t stream);

/*
 * NVFP4 GEMM: packed E2M1 elements, E4M3 block scales sA (M x K/16) and sB
 * (N x K/16), per-tensor fp32 scales tA, tB; D = bf16(tA*tB * sum).  K must
 * be a multiple of 16 (the format's block), at most 2^22.  MN-major operands
 * (see dbs_layout) run on kernels that stage the packed codes and decode them
 * in registers; there a K-major operand beside an MN-major one needs K a
 * multiple of 32 (DBS_EUNSUPPORTED otherwise).
 */
dbs_status gemm_nvfp4(const void *A, const uint8_t *sA, float tA,
                      const void *B, const uint8_t *sB, float tB, void *D,
                      int64_t M, int64_t N, int64_t K,
                      dbs_layout la, dbs_layout lb, hipStream_t stream);

/*
 * FP8-rate NVFP4 GEMM (opt-in, LOSSY): the NVFP4 operands of gemm_nvfp4 are
 * first requantised to MXFP8 in `workspace` -- per block of 32 K elements
 * (two 16-element groups with E4M3 scales s0, s1) the E8M0 exponent is
 * E = floor(log2(max |s_g|)) and each element a becomes the nearest E4M3
 * code of a * s_g * 2^-E (ties to even) -- and the MXFP8 GEMM then runs at
 * the 8-bit MFMA rate, with tA * tB applied to its result.  This is the
 * FP8-rate form of the NVFP4 rescale step ("ThunderKittens 2.0", section
 * 2.1, NVFP4 scale handling), for hardware whose scaled MFMA takes only
 * E8M0 scales per 32.  Each requantised element is within 2^-4 of its exact
 * value relative to that value (half a subnormal E4M3 step, 2^-10 * 2^E,
 * absolutely, below 2^-6 * 2^E), so |D - D_exact| <= (2^-3 + 2^-8) *
 * sum_k |dA dB| + the subnormal terms; with unit scales it is exact.  K a
 * multiple of 32 (DBS_EUNSUPPORTED for K = 16 mod 32), K-major operands.
 * workspace: device memory of at least gemm_nvfp4_fp8_workspace(M, N, K)
 * bytes, 256-byte aligned, owned by the caller (overwritten, not read
 * before being written; calls that share one workspace must not overlap).
 * Two requantisation kernels and the GEMM are enqueued on `stream`.
 */
size_t gemm_nvfp4_fp8_workspace(int64_t M, int64_t N, int64_t K);    /* 0 for invalid sizes */
dbs_status gemm_nvfp4_fp8(const void *A, const uint8_t *sA, float tA,
                          const void *B, const uint8_t *sB, float tB, void *D,
                          int64_t M, int64_t N, int64_t K,
                          dbs_layout la, dbs_layout lb,
                          void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * FP4-rate NVFP4 GEMM (opt-in, LOSSY): the NVFP4 operands of gemm_nvfp4 are
 * requantised to MXFP6 E2M3 in `workspace` and multiplied at the FP6 rate of
 * gfx950's scaled MFMA, which equals its FP4 rate.  Per block of 32 K
 * elements (two 16-element groups with E4M3 scales s0, s1; m = max(|s0|,
 * |s1|)) the E8M0 exponent E is the smallest integer with 6 m <= 7.5 * 2^E
 * (the block's largest possible magnitude then fits E2M3's largest value,
 * 7.5, without saturating), and each element a becomes the nearest E2M3 code
 * of a * s_g * 2^-E (ties to even); tA * tB scales the result.  This is the
 * FP4-rate form of the NVFP4 rescale step ("ThunderKittens 2.0", section
 * 2.1) for hardware whose scaled MFMA takes only E8M0 scales per 32.  E2M3
 * keeps E4M3's three mantissa bits but only two exponent bits: each
 * requantised element is within max(2^-4 |a s_g|, 2^-4 * 2^E) of its exact
 * value, 2^E < 1.6 m, so |D - D_exact| <= sum_k (|a_k| e_b,k + |b_k| e_a,k +
 * e_a,k e_b,k) * |tA tB| plus the fp32/bf16 terms of any GEMM; with unit
 * scales it is exact.  K a multiple of 32 (DBS_EUNSUPPORTED for K = 16 mod
 * 32), K-major operands.  workspace: device memory of at least
 * gemm_nvfp4_fp6_workspace(M, N, K) bytes, 256-byte aligned, owned by the
 * caller (overwritten, not read before being written; calls sharing one
 * workspace must not overlap; its layout is internal to the library).  Two
 * requantisation kernels and the GEMM are enqueued on `stream`; the GEMM
 * runs at the FP6 rate on 256 x 256 tiles when K is a multiple of 128 and
 * those tiles fill at least a quarter of the CUs (the requantised codes are
 * then stored in that kernel's stage-blocked order), else widened to 8 bits
 * on 256 x 64 tiles (gemm_mx_mixed's FP6 paths).
 */
size_t gemm_nvfp4_fp6_workspace(int64_t M, int64_t N, int64_t K);    /* 0 for invalid sizes */
dbs_status gemm_nvfp4_fp6(const void *A, const uint8_t *sA, float tA,
                          const void *B, const uint8_t *sB, float tB, void *D,
                          int64_t M, int64_t N, int64_t K,
                          dbs_layout la, dbs_layout lb,
                          void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * gemm_nvfp4_fp8 for callers that cannot allocate device memory or pass a
 * workspace: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation.  Same arguments, validation, arithmetic and result
 * as gemm_nvfp4_fp8 (bit for bit), except that the requantisation workspace
 * is the library's own static device array of DBS_NOALLOC_WORKSPACE_BYTES
 * (64 MiB): each GPU the library runs on holds one copy from the first call
 * on it until the process ends.  A call whose gemm_nvfp4_fp8_workspace(M, N,
 * K) exceeds that returns DBS_EINVAL before any device work (use
 * gemm_nvfp4_fp8 with a caller workspace instead).  The call allocates
 * nothing: the array's device address is looked up once per device, on the
 * first call with that device current (DBS_EHIP if that fails).  Every call
 * on one GPU uses the same array, which keeps the last call's contents (each
 * call overwrites what it reads); calls that overlap on one GPU -- on
 * different streams, or from different host threads without ordering --
 * race for it and must not be issued.
 */
#define DBS_NOALLOC_WORKSPACE_BYTES ((size_t)64 << 20)
dbs_status gemm_nvfp4_fp8_noalloc(const void *A, const uint8_t *sA, float tA,
                                  const void *B, const uint8_t *sB, float tB, void *D,
                                  int64_t M, int64_t N, int64_t K,
                                  dbs_layout la, dbs_layout lb, hipStream_t stream);

/*
 * Grouped GEMMs (mixture-of-experts layout): G groups (1 <= G <= 64) share N
 * and K.  Group g owns rows offsets[g] .. offsets[g+1]-1 of A and of D (and
 * of sA), and the g-th block of N rows of B (B holds G x N rows of K
 * elements, sB G x N scale rows):  D_g = bf16(alpha_g (sA_g (.) A_g) .
 * (sB_g (.) B_g)^T).  offsets (G + 1 values, offsets[0] = 0, non-decreasing,
 * empty groups allowed) and tB (G values) are HOST arrays; everything else
 * is as for the single GEMMs (K-major operands only; gemm_grouped_mx takes
 * E4M3, E5M2 or E2M1 for both operands).  alpha_g = 1, or
 * tA * tB[g] for NVFP4.  One kernel launch covers every group's tiles.  The
 * grouped GEMM is the mixture-of-experts workload the "ThunderKittens 2.0"
 * post points to (section on what comes next).
 */
dbs_status gemm_grouped_bf16(const void *A, const void *B, void *D, const int64_t *offsets, int64_t G, int64_t N,
                             int64_t K, hipStream_t stream);
dbs_status gemm_grouped_mx(dbs_mx_elem elem, const void *A, const uint8_t *sA, const void *B, const uint8_t *sB,
                           void *D, const int64_t *offsets, int64_t G, int64_t N, int64_t K, hipStream_t stream);
dbs_status gemm_grouped_nvfp4(const void *A, const uint8_t *sA, float tA, const void *B, const uint8_t *sB,
                              const float *tB, void *D, const int64_t *offsets, int64_t G, int64_t N, int64_t K,
                              hipStream_t stream);

/*
 * Quantisers: fp32 -> the GEMM's input formats, on the GPU.  x holds `rows`
 * rows of K fp32 values (row-major, finite); x and codes must be 16-byte
 * aligned.  Every call enqueues its kernels on `stream` and returns.
 *
 * quant_mx: K a multiple of 32.  Per block of 32 consecutive elements of a
 *   row, E8M0 scale 2^e with e = floor(log2(amax / emax)) (emax = 448 for
 *   DBS_E4M3, 57344 for DBS_E5M2, 6 for DBS_E2M1; e clamped to [-127, 127];
 *   scale 1 for an all-zero block), then each element the nearest E4M3 /
 *   E5M2 / E2M1 code of x / 2^e.  codes: rows x K bytes (E4M3, E5M2) or
 *   rows x K/2 packed bytes (E2M1,
 *   element 2j in the low nibble); scales: rows x K/32 bytes.  The scale rule
 *   follows the MX scale definition (OCP MX v1.0) with the workloads'
 *   floor(log2(amax / emax)) exponent.  FP6 (DBS_E2M3, DBS_E3M2): e =
 *   floor(log2(amax)) - 2 (E2M3) or - 4 (E3M2), the OCP recipe; codes rows x
 *   3K/4 packed bytes (see dbs_mx_elem).
 * quant_nvfp4: K a multiple of 16.  t (device, one float, out) = amax /
 *   (6 * 448) over the whole array (1 if it is all zero); per block of 16 the
 *   E4M3 scale s = nearest(amax_block / (6 t)); each element the nearest E2M1
 *   code of x / (s t); every step in correctly rounded fp32.  codes: rows x
 *   K/2 packed bytes; scales: rows x K/16 bytes.  t doubles as the amax
 *   accumulator while the call's kernels run (four launches on `stream`).
 *   The per-tensor plus per-16 E4M3 layout is the NVFP4 format of the
 *   "ThunderKittens 2.0" post (section 2.1).
 * quant_bf16: n a multiple of 8; out: n bf16 values (uint16), nearest even.
 *
 * "Nearest" rounds to the closest representable value, ties to the code with
 * an even mantissa, saturating at the largest finite value and keeping the
 * sign of zero.  Errors as for the GEMMs (DBS_EINVAL before any device work).
 */
dbs_status quant_mx(dbs_mx_elem elem, const float *x, int64_t rows, int64_t K, void *codes, uint8_t *scales,
                    hipStream_t stream);
dbs_status quant_nvfp4(const float *x, int64_t rows, int64_t K, void *codes, uint8_t *scales, float *t,
                       hipStream_t stream);
dbs_status quant_bf16(const float *x, int64_t n, void *out, hipStream_t stream);

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
