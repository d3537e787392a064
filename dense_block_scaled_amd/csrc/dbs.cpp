// dbs.cpp -- the C ABI declared in include/dbs.h: argument validation, tile
// configuration and launch of the gfx950 kernels in gemm.hip.
#include "dbs.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdio>
#include <cstring>

#include "launch.h"

namespace {

thread_local char g_err[512] = "";

dbs_status fail(dbs_status st, const char *msg)
{
    std::snprintf(g_err, sizeof(g_err), "%s", msg);
    return st;
}

dbs_status fail_hip(hipError_t e, const char *what)
{
    std::snprintf(g_err, sizeof(g_err), "%s: %s", what, hipGetErrorString(e));
    return DBS_EHIP;
}

// CU count per device, looked up once (the library's only state).
constexpr int kMaxDevices = 64;
std::atomic<int> g_cus[kMaxDevices];

dbs_status device_cus(int *cus)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail_hip(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(DBS_EHIP, "device index out of range");
    int c = g_cus[dev].load(std::memory_order_relaxed);
    if (c <= 0) {
        e = hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return fail_hip(e, "hipDeviceGetAttribute");
        if (c <= 0) return fail(DBS_EHIP, "device reports no compute units");
        g_cus[dev].store(c, std::memory_order_relaxed);
    }
    *cus = c;
    return DBS_OK;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

dbs_status check_common(const void *A, const void *B, const void *D, int64_t M, int64_t N, int64_t K,
                        dbs_layout la, dbs_layout lb, int64_t kmax)
{
    if (!A || !B || !D) return fail(DBS_EINVAL, "null pointer argument");
    if (M <= 0 || N <= 0 || K <= 0) return fail(DBS_EINVAL, "M, N and K must be positive");
    if (M > (int64_t(1) << 25) || N > (int64_t(1) << 25)) return fail(DBS_EINVAL, "M or N above 2^25");
    if (K > kmax) return fail(DBS_EINVAL, "K above the supported maximum");
    if ((la != DBS_K_MAJOR && la != DBS_MN_MAJOR) || (lb != DBS_K_MAJOR && lb != DBS_MN_MAJOR))
        return fail(DBS_EINVAL, "unknown layout value");
    if (!aligned(A, 16) || !aligned(B, 16)) return fail(DBS_EINVAL, "A and B must be 16-byte aligned");
    if (!aligned(D, 2)) return fail(DBS_EINVAL, "D must be 2-byte aligned");
    return DBS_OK;
}

// MN-major operands (stored K x M for A, K x N for B): each K-row of `rows`
// elements must be whole 16-byte chunks, and the operand must stay below
// 2^31 bytes with a stage of slack (the kernels address it with 32-bit
// offsets from a tile's first column).
dbs_status check_mn(dbs_layout la, dbs_layout lb, int64_t M, int64_t N, int64_t K, int elem_bits)
{
    auto one = [&](dbs_layout l, int64_t rows, const char *what) -> dbs_status {
        if (l != DBS_MN_MAJOR) return DBS_OK;
        if ((rows * elem_bits) % 128)
            return fail(DBS_EUNSUPPORTED, what);
        if ((K + 256) * (rows * elem_bits / 8) >= (int64_t(1) << 31))
            return fail(DBS_EUNSUPPORTED, "MN-major operand of 2 GiB or more");
        return DBS_OK;
    };
    dbs_status st = one(la, M, "MN-major A needs M * element bits to be a multiple of 128 (16-byte rows)");
    if (st != DBS_OK) return st;
    return one(lb, N, "MN-major B needs N * element bits to be a multiple of 128 (16-byte rows)");
}

// Groups of a grouped GEMM (host arrays): G + 1 row offsets and one output
// scale per group.
struct Groups {
    const int64_t *off;
    int64_t G;
    const float *alpha;
};

dbs_status run(int fmt, const void *A, const uint8_t *sA, const void *B, const uint8_t *sB, void *D, int64_t M,
               int64_t N, int64_t K, float alpha, int elem_bits, int block, hipStream_t stream,
               const Groups *groups = nullptr, dbs_layout la = DBS_K_MAJOR, dbs_layout lb = DBS_K_MAJOR,
               int ec = 0, int cv = 0, int blk6 = 0)
{
    int cus = 0;
    dbs_status st = device_cus(&cus);
    if (st != DBS_OK) return st;

    dbs::Params p{};
    p.A = static_cast<const uint8_t *>(A);
    p.B = static_cast<const uint8_t *>(B);
    p.sA = sA;
    p.sB = sB;
    p.D = static_cast<uint16_t *>(D);
    p.M = (int)M;
    p.N = (int)N;
    p.K = (int)K;
    p.lda = (int)(K * elem_bits / 8);
    p.sld = block ? (int)(K / block) : 0;
    p.lay = (la == DBS_MN_MAJOR ? 1 : 0) | (lb == DBS_MN_MAJOR ? 2 : 0);
    // (an E2M1 operand of an 8-bit kernel, cv: K-rows of M / 2 or N / 2 bytes)
    p.ldam = (int)((cv & 3) == 1 ? M / 2 : M * elem_bits / 8);
    p.ldbm = (int)((cv >> 2) == 1 ? N / 2 : N * elem_bits / 8);
    p.ec = ec;
    p.cv = cv;
    p.blk6 = blk6;
    // rows of a widened operand: E2M1 K/2 bytes, FP6 3K/4
    p.ldc = (int)(((cv & 3) >= 2 || (cv >> 2) >= 2) ? K / 4 * 3 : K / 2);
    // square tiles unless they would fill at most half of the CUs
    auto tiles_of = [&](int64_t rows, int64_t tm_, int64_t tn_) { return ((rows + tm_ - 1) / tm_) * ((N + tn_ - 1) / tn_); };
    int64_t sq_tiles = 0;
    if (groups) {
        for (int64_t g = 0; g < groups->G; ++g)
            sq_tiles += tiles_of(groups->off[g + 1] - groups->off[g], dbs::kSquareTM, dbs::kSquareTN);
    } else {
        sq_tiles = tiles_of(M, dbs::kSquareTM, dbs::kSquareTN);
    }
    // FP6 operands (widened through registers) run on 256 x 64 tiles: on
    // 256 x 256 tiles their staging registers spill.  The MX kernels (no
    // widened operand) keep square tiles down to a quarter of the CUs: at
    // half of them (128 tiles) the square kernels measured 20-27% faster
    // than 256 x 64 tiles, BF16 and NVFP4 10% slower.
    const bool fp6 = (cv & 3) >= 2 || (cv >> 2) >= 2;
    const bool mx = (fmt == dbs::kMXFP8 || fmt == dbs::kMXFP4 || fmt == dbs::kMXFP6) && cv == 0;
    // (the early-A BF16 kernel and the FP6-rate kernel have square tiles
    // only; fp6_native decides when the latter runs)
    const int shape = (fmt == dbs::kBF16EA || fmt == dbs::kBF16EL || fmt == dbs::kMXFP6) ? dbs::kShapeSquare
                      : ((mx ? 4 : 2) * sq_tiles <= cus || fp6) ? dbs::kShapeSkinny : dbs::kShapeSquare;
    const int tm = shape == dbs::kShapeSkinny ? dbs::kSkinnyTM : dbs::kSquareTM;
    const int tn = shape == dbs::kShapeSkinny ? dbs::kSkinnyTN : dbs::kSquareTN;
    p.tiles_m = (int)((M + tm - 1) / tm);
    p.tiles_n = (int)((N + tn - 1) / tn);
    if (groups) {
        // every group's tiles in sequence: tiles_m holds the total
        int64_t acc = 0;
        p.ngroups = (int)groups->G;
        for (int64_t g = 0; g < groups->G; ++g) {
            p.goff[g] = (int)groups->off[g];
            p.gtiles[g] = (int)acc;
            p.galpha[g] = groups->alpha ? groups->alpha[g] : alpha;
            acc += tiles_of(groups->off[g + 1] - groups->off[g], tm, tn);
        }
        p.goff[groups->G] = (int)groups->off[groups->G];
        p.gtiles[groups->G] = (int)std::min<int64_t>(acc, INT32_MAX);
        if (acc == 0) return DBS_OK;       // all groups empty: nothing to compute
        if (acc > INT32_MAX) return fail(DBS_EINVAL, "too many output tiles");
        p.tiles_m = (int)acc;
        p.tiles_n = 1;
    }
    p.group_m = 4;
    p.vec_store = (N % 4 == 0 && aligned(D, 8)) ? 1 : 0;
    p.vec16 = (N % 8 == 0 && aligned(D, 16)) ? 1 : 0;
    p.scales_aligned = (block == 0 || (p.sld % 4 == 0 && aligned(sA, 4) && aligned(sB, 4))) ? 1 : 0;
    p.alpha = alpha;

    const int64_t tiles = (int64_t)p.tiles_m * p.tiles_n;
    if (tiles > INT32_MAX) return fail(DBS_EINVAL, "too many output tiles");
    const int grid = (int)std::min<int64_t>(tiles, cus);
    hipError_t e = dbs::launch_gemm(fmt, shape, p, grid, stream);
    if (e == hipErrorNotSupported)
        return fail(DBS_EUNSUPPORTED, "no kernel for this element format pair, layout and tile shape");
    if (e != hipSuccess) return fail_hip(e, "kernel launch");
    g_err[0] = '\0';
    return DBS_OK;
}

// The f8f6f4 MFMA format code of an 8-bit MX element (0 E4M3, 1 E5M2).
int mx8_code(dbs_mx_elem e) { return e == DBS_E5M2 ? 1 : 0; }

bool mx_elem_known(dbs_mx_elem e)
{
    return e == DBS_E4M3 || e == DBS_E5M2 || e == DBS_E2M1 || e == DBS_E2M3 || e == DBS_E3M2;
}

bool is_fp6(dbs_mx_elem e) { return e == DBS_E2M3 || e == DBS_E3M2; }

// An operand that the 8-bit kernels widen on its way into LDS: its source
// code (1 E2M1, 2 E2M3, 3 E3M2; 0 for E4M3 / E5M2) and the MFMA code of the
// 8-bit format it is widened to (E2M1, E2M3 -> E4M3; E3M2 -> E5M2).
int cv_source(dbs_mx_elem e) { return e == DBS_E2M1 ? 1 : e == DBS_E2M3 ? 2 : e == DBS_E3M2 ? 3 : 0; }
int mfma8_code(dbs_mx_elem e) { return (e == DBS_E5M2 || e == DBS_E3M2) ? 1 : 0; }

int64_t align256(int64_t x) { return (x + 255) / 256 * 256; }

// Workspace layout: A codes (M x K), B codes (N x K), A scales (M x K/32),
// B scales (N x K/32), each starting on a 256-byte boundary.
struct Fp8Ws {
    uint8_t *a, *b, *sa, *sb;
    int64_t bytes;
};

Fp8Ws fp8_ws(void *base, int64_t M, int64_t N, int64_t K)
{
    const int64_t ob = align256(M * K), osa = ob + align256(N * K), osb = osa + align256(M * K / 32);
    Fp8Ws w;
    w.bytes = osb + align256(N * K / 32);
    uint8_t *p = static_cast<uint8_t *>(base);
    w.a = p;
    w.b = p ? p + ob : nullptr;
    w.sa = p ? p + osa : nullptr;
    w.sb = p ? p + osb : nullptr;
    return w;
}

int64_t round8(int64_t x) { return (x + 7) / 8 * 8; }

// Workspace layout of the FP4-rate path: A codes (M x 3K/4, rows padded to a
// multiple of 8: the FP6-rate kernel's stage-blocked layout needs whole
// groups of 8), B codes (N x 3K/4, likewise), A scales (M x K/32), B scales
// (N x K/32), each on a 256-byte boundary.
Fp8Ws fp6_ws(void *base, int64_t M, int64_t N, int64_t K)
{
    const int64_t ob = align256(round8(M) * K / 4 * 3), osa = ob + align256(round8(N) * K / 4 * 3),
                  osb = osa + align256(M * K / 32);
    Fp8Ws w;
    w.bytes = osb + align256(N * K / 32);
    uint8_t *p = static_cast<uint8_t *>(base);
    w.a = p;
    w.b = p ? p + ob : nullptr;
    w.sa = p ? p + osa : nullptr;
    w.sb = p ? p + osb : nullptr;
    return w;
}

// Whether FP6 x FP6 (K-major) runs at the FP6 rate: on 256 x 256 tiles when
// those occupy at least a quarter of the CUs, K is whole 128-K stages and
// the scale rows start on 4-byte boundaries.  At exactly a quarter (the
// 256 x 16384 x 8192 FP4-rate NVFP4 shape: 64 tiles) the FP6-rate kernel on
// 64 CUs measured 4% faster than the widening kernel's 256 tiles of 256 x 64.
dbs_status fp6_native(int64_t M, int64_t N, int64_t K, const uint8_t *sA, const uint8_t *sB, bool *native)
{
    *native = false;
    if (K % dbs::kFp6StageK || !aligned(sA, 4) || !aligned(sB, 4)) return DBS_OK;
    int cus = 0;
    dbs_status st = device_cus(&cus);
    if (st != DBS_OK) return st;
    const int64_t sq = ((M + dbs::kSquareTM - 1) / dbs::kSquareTM) * ((N + dbs::kSquareTN - 1) / dbs::kSquareTN);
    *native = 4 * sq >= cus;
    return DBS_OK;
}

// FP6 on both sides, K-major (elements ea, eb: E2M3 or E3M2): at the FP6
// rate where fp6_native says so, otherwise widened to 8 bits on 256 x 64
// tiles.  blocked: the operands are stage-blocked (only the FP6-rate kernel
// reads that layout; the caller has checked fp6_native).
dbs_status fp6_gemm(dbs_mx_elem ea, dbs_mx_elem eb, const void *A, const uint8_t *sA, const void *B,
                    const uint8_t *sB, void *D, int64_t M, int64_t N, int64_t K, float alpha, hipStream_t stream,
                    bool blocked = false)
{
    bool native = false;
    dbs_status st = fp6_native(M, N, K, sA, sB, &native);
    if (st != DBS_OK) return st;
    if (native)
        return run(dbs::kMXFP6, A, sA, B, sB, D, M, N, K, alpha, 6, 32, stream, nullptr, DBS_K_MAJOR, DBS_K_MAJOR,
                   (int)ea | ((int)eb << 3), 0, blocked ? 1 : 0);
    if (blocked) return fail(DBS_EINVAL, "stage-blocked FP6 operands need the FP6-rate kernel");
    const int cv = cv_source(ea) | (cv_source(eb) << 2);
    const int ec = mfma8_code(ea) | (mfma8_code(eb) << 3);
    return run(dbs::kMXFP8, A, sA, B, sB, D, M, N, K, alpha, 8, 32, stream, nullptr, DBS_K_MAJOR, DBS_K_MAJOR, ec,
               cv);
}

}  // namespace

namespace dbs {

void set_error(const char *msg) { std::snprintf(g_err, sizeof(g_err), "%s", msg); }

int nvfp4_fp8_check(const void *A, const uint8_t *sA, const void *B, const uint8_t *sB, const void *D, int64_t M,
                    int64_t N, int64_t K, int la, int lb)
{
    if (!sA || !sB) return fail(DBS_EINVAL, "null pointer argument");
    dbs_status st = check_common(A, B, D, M, N, K, static_cast<dbs_layout>(la), static_cast<dbs_layout>(lb),
                                 int64_t(1) << 22);
    if (st != DBS_OK) return st;
    if (K % 16) return fail(DBS_EINVAL, "nvfp4: K must be a multiple of 16");
    if (K % 32) return fail(DBS_EUNSUPPORTED, "nvfp4 requantised: K must be a multiple of 32 (whole MX blocks)");
    if (la != DBS_K_MAJOR || lb != DBS_K_MAJOR)
        return fail(DBS_EUNSUPPORTED, "nvfp4 requantised: only K-major A and B are implemented");
    return DBS_OK;
}

int64_t nvfp4_fp8_workspace_bytes(int64_t M, int64_t N, int64_t K) { return fp8_ws(nullptr, M, N, K).bytes; }

int nvfp4_fp8_run(const void *A, const uint8_t *sA, float tA, const void *B, const uint8_t *sB, float tB, void *D,
                  int64_t M, int64_t N, int64_t K, void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    if (!aligned(workspace, 256)) return fail(DBS_EINVAL, "workspace must be 256-byte aligned");
    const Fp8Ws w = fp8_ws(workspace, M, N, K);
    if ((int64_t)workspace_bytes < w.bytes) return fail(DBS_EINVAL, "workspace smaller than gemm_nvfp4_fp8_workspace()");
    int cus = 0;
    dbs_status st = device_cus(&cus);
    if (st != DBS_OK) return st;
    hipError_t e = launch_requant_nvfp4_mx8(static_cast<const uint8_t *>(A), sA, M * K, w.a, w.sa, cus, stream);
    if (e == hipSuccess)
        e = launch_requant_nvfp4_mx8(static_cast<const uint8_t *>(B), sB, N * K, w.b, w.sb, cus, stream);
    if (e != hipSuccess) return fail_hip(e, "kernel launch");
    return run(kMXFP8, w.a, w.sa, w.b, w.sb, D, M, N, K, tA * tB, 8, 32, stream);
}

}  // namespace dbs

extern "C" {

dbs_status gemm_bf16(const void *A, const void *B, void *D, int64_t M, int64_t N, int64_t K, dbs_layout la,
                     dbs_layout lb, hipStream_t stream)
{
    dbs_status st = check_common(A, B, D, M, N, K, la, lb, int64_t(1) << 21);
    if (st != DBS_OK) return st;
    if (K % 8) return fail(DBS_EINVAL, "bf16: K must be a multiple of 8");
    if ((st = check_mn(la, lb, M, N, K, 16)) != DBS_OK) return st;
    return run(dbs::kBF16, A, nullptr, B, nullptr, D, M, N, K, 1.0f, 16, 0, stream, nullptr, la, lb);
}

dbs_status gemm_bf16_decoupled(const void *A, const void *B, void *D, int64_t M, int64_t N, int64_t K,
                               int early_release_a, hipStream_t stream)
{
    dbs_status st = check_common(A, B, D, M, N, K, DBS_K_MAJOR, DBS_K_MAJOR, int64_t(1) << 21);
    if (st != DBS_OK) return st;
    if (K % 8) return fail(DBS_EINVAL, "bf16: K must be a multiple of 8");
    if (early_release_a != 0 && early_release_a != 1) return fail(DBS_EINVAL, "early_release_a must be 0 or 1");
    if (K <= 64) return fail(DBS_EUNSUPPORTED, "bf16 decoupled rings: K must exceed 64 (two stages)");
    return run(early_release_a ? dbs::kBF16EA : dbs::kBF16EL, A, nullptr, B, nullptr, D, M, N, K, 1.0f, 16, 0,
               stream);
}

dbs_status gemm_mx_mixed(dbs_mx_elem elem_a, dbs_mx_elem elem_b, const void *A, const uint8_t *sA, const void *B,
                         const uint8_t *sB, void *D, int64_t M, int64_t N, int64_t K, dbs_layout la, dbs_layout lb,
                         hipStream_t stream)
{
    if (!mx_elem_known(elem_a) || !mx_elem_known(elem_b)) return fail(DBS_EINVAL, "mx: unknown element format");
    if (!sA || !sB) return fail(DBS_EINVAL, "null pointer argument");
    dbs_status st = check_common(A, B, D, M, N, K, la, lb, int64_t(1) << 22);
    if (st != DBS_OK) return st;
    if (K % 32) return fail(DBS_EINVAL, "mx: K must be a multiple of 32");
    const bool fp4_a = elem_a == DBS_E2M1, fp4_b = elem_b == DBS_E2M1;
    const bool fp6_a = is_fp6(elem_a), fp6_b = is_fp6(elem_b);
    if ((fp4_a && fp6_b) || (fp6_a && fp4_b))
        return fail(DBS_EUNSUPPORTED, "mx: E2M1 with an FP6 operand is not implemented");
    if ((fp6_a || fp6_b) && (la != DBS_K_MAJOR || lb != DBS_K_MAJOR))
        return fail(DBS_EUNSUPPORTED, "mx: FP6 operands are K-major only");
    // E2M1 x E2M1 is the MXFP4 kernel; otherwise the 8-bit kernels, where an
    // E2M1 or FP6 operand is widened to the 8-bit format that holds its
    // values exactly (cv, per operand) and E2M1 beside an 8-bit operand goes
    // packed to the MFMA when K % 256 == 0 (the kernels pick)
    const int cv = fp4_a && fp4_b ? 0 : cv_source(elem_a) | (cv_source(elem_b) << 2);
    const int ec = fp4_a && fp4_b ? 0 : mfma8_code(elem_a) | (mfma8_code(elem_b) << 3);
    if (cv != 0 && (la != DBS_K_MAJOR || lb != DBS_K_MAJOR) && K % 256)
        return fail(DBS_EUNSUPPORTED, "mx: 8-bit x E2M1 pairs with an MN-major operand need K % 256 == 0");
    const int bits = fp4_a && fp4_b ? 4 : 8;
    if (fp6_a && fp6_b) return fp6_gemm(elem_a, elem_b, A, sA, B, sB, D, M, N, K, 1.0f, stream);
    if ((st = check_mn(la, DBS_K_MAJOR, M, N, K, fp4_a ? 4 : 8)) != DBS_OK) return st;
    if ((st = check_mn(DBS_K_MAJOR, lb, M, N, K, fp4_b ? 4 : 8)) != DBS_OK) return st;
    return run(bits == 8 ? dbs::kMXFP8 : dbs::kMXFP4, A, sA, B, sB, D, M, N, K, 1.0f, bits, 32, stream, nullptr,
               la, lb, ec, cv);
}

dbs_status gemm_mx(dbs_mx_elem elem, const void *A, const uint8_t *sA, const void *B, const uint8_t *sB, void *D,
                   int64_t M, int64_t N, int64_t K, dbs_layout la, dbs_layout lb, hipStream_t stream)
{
    return gemm_mx_mixed(elem, elem, A, sA, B, sB, D, M, N, K, la, lb, stream);
}

dbs_status gemm_nvfp4(const void *A, const uint8_t *sA, float tA, const void *B, const uint8_t *sB, float tB,
                      void *D, int64_t M, int64_t N, int64_t K, dbs_layout la, dbs_layout lb, hipStream_t stream)
{
    if (!sA || !sB) return fail(DBS_EINVAL, "null pointer argument");
    dbs_status st = check_common(A, B, D, M, N, K, la, lb, int64_t(1) << 22);
    if (st != DBS_OK) return st;
    if (K % 16) return fail(DBS_EINVAL, "nvfp4: K must be a multiple of 16");
    // K % 32 == 0 or an MN-major operand: the raw kernels (codes staged as
    // they are, decoded in registers), which stage K-major rows in 16-byte
    // pieces (whole 32-element half-rows); the launcher sends K-major
    // problems they do not suit back to the NVFP4 kernels
    if (la == DBS_K_MAJOR && lb == DBS_K_MAJOR && K % 32)
        return run(dbs::kNVFP4, A, sA, B, sB, D, M, N, K, tA * tB, 4, 16, stream);
    if ((la == DBS_K_MAJOR || lb == DBS_K_MAJOR) && K % 32)
        return fail(DBS_EUNSUPPORTED, "nvfp4: a K-major operand beside an MN-major one needs K % 32 == 0");
    if ((st = check_mn(la, lb, M, N, K, 4)) != DBS_OK) return st;
    return run(dbs::kNVFP4R, A, sA, B, sB, D, M, N, K, tA * tB, 4, 16, stream, nullptr, la, lb);
}

// ---- FP8-rate NVFP4 (opt-in, lossy) ---------------------------------------------

size_t gemm_nvfp4_fp8_workspace(int64_t M, int64_t N, int64_t K)
{
    if (M <= 0 || N <= 0 || K <= 0 || K % 32 || M > (int64_t(1) << 25) || N > (int64_t(1) << 25) ||
        K > (int64_t(1) << 22))
        return 0;
    return (size_t)fp8_ws(nullptr, M, N, K).bytes;
}

dbs_status gemm_nvfp4_fp8(const void *A, const uint8_t *sA, float tA, const void *B, const uint8_t *sB, float tB,
                          void *D, int64_t M, int64_t N, int64_t K, dbs_layout la, dbs_layout lb, void *workspace,
                          size_t workspace_bytes, hipStream_t stream)
{
    if (!workspace) return fail(DBS_EINVAL, "null pointer argument");
    dbs_status st = static_cast<dbs_status>(dbs::nvfp4_fp8_check(A, sA, B, sB, D, M, N, K, la, lb));
    if (st != DBS_OK) return st;
    return static_cast<dbs_status>(
        dbs::nvfp4_fp8_run(A, sA, tA, B, sB, tB, D, M, N, K, workspace, workspace_bytes, stream));
}

// ---- FP4-rate NVFP4 (opt-in, lossy) ---------------------------------------------

size_t gemm_nvfp4_fp6_workspace(int64_t M, int64_t N, int64_t K)
{
    if (M <= 0 || N <= 0 || K <= 0 || K % 32 || M > (int64_t(1) << 25) || N > (int64_t(1) << 25) ||
        K > (int64_t(1) << 22))
        return 0;
    return (size_t)fp6_ws(nullptr, M, N, K).bytes;
}

dbs_status gemm_nvfp4_fp6(const void *A, const uint8_t *sA, float tA, const void *B, const uint8_t *sB, float tB,
                          void *D, int64_t M, int64_t N, int64_t K, dbs_layout la, dbs_layout lb, void *workspace,
                          size_t workspace_bytes, hipStream_t stream)
{
    if (!workspace) return fail(DBS_EINVAL, "null pointer argument");
    dbs_status st = static_cast<dbs_status>(dbs::nvfp4_fp8_check(A, sA, B, sB, D, M, N, K, la, lb));
    if (st != DBS_OK) return st;
    if (!aligned(workspace, 256)) return fail(DBS_EINVAL, "workspace must be 256-byte aligned");
    const Fp8Ws w = fp6_ws(workspace, M, N, K);
    if ((int64_t)workspace_bytes < w.bytes) return fail(DBS_EINVAL, "workspace smaller than gemm_nvfp4_fp6_workspace()");
    int cus = 0;
    if ((st = device_cus(&cus)) != DBS_OK) return st;
    // the FP6-rate kernel reads the requantised codes stage-blocked
    bool blocked = false;
    if ((st = fp6_native(M, N, K, w.sa, w.sb, &blocked)) != DBS_OK) return st;
    hipError_t e = dbs::launch_requant_nvfp4_e2m3(static_cast<const uint8_t *>(A), sA, M, K, blocked, w.a, w.sa, cus,
                                                  stream);
    if (e == hipSuccess)
        e = dbs::launch_requant_nvfp4_e2m3(static_cast<const uint8_t *>(B), sB, N, K, blocked, w.b, w.sb, cus, stream);
    if (e != hipSuccess) return fail_hip(e, "kernel launch");
    return fp6_gemm(DBS_E2M3, DBS_E2M3, w.a, w.sa, w.b, w.sb, D, M, N, K, tA * tB, stream, blocked);
}

// ---- quantisers ----------------------------------------------------------------

static dbs_status check_quant(const float *x, const void *codes, int64_t rows, int64_t K, int64_t block)
{
    if (!x || !codes) return fail(DBS_EINVAL, "null pointer argument");
    if (rows <= 0 || K <= 0) return fail(DBS_EINVAL, "rows and K must be positive");
    if (K % block) return fail(DBS_EINVAL, "K must be a multiple of the block size");
    if (rows > (int64_t(1) << 31) || K > (int64_t(1) << 31) || rows * K > (int64_t(1) << 40))
        return fail(DBS_EINVAL, "array too large");
    if (!aligned(x, 16) || !aligned(codes, 16)) return fail(DBS_EINVAL, "x and codes must be 16-byte aligned");
    return DBS_OK;
}

dbs_status quant_mx(dbs_mx_elem elem, const float *x, int64_t rows, int64_t K, void *codes, uint8_t *scales,
                    hipStream_t stream)
{
    if (!mx_elem_known(elem)) return fail(DBS_EINVAL, "mx: unknown element format");
    dbs_status st = check_quant(x, codes, rows, K, 32);
    if (st != DBS_OK) return st;
    if (!scales) return fail(DBS_EINVAL, "null pointer argument");
    int cus = 0;
    if ((st = device_cus(&cus)) != DBS_OK) return st;
    // the quantiser's element codes: 0 E2M1, 1 E4M3, 2 E5M2, 3 E2M3, 4 E3M2
    const int qe = elem == DBS_E2M1 ? 0 : elem == DBS_E4M3 ? 1 : elem == DBS_E5M2 ? 2 : elem == DBS_E2M3 ? 3 : 4;
    hipError_t e = dbs::launch_quant_mx(qe, x, rows * K, static_cast<uint8_t *>(codes), scales, cus, stream);
    if (e != hipSuccess) return fail_hip(e, "kernel launch");
    g_err[0] = '\0';
    return DBS_OK;
}

dbs_status quant_nvfp4(const float *x, int64_t rows, int64_t K, void *codes, uint8_t *scales, float *t,
                       hipStream_t stream)
{
    dbs_status st = check_quant(x, codes, rows, K, 16);
    if (st != DBS_OK) return st;
    if (!scales || !t) return fail(DBS_EINVAL, "null pointer argument");
    if (!aligned(t, 4)) return fail(DBS_EINVAL, "t must be 4-byte aligned");
    int cus = 0;
    if ((st = device_cus(&cus)) != DBS_OK) return st;
    hipError_t e = dbs::launch_quant_nvfp4(x, rows * K, static_cast<uint8_t *>(codes), scales, t, cus, stream);
    if (e != hipSuccess) return fail_hip(e, "kernel launch");
    g_err[0] = '\0';
    return DBS_OK;
}

dbs_status quant_bf16(const float *x, int64_t n, void *out, hipStream_t stream)
{
    dbs_status st = check_quant(x, out, 1, n, 8);
    if (st != DBS_OK) return st;
    int cus = 0;
    if ((st = device_cus(&cus)) != DBS_OK) return st;
    hipError_t e = dbs::launch_quant_bf16(x, n, static_cast<uint16_t *>(out), cus, stream);
    if (e != hipSuccess) return fail_hip(e, "kernel launch");
    g_err[0] = '\0';
    return DBS_OK;
}

// ---- grouped GEMM ---------------------------------------------------------------

static dbs_status check_groups(const int64_t *offsets, int64_t G, int64_t *M)
{
    if (!offsets) return fail(DBS_EINVAL, "null offsets");
    if (G < 1 || G > dbs::kMaxGroups) return fail(DBS_EINVAL, "group count outside 1 .. 64");
    if (offsets[0] != 0) return fail(DBS_EINVAL, "offsets[0] must be 0");
    for (int64_t g = 0; g < G; ++g)
        if (offsets[g + 1] < offsets[g]) return fail(DBS_EINVAL, "offsets must be non-decreasing");
    *M = offsets[G];
    if (*M <= 0) return fail(DBS_EINVAL, "the groups hold no rows");
    return DBS_OK;
}

dbs_status gemm_grouped_bf16(const void *A, const void *B, void *D, const int64_t *offsets, int64_t G, int64_t N,
                             int64_t K, hipStream_t stream)
{
    int64_t M = 0;
    dbs_status st = check_groups(offsets, G, &M);
    if (st != DBS_OK) return st;
    if ((st = check_common(A, B, D, M, N, K, DBS_K_MAJOR, DBS_K_MAJOR, int64_t(1) << 21)) != DBS_OK) return st;
    if (K % 8) return fail(DBS_EINVAL, "bf16: K must be a multiple of 8");
    const Groups gr{offsets, G, nullptr};
    return run(dbs::kBF16, A, nullptr, B, nullptr, D, M, N, K, 1.0f, 16, 0, stream, &gr);
}

dbs_status gemm_grouped_mx(dbs_mx_elem elem, const void *A, const uint8_t *sA, const void *B, const uint8_t *sB,
                           void *D, const int64_t *offsets, int64_t G, int64_t N, int64_t K, hipStream_t stream)
{
    if (!mx_elem_known(elem)) return fail(DBS_EINVAL, "mx: unknown element format");
    if (is_fp6(elem)) return fail(DBS_EUNSUPPORTED, "grouped mx: FP6 elements are not implemented");
    if (!sA || !sB) return fail(DBS_EINVAL, "null pointer argument");
    int64_t M = 0;
    dbs_status st = check_groups(offsets, G, &M);
    if (st != DBS_OK) return st;
    if ((st = check_common(A, B, D, M, N, K, DBS_K_MAJOR, DBS_K_MAJOR, int64_t(1) << 22)) != DBS_OK) return st;
    if (K % 32) return fail(DBS_EINVAL, "mx: K must be a multiple of 32");
    const Groups gr{offsets, G, nullptr};
    if (elem != DBS_E2M1)
        return run(dbs::kMXFP8, A, sA, B, sB, D, M, N, K, 1.0f, 8, 32, stream, &gr, DBS_K_MAJOR, DBS_K_MAJOR,
                   mx8_code(elem) * 9);
    return run(dbs::kMXFP4, A, sA, B, sB, D, M, N, K, 1.0f, 4, 32, stream, &gr);
}

dbs_status gemm_grouped_nvfp4(const void *A, const uint8_t *sA, float tA, const void *B, const uint8_t *sB,
                              const float *tB, void *D, const int64_t *offsets, int64_t G, int64_t N, int64_t K,
                              hipStream_t stream)
{
    if (!sA || !sB || !tB) return fail(DBS_EINVAL, "null pointer argument");
    int64_t M = 0;
    dbs_status st = check_groups(offsets, G, &M);
    if (st != DBS_OK) return st;
    if ((st = check_common(A, B, D, M, N, K, DBS_K_MAJOR, DBS_K_MAJOR, int64_t(1) << 22)) != DBS_OK) return st;
    if (K % 16) return fail(DBS_EINVAL, "nvfp4: K must be a multiple of 16");
    float alpha[dbs::kMaxGroups];
    for (int64_t g = 0; g < G; ++g) alpha[g] = tA * tB[g];
    const Groups gr{offsets, G, alpha};
    // K % 32 == 0: the raw kernels of gemm_nvfp4 (codes staged as they are,
    // decoded in registers); else the kernels that decode into LDS
    return run(K % 32 ? dbs::kNVFP4 : dbs::kNVFP4R, A, sA, B, sB, D, M, N, K, 1.0f, 4, 16, stream, &gr);
}

const char *dbs_status_str(dbs_status st)
{
    switch (st) {
    case DBS_OK: return "DBS_OK: success";
    case DBS_EINVAL: return "DBS_EINVAL: invalid argument";
    case DBS_EUNSUPPORTED: return "DBS_EUNSUPPORTED: valid request not implemented";
    case DBS_EHIP: return "DBS_EHIP: HIP runtime error";
    }
    return "unknown status";
}

const char *dbs_last_error(void) { return g_err; }

int dbs_version(void) { return 102; }

}  // extern "C"
