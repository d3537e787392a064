/*
 * oracle.c -- plain, slow, fp64 CPU oracle for the block-scaled GEMM
 *
 *     D[m,n] = alpha * sum_{k=0}^{K-1} dA[m,k] * dB[n,k]        (k ascending, fp64)
 *     dX[r,k] = value(X[r,k]) * value(sX[r, k / bs])
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark use it.  It shares no code, header, table or constant with the
 * HIP kernels.
 *
 * What it follows:
 *  - The operation is A times B-transposed on two K-major operands: the
 *    "ThunderKittens Now on NVIDIA Vera Rubin NVL72" post builds its GEMMs on
 *    mma_ABt (section "New features of the Vera Rubin platform", item 1).
 *  - Block scales are separate tensors in global memory loaded next to the
 *    operand tiles and applied per block along K ("ThunderKittens 2.0", sec.
 *    1.2 and 2.1: MXFP8/NVFP4 GEMMs stage the A/B scale factors alongside the
 *    A/B tiles).
 *  - Two FP4 values share one byte ("Dissecting ThunderKittens", tile
 *    abstractions, fp4e2m1_2).  Element 2j is the low nibble (the pages do not
 *    fix the order; this reading is documented with the build).
 *  - The element/scale bit layouts are the OCP Microscaling (MX) v1.0
 *    definitions of E2M1, E4M3 (the "FN" variant: no infinities, S.1111.111 is
 *    NaN, max 448), E5M2 (IEEE-like: bias 15, S.11111.00 infinite, S.11111.xx
 *    NaN otherwise, max 57344), E2M3 and E3M2 (FP6: bias 1 / 3, no
 *    infinities or NaNs, max 7.5 / 28) and E8M0 (2^(e-127), 0xFF is NaN); bf16 is the
 *    upper half of an IEEE binary32.  The pages name only E4M3 and E2M1; E5M2
 *    is the other MXFP8 element the OCP format defines, and each operand of a
 *    GEMM may carry its own MX element format.
 *  - Blocks: 32 elements per E8M0 scale (MXFP8, MXFP4); 16 elements per E4M3
 *    scale plus one fp32 scale per tensor, alpha = tA*tB (NVFP4).
 *
 * Every decoded element and every product is exact in fp64 (at most 16
 * significant bits, exponents far inside the fp64 range), so the only error
 * is the fp64 summation itself.
 *
 * A planted-mistake switch (orc_set_mutation) lets the CPU tests verify that
 * the pins catch plausible errors; it is 0 (off) except inside those tests.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_BF16 = 0, ORC_MXFP8 = 1, ORC_MXFP4 = 2, ORC_NVFP4 = 3, ORC_MXE5M2 = 4, ORC_MXE2M3 = 5, ORC_MXE3M2 = 6 };

enum {
    MUT_NONE = 0,
    MUT_SCALE_BLOCK = 2,    /* scale of the next block applied                 */
    MUT_DROP_ALPHA = 3,     /* NVFP4: tensor scales ignored                    */
    MUT_B_NOT_T = 4,        /* B read as K x N (A*B instead of A*B^T)          */
    MUT_E4M3_BIAS = 5,      /* E4M3 exponent bias 8 instead of 7               */
    MUT_E2M1_SUBN = 6,      /* E2M1 subnormal decoded as 1.0 instead of 0.5    */
    MUT_FP32_SUM = 7,       /* accumulate in fp32                              */
    MUT_E8M0_BIAS = 8,      /* E8M0 bias 128                                   */
    MUT_DROP_LAST_K = 9,    /* last term of the sum dropped                    */
    MUT_E4M3_SIGN = 10,     /* E4M3 sign bit ignored                           */
    MUT_BF16_MANT = 11,     /* bf16 mantissa read as 6 bits                    */
    MUT_E5M2_BIAS = 12,     /* E5M2 exponent bias 16 instead of 15             */
    MUT_E5M2_SUBN = 13,     /* E5M2 subnormals read as normals (1.M)            */
    MUT_E2M3_BIAS = 14,     /* E2M3 exponent bias 2 instead of 1               */
    MUT_E3M2_SUBN = 15,     /* E3M2 subnormals read as normals (1.M)            */
    MUT_FP6_ORDER = 16,     /* FP6 codes read from the high end of each group  */
    MUT_FP6_SCALE = 17,     /* FP6 scale by floor(log2(amax / largest value))  */
    MUT_NV_S16_TRUNC = 18,  /* NVFP4 block scale rounded toward zero           */
    MUT_E5M2_EMAX = 19,     /* E5M2 scale recipe with E4M3's largest value     */
    MUT_E2M3_REQ_E = 20,    /* E2M3 requantisation exponent floor(log2 m)      */
};
static int g_mut = MUT_NONE;
void orc_set_mutation(int m) { g_mut = m; }

/* ---------------------------------------------------------------- formats */

double orc_decode_e2m1(unsigned c)
{
    c &= 0xFu;
    int s = (c >> 3) & 1, e = (c >> 1) & 3, m = c & 1;
    double mag;
    if (e == 0)
        mag = (g_mut == MUT_E2M1_SUBN ? 1.0 : 0.5) * m;      /* 0.M * 2^(1-1) */
    else
        mag = ldexp(1.0 + m / 2.0, e - 1);                    /* 1.M * 2^(e-1) */
    return s ? -mag : mag;
}

double orc_decode_e4m3(unsigned c)
{
    c &= 0xFFu;
    int s = (c >> 7) & 1, e = (c >> 3) & 0xF, m = c & 7;
    int bias = (g_mut == MUT_E4M3_BIAS) ? 8 : 7;
    if (e == 15 && m == 7) return NAN;
    double mag = (e == 0) ? ldexp(m / 8.0, 1 - bias) : ldexp(1.0 + m / 8.0, e - bias);
    if (g_mut == MUT_E4M3_SIGN) s = 0;
    return s ? -mag : mag;
}

double orc_decode_e5m2(unsigned c)
{
    c &= 0xFFu;
    int s = (c >> 7) & 1, e = (c >> 2) & 0x1F, m = c & 3;
    int bias = (g_mut == MUT_E5M2_BIAS) ? 16 : 15;
    double mag;
    if (e == 31) mag = m ? NAN : INFINITY;
    else if (e == 0 && g_mut != MUT_E5M2_SUBN) mag = ldexp(m / 4.0, 1 - bias);   /* 0.M * 2^(1-15) */
    else mag = ldexp(1.0 + m / 4.0, e - bias);                                  /* 1.M * 2^(e-15) */
    return s ? -mag : mag;
}

/* FP6 (OCP MX v1.0): no infinities or NaNs.  E2M3: bias 1, max 7.5; E3M2:
 * bias 3, max 28. */
double orc_decode_e2m3(unsigned c)
{
    c &= 0x3Fu;
    int s = (c >> 5) & 1, e = (c >> 3) & 3, m = c & 7;
    int bias = (g_mut == MUT_E2M3_BIAS) ? 2 : 1;
    double mag = (e == 0) ? ldexp(m / 8.0, 1 - bias) : ldexp(1.0 + m / 8.0, e - bias);
    return s ? -mag : mag;
}

double orc_decode_e3m2(unsigned c)
{
    c &= 0x3Fu;
    int s = (c >> 5) & 1, e = (c >> 2) & 7, m = c & 3;
    double mag = (e == 0 && g_mut != MUT_E3M2_SUBN) ? ldexp(m / 4.0, 1 - 3) : ldexp(1.0 + m / 4.0, e - 3);
    return s ? -mag : mag;
}

double orc_decode_e8m0(unsigned c)
{
    c &= 0xFFu;
    if (c == 0xFF) return NAN;
    return ldexp(1.0, (int)c - (g_mut == MUT_E8M0_BIAS ? 128 : 127));
}

double orc_decode_bf16(unsigned b)
{
    b &= 0xFFFFu;
    int s = (b >> 15) & 1, e = (b >> 7) & 0xFF, m = b & 0x7F;
    if (g_mut == MUT_BF16_MANT) m &= 0x7E;
    double mag;
    if (e == 0xFF) mag = m ? NAN : INFINITY;
    else if (e == 0) mag = ldexp(m / 128.0, -126);
    else mag = ldexp(1.0 + m / 128.0, e - 127);
    return s ? -mag : mag;
}

/* Nearest code by exhaustive search over the non-negative codes 0..maxcode,
 * ties to the code with an even mantissa (its lowest bit clear).  Magnitudes
 * beyond the largest finite code land on it (saturation). */
static unsigned encode_nearest(double x, double (*dec)(unsigned), unsigned maxcode,
                               unsigned signbit_code)
{
    double a = fabs(x);
    unsigned best = 0;
    double bestd = INFINITY;
    for (unsigned c = 0; c <= maxcode; ++c) {
        double d = fabs(dec(c) - a);
        if (d < bestd || (d == bestd && (c & 1u) == 0 && (best & 1u) == 1)) {
            best = c;
            bestd = d;
        }
    }
    return signbit(x) ? (best | signbit_code) : best;
}

unsigned orc_encode_e2m1(double x) { return encode_nearest(x, orc_decode_e2m1, 0x7, 0x8); }
unsigned orc_encode_e4m3(double x) { return encode_nearest(x, orc_decode_e4m3, 0x7E, 0x80); }
unsigned orc_encode_e5m2(double x) { return encode_nearest(x, orc_decode_e5m2, 0x7B, 0x80); }
unsigned orc_encode_e2m3(double x) { return encode_nearest(x, orc_decode_e2m3, 0x1F, 0x20); }
unsigned orc_encode_e3m2(double x) { return encode_nearest(x, orc_decode_e3m2, 0x1F, 0x20); }

/* FP6 packing: four consecutive elements of a row in three bytes, element j
 * of the row at bits 6j .. 6j+5 of the row's bytes read as one little-endian
 * bit string (the pages define no FP6 layout; this is the plainest one). */
unsigned orc_fp6_get(const uint8_t *row, int64_t j)
{
    if (g_mut == MUT_FP6_ORDER) j = (j & ~(int64_t)3) + (3 - (j & 3));
    const uint8_t *g = row + (j / 4) * 3;
    uint32_t bits = (uint32_t)g[0] | ((uint32_t)g[1] << 8) | ((uint32_t)g[2] << 16);
    return (bits >> (6 * (j % 4))) & 0x3Fu;
}

static void fp6_put(uint8_t *row, int64_t j, unsigned c)
{
    uint8_t *g = row + (j / 4) * 3;
    uint32_t bits = (uint32_t)g[0] | ((uint32_t)g[1] << 8) | ((uint32_t)g[2] << 16);
    const int sh = 6 * (int)(j % 4);
    bits = (bits & ~(0x3Fu << sh)) | ((c & 0x3Fu) << sh);
    g[0] = (uint8_t)bits;
    g[1] = (uint8_t)(bits >> 8);
    g[2] = (uint8_t)(bits >> 16);
}

/* fp64 -> bf16 bits, round to nearest even (used to state the bit-exact
 * expectation of results that are exactly representable). */
unsigned orc_encode_bf16(double x)
{
    unsigned sign = signbit(x) ? 0x8000u : 0u;
    double a = fabs(x);
    if (isnan(x)) return 0x7FC0u;
    if (a == 0.0) return sign;
    int e;
    frexp(a, &e);                       /* a in [2^(e-1), 2^e) */
    int ex = e - 1;
    if (ex < -126) ex = -126;           /* subnormal binade */
    double q = ldexp(1.0, ex - 7);      /* 7 stored mantissa bits */
    double r = rint(a / q) * q;         /* default rounding mode: nearest even */
    if (r == 0.0) return sign;          /* below half the smallest subnormal */
    if (r >= ldexp(1.0, 128)) return sign | 0x7F80u;
    frexp(r, &e);
    ex = e - 1;
    if (ex < -126) return sign | (unsigned)(r / ldexp(1.0, -133));
    unsigned man = (unsigned)((r / ldexp(1.0, ex) - 1.0) * 128.0);
    return sign | ((unsigned)(ex + 127) << 7) | man;
}

void orc_decode_array(int fmt, const uint8_t *codes, int64_t n, double *out)
{
    /* fmt: 0 = E2M1 (one code per byte), 1 = E4M3, 2 = E8M0, 3 = bf16 (n uint16), 4 = E5M2,
     * 5 = E2M3, 6 = E3M2 (one code per byte) */
    for (int64_t i = 0; i < n; ++i) {
        switch (fmt) {
        case 0: out[i] = orc_decode_e2m1(codes[i]); break;
        case 1: out[i] = orc_decode_e4m3(codes[i]); break;
        case 2: out[i] = orc_decode_e8m0(codes[i]); break;
        case 4: out[i] = orc_decode_e5m2(codes[i]); break;
        case 5: out[i] = orc_decode_e2m3(codes[i]); break;
        case 6: out[i] = orc_decode_e3m2(codes[i]); break;
        default: out[i] = orc_decode_bf16(((const uint16_t *)codes)[i]); break;
        }
    }
}

void orc_encode_array(int fmt, const double *x, int64_t n, uint8_t *out)
{
    /* fmt: 0 = E2M1 (one code per byte), 1 = E4M3, 3 = bf16 (n uint16), 4 = E5M2, 5 = E2M3,
     * 6 = E3M2 */
    for (int64_t i = 0; i < n; ++i) {
        switch (fmt) {
        case 0: out[i] = (uint8_t)orc_encode_e2m1(x[i]); break;
        case 1: out[i] = (uint8_t)orc_encode_e4m3(x[i]); break;
        case 4: out[i] = (uint8_t)orc_encode_e5m2(x[i]); break;
        case 5: out[i] = (uint8_t)orc_encode_e2m3(x[i]); break;
        case 6: out[i] = (uint8_t)orc_encode_e3m2(x[i]); break;
        default: ((uint16_t *)out)[i] = (uint16_t)orc_encode_bf16(x[i]); break;
        }
    }
}

/* --------------------------------------------------------------- operands */

typedef struct {
    int kind;
    const void *X;          /* rows x K elements, K-major (FP4: rows x K/2 bytes, FP6: rows x 3K/4) */
    const uint8_t *sX;      /* rows x K/bs scale codes (MX: E8M0, NVFP4: E4M3)    */
    int64_t rows, K;
} operand;

static int block_size(int kind) { return kind == ORC_NVFP4 ? 16 : 32; }

/* value of the (r, k) element: decoded element times decoded block scale */
static double element(const operand *op, int64_t r, int64_t k)
{
    const int64_t K = op->K;
    if (op->kind == ORC_BF16)
        return orc_decode_bf16(((const uint16_t *)op->X)[r * K + k]);

    int bs = block_size(op->kind);
    int64_t nblk = K / bs;
    int64_t blk = k / bs;
    if (g_mut == MUT_SCALE_BLOCK) blk = (blk + 1) % nblk;
    uint8_t sc = op->sX[r * nblk + blk];

    double v;
    if (op->kind == ORC_MXFP8) {
        v = orc_decode_e4m3(((const uint8_t *)op->X)[r * K + k]);
    } else if (op->kind == ORC_MXE5M2) {
        v = orc_decode_e5m2(((const uint8_t *)op->X)[r * K + k]);
    } else if (op->kind == ORC_MXE2M3 || op->kind == ORC_MXE3M2) {
        unsigned c = orc_fp6_get((const uint8_t *)op->X + r * (K / 4 * 3), k);
        v = op->kind == ORC_MXE2M3 ? orc_decode_e2m3(c) : orc_decode_e3m2(c);
    } else {
        uint8_t byte = ((const uint8_t *)op->X)[r * (K / 2) + k / 2];
        v = orc_decode_e2m1((k & 1) ? (byte >> 4) : (byte & 0xF));
    }
    double s = (op->kind == ORC_NVFP4) ? orc_decode_e4m3(sc) : orc_decode_e8m0(sc);
    return v * s;
}

static void decode_row(const operand *op, int64_t r, double *out)
{
    for (int64_t k = 0; k < op->K; ++k) out[k] = element(op, r, k);
}

/* B row n as the GEMM reads it.  The planted A*B mistake (bf16 only) reads
 * column n of a K x N matrix instead. */
static void decode_b_row(const operand *op, int64_t n, int64_t N, double *out)
{
    if (g_mut == MUT_B_NOT_T && op->kind == ORC_BF16) {
        for (int64_t k = 0; k < op->K; ++k)
            out[k] = orc_decode_bf16(((const uint16_t *)op->X)[k * N + n]);
        return;
    }
    decode_row(op, n, out);
}

static double dot(const double *a, const double *b, int64_t K)
{
    int64_t kend = (g_mut == MUT_DROP_LAST_K && K > 0) ? K - 1 : K;
    if (g_mut == MUT_FP32_SUM) {
        float s = 0.0f;
        for (int64_t k = 0; k < kend; ++k) s += (float)(a[k] * b[k]);
        return s;
    }
    double s = 0.0;
    for (int64_t k = 0; k < kend; ++k) s += a[k] * b[k];
    return s;
}

static double norm2(const double *a, int64_t K)
{
    double s = 0.0;
    for (int64_t k = 0; k < K; ++k) s += a[k] * a[k];
    return sqrt(s);
}

/* ------------------------------------------------------------ GEMM entries */

typedef struct {
    operand a, b;
    int64_t N;
    double alpha, ta, tb;
    const int64_t *em, *en;
    int64_t begin, end;
    double *d, *anorm, *bnorm;
    int status;
} job;

static void *entries_worker(void *p)
{
    job *j = (job *)p;
    const int64_t K = j->a.K;
    double *ra = malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
    double *rb = malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
    if (!ra || !rb) { j->status = -1; free(ra); free(rb); return NULL; }
    int64_t last_m = -1, last_n = -1;
    double na = 0.0, nb = 0.0;
    for (int64_t i = j->begin; i < j->end; ++i) {
        int64_t m = j->em[i], n = j->en[i];
        if (m != last_m) { decode_row(&j->a, m, ra); na = norm2(ra, K); last_m = m; }
        if (n != last_n) { decode_b_row(&j->b, n, j->N, rb); nb = norm2(rb, K); last_n = n; }
        j->d[i] = j->alpha * dot(ra, rb, K);
        if (j->anorm) j->anorm[i] = na * fabs(j->ta);
        if (j->bnorm) j->bnorm[i] = nb * fabs(j->tb);
    }
    free(ra);
    free(rb);
    j->status = 0;
    return NULL;
}

/* Operand kinds a GEMM may pair: equal kinds, or any two MX kinds (E4M3,
 * E5M2, E2M3, E3M2 or E2M1 elements, all with E8M0 scales per 32). */
static int is_mx(int k)
{
    return k == ORC_MXFP8 || k == ORC_MXE5M2 || k == ORC_MXFP4 || k == ORC_MXE2M3 || k == ORC_MXE3M2;
}

static int kinds_ok(int ka, int kb)
{
    if (ka < 0 || ka > 6 || kb < 0 || kb > 6) return 0;
    return ka == kb || (is_mx(ka) && is_mx(kb));
}

/*
 * Computes D at the listed entries (em[i], en[i]) for i < count.
 *   kind_a, kind_b : the operands' kinds: 0 bf16 (uint16), 1 MXFP8 (uint8
 *            E4M3 + E8M0 scales), 2 MXFP4 (packed E2M1 + E8M0), 3 NVFP4
 *            (packed E2M1 + E4M3, tA, tB), 4 MX with E5M2 elements (uint8 +
 *            E8M0), 5 / 6 MX with E2M3 / E3M2 elements (FP6 packed four to
 *            three bytes + E8M0); see kinds_ok for the pairs
 *   d      : D_ref per entry (alpha applied)
 *   anorm  : ||dA_m||_2 * |tA| per entry (may be NULL)
 *   bnorm  : ||dB_n||_2 * |tB| per entry (may be NULL)
 * Returns 0, or -1 on bad arguments / allocation failure.
 */
int orc_gemm_entries2(int kind_a, int kind_b, const void *A, const uint8_t *sA, double tA,
                      const void *B, const uint8_t *sB, double tB,
                      int64_t M, int64_t N, int64_t K,
                      const int64_t *em, const int64_t *en, int64_t count,
                      double *d, double *anorm, double *bnorm, int nthreads)
{
    const int kind = kind_a;
    if (!kinds_ok(kind_a, kind_b) || M < 0 || N < 0 || K < 0 || count < 0) return -1;
    if (kind != ORC_BF16 && K % block_size(kind)) return -1;
    for (int64_t i = 0; i < count; ++i)
        if (em[i] < 0 || em[i] >= M || en[i] < 0 || en[i] >= N) return -1;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (count < (int64_t)nthreads) nthreads = count > 0 ? (int)count : 1;

    double alpha = (kind == ORC_NVFP4 && g_mut != MUT_DROP_ALPHA) ? tA * tB : 1.0;
    double ta = (kind == ORC_NVFP4) ? tA : 1.0, tb = (kind == ORC_NVFP4) ? tB : 1.0;
    operand oa = {kind_a, A, sA, M, K}, ob = {kind_b, B, sB, N, K};

    job *jobs = calloc((size_t)nthreads, sizeof(job));
    pthread_t *th = calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !th) { free(jobs); free(th); return -1; }
    int64_t per = (count + nthreads - 1) / nthreads;
    for (int t = 0; t < nthreads; ++t) {
        job *j = &jobs[t];
        j->a = oa; j->b = ob; j->N = N;
        j->alpha = alpha; j->ta = ta; j->tb = tb;
        j->em = em; j->en = en;
        j->begin = (int64_t)t * per;
        j->end = j->begin + per < count ? j->begin + per : count;
        if (j->begin > count) j->begin = count;
        j->d = d; j->anorm = anorm; j->bnorm = bnorm;
        j->status = -1;
    }
    int rc = 0;
    if (nthreads == 1) {
        entries_worker(&jobs[0]);
        rc = jobs[0].status;
    } else {
        for (int t = 0; t < nthreads; ++t) pthread_create(&th[t], NULL, entries_worker, &jobs[t]);
        for (int t = 0; t < nthreads; ++t) { pthread_join(th[t], NULL); if (jobs[t].status) rc = -1; }
    }
    free(jobs);
    free(th);
    return rc;
}

int orc_gemm_entries(int kind, const void *A, const uint8_t *sA, double tA,
                     const void *B, const uint8_t *sB, double tB,
                     int64_t M, int64_t N, int64_t K,
                     const int64_t *em, const int64_t *en, int64_t count,
                     double *d, double *anorm, double *bnorm, int nthreads)
{
    return orc_gemm_entries2(kind, kind, A, sA, tA, B, sB, tB, M, N, K, em, en, count, d, anorm, bnorm, nthreads);
}

/* ---------------------------------------------------------- full GEMM D */

typedef struct {
    operand a;
    const double *bdec;   /* N x K decoded B rows */
    const double *bn;     /* N row norms of B (times |tB|) */
    int64_t N;
    double alpha, ta;
    int64_t m_begin, m_end;
    double *d, *anorm, *bnorm;
    int status;
} fjob;

static void *full_worker(void *p)
{
    fjob *j = (fjob *)p;
    const int64_t K = j->a.K, N = j->N;
    double *ra = malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
    if (!ra) { j->status = -1; return NULL; }
    for (int64_t m = j->m_begin; m < j->m_end; ++m) {
        decode_row(&j->a, m, ra);
        double na = norm2(ra, K) * fabs(j->ta);
        for (int64_t n = 0; n < N; ++n) {
            j->d[m * N + n] = j->alpha * dot(ra, j->bdec + n * K, K);
            if (j->anorm) j->anorm[m * N + n] = na;
            if (j->bnorm) j->bnorm[m * N + n] = j->bn[n];
        }
    }
    free(ra);
    j->status = 0;
    return NULL;
}

/* All M x N entries, row-major into d (and the per-entry norms if non-NULL).
 * B is decoded once (N*K doubles).  Kinds as for orc_gemm_entries2. */
int orc_gemm_full2(int kind_a, int kind_b, const void *A, const uint8_t *sA, double tA,
                   const void *B, const uint8_t *sB, double tB,
                   int64_t M, int64_t N, int64_t K,
                   double *d, double *anorm, double *bnorm, int nthreads)
{
    const int kind = kind_a;
    if (!kinds_ok(kind_a, kind_b) || M < 0 || N < 0 || K < 0) return -1;
    if (kind != ORC_BF16 && K % block_size(kind)) return -1;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (M < (int64_t)nthreads) nthreads = M > 0 ? (int)M : 1;

    double alpha = (kind == ORC_NVFP4 && g_mut != MUT_DROP_ALPHA) ? tA * tB : 1.0;
    double ta = (kind == ORC_NVFP4) ? tA : 1.0, tb = (kind == ORC_NVFP4) ? tB : 1.0;
    operand oa = {kind_a, A, sA, M, K}, ob = {kind_b, B, sB, N, K};

    double *bdec = malloc(sizeof(double) * (size_t)(N * K > 0 ? N * K : 1));
    double *bn = malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
    fjob *jobs = calloc((size_t)nthreads, sizeof(fjob));
    pthread_t *th = calloc((size_t)nthreads, sizeof(pthread_t));
    if (!bdec || !bn || !jobs || !th) { free(bdec); free(bn); free(jobs); free(th); return -1; }
    for (int64_t n = 0; n < N; ++n) {
        decode_b_row(&ob, n, N, bdec + n * K);
        bn[n] = norm2(bdec + n * K, K) * fabs(tb);
    }
    int64_t per = (M + nthreads - 1) / nthreads;
    for (int t = 0; t < nthreads; ++t) {
        fjob *j = &jobs[t];
        j->a = oa; j->bdec = bdec; j->bn = bn; j->N = N;
        j->alpha = alpha; j->ta = ta;
        j->m_begin = (int64_t)t * per < M ? (int64_t)t * per : M;
        j->m_end = j->m_begin + per < M ? j->m_begin + per : M;
        j->d = d; j->anorm = anorm; j->bnorm = bnorm;
        j->status = -1;
    }
    int rc = 0;
    if (nthreads == 1) {
        full_worker(&jobs[0]);
        rc = jobs[0].status;
    } else {
        for (int t = 0; t < nthreads; ++t) pthread_create(&th[t], NULL, full_worker, &jobs[t]);
        for (int t = 0; t < nthreads; ++t) { pthread_join(th[t], NULL); if (jobs[t].status) rc = -1; }
    }
    free(bdec); free(bn); free(jobs); free(th);
    return rc;
}

int orc_gemm_full(int kind, const void *A, const uint8_t *sA, double tA,
                  const void *B, const uint8_t *sB, double tB,
                  int64_t M, int64_t N, int64_t K,
                  double *d, double *anorm, double *bnorm, int nthreads)
{
    return orc_gemm_full2(kind, kind, A, sA, tA, B, sB, tB, M, N, K, d, anorm, bnorm, nthreads);
}

/* ------------------------------------------------- quantisation recipes */
/* Written independently of the input generator so the CPU tests can confirm
 * that the generator's codes follow the stated recipes. */

/* largest integer e with emax * 2^e <= amax (amax > 0), by stepping */
static int floor_log2_ratio(double amax, double emax)
{
    int e = 0;
    while (ldexp(emax, e) > amax) --e;
    while (ldexp(emax, e + 1) <= amax) ++e;
    return e;
}

/* MX recipe: per 32-block, scale 2^floor(log2(amax/emax)) clamped to
 * [-127, 127] (code 127 for an all-zero block); elements RNE + saturate.
 * elem: 0 = E2M1 (codes out: rows x K/2 packed), 1 = E4M3 (rows x K),
 * 2 = E5M2 (rows x K; emax 57344, the same recipe with E5M2's largest
 * finite value), 3 = E2M3 / 4 = E3M2 (rows x 3K/4 packed).  The FP6 scales
 * follow the OCP MX recipe, 2^(floor(log2 amax) - emax) with emax the
 * element's largest normal exponent (2 / 4), i.e. the ratio to 4 / 16: no
 * configuration fixes a recipe for them, and this one clips only values in
 * [7.5, 8) / [28, 32) of the scaled block maximum. */
int orc_quant_mx(int elem, const float *x, int64_t rows, int64_t K, uint8_t *codes, uint8_t *scales)
{
    if (K % 32 || elem < 0 || elem > 4) return -1;
    const double emaxs[5] = {6.0, 448.0, 57344.0, 4.0, 16.0};
    double emax = emaxs[elem];
    if (g_mut == MUT_FP6_SCALE && elem >= 3) emax = elem == 3 ? 7.5 : 28.0;
    if (g_mut == MUT_E5M2_EMAX && elem == 2) emax = 448.0;
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t b = 0; b < K / 32; ++b) {
            const float *xb = x + r * K + b * 32;
            double amax = 0.0;
            for (int i = 0; i < 32; ++i) amax = fmax(amax, fabs((double)xb[i]));
            int e = amax > 0.0 ? floor_log2_ratio(amax, emax) : 0;
            if (e < -127) e = -127;
            if (e > 127) e = 127;
            scales[r * (K / 32) + b] = (uint8_t)(e + 127);
            for (int i = 0; i < 32; ++i) {
                double v = ldexp((double)xb[i], -e);
                int64_t k = b * 32 + i;
                if (elem == 1) {
                    codes[r * K + k] = (uint8_t)orc_encode_e4m3(v);
                } else if (elem == 2) {
                    codes[r * K + k] = (uint8_t)orc_encode_e5m2(v);
                } else if (elem >= 3) {
                    fp6_put(codes + r * (K / 4 * 3), k, elem == 3 ? orc_encode_e2m3(v) : orc_encode_e3m2(v));
                } else {
                    uint8_t c = (uint8_t)orc_encode_e2m1(v);
                    uint8_t *byte = &codes[r * (K / 2) + k / 2];
                    if (k & 1) *byte = (uint8_t)((*byte & 0x0F) | (c << 4));
                    else *byte = (uint8_t)((*byte & 0xF0) | c);
                }
            }
        }
    }
    return 0;
}

/* NVFP4 recipe, every step in fp32: t = amax/(6*448) (1 if amax = 0);
 * s16 = RNE_e4m3(amax_blk / (6*t)); q = RNE_e2m1(x / (value(s16) * t)). */
int orc_quant_nvfp4(const float *x, int64_t rows, int64_t K, uint8_t *codes, uint8_t *scales, float *t_out)
{
    if (K % 16) return -1;
    float amax = 0.0f;
    for (int64_t i = 0; i < rows * K; ++i) amax = fmaxf(amax, fabsf(x[i]));
    const float six = 6.0f, prod = 2688.0f;
    float t = amax > 0.0f ? amax / prod : 1.0f;
    *t_out = t;
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t b = 0; b < K / 16; ++b) {
            const float *xb = x + r * K + b * 16;
            float ab = 0.0f;
            for (int i = 0; i < 16; ++i) ab = fmaxf(ab, fabsf(xb[i]));
            float six_t = six * t;
            float v = ab / six_t;
            uint8_t sc = (uint8_t)orc_encode_e4m3((double)v);
            if (g_mut == MUT_NV_S16_TRUNC && orc_decode_e4m3(sc) > (double)v && sc > 0) --sc;
            scales[r * (K / 16) + b] = sc;
            float denom = (float)orc_decode_e4m3(sc) * t;
            for (int i = 0; i < 16; ++i) {
                float q = denom > 0.0f ? xb[i] / denom : xb[i] * 0.0f;
                uint8_t c = (uint8_t)orc_encode_e2m1((double)q);
                int64_t k = b * 16 + i;
                uint8_t *byte = &codes[r * (K / 2) + k / 2];
                if (k & 1) *byte = (uint8_t)((*byte & 0x0F) | (c << 4));
                else *byte = (uint8_t)((*byte & 0xF0) | c);
            }
        }
    }
    return 0;
}

/* bf16 recipe: fp32 -> bf16 RNE */
/* NVFP4 -> MXFP8 requantisation (the opt-in FP8-rate NVFP4 GEMM): per
 * 32-element block of a row, made of two 16-element groups with E4M3 scales
 * s0, s1, the E8M0 exponent is E = floor(log2(max(|s0|, |s1|))) (0 when both
 * are zero), and each element a (E2M1) of group g becomes the nearest E4M3
 * code of a * s_g * 2^-E (ties to even).  That value is below 12 in
 * magnitude, so E4M3 never saturates; values under E4M3's subnormal step
 * lose precision.  The scale code is E + 127.  Codes in: rows x K/2 packed
 * E2M1, rows x K/16 E4M3; out: rows x K E4M3, rows x K/32 E8M0.  K % 32 == 0.
 * (The tensor scales are applied to the GEMM result, as for NVFP4.) */
int orc_requant_nvfp4_mx8(const uint8_t *codes, const uint8_t *scales, int64_t rows, int64_t K, uint8_t *out,
                          uint8_t *out_scales)
{
    if (K % 32) return -1;
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t b = 0; b < K / 32; ++b) {
            double s0 = orc_decode_e4m3(scales[r * (K / 16) + 2 * b]);
            double s1 = orc_decode_e4m3(scales[r * (K / 16) + 2 * b + 1]);
            double m = fmax(fabs(s0), fabs(s1));
            int E = 0;
            if (m > 0.0) {
                int ex;
                frexp(m, &ex);              /* m in [2^(ex-1), 2^ex) */
                E = ex - 1;
            }
            out_scales[r * (K / 32) + b] = (uint8_t)(E + 127);
            for (int i = 0; i < 32; ++i) {
                int64_t k = b * 32 + i;
                uint8_t byte = codes[r * (K / 2) + k / 2];
                double a = orc_decode_e2m1((k & 1) ? (byte >> 4) : (byte & 0xF));
                double v = ldexp(a * (i < 16 ? s0 : s1), -E);      /* exact */
                out[r * K + k] = (uint8_t)orc_encode_e4m3(v);
            }
        }
    }
    return 0;
}

/* NVFP4 -> MXFP6 (E2M3) requantisation (the opt-in FP4-rate NVFP4 GEMM):
 * per 32-element block of a row (two 16-element groups with E4M3 scales s0,
 * s1; m = max(|s0|, |s1|)), the E8M0 exponent E is the smallest integer with
 * 6 m <= 7.5 * 2^E, i.e. the block's largest possible magnitude fits E2M3's
 * largest value (never saturating) as high in its range as it goes: with
 * e0 = floor(log2 m), E = e0 if m <= 1.25 * 2^e0, else e0 + 1 (E = 0 when
 * both scales are zero).  Each element a (E2M1) of group g becomes the
 * nearest E2M3 code of a * s_g * 2^-E (ties to even).  Codes in: rows x K/2
 * packed E2M1, rows x K/16 E4M3; out: rows x 3K/4 packed E2M3 (element j at
 * bits 6j .. 6j+5 of the row), rows x K/32 E8M0.  K % 32 == 0.  (The tensor
 * scales are applied to the GEMM result, as for NVFP4.) */
int orc_requant_nvfp4_e2m3(const uint8_t *codes, const uint8_t *scales, int64_t rows, int64_t K, uint8_t *out,
                           uint8_t *out_scales)
{
    if (K % 32) return -1;
    for (int64_t r = 0; r < rows; ++r) {
        uint8_t *orow = out + r * (K / 4 * 3);
        for (int64_t b = 0; b < K / 32; ++b) {
            double s0 = orc_decode_e4m3(scales[r * (K / 16) + 2 * b]);
            double s1 = orc_decode_e4m3(scales[r * (K / 16) + 2 * b + 1]);
            double m = fmax(fabs(s0), fabs(s1));
            int E = 0;
            if (m > 0.0) {
                int ex;
                frexp(m, &ex);              /* m in [2^(ex-1), 2^ex) */
                E = ex - 1;
                if (g_mut != MUT_E2M3_REQ_E && m > ldexp(1.25, E)) E += 1;
            }
            out_scales[r * (K / 32) + b] = (uint8_t)(E + 127);
            for (int i = 0; i < 32; ++i) {
                int64_t k = b * 32 + i;
                uint8_t byte = codes[r * (K / 2) + k / 2];
                double a = orc_decode_e2m1((k & 1) ? (byte >> 4) : (byte & 0xF));
                double v = ldexp(a * (i < 16 ? s0 : s1), -E);      /* exact */
                fp6_put(orow, k, orc_encode_e2m3(v));
            }
        }
    }
    return 0;
}

void orc_quant_bf16(const float *x, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = (uint16_t)orc_encode_bf16((double)x[i]);
}
