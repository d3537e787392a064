// quant.hip -- gfx950 kernels that quantise fp32 operands into the GEMM's
// input formats (the step upstream of the block-scaled GEMM):
//
//   MXFP8 / MXFP4: per block of 32 consecutive K elements, the E8M0 scale
//     2^e with e = floor(log2(amax / emax)) (emax = 448 for E4M3, 57344 for
//     E5M2, 6 for E2M1; e clamped to [-127, 127]; an all-zero block gets
//     scale 1), then each element x -> nearest E4M3 / E5M2 / E2M1 value of
//     x * 2^-e.  This is the scale
//     rule stated with the workloads of the "ThunderKittens 2.0" MXFP8 GEMM
//     (section 2.1: an E8M0 scale per 32 elements) and the OCP MX v1.0
//     definition of the scale as a power of two.
//   NVFP4: one fp32 tensor scale t = amax / (6 * 448) (t = 1 when the tensor
//     is zero), per block of 16 the E4M3 scale s = nearest(amax_block / (6 t)),
//     then each element x -> nearest E2M1 value of x / (s * t); every step in
//     fp32 with correctly rounded operations.
//   BF16: fp32 -> bf16, round to nearest even.
//
// "Nearest" is round-to-nearest with ties to the even code (the code with its
// lowest bit clear), saturating at the largest finite value (448, 6) and
// keeping the sign of zero.  Inputs must be finite.  (E5M2's saturating
// rounding never produces its infinity code.)
//
// All kernels are bandwidth-bound streams over the flat element array
// (K is a multiple of the block size, so blocks never straddle rows): four
// lanes per MX block or two per NVFP4 block, eight consecutive elements per
// lane read as two 16-byte loads, block maxima combined across the lanes
// with cross-lane moves, codes written as one 8-byte (E4M3) or 4-byte (E2M1)
// store per lane.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace dbs {
namespace {

typedef __attribute__((ext_vector_type(4))) float f32x4;

// |x| rounded to the nearest E4M3 code (0..0x7E), ties to even, saturating.
// The grid step in x's binade is 2^(E-3) for x >= 2^-6 (E = its exponent),
// 2^-9 below (subnormals); rint() of x / step in fp32 is exact and rounds
// ties to even, and the code of a grid value v is v / 2^-9 below 2^-6 and
// ((E + 7) << 3) + mantissa above.
__device__ __forceinline__ uint32_t enc_e4m3_abs(float a)
{
    if (a >= 448.0f) return 0x7Eu;
    int E;
    (void)__builtin_frexpf(a, &E);          // a in [2^(E-1), 2^E)
    const int e = a < 0x1p-6f ? -6 : E - 1;
    const float v = __builtin_rintf(__builtin_ldexpf(a, 3 - e)) ;   // grid units of 2^(e-3)
    // v in [0, 16]; v == 16 moves to the next binade (mantissa 0)
    if (e == -6 && v < 8.0f) return (uint32_t)v;                   // subnormal (or zero)
    const int ee = v >= 16.0f ? e + 1 : e;
    const uint32_t m = v >= 16.0f ? 0u : (uint32_t)v - 8u;
    const uint32_t code = ((uint32_t)(ee + 7) << 3) | m;
    return code > 0x7Eu ? 0x7Eu : code;
}

// |x| rounded to the nearest E5M2 code (0..0x7B), ties to even, saturating:
// as for E4M3 with two mantissa bits, a minimum normal exponent of -14 and
// subnormal steps of 2^-16 (OCP MX v1.0 E5M2, bias 15).
__device__ __forceinline__ uint32_t enc_e5m2_abs(float a)
{
    if (a >= 57344.0f) return 0x7Bu;
    int E;
    (void)__builtin_frexpf(a, &E);
    const int e = a < 0x1p-14f ? -14 : E - 1;
    const float v = __builtin_rintf(__builtin_ldexpf(a, 2 - e));      // grid units of 2^(e-2)
    if (e == -14 && v < 4.0f) return (uint32_t)v;                      // subnormal (or zero)
    const int ee = v >= 8.0f ? e + 1 : e;
    const uint32_t m = v >= 8.0f ? 0u : (uint32_t)v - 4u;
    const uint32_t code = ((uint32_t)(ee + 15) << 2) | m;
    return code > 0x7Bu ? 0x7Bu : code;
}

// |x| rounded to the nearest E2M1 code (0..7), ties to even, saturating.
// Values 0, 0.5, 1, 1.5, 2, 3, 4, 6: step 0.5 below 2, 1 in [2, 4), 2 above.
__device__ __forceinline__ uint32_t enc_e2m1_abs(float a)
{
    if (a >= 6.0f) return 7u;
    if (a < 2.0f) return (uint32_t)__builtin_rintf(a * 2.0f);           // 0..4 -> codes 0..4 (4 = 2.0)
    if (a < 4.0f) return 2u + (uint32_t)__builtin_rintf(a);             // 2..4 -> codes 4..6
    return 4u + (uint32_t)__builtin_rintf(a * 0.5f);                    // 2..3 -> codes 6..7
}

// |x| rounded to the nearest FP6 code (0..0x1F), ties to even, saturating:
// MB mantissa bits, smallest normal exponent EMIN (subnormal steps of
// 2^(EMIN - MB)), bias 1 - EMIN, largest value VMAX (OCP MX v1.0 E2M3: MB 3,
// EMIN 0, max 7.5; E3M2: MB 2, EMIN -2, max 28).
template <int MB, int EMIN>
__device__ __forceinline__ uint32_t enc_fp6_abs(float a, float vmax)
{
    if (a >= vmax) return 0x1Fu;
    int E;
    (void)__builtin_frexpf(a, &E);
    const int e = a < __builtin_ldexpf(1.0f, EMIN) ? EMIN : E - 1;
    const float v = __builtin_rintf(__builtin_ldexpf(a, MB - e));      // grid units of 2^(e-MB)
    if (e == EMIN && v < (float)(1 << MB)) return (uint32_t)v;        // subnormal (or zero)
    const int ee = v >= (float)(2 << MB) ? e + 1 : e;
    const uint32_t m = v >= (float)(2 << MB) ? 0u : (uint32_t)v - (1u << MB);
    const uint32_t code = ((uint32_t)(ee + 1 - EMIN) << MB) | m;
    return code > 0x1Fu ? 0x1Fu : code;
}

__device__ __forceinline__ uint32_t sign_of(float x) { return __builtin_bit_cast(uint32_t, x) >> 31; }

__device__ __forceinline__ uint32_t enc_e4m3(float x) { return (sign_of(x) << 7) | enc_e4m3_abs(__builtin_fabsf(x)); }
__device__ __forceinline__ uint32_t enc_e2m1(float x) { return (sign_of(x) << 3) | enc_e2m1_abs(__builtin_fabsf(x)); }
__device__ __forceinline__ uint32_t enc_e5m2(float x) { return (sign_of(x) << 7) | enc_e5m2_abs(__builtin_fabsf(x)); }

// Element formats of the MX quantiser.
constexpr int kQE2M1 = 0, kQE4M3 = 1, kQE5M2 = 2, kQE2M3 = 3, kQE3M2 = 4;

template <int ELEM>
__device__ __forceinline__ uint32_t enc_fp6(float x)
{
    const float a = __builtin_fabsf(x);
    const uint32_t c = ELEM == kQE2M3 ? enc_fp6_abs<3, 0>(a, 7.5f) : enc_fp6_abs<2, -2>(a, 28.0f);
    return (sign_of(x) << 5) | c;
}

// E4M3 code (finite, non-negative) -> its fp32 value.
__device__ __forceinline__ float dec_e4m3_pos(uint32_t c)
{
    const uint32_t e = (c >> 3) & 0xF, m = c & 7;
    return e == 0 ? __builtin_ldexpf((float)m, -9) : __builtin_ldexpf((float)(8 + m), (int)e - 10);
}

// Maximum over the `lanes` consecutive lanes that share a block (lanes = 2
// or 4, groups aligned to it).
template <int LANES>
__device__ __forceinline__ float group_max(float v)
{
    v = __builtin_fmaxf(v, __shfl_xor(v, 1));
    if constexpr (LANES == 4) v = __builtin_fmaxf(v, __shfl_xor(v, 2));
    return v;
}

// e = floor(log2(amax / emax)) for amax > 0, exactly: amax = f 2^E with f in
// [1, 2) (frexp gives f/2 in [0.5, 1)); emax = 1.75 * 2^8 (E4M3), 1.75 *
// 2^15 (E5M2) or 1.5 * 2^2 (E2M1).  FP6 follows the OCP recipe
// floor(log2 amax) - emax with emax = 2 (E2M3) or 4 (E3M2).
template <int ELEM>
__device__ __forceinline__ int mx_exponent(float amax)
{
    int E;
    const float f = 2.0f * __builtin_frexpf(amax, &E);
    --E;
    if constexpr (ELEM == kQE4M3) return E - 8 - (f < 1.75f ? 1 : 0);
    if constexpr (ELEM == kQE5M2) return E - 15 - (f < 1.75f ? 1 : 0);
    if constexpr (ELEM == kQE2M3) return E - 2;
    if constexpr (ELEM == kQE3M2) return E - 4;
    return E - 2 - (f < 1.5f ? 1 : 0);
}

// Elements 8 l .. 8 l + 7 of the flat array for lane index l (grid-stride).
template <int ELEM>
__global__ __launch_bounds__(256) void quant_mx_kernel(const float *__restrict__ x, uint8_t *__restrict__ codes,
                                                       uint8_t *__restrict__ scales, int64_t nlanes)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t l = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; l - (threadIdx.x & 3) < nlanes; l += stride) {
        // groups of four lanes stay together: nlanes is a multiple of 4 and
        // the loop bound is taken at the group's first lane
        const f32x4 v0 = *reinterpret_cast<const f32x4 *>(x + 8 * l);
        const f32x4 v1 = *reinterpret_cast<const f32x4 *>(x + 8 * l + 4);
        float a = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) a = __builtin_fmaxf(a, __builtin_fmaxf(__builtin_fabsf(v0[i]), __builtin_fabsf(v1[i])));
        a = group_max<4>(a);
        int e = a > 0.0f ? mx_exponent<ELEM>(a) : 0;
        e = e < -127 ? -127 : (e > 127 ? 127 : e);
        if ((threadIdx.x & 3) == 0) scales[l >> 2] = (uint8_t)(e + 127);
        float y[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            y[i] = __builtin_ldexpf(v0[i], -e);
            y[4 + i] = __builtin_ldexpf(v1[i], -e);
        }
        if constexpr (ELEM == kQE2M3 || ELEM == kQE3M2) {
            // eight 6-bit codes = 48 bits: bytes 6 l .. 6 l + 5 of the row
            // stream (element j at bits 6j..), written as three halfwords
            uint32_t lo = 0, hi = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                lo |= enc_fp6<ELEM>(y[i]) << (6 * i);
                hi |= enc_fp6<ELEM>(y[4 + i]) << (6 * i);
            }
            uint16_t *o = reinterpret_cast<uint16_t *>(codes + 6 * l);
            o[0] = (uint16_t)lo;
            o[1] = (uint16_t)((lo >> 16) | (hi << 8));
            o[2] = (uint16_t)(hi >> 8);
        } else if constexpr (ELEM != kQE2M1) {
            uint32_t lo = 0, hi = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                lo |= (ELEM == kQE4M3 ? enc_e4m3(y[i]) : enc_e5m2(y[i])) << (8 * i);
                hi |= (ELEM == kQE4M3 ? enc_e4m3(y[4 + i]) : enc_e5m2(y[4 + i])) << (8 * i);
            }
            *reinterpret_cast<uint2 *>(codes + 8 * l) = uint2{lo, hi};
        } else {
            uint32_t w = 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) w |= enc_e2m1(y[i]) << (4 * i);
            *reinterpret_cast<uint32_t *>(codes + 4 * l) = w;
        }
    }
}

// Tensor amax of n elements (n a multiple of 8) into *amax_bits as the bit
// pattern of a non-negative float (ordered like an unsigned integer); the
// caller zeroes it first.
__global__ __launch_bounds__(256) void amax_kernel(const float *__restrict__ x, int64_t n8, uint32_t *amax_bits)
{
    float a = 0.0f;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t l = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; l < n8; l += stride) {
        const f32x4 v0 = *reinterpret_cast<const f32x4 *>(x + 8 * l);
        const f32x4 v1 = *reinterpret_cast<const f32x4 *>(x + 8 * l + 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) a = __builtin_fmaxf(a, __builtin_fmaxf(__builtin_fabsf(v0[i]), __builtin_fabsf(v1[i])));
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) a = __builtin_fmaxf(a, __shfl_xor(a, o));
    if ((threadIdx.x & 63) == 0) atomicMax(amax_bits, __builtin_bit_cast(uint32_t, a));
}

__global__ void zero_kernel(uint32_t *p) { *p = 0u; }

// t = amax / 2688 (1 for a zero tensor), in fp32, correctly rounded.
__device__ __forceinline__ float tensor_scale(uint32_t amax_bits)
{
    const float amax = __builtin_bit_cast(float, amax_bits);
    return amax > 0.0f ? __fdiv_rn(amax, 2688.0f) : 1.0f;
}

// NVFP4 blocks of 16: two lanes per block, eight elements each.
__global__ __launch_bounds__(256) void quant_nvfp4_kernel(const float *__restrict__ x, uint8_t *__restrict__ codes,
                                                          uint8_t *__restrict__ scales, int64_t nlanes,
                                                          const uint32_t *amax_bits)
{
    const float t = tensor_scale(*amax_bits);
    const float six_t = __fmul_rn(6.0f, t);
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t l = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; l - (threadIdx.x & 1) < nlanes; l += stride) {
        const f32x4 v0 = *reinterpret_cast<const f32x4 *>(x + 8 * l);
        const f32x4 v1 = *reinterpret_cast<const f32x4 *>(x + 8 * l + 4);
        float a = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) a = __builtin_fmaxf(a, __builtin_fmaxf(__builtin_fabsf(v0[i]), __builtin_fabsf(v1[i])));
        a = group_max<2>(a);
        const uint32_t sc = enc_e4m3(__fdiv_rn(a, six_t));
        if ((threadIdx.x & 1) == 0) scales[l >> 1] = (uint8_t)sc;
        const float denom = __fmul_rn(dec_e4m3_pos(sc & 0x7F), t);
        uint32_t w = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float xi = i < 4 ? v0[i] : v1[i - 4];
            const float q = denom > 0.0f ? __fdiv_rn(xi, denom) : xi * 0.0f;
            w |= enc_e2m1(q) << (4 * i);
        }
        *reinterpret_cast<uint32_t *>(codes + 4 * l) = w;
    }
}

// NVFP4 -> MXFP8 requantisation for the FP8-rate NVFP4 GEMM: lane l takes
// block l of 32 elements of the flat operand (two E4M3 group scales, 16
// packed bytes), picks E = floor(log2(max |s_g|)) (0 for two zero scales)
// and writes the 32 nearest E4M3 codes of a * s_g * 2^-E (ties to even) and
// the E8M0 code E + 127.  a * s_g * 2^-E has at most 6 significant bits, so
// it is exact in fp32 and the rounding is the only inexact step (checked bit
// for bit against the oracle's recipe over every pair of positive E4M3 group
// scales and every E2M1 code).  Inputs must be finite.
__device__ __forceinline__ float dec_e4m3(uint32_t c)
{
    const float v = dec_e4m3_pos(c & 0x7F);
    return (c & 0x80) ? -v : v;
}

__global__ __launch_bounds__(256) void requant_nvfp4_mx8_kernel(const uint8_t *__restrict__ codes,
                                                                const uint8_t *__restrict__ scales,
                                                                uint8_t *__restrict__ out,
                                                                uint8_t *__restrict__ out_scales, int64_t nblocks)
{
    typedef __attribute__((ext_vector_type(2))) float f32x2;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nblocks; b += stride) {
        const uint4 c = *reinterpret_cast<const uint4 *>(codes + 16 * b);
        const float s0 = dec_e4m3(scales[2 * b]), s1 = dec_e4m3(scales[2 * b + 1]);
        const float m = __builtin_fmaxf(__builtin_fabsf(s0), __builtin_fabsf(s1));
        int E = 0;
        if (m > 0.0f) {
            (void)__builtin_frexpf(m, &E);     // m in [2^(E-1), 2^E)
            --E;
        }
        out_scales[b] = (uint8_t)(E + 127);
        const float f0 = __builtin_ldexpf(s0, -E), f1 = __builtin_ldexpf(s1, -E);
        const uint32_t cw[4] = {c.x, c.y, c.z, c.w};
        uint32_t o[8];
        // byte j of an input dword holds two elements (low nibble first),
        // decoded exactly (unit scale); the products go to E4M3 through the
        // hardware conversion, which rounds to nearest even (the default
        // mode) and never sees a magnitude near E4M3's maximum here
        auto elems = [](uint32_t w, int j) -> f32x2 {
            switch (j) {
            case 0: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
            case 1: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
            case 2: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
            default: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
            }
        };
        auto four = [&](uint32_t w, float f, int j) -> uint32_t {   // bytes j, j+1 -> 4 codes
            const f32x2 lo = elems(w, j), hi = elems(w, j + 1);
            const int r = __builtin_amdgcn_cvt_pk_fp8_f32(lo[0] * f, lo[1] * f, 0, false);
            return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(hi[0] * f, hi[1] * f, r, true);
        };
#pragma unroll
        for (int d = 0; d < 4; ++d) {             // dword d: elements 8d .. 8d+7, group d / 2
            const float f = d < 2 ? f0 : f1;
            o[2 * d] = four(cw[d], f, 0);
            o[2 * d + 1] = four(cw[d], f, 2);
        }
        *reinterpret_cast<uint4 *>(out + 32 * b) = uint4{o[0], o[1], o[2], o[3]};
        *reinterpret_cast<uint4 *>(out + 32 * b + 16) = uint4{o[4], o[5], o[6], o[7]};
    }
}

// NVFP4 -> MXFP6 (E2M3) requantisation (the FP4-rate NVFP4 GEMM), one lane
// per 32-element block: with m the larger |scale| of the block's two groups
// and e0 = floor(log2 m), the E8M0 exponent is E = e0 if m <= 1.25 * 2^e0,
// else e0 + 1 -- the smallest E with 6 m <= 7.5 * 2^E, so that the block's
// largest possible value a * s_g * 2^-E (exact in fp32) never exceeds E2M3's
// 7.5 -- and each value goes to E2M3 through the hardware conversion of 32
// fp32 values to packed FP6 (round to nearest even at unit scale, both
// established with a one-wave probe; element j of the block lands at bits
// 6j .. 6j+5 of 24 bytes, the rows' own packing).  Checked
// bit for bit against the oracle's recipe over every pair of finite E4M3
// group scales and every E2M1 code.
//
// Output order: lane b writes the 24 bytes at 24 b.  Row-major (nk = 0) that
// is block b of the rows; stage-blocked (nk = stages of 128 elements a row,
// the FP6 kernel's layout) b counts the four blocks of a stage of a row, the
// eight rows of a group, the stages, then the groups, so the 768 bytes of one
// stage of rows 8g .. 8g+7 lie together; padding rows past the last
// (rows rounded up to 8) get zero codes.  Scales stay row-major either way.
__global__ __launch_bounds__(256) void requant_nvfp4_e2m3_kernel(const uint8_t *__restrict__ codes,
                                                                 const uint8_t *__restrict__ scales,
                                                                 uint8_t *__restrict__ out,
                                                                 uint8_t *__restrict__ out_scales, int64_t rows,
                                                                 int kbr, int nk)
{
    typedef __attribute__((ext_vector_type(2))) float f32x2;
    typedef __attribute__((ext_vector_type(16))) float f32x16;
    typedef __attribute__((ext_vector_type(6))) unsigned int u32x6;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t nblocks = (nk ? (rows + 7) / 8 * 8 : rows) * kbr;
    for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nblocks; b += stride) {
        uint2 *dst = reinterpret_cast<uint2 *>(out + 24 * b);
        int64_t sb = b;         // the block's index in the row-major order of the input
        if (nk) {
            const int64_t t = b >> 5;
            const int64_t g = t / nk;
            const int64_t row = 8 * g + ((b >> 2) & 7);
            if (row >= rows) {
                dst[0] = dst[1] = dst[2] = uint2{0u, 0u};
                continue;
            }
            sb = row * kbr + 4 * (t - g * nk) + (b & 3);
        }
        const uint4 c = *reinterpret_cast<const uint4 *>(codes + 16 * sb);
        const float s0 = dec_e4m3(scales[2 * sb]), s1 = dec_e4m3(scales[2 * sb + 1]);
        const float m = __builtin_fmaxf(__builtin_fabsf(s0), __builtin_fabsf(s1));
        int E = 0;
        if (m > 0.0f) {
            (void)__builtin_frexpf(m, &E);     // m in [2^(E-1), 2^E)
            --E;
            if (m > __builtin_ldexpf(1.25f, E)) ++E;
        }
        out_scales[sb] = (uint8_t)(E + 127);
        const float f0 = __builtin_ldexpf(s0, -E), f1 = __builtin_ldexpf(s1, -E);
        const uint32_t cw[4] = {c.x, c.y, c.z, c.w};
        // the conversion packs its two 16-value inputs interleaved (output
        // element 2i from the first's value i, 2i + 1 from the second's;
        // established with a one-wave probe), so the even elements go in
        // the first, the odd ones in the second
        f32x16 ev, od;
#pragma unroll
        for (int d = 0; d < 4; ++d) {             // dword d: elements 8d .. 8d+7, group d / 2
            const float f = d < 2 ? f0 : f1;
#pragma unroll
            for (int t = 0; t < 4; ++t) {         // byte t: elements 8d + 2t (low nibble), 8d + 2t + 1
                const f32x2 e = t == 0   ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[d], 1.0f, 0)
                                : t == 1 ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[d], 1.0f, 1)
                                : t == 2 ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[d], 1.0f, 2)
                                         : __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[d], 1.0f, 3);
                ev[4 * d + t] = e[0] * f;
                od[4 * d + t] = e[1] * f;
            }
        }
        const u32x6 r = __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(ev, od, 1.0f);
        dst[0] = uint2{r[0], r[1]};
        dst[1] = uint2{r[2], r[3]};
        dst[2] = uint2{r[4], r[5]};
    }
}

// *t: the tensor amax's bit pattern -> the tensor scale.
__global__ void finish_scale_kernel(uint32_t *t) { *t = __builtin_bit_cast(uint32_t, tensor_scale(*t)); }

__global__ __launch_bounds__(256) void quant_bf16_kernel(const float *__restrict__ x, uint16_t *__restrict__ out,
                                                         int64_t n8)
{
    typedef __attribute__((ext_vector_type(2))) float f32x2;
    typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t l = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; l < n8; l += stride) {
        const f32x4 v0 = *reinterpret_cast<const f32x4 *>(x + 8 * l);
        const f32x4 v1 = *reinterpret_cast<const f32x4 *>(x + 8 * l + 4);
        uint32_t w[4];
        w[0] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{v0[0], v0[1]}, bf16x2));
        w[1] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{v0[2], v0[3]}, bf16x2));
        w[2] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{v1[0], v1[1]}, bf16x2));
        w[3] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{v1[2], v1[3]}, bf16x2));
        *reinterpret_cast<uint4 *>(out + 8 * l) = uint4{w[0], w[1], w[2], w[3]};
    }
}

int grid_for(int64_t lanes, int cus)
{
    const int64_t blocks = (lanes + 255) / 256;
    const int64_t cap = (int64_t)cus * 8;
    return (int)(blocks < cap ? (blocks > 0 ? blocks : 1) : cap);
}

}  // namespace

hipError_t launch_quant_mx(int elem, const float *x, int64_t n, uint8_t *codes, uint8_t *scales, int cus,
                           hipStream_t stream)
{
    const int64_t lanes = n / 8;
    const int grid = grid_for(lanes, cus);
    switch (elem) {
    case kQE2M1: hipLaunchKernelGGL(quant_mx_kernel<kQE2M1>, dim3(grid), dim3(256), 0, stream, x, codes, scales, lanes); break;
    case kQE4M3: hipLaunchKernelGGL(quant_mx_kernel<kQE4M3>, dim3(grid), dim3(256), 0, stream, x, codes, scales, lanes); break;
    case kQE5M2: hipLaunchKernelGGL(quant_mx_kernel<kQE5M2>, dim3(grid), dim3(256), 0, stream, x, codes, scales, lanes); break;
    case kQE2M3: hipLaunchKernelGGL(quant_mx_kernel<kQE2M3>, dim3(grid), dim3(256), 0, stream, x, codes, scales, lanes); break;
    case kQE3M2: hipLaunchKernelGGL(quant_mx_kernel<kQE3M2>, dim3(grid), dim3(256), 0, stream, x, codes, scales, lanes); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_requant_nvfp4_mx8(const uint8_t *codes, const uint8_t *scales, int64_t n, uint8_t *out,
                                    uint8_t *out_scales, int cus, hipStream_t stream)
{
    const int64_t nblocks = n / 32;
    const int grid = grid_for(nblocks, cus);
    hipLaunchKernelGGL(requant_nvfp4_mx8_kernel, dim3(grid), dim3(256), 0, stream, codes, scales, out, out_scales,
                       nblocks);
    return hipGetLastError();
}

hipError_t launch_requant_nvfp4_e2m3(const uint8_t *codes, const uint8_t *scales, int64_t rows, int64_t K,
                                     bool blocked, uint8_t *out, uint8_t *out_scales, int cus, hipStream_t stream)
{
    if (K % 32 || (blocked && K % 128)) return hipErrorInvalidValue;
    const int64_t nblocks = (blocked ? (rows + 7) / 8 * 8 : rows) * (K / 32);
    const int grid = grid_for(nblocks, cus);
    hipLaunchKernelGGL(requant_nvfp4_e2m3_kernel, dim3(grid), dim3(256), 0, stream, codes, scales, out, out_scales,
                       rows, (int)(K / 32), blocked ? (int)(K / 128) : 0);
    return hipGetLastError();
}

hipError_t launch_quant_nvfp4(const float *x, int64_t n, uint8_t *codes, uint8_t *scales, float *t, int cus,
                              hipStream_t stream)
{
    const int64_t lanes = n / 8;
    const int grid = grid_for(lanes, cus);
    uint32_t *tb = reinterpret_cast<uint32_t *>(t);
    hipLaunchKernelGGL(zero_kernel, dim3(1), dim3(1), 0, stream, tb);
    hipLaunchKernelGGL(amax_kernel, dim3(grid), dim3(256), 0, stream, x, lanes, tb);
    hipLaunchKernelGGL(quant_nvfp4_kernel, dim3(grid), dim3(256), 0, stream, x, codes, scales, lanes, tb);
    hipLaunchKernelGGL(finish_scale_kernel, dim3(1), dim3(1), 0, stream, tb);
    return hipGetLastError();
}

hipError_t launch_quant_bf16(const float *x, int64_t n, uint16_t *out, int cus, hipStream_t stream)
{
    const int64_t lanes = n / 8;
    hipLaunchKernelGGL(quant_bf16_kernel, dim3(grid_for(lanes, cus)), dim3(256), 0, stream, x, out, lanes);
    return hipGetLastError();
}

}  // namespace dbs
