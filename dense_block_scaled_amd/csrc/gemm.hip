// gemm.hip -- gfx950 (MI355X, CDNA4) kernels for the block-scaled GEMM
//
//     D[m, n] = bf16( alpha * sum_k dA[m, k] * dB[n, k] ),   fp32 accumulation
//
// One persistent kernel template serves the four formats.  Design (and where
// it departs from the Blackwell kernels the pages describe):
//
// * Scheduling.  A persistent grid of at most one workgroup per CU walks the
//   256 x 256 output tiles (cf. the persistent tile loop in "ThunderKittens Now
//   on NVIDIA Vera Rubin NVL72", Blackwell GEMM recap, and the static
//   persistent scheduler in "Dissecting ThunderKittens").  Workgroups are
//   dispatched round-robin over the 8 XCDs, so workgroup ids are remapped to
//   give every XCD a contiguous run of tile ids, and tile ids are rastered in
//   groups of `group_m` tile rows: the tiles one XCD runs at the same time
//   share A and B panels in that XCD's L2 (the locality concern of the
//   "ThunderKittens 2.0" notes, section 6, and the raster-order tuning of the
//   Vera Rubin post, final optimisations).
// * Staging.  Each stage moves a 256-row x 128-byte slab of A and of B from
//   HBM through registers into a two-slot LDS ring (2 x 64 KiB of the 160 KiB
//   LDS; cf. the stage-count discussion of "Async Tensor Core: Hopper wgmma ->
//   Blackwell tcgen05", sections 3.1 and 4.3).  Buffer loads return zero for
//   out-of-range rows and K columns, which handles ragged M, N and K.  16-byte
//   chunks are XOR-swizzled per row so fragment reads are bank-conflict-free.
//   One barrier per stage; no fences (cf. "ThunderKittens 2.0", section 1).
// * Scales.  MX scale bytes ride the same stage as their operand slab: they
//   are loaded one stage ahead straight into VGPRs and fed to the scaled MFMA
//   as its per-lane E8M0 operand (the gfx950 counterpart of issuing the scale
//   copy in the same thread as the MMA, "ThunderKittens 2.0", section 2.1).
// * Math.  Each of the 4 waves owns a 128 x 128 sub-tile as 4 x 4 MFMA
//   32x32 blocks (256 fp32 accumulators per lane) and reuses every A and B
//   fragment four times from VGPRs (cf. dual accumulation, "ThunderKittens
//   2.0", section 2.2).  BF16: v_mfma_f32_32x32x16_bf16.  MXFP8/MXFP4:
//   v_mfma_scale_f32_32x32x64_f8f6f4.  NVFP4: gfx950's scaled MFMA takes only
//   E8M0 per 32, so the loader decodes E2M1 x E4M3 exactly into fp16 (a product
//   of 2- and 4-bit significands with magnitude in [2^-10, 2688]) while filling
//   LDS, the math is v_mfma_f32_32x32x16_f16, and tA*tB is applied in the
//   epilogue.
// * Epilogue.  alpha * acc -> bf16 (round to nearest even) -> global, fused in
//   the same kernel.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace dbs {
namespace {

typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;

constexpr int kThreads = 256;                  // 4 waves of 64
constexpr int kRowBytes = 128;                 // bytes of one tile row per stage
constexpr int kTileBytes = kTileM * kRowBytes; // 32 KiB per operand per stage
constexpr int kStageBytes = 2 * kTileBytes;    // A + B
constexpr int kStages = 2;
constexpr uint32_t kOOB = 0x80000000u;         // beyond every num_records we set

// Buffer resource over [base, base + bytes): loads at offsets >= bytes return
// zero, stores there are dropped.  Word 3 = 0x00020000 is the gfx9-family
// raw-buffer configuration (32-bit data format, no swizzle, no stride).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// LDS byte offset of 16-byte chunk `chunk` (0..7) of tile row `row`.  The XOR
// pattern gives 8 (and 16) consecutive rows reading the same logical chunk
// distinct bank groups.
__device__ __forceinline__ int lds_off(int row, int chunk)
{
    const int swz = (row ^ (row >> 3)) & 7;
    return row * kRowBytes + ((chunk ^ swz) << 4);
}

// Output tile of linear id `tile`: groups of `group_m` tile rows, column-major
// inside a group.
__device__ __forceinline__ void tile_coords(int tile, const Params &p, int &tm, int &tn)
{
    const int per_group = p.group_m * p.tiles_n;
    const int g = tile / per_group;
    const int first = g * p.group_m;
    const int rows = min(p.tiles_m - first, p.group_m);
    const int idx = tile - g * per_group;
    tm = first + idx % rows;
    tn = idx / rows;
}

// ---------------------------------------------------------------- loaders

// 128-byte-row formats (bf16, E4M3, E2M1): thread t copies chunk t%8 of rows
// t/8 + 32 i, i < 8, for A and for B.
struct SlabRegs {
    i32x4 a[8], b[8];
};

__device__ __forceinline__ void load_slab(SlabRegs &r, __amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb,
                                          int lda, int s, int t)
{
    const int kb = s * kRowBytes + (t & 7) * 16;
    const bool ok = kb < lda;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int row = (t >> 3) + 32 * i;
        const uint32_t off = ok ? (uint32_t)(row * lda + kb) : kOOB;
        r.a[i] = __builtin_amdgcn_raw_buffer_load_b128(ra, off, 0, 0);
        r.b[i] = __builtin_amdgcn_raw_buffer_load_b128(rb, off, 0, 0);
    }
}

__device__ __forceinline__ void store_slab(const SlabRegs &r, uint8_t *stage, int t)
{
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int row = (t >> 3) + 32 * i;
        const int o = lds_off(row, t & 7);
        *reinterpret_cast<i32x4 *>(stage + o) = r.a[i];
        *reinterpret_cast<i32x4 *>(stage + kTileBytes + o) = r.b[i];
    }
}

// NVFP4: a stage covers 64 K elements = 32 packed bytes per row.  Thread t
// copies half t%2 (32 elements) of rows t/2 and t/2 + 128 of A and of B, with
// the two E4M3 scales of those 32 elements, and expands them to 64 bytes of
// fp16 (4 LDS chunks).
struct Fp4Regs {
    i32x4 a[2], b[2];
    uint32_t sa[2], sb[2];
};

__device__ __forceinline__ void load_fp4(Fp4Regs &r, __amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb,
                                         __amdgpu_buffer_rsrc_t rsa, __amdgpu_buffer_rsrc_t rsb,
                                         int lda, int sld, int s, int t)
{
    const int half = t & 1;
    const int kb = s * 32 + half * 16;         // packed byte within the row
    const int sb = s * 4 + half * 2;           // first of the two scale bytes
    const bool ok = kb < lda;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int row = (t >> 1) + 128 * i;
        const uint32_t off = ok ? (uint32_t)(row * lda + kb) : kOOB;
        const uint32_t soff = ok ? (uint32_t)(row * sld + sb) : kOOB;
        r.a[i] = __builtin_amdgcn_raw_buffer_load_b128(ra, off, 0, 0);
        r.b[i] = __builtin_amdgcn_raw_buffer_load_b128(rb, off, 0, 0);
        r.sa[i] = __builtin_amdgcn_raw_buffer_load_b16(rsa, soff, 0, 0);
        r.sb[i] = __builtin_amdgcn_raw_buffer_load_b16(rsb, soff, 0, 0);
    }
}

// E4M3 scale byte -> fp16 (exact: E4M3 values lie inside fp16's normal range).
__device__ __forceinline__ f16x2 e4m3_pair(uint32_t byte)
{
    const _Float16 v = (_Float16)__builtin_amdgcn_cvt_f32_fp8((int)byte, 0);
    return f16x2{v, v};
}

// 8 E2M1 codes (one dword) times one scale -> 8 fp16 (one 16-byte chunk).
// The conversion runs with unit scale, so it is exact; the product by the
// E4M3 scale is exact in fp16 as well.
__device__ __forceinline__ i32x4 expand8(uint32_t codes, f16x2 s)
{
    const f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 0) * s;
    const f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 1) * s;
    const f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 2) * s;
    const f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 3) * s;
    return i32x4{__builtin_bit_cast(int, p0), __builtin_bit_cast(int, p1),
                 __builtin_bit_cast(int, p2), __builtin_bit_cast(int, p3)};
}

__device__ __forceinline__ void store_fp4(const Fp4Regs &r, uint8_t *stage, int t)
{
    const int half = t & 1;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int row = (t >> 1) + 128 * i;
        const f16x2 alo = e4m3_pair(r.sa[i] & 0xFF), ahi = e4m3_pair((r.sa[i] >> 8) & 0xFF);
        const f16x2 blo = e4m3_pair(r.sb[i] & 0xFF), bhi = e4m3_pair((r.sb[i] >> 8) & 0xFF);
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const int o = lds_off(row, half * 4 + d);
            *reinterpret_cast<i32x4 *>(stage + o) = expand8((uint32_t)r.a[i][d], d < 2 ? alo : ahi);
            *reinterpret_cast<i32x4 *>(stage + kTileBytes + o) = expand8((uint32_t)r.b[i][d], d < 2 ? blo : bhi);
        }
    }
}

// MX scales for one stage, per lane: the E8M0 byte of each of the wave's 4 A
// (and B) row blocks for each MFMA k-step.  Lane l of a 32x32x64 scaled MFMA
// supplies the scale of K block l/32 of row l%32 (for E2M1 those are exactly
// the 32 elements the lane holds; for E4M3 see math_fp8).
template <int KSTEPS>
struct MxScales {
    int a[4][KSTEPS], b[4][KSTEPS];
};

template <int KSTEPS>
__device__ __forceinline__ void load_mx_scales(MxScales<KSTEPS> &sc, __amdgpu_buffer_rsrc_t rsa,
                                               __amdgpu_buffer_rsrc_t rsb, int sld, int s, int wm, int wn,
                                               int lr, int h)
{
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
        const int blk = s * (2 * KSTEPS) + kk * 2 + h;
        const bool ok = blk < sld;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int ra = wm * 128 + i * 32 + lr, rb = wn * 128 + i * 32 + lr;
            sc.a[i][kk] = __builtin_amdgcn_raw_buffer_load_b8(rsa, ok ? (uint32_t)(ra * sld + blk) : kOOB, 0, 0);
            sc.b[i][kk] = __builtin_amdgcn_raw_buffer_load_b8(rsb, ok ? (uint32_t)(rb * sld + blk) : kOOB, 0, 0);
        }
    }
}

// ----------------------------------------------------------------- math

// 16-bit formats: 4 k-steps of 16 per stage; lane l reads the 8 elements of
// chunk (2 kk + l/32) of its row.  The MFMA's first operand is the B
// fragment, so each lane ends up holding 4 consecutive output columns.
template <typename V, bool F16>
__device__ __forceinline__ void math_16bit(f32x16 (&acc)[4][4], const uint8_t *stage, int wm, int wn, int lr, int h)
{
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        V a[4], b[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            a[i] = *reinterpret_cast<const V *>(stage + lds_off(wm * 128 + i * 32 + lr, kk * 2 + h));
            b[i] = *reinterpret_cast<const V *>(stage + kTileBytes + lds_off(wn * 128 + i * 32 + lr, kk * 2 + h));
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if constexpr (F16)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(b[j], a[i], acc[i][j], 0, 0, 0);
                else
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[j], a[i], acc[i][j], 0, 0, 0);
            }
    }
}

// E4M3: 2 k-steps of 64 per stage.  In the 32x32x64 scaled MFMA with 8-bit
// elements, lane half h holds K positions [16h, 16h+16) in bytes 0..15 and
// [32+16h, 32+16h+16) in bytes 16..31, and its scale applies to K block h,
// i.e. bytes 16h..16h+15 of both halves (established with a one-instruction
// probe).  So lane half h reads chunks 4 kk + h and 4 kk + 2 + h and supplies
// the scale of block 2 kk + h.
__device__ __forceinline__ void math_fp8(f32x16 (&acc)[4][4], const uint8_t *stage, const MxScales<2> &sc,
                                         int wm, int wn, int lr, int h)
{
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        i32x8 a[4], b[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int ra = wm * 128 + i * 32 + lr, rb = wn * 128 + i * 32 + lr;
            const i32x4 a0 = *reinterpret_cast<const i32x4 *>(stage + lds_off(ra, kk * 4 + h));
            const i32x4 a1 = *reinterpret_cast<const i32x4 *>(stage + lds_off(ra, kk * 4 + 2 + h));
            const i32x4 b0 = *reinterpret_cast<const i32x4 *>(stage + kTileBytes + lds_off(rb, kk * 4 + h));
            const i32x4 b1 = *reinterpret_cast<const i32x4 *>(stage + kTileBytes + lds_off(rb, kk * 4 + 2 + h));
            a[i] = i32x8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
            b[i] = i32x8{b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    b[j], a[i], acc[i][j], 0, 0, 0, sc.b[j][kk], 0, sc.a[i][kk]);
    }
}

// E2M1: 4 k-steps of 64 per stage, 16 bytes (32 elements) per lane in the
// low half of the 8-dword operand.
__device__ __forceinline__ void math_fp4(f32x16 (&acc)[4][4], const uint8_t *stage, const MxScales<4> &sc,
                                         int wm, int wn, int lr, int h)
{
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        i32x8 a[4], b[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const i32x4 a0 = *reinterpret_cast<const i32x4 *>(stage + lds_off(wm * 128 + i * 32 + lr, kk * 2 + h));
            const i32x4 b0 =
                *reinterpret_cast<const i32x4 *>(stage + kTileBytes + lds_off(wn * 128 + i * 32 + lr, kk * 2 + h));
            a[i] = i32x8{a0[0], a0[1], a0[2], a0[3], 0, 0, 0, 0};
            b[i] = i32x8{b0[0], b0[1], b0[2], b0[3], 0, 0, 0, 0};
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    b[j], a[i], acc[i][j], 4, 4, 0, sc.b[j][kk], 0, sc.a[i][kk]);
    }
}

// ------------------------------------------------------------- epilogue

// acc[i][j] holds, for output row m = wm*128 + 32 i + lane%32, the columns
// n = wn*128 + 32 j + 8 g + 4 (lane/32) + q in register 4 g + q.
__device__ __forceinline__ void store_tile(const f32x16 (&acc)[4][4], const Params &p, int m0, int n0, int wm,
                                           int wn, int lr, int h)
{
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int m = m0 + wm * 128 + i * 32 + lr;
        if (m >= p.M) continue;
        uint16_t *drow = p.D + (int64_t)m * p.N;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int n = n0 + wn * 128 + j * 32 + g * 8 + h * 4;
                uint16_t v[4];
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    v[q] = __builtin_bit_cast(uint16_t, (__bf16)(acc[i][j][4 * g + q] * p.alpha));
                if (p.vec_store) {
                    if (n < p.N) {
                        const uint2 pk = {(uint32_t)v[0] | ((uint32_t)v[1] << 16),
                                          (uint32_t)v[2] | ((uint32_t)v[3] << 16)};
                        *reinterpret_cast<uint2 *>(drow + n) = pk;
                    }
                } else {
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        if (n + q < p.N) drow[n + q] = v[q];
                }
            }
        }
    }
}

// ---------------------------------------------------------------- kernel

template <int FMT>
__global__ __launch_bounds__(kThreads, 1) void gemm_kernel(Params p)
{
    __shared__ __attribute__((aligned(16))) uint8_t lds[kStages * kStageBytes];

    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int h = lane >> 5, lr = lane & 31;
    const int wm = w >> 1, wn = w & 1;
    const int ntiles = p.tiles_m * p.tiles_n;
    const int nwg = gridDim.x, wg = blockIdx.x;
    // hardware places workgroup wg on XCD wg % 8: give each XCD a contiguous
    // range of logical ids
    const int lid = (nwg & 7) == 0 ? (wg & 7) * (nwg >> 3) + (wg >> 3) : wg;

    for (int tile = lid; tile < ntiles; tile += nwg) {
        int tm, tn;
        tile_coords(tile, p, tm, tn);
        const int m0 = tm * kTileM, n0 = tn * kTileN;
        const int rows_a = min(p.M - m0, kTileM), rows_b = min(p.N - n0, kTileN);
        const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.A + (int64_t)m0 * p.lda, (uint32_t)(rows_a * p.lda));
        const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.B + (int64_t)n0 * p.lda, (uint32_t)(rows_b * p.lda));

        f32x16 acc[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

        if constexpr (FMT == kBF16 || FMT == kMXFP8 || FMT == kMXFP4) {
            constexpr int KS = FMT == kMXFP8 ? 2 : 4;
            __amdgpu_buffer_rsrc_t rsa = ra, rsb = rb;
            if constexpr (FMT != kBF16) {
                rsa = make_rsrc(p.sA + (int64_t)m0 * p.sld, (uint32_t)(rows_a * p.sld));
                rsb = make_rsrc(p.sB + (int64_t)n0 * p.sld, (uint32_t)(rows_b * p.sld));
            }
            SlabRegs regs;
            MxScales<KS> sc_cur, sc_next;
            load_slab(regs, ra, rb, p.lda, 0, t);
            if constexpr (FMT != kBF16) load_mx_scales<KS>(sc_cur, rsa, rsb, p.sld, 0, wm, wn, lr, h);
            store_slab(regs, lds, t);
            __syncthreads();
            for (int s = 0; s < p.nk; ++s) {
                const uint8_t *stage = lds + (s & 1) * kStageBytes;
                const bool more = s + 1 < p.nk;
                if (more) {
                    load_slab(regs, ra, rb, p.lda, s + 1, t);
                    if constexpr (FMT != kBF16) load_mx_scales<KS>(sc_next, rsa, rsb, p.sld, s + 1, wm, wn, lr, h);
                }
                if constexpr (FMT == kBF16)
                    math_16bit<bf16x8, false>(acc, stage, wm, wn, lr, h);
                else if constexpr (FMT == kMXFP8)
                    math_fp8(acc, stage, sc_cur, wm, wn, lr, h);
                else
                    math_fp4(acc, stage, sc_cur, wm, wn, lr, h);
                if (more) {
                    store_slab(regs, lds + ((s + 1) & 1) * kStageBytes, t);
                    if constexpr (FMT != kBF16) sc_cur = sc_next;
                }
                __syncthreads();
            }
        } else {  // NVFP4
            const __amdgpu_buffer_rsrc_t rsa = make_rsrc(p.sA + (int64_t)m0 * p.sld, (uint32_t)(rows_a * p.sld));
            const __amdgpu_buffer_rsrc_t rsb = make_rsrc(p.sB + (int64_t)n0 * p.sld, (uint32_t)(rows_b * p.sld));
            Fp4Regs regs;
            load_fp4(regs, ra, rb, rsa, rsb, p.lda, p.sld, 0, t);
            store_fp4(regs, lds, t);
            __syncthreads();
            for (int s = 0; s < p.nk; ++s) {
                const uint8_t *stage = lds + (s & 1) * kStageBytes;
                const bool more = s + 1 < p.nk;
                if (more) load_fp4(regs, ra, rb, rsa, rsb, p.lda, p.sld, s + 1, t);
                math_16bit<f16x8, true>(acc, stage, wm, wn, lr, h);
                if (more) store_fp4(regs, lds + ((s + 1) & 1) * kStageBytes, t);
                __syncthreads();
            }
        }

        store_tile(acc, p, m0, n0, wm, wn, lr, h);
    }
}

}  // namespace

hipError_t launch_gemm(int fmt, const Params &p, int grid, hipStream_t stream)
{
    const dim3 g(grid), b(kThreads);
    switch (fmt) {
    case kBF16: hipLaunchKernelGGL(gemm_kernel<kBF16>, g, b, 0, stream, p); break;
    case kMXFP8: hipLaunchKernelGGL(gemm_kernel<kMXFP8>, g, b, 0, stream, p); break;
    case kMXFP4: hipLaunchKernelGGL(gemm_kernel<kMXFP4>, g, b, 0, stream, p); break;
    case kNVFP4: hipLaunchKernelGGL(gemm_kernel<kNVFP4>, g, b, 0, stream, p); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace dbs
