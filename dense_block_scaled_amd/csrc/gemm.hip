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
// * Staging.  Each stage moves a 256-row x 128-byte slab of A and of B into
//   one slot of a two-slot LDS ring (2 x 64 KiB of the 160 KiB LDS; cf. the
//   stage-count discussion of "Async Tensor Core: Hopper wgmma -> Blackwell
//   tcgen05", sections 3.1 and 4.3).  BF16/E4M3/E2M1 slabs go straight from
//   HBM to LDS (buffer_load_dwordx4 ... lds), so staging costs no VGPRs and no
//   LDS-write instructions; the load for stage s+1 is issued at the start of
//   stage s.  Each lane fetches the global chunk that belongs at its fixed LDS
//   position under an XOR swizzle of the 16-byte chunks, which keeps fragment
//   reads bank-conflict-free.  Buffer loads return zero for rows past M and
//   for K columns past K (ragged shapes).  One barrier per stage and no
//   fences (cf. "ThunderKittens 2.0", section 1).
// * Scales.  MX scale bytes ride the same stage as their operand slab: they
//   are loaded one stage ahead straight into VGPRs and fed to the scaled MFMA
//   as its per-lane E8M0 operand (the gfx950 counterpart of issuing the scale
//   copy from the same thread as the MMA, "ThunderKittens 2.0", section 2.1).
// * Math.  Each of the 4 waves owns a 128 x 128 sub-tile as 4 x 4 MFMA 32x32
//   blocks (256 fp32 accumulators per lane) and reuses every A and B fragment
//   four times from VGPRs (cf. dual accumulation, "ThunderKittens 2.0",
//   section 2.2).  Fragments are double-buffered in VGPRs: the reads for
//   k-step kk+1 are in flight while the MFMAs of kk issue, and the MFMAs of a
//   stage's last k-step are issued after the barrier, behind the next stage's
//   first reads.  BF16: v_mfma_f32_32x32x16_bf16.  MXFP8/MXFP4:
//   v_mfma_scale_f32_32x32x64_f8f6f4.  NVFP4: gfx950's scaled MFMA takes only
//   E8M0 per 32, so its loader stages through VGPRs and decodes E2M1 x E4M3
//   exactly into fp16 (a product of 2- and 4-bit significands with magnitude
//   in [2^-10, 2688]) on the way into LDS; the math is
//   v_mfma_f32_32x32x16_f16 and tA*tB is applied in the epilogue.
// * Epilogue.  alpha * acc -> bf16 (round to nearest even) -> global with
//   buffer stores (out-of-range rows and columns dropped), in the same kernel.
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
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kThreads = 256;                  // 4 waves of 64
constexpr int kRowBytes = 128;                 // bytes of one tile row per stage
constexpr int kTileBytes = kTileM * kRowBytes; // 32 KiB per operand per stage
constexpr uint32_t kOOB = 0x80000000u;         // beyond every num_records we set

#define DBS_FENCE() __builtin_amdgcn_sched_barrier(0)

// Buffer resource over [base, base + bytes): loads at offsets >= bytes return
// zero, stores there are dropped.  Word 3 = 0x00020000 is the gfx9-family
// raw-buffer configuration (32-bit data format, no swizzle, no stride).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// XOR swizzle of the 8 16-byte chunks of a tile row: 8 (and 16) consecutive
// rows reading the same logical chunk hit distinct bank groups.
__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }

__device__ __forceinline__ int lds_off(int row, int chunk) { return row * kRowBytes + ((chunk ^ swz(row)) << 4); }

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

// LDS map: A slot 0 | A slot 1 | B slot 0 | B slot 1, 32 KiB each; 1 KiB
// that L2-prefetch loads land in (never read); then for the MX formats the
// scale slots SA 0 | SA 1 | SB 0 | SB 1 of 256 rows x BPS bytes.  (Planes of
// 4-byte columns avoid the 2-way bank conflicts of the 8-byte E2M1 rows but
// measured slower.)  Slot 1 of the operands is reached through the 16-bit
// immediate offset of ds_read.
constexpr int kLdsA = 0;
constexpr int kLdsB = 2 * kTileBytes;
constexpr int kSlotStride = kTileBytes;
constexpr int kLdsJunk = 4 * kTileBytes;
constexpr int kLdsS = kLdsJunk + 1024;

// MX scale bytes per row per stage (2 blocks of 32 per 64-K k-step).
template <int FMT>
constexpr int scale_bps() { return FMT == kMXFP8 ? 4 : FMT == kMXFP4 ? 8 : 0; }
template <int FMT>
constexpr int lds_bytes() { return kLdsS + 4 * kTileM * scale_bps<FMT>(); }

// Stages ahead that an L2 prefetch touches: the direct-to-LDS load of stage
// s+1 then mostly hits L2 instead of waiting on the Infinity Cache or HBM.
#ifndef DBS_L2_PREFETCH
#define DBS_L2_PREFETCH 0
#endif
constexpr int kPrefetch = DBS_L2_PREFETCH;   // 0: off

// Per-lane constants of one workgroup.  w, wm, wn are wave-uniform.
struct Ctx {
    int t, lane, h, lr;
    int w, wm, wn;
    uint32_t fa[4], fb[4];   // LDS address of fragment reads at k-step 0, slot 0
    uint32_t sa[4], sb[4];   // LDS address of the lane's MX scale byte, k-step 0, slot 0
    uint32_t voff[8];        // direct-to-LDS source offsets at stage 0
    int kc[8];               // the K byte (within a stage) those loads fetch
};

// What a stage's loads fetch: stage `s` of the tile whose operand and scale
// rows start at the four buffer resources.  inval = kOOB turns every load of
// the target into a zero read (used when a workgroup has nothing left).
struct Target {
    __amdgpu_buffer_rsrc_t ra, rb, rsa, rsb;
    int s;
    uint32_t inval;
};

// ------------------------------------------------------------ format traits

template <int FMT>
struct Fmt;
template <>
struct Fmt<kBF16> {
    static constexpr int KK = 4;           // MFMA k-steps per stage (16 K each)
    using Frag = bf16x8;
};
template <>
struct Fmt<kNVFP4> {
    static constexpr int KK = 4;           // fp16 in LDS, same geometry as bf16
    using Frag = f16x8;
};
template <>
struct Fmt<kMXFP8> {
    static constexpr int KK = 2;           // 64 K per k-step, 32 bytes per lane
    using Frag = i32x8;
};
template <>
struct Fmt<kMXFP4> {
    static constexpr int KK = 4;           // 64 K per k-step, 16 bytes per lane
    using Frag = i32x4;
};

template <int FMT>
struct Frags {
    typename Fmt<FMT>::Frag a[4], b[4];
    uint32_t sa[4], sb[4];   // MX: E8M0 byte of each row block for this k-step
};

template <typename V>
__device__ __forceinline__ V lds_read(const uint8_t *lds, uint32_t addr)
{
    return *reinterpret_cast<const V *>(lds + addr);
}

// Fragment reads for k-step kk from ring slot `slot`.  16-bit formats: lane l
// holds the 8 elements of chunk 2 kk + l/32 of its row.  E2M1: 32 elements,
// chunk 2 kk + l/32.  E4M3: in the 32x32x64 scaled MFMA with 8-bit elements,
// lane half h holds K positions [16h, 16h+16) in bytes 0..15 and
// [32+16h, 48+16h) in bytes 16..31, and its scale applies to K block h, i.e.
// bytes 16h..16h+15 of both halves (established with a one-instruction
// probe); so lane half h reads chunks 4 kk + h and 4 kk + 2 + h.  With the
// XOR swizzle, chunk 2 kk + h of a row sits at fa ^ (kk << 5) and chunk
// 4 kk + h at fa ^ (kk << 6).  MX scales: lane l of a 32x32x64 scaled MFMA
// supplies the E8M0 scale of K block l/32 of row l%32 in bits [7:0]; for
// k-step kk that is byte 2 kk + l/32 of the row's stage scales.
template <int FMT>
__device__ __forceinline__ void read_one(typename Fmt<FMT>::Frag &v, uint32_t &sc, const uint8_t *lds, uint32_t fbase,
                                         uint32_t sbase, int slot, int kk)
{
    const uint32_t so = (uint32_t)(slot * kSlotStride);
    if constexpr (FMT == kMXFP8) {
        const uint32_t x = (fbase ^ (uint32_t)(kk << 6)) + so;
        const i32x4 v0 = lds_read<i32x4>(lds, x), v1 = lds_read<i32x4>(lds, x ^ 32u);
        v = i32x8{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
    } else {
        v = lds_read<typename Fmt<FMT>::Frag>(lds, (fbase ^ (uint32_t)(kk << 5)) + so);
    }
    if constexpr (FMT == kMXFP8 || FMT == kMXFP4)
        sc = lds[sbase + (uint32_t)(slot * kTileM * scale_bps<FMT>() + 2 * kk)];
}

template <int FMT>
__device__ __forceinline__ void read_a(Frags<FMT> &f, int i, const uint8_t *lds, int slot, int kk, const Ctx &c)
{
    read_one<FMT>(f.a[i], f.sa[i], lds, c.fa[i], c.sa[i], slot, kk);
}

template <int FMT>
__device__ __forceinline__ void read_b(Frags<FMT> &f, int j, const uint8_t *lds, int slot, int kk, const Ctx &c)
{
    read_one<FMT>(f.b[j], f.sb[j], lds, c.fb[j], c.sb[j], slot, kk);
}

template <int FMT>
__device__ __forceinline__ void read_frags(Frags<FMT> &f, const uint8_t *lds, int slot, int kk, const Ctx &c)
{
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        read_a(f, i, lds, slot, kk, c);
        read_b(f, i, lds, slot, kk, c);
    }
}

// ------------------------------------------------------------------ scales

// MX scales of the target stage for the workgroup's 256 A rows and 256 B
// rows go to scale slot `slot` as 256 rows x BPS bytes per operand.
//
// Rows whose stage scales are whole dwords (row stride K/32 a multiple of 4):
// direct-to-LDS dword loads.  A dword wave-load writes 64 lanes x 4 bytes, so
// for E4M3 (BPS = 4) lane i of wave w carries row 64w + i, and for E2M1
// (BPS = 8) wave-load j carries rows 64w + 32j + i/2, dword i%2.  A dword
// past the row's last block (partial last stage) reads zero.
template <int FMT>
__device__ __forceinline__ void dma_scales(uint8_t *lds, int slot, const Target &tg, const Ctx &c, int sld)
{
    constexpr int BPS = scale_bps<FMT>();
    constexpr int NW = BPS / 4;                      // wave-loads per wave per operand
#pragma unroll
    for (int j = 0; j < NW; ++j) {
        const int row = c.w * 64 + (NW == 1 ? c.lane : j * 32 + (c.lane >> 1));
        const int word = NW == 1 ? 0 : (c.lane & 1);
        const int o = tg.s * BPS + 4 * word;
        const uint32_t off = ((uint32_t)(row * sld + o) | (o < sld ? 0u : kOOB)) | tg.inval;
        const int dst = slot * kTileM * BPS + (c.w * NW + j) * 256;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(tg.rsa, (lds_void *)(lds + kLdsS + dst), 4, off, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(tg.rsb, (lds_void *)(lds + kLdsS + 2 * kTileM * BPS + dst), 4,
                                                 off, 0, 0, 0);
    }
}

// Any other row stride: thread t fetches the BPS bytes of A row t and B row
// t one by one (bytes past the row's last block read zero) and writes them
// to LDS before the stage's barrier.
template <int FMT>
struct ScaleBytes {
    uint32_t a[scale_bps<FMT>() > 0 ? scale_bps<FMT>() : 1], b[scale_bps<FMT>() > 0 ? scale_bps<FMT>() : 1];
};

template <int FMT>
__device__ __forceinline__ void load_scale_bytes(ScaleBytes<FMT> &r, const Target &tg, int t, int sld)
{
    constexpr int BPS = scale_bps<FMT>();
#pragma unroll
    for (int b = 0; b < BPS; ++b) {
        const int o = tg.s * BPS + b;
        const uint32_t off = ((uint32_t)(t * sld + o) | (o < sld ? 0u : kOOB)) | tg.inval;
        r.a[b] = __builtin_amdgcn_raw_buffer_load_b8(tg.rsa, off, 0, 0);
        r.b[b] = __builtin_amdgcn_raw_buffer_load_b8(tg.rsb, off, 0, 0);
    }
}

template <int FMT>
__device__ __forceinline__ void store_scale_bytes(const ScaleBytes<FMT> &r, uint8_t *lds, int slot, int t)
{
    constexpr int BPS = scale_bps<FMT>();
    uint8_t *sa = lds + kLdsS + slot * kTileM * BPS + t * BPS;
#pragma unroll
    for (int b = 0; b < BPS; ++b) {
        sa[b] = (uint8_t)r.a[b];
        sa[2 * kTileM * BPS + b] = (uint8_t)r.b[b];
    }
}

// ------------------------------------------------------------------- math

// One 32x32 block: acc[i][j] += A block i x B block j for one k-step.  The
// MFMA's first operand is the B fragment, so each lane ends up holding 4
// consecutive output columns.
template <int FMT>
__device__ __forceinline__ void mma1(f32x16 &acc, const Frags<FMT> &f, int i, int j)
{
    if constexpr (FMT == kBF16) {
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[j], f.a[i], acc, 0, 0, 0);
    } else if constexpr (FMT == kNVFP4) {
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(f.b[j], f.a[i], acc, 0, 0, 0);
    } else if constexpr (FMT == kMXFP8) {
        acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.b[j], f.a[i], acc, 0, 0, 0, (int)f.sb[j], 0,
                                                              (int)f.sa[i]);
    } else {
        const i32x8 bb = {f.b[j][0], f.b[j][1], f.b[j][2], f.b[j][3], 0, 0, 0, 0};
        const i32x8 aa = {f.a[i][0], f.a[i][1], f.a[i][2], f.a[i][3], 0, 0, 0, 0};
        acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bb, aa, acc, 4, 4, 0, (int)f.sb[j], 0, (int)f.sa[i]);
    }
}

template <int FMT>
__device__ __forceinline__ void mma(f32x16 (&acc)[4][4], const Frags<FMT> &f)
{
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) mma1(acc[i][j], f, i, j);
}

// ------------------------------------------------------ direct-to-LDS loads

// One wave-load pair (A and B) of the target stage into ring slot `slot`.
// Wave w issues the 8 wave-loads q of rows 64w .. 64w+63 of each operand; a
// wave-load writes 64 lanes x 16 bytes to consecutive LDS bytes, i.e. 8 rows
// x 8 chunks, so lane i lands on row 64w + 8q + i/8, physical chunk i%8, and
// fetches the logical chunk the swizzle places there (c.voff[q] at stage 0,
// K byte c.kc[q] within the stage).  Chunks past the row end (a partial
// last stage) read zeros.
__device__ __forceinline__ void dma_pair(uint8_t *lds, int slot, const Target &tg, const Ctx &c, int q, int lda)
{
    const int k0 = tg.s * kRowBytes;
    const uint32_t off = ((c.voff[q] + (uint32_t)k0) | (k0 + c.kc[q] < lda ? 0u : kOOB)) | tg.inval;
    const int dst = slot * kSlotStride + (c.w * 8 + q) * 1024;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(tg.ra, (lds_void *)(lds + kLdsA + dst), 16, off, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(tg.rb, (lds_void *)(lds + kLdsB + dst), 16, off, 0, 0, 0);
}

// ---------------------------------------------------------- NVFP4 staging

// A stage covers 64 K elements = 32 packed bytes per row.  Thread t loads
// half t%2 (32 elements) of rows t/2 and t/2 + 128 of A and of B, with the
// two E4M3 scales of those 32 elements, and expands them to 64 bytes of fp16
// (4 LDS chunks).
struct Fp4Regs {
    i32x4 a[2], b[2];
    uint32_t sa[2], sb[2];
};

__device__ __forceinline__ void load_fp4(Fp4Regs &r, const Target &tg, int lda, int sld, int t)
{
    const int half = t & 1;
    const int kb = tg.s * 32 + half * 16;      // packed byte within the row
    const int sb = tg.s * 4 + half * 2;        // first of the two scale bytes
    // K%32 == 0: a chunk is all in or all out
    const uint32_t pad = (kb < lda ? 0u : kOOB) | tg.inval;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int row = (t >> 1) + 128 * i;
        const uint32_t off = (uint32_t)(row * lda + kb) | pad;
        const uint32_t soff = (uint32_t)(row * sld + sb) | pad;
        r.a[i] = __builtin_amdgcn_raw_buffer_load_b128(tg.ra, off, 0, 0);
        r.b[i] = __builtin_amdgcn_raw_buffer_load_b128(tg.rb, off, 0, 0);
        r.sa[i] = __builtin_amdgcn_raw_buffer_load_b16(tg.rsa, soff, 0, 0);
        r.sb[i] = __builtin_amdgcn_raw_buffer_load_b16(tg.rsb, soff, 0, 0);
    }
}

// E4M3 scale byte -> fp16 (exact: E4M3 values lie inside fp16's normal range).
__device__ __forceinline__ f16x2 e4m3_pair(uint32_t byte)
{
    const _Float16 v = (_Float16)__builtin_amdgcn_cvt_f32_fp8((int)byte, 0);
    return f16x2{v, v};
}

// 8 E2M1 codes (one dword) times one scale -> 8 fp16 (one 16-byte chunk).
// The conversion instruction uses only the exponent of its scale operand, so
// it runs with unit scale (exact) and the E4M3 scale is applied by an fp16
// multiply, also exact.  Low nibble first.
__device__ __forceinline__ i32x4 expand8(uint32_t codes, f16x2 s)
{
    const f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 0) * s;
    const f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 1) * s;
    const f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 2) * s;
    const f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 3) * s;
    return i32x4{__builtin_bit_cast(int, p0), __builtin_bit_cast(int, p1), __builtin_bit_cast(int, p2),
                 __builtin_bit_cast(int, p3)};
}

__device__ __forceinline__ void store_fp4(const Fp4Regs &r, uint8_t *lds, int slot, int t)
{
    const int half = t & 1;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int row = (t >> 1) + 128 * i;
        const f16x2 alo = e4m3_pair(r.sa[i] & 0xFF), ahi = e4m3_pair((r.sa[i] >> 8) & 0xFF);
        const f16x2 blo = e4m3_pair(r.sb[i] & 0xFF), bhi = e4m3_pair((r.sb[i] >> 8) & 0xFF);
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const int o = slot * kSlotStride + lds_off(row, half * 4 + d);
            *reinterpret_cast<i32x4 *>(lds + kLdsA + o) = expand8((uint32_t)r.a[i][d], d < 2 ? alo : ahi);
            *reinterpret_cast<i32x4 *>(lds + kLdsB + o) = expand8((uint32_t)r.b[i][d], d < 2 ? blo : bhi);
        }
    }
}

// --------------------------------------------------------------- epilogue

// acc[i][j] holds, for output row m = wm*128 + 32 i + lane%32, the columns
// n = wn*128 + 32 j + 8 g + 4 (lane/32) + q in register 4 g + q.  Each
// 32-row block is stored through its own buffer resource, so rows past M
// and columns past N are dropped by the hardware range check.
__device__ __forceinline__ uint32_t pack_bf16(float x, float y)
{
    typedef __attribute__((ext_vector_type(2))) float f32x2;
    typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x, y}, bf16x2));
}

__device__ __forceinline__ void store_tile(const f32x16 (&acc)[4][4], const Params &p, int m0, int n0,
                                           const Ctx &c)
{
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r0 = m0 + c.wm * 128 + i * 32;
        const uint32_t bytes = __builtin_amdgcn_readfirstlane((uint32_t)max(0, min(32, p.M - r0)) * (uint32_t)p.N * 2u);
        const __amdgpu_buffer_rsrc_t rd = make_rsrc(p.D + (int64_t)r0 * p.N, bytes);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int n = n0 + c.wn * 128 + j * 32 + g * 8 + c.h * 4;
                const f32x16 &a = acc[i][j];
                const uint32_t lo = pack_bf16(a[4 * g] * p.alpha, a[4 * g + 1] * p.alpha);
                const uint32_t hi = pack_bf16(a[4 * g + 2] * p.alpha, a[4 * g + 3] * p.alpha);
                const uint32_t base = (uint32_t)(c.lr * p.N + n) * 2u;
                if (p.vec_store) {
                    // N % 4 == 0 and n % 4 == 0: the 4 columns are all in or all out
                    __builtin_amdgcn_raw_buffer_store_b64(u32x2{lo, hi}, rd, n < p.N ? base : kOOB, 0, 0);
                } else {
                    const uint16_t v[4] = {(uint16_t)lo, (uint16_t)(lo >> 16), (uint16_t)hi, (uint16_t)(hi >> 16)};
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        __builtin_amdgcn_raw_buffer_store_b16(v[q], rd, n + q < p.N ? base + 2 * q : kOOB, 0, 0);
                }
            }
        }
    }
}

// ------------------------------------------------------------------ kernel

// L2 prefetch of stage pf.s of the current tile: one dword per thread of A
// row t and of B row t, i.e. the first bytes of each row's stage slab (one
// 128-byte line when the row stride is a multiple of 128).  The dwords land
// in the junk LDS area and are never waited for or read.
__device__ __forceinline__ void l2_prefetch(uint8_t *lds, const Target &pf, const Ctx &c, int lda)
{
    const int k0 = pf.s * kRowBytes;
    const uint32_t off = ((uint32_t)(c.t * lda + k0) | (k0 < lda ? 0u : kOOB)) | pf.inval;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(pf.ra, (lds_void *)(lds + kLdsJunk + c.w * 256), 4, off, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(pf.rb, (lds_void *)(lds + kLdsJunk + c.w * 256), 4, off, 0, 0, 0);
}

// End of a stage: this wave's LDS reads and writes are done and all of its
// loads except the two newest (the L2 prefetch) have landed; then all waves
// meet.  After it the slot just read may be refilled and the slot just
// loaded may be read.
__device__ __forceinline__ void stage_barrier()
{
    if constexpr (kPrefetch > 0)
        asm volatile("s_waitcnt vmcnt(2) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    else
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// State threaded through the stage function.
template <int FMT>
struct Pipe {
    Frags<FMT> F0, F1;                       // k-step fragments, double-buffered
    Fp4Regs fp4;
    ScaleBytes<FMT> sbytes;
};

// Load piece q (of 8) of the target stage into ring slot `slot`, so the
// caller can interleave the pieces with MFMAs.
template <int FMT, bool ALIGNED>
__device__ __forceinline__ void load_piece(Pipe<FMT> &P, uint8_t *lds, int slot, const Target &tg, const Params &p,
                                           const Ctx &c, int q)
{
    if constexpr (FMT == kNVFP4) {
        if (q == 0) load_fp4(P.fp4, tg, p.lda, p.sld, c.t);
    } else {
        dma_pair(lds, slot, tg, c, q, p.lda);
        if constexpr (FMT == kMXFP8 || FMT == kMXFP4) {
            if (q == 7) {
                if constexpr (ALIGNED)
                    dma_scales<FMT>(lds, slot, tg, c, p.sld);
                else
                    load_scale_bytes(P.sbytes, tg, c.t, p.sld);
            }
        }
    }
}

// Register-staged parts of a stage (NVFP4 data, unaligned MX scales) go to
// LDS before the stage's barrier.
template <int FMT, bool ALIGNED>
__device__ __forceinline__ void commit_stage(Pipe<FMT> &P, uint8_t *lds, int slot, const Ctx &c)
{
    if constexpr (FMT == kNVFP4) store_fp4(P.fp4, lds, slot, c.t);
    if constexpr ((FMT == kMXFP8 || FMT == kMXFP4) && !ALIGNED) store_scale_bytes<FMT>(P.sbytes, lds, slot, c.t);
}

// Fragments are 8 VGPRs for E4M3 (two sets do not fit beside the 256
// accumulators), 4 for the other formats.
template <int FMT>
constexpr bool rolling() { return FMT == kMXFP8; }

// One phase: the 16 MFMAs of fragment set `cur` while set `nxt` is read
// (k-step rkk of slot rslot, if rd) and, if tg is given, the target stage is
// loaded into slot lslot in eight pieces between MFMA pairs, followed by the
// L2 prefetch pf.  Without
// rolling, `nxt` is read before the MFMAs.  With rolling, the MFMAs go in
// 2x2 groups and each next fragment is read as soon as the register it
// replaces is dead: A0/A1 after the second group, B0/B1 after the third,
// the rest after the fourth; every fragment is read at least four MFMAs
// before its first use in the next phase.
template <int FMT, bool ALIGNED>
__device__ __forceinline__ void phase(f32x16 (&acc)[4][4], Pipe<FMT> &P, const Frags<FMT> &cur, Frags<FMT> &nxt,
                                      uint8_t *lds, const Params &p, const Ctx &c, bool rd, int rslot, int rkk,
                                      const Target *tg, int lslot, const Target *pf = nullptr)
{
    if constexpr (!rolling<FMT>()) {
        if (rd) read_frags(nxt, lds, rslot, rkk, c);
        DBS_FENCE();
    }
    constexpr int gi[4] = {0, 0, 2, 2}, gj[4] = {0, 2, 0, 2};
#pragma unroll
    for (int g = 0; g < 4; ++g) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int i = gi[g] + (u >> 1), j = gj[g] + (u & 1);
            mma1(acc[i][j], cur, i, j);
            if ((u & 1) && tg) {
                DBS_FENCE();
                load_piece<FMT, ALIGNED>(P, lds, lslot, *tg, p, c, 2 * g + (u >> 1));
                DBS_FENCE();
            }
        }
        if (kPrefetch > 0 && g == 3 && pf) {
            DBS_FENCE();
            l2_prefetch(lds, *pf, c, p.lda);
            DBS_FENCE();
        }
        if constexpr (rolling<FMT>()) {
            if (rd) {
                if (g == 1) { read_a(nxt, 0, lds, rslot, rkk, c); read_a(nxt, 1, lds, rslot, rkk, c); }
                if (g == 2) { read_b(nxt, 0, lds, rslot, rkk, c); read_b(nxt, 1, lds, rslot, rkk, c); }
                if (g == 3) {
                    read_a(nxt, 2, lds, rslot, rkk, c); read_a(nxt, 3, lds, rslot, rkk, c);
                    read_b(nxt, 2, lds, rslot, rkk, c); read_b(nxt, 3, lds, rslot, rkk, c);
                }
            }
            DBS_FENCE();
        }
    }
}

// One stage read from ring slot `slot` while the target stage is loaded into
// the other slot.  On entry F1 holds the last k-step of the previous stage
// (zeros at a tile's first stage): its MFMAs form the first phase,
// interleaved with the loads and with the reads of k-step 0 of this stage.
template <int FMT, bool ALIGNED>
__device__ __forceinline__ void stage(Pipe<FMT> &P, f32x16 (&acc)[4][4], uint8_t *lds, int slot, const Params &p,
                                      const Ctx &c, const Target &tg, const Target &pf)
{
    constexpr int KK = Fmt<FMT>::KK;
    const int nxt = slot ^ 1;
    phase<FMT, ALIGNED>(acc, P, P.F1, P.F0, lds, p, c, true, slot, 0, &tg, nxt, &pf);
#pragma unroll
    for (int kk = 0; kk < KK - 1; ++kk) {
        if (kk & 1)
            phase<FMT, ALIGNED>(acc, P, P.F1, P.F0, lds, p, c, true, slot, kk + 1, nullptr, 0);
        else
            phase<FMT, ALIGNED>(acc, P, P.F0, P.F1, lds, p, c, true, slot, kk + 1, nullptr, 0);
    }
    commit_stage<FMT, ALIGNED>(P, lds, nxt, c);
    stage_barrier();
}

// Buffer resources of output tile `tile`: A/B rows and their scale rows.
template <int FMT>
__device__ __forceinline__ Target tile_target(const Params &p, int tile, int s)
{
    int tm, tn;
    tile_coords(tile, p, tm, tn);
    const int m0 = tm * kTileM, n0 = tn * kTileN;
    const int rows_a = min(p.M - m0, kTileM), rows_b = min(p.N - n0, kTileN);
    Target t;
    t.ra = make_rsrc(p.A + (int64_t)m0 * p.lda, (uint32_t)(rows_a * p.lda));
    t.rb = make_rsrc(p.B + (int64_t)n0 * p.lda, (uint32_t)(rows_b * p.lda));
    t.rsa = t.ra;
    t.rsb = t.rb;
    if constexpr (FMT != kBF16) {
        t.rsa = make_rsrc(p.sA + (int64_t)m0 * p.sld, (uint32_t)(rows_a * p.sld));
        t.rsb = make_rsrc(p.sB + (int64_t)n0 * p.sld, (uint32_t)(rows_b * p.sld));
    }
    t.s = s;
    t.inval = 0;
    return t;
}

template <int FMT, bool ALIGNED>
__global__ __launch_bounds__(kThreads, 1) void gemm_kernel(Params p)
{
    __shared__ __attribute__((aligned(1024))) uint8_t lds[lds_bytes<FMT>()];
    constexpr int BPS = scale_bps<FMT>();

    Ctx c;
    c.t = threadIdx.x;
    c.lane = c.t & 63;
    c.h = c.lane >> 5;
    c.lr = c.lane & 31;
    c.w = __builtin_amdgcn_readfirstlane(c.t >> 6);
    c.wm = c.w >> 1;
    c.wn = c.w & 1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int ra = c.wm * 128 + i * 32 + c.lr, rb = c.wn * 128 + i * 32 + c.lr;
        c.fa[i] = (uint32_t)(kLdsA + ra * kRowBytes + ((c.h ^ swz(ra)) << 4));
        c.fb[i] = (uint32_t)(kLdsB + rb * kRowBytes + ((c.h ^ swz(rb)) << 4));
        c.sa[i] = (uint32_t)(kLdsS + ra * BPS + c.h);
        c.sb[i] = (uint32_t)(kLdsS + 2 * kTileM * BPS + rb * BPS + c.h);
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const int row = c.w * 64 + q * 8 + (c.lane >> 3);
        c.kc[q] = ((c.lane & 7) ^ swz(row)) << 4;
        c.voff[q] = (uint32_t)(row * p.lda + c.kc[q]);
    }

    const int ntiles = p.tiles_m * p.tiles_n;
    const int nwg = gridDim.x, wg = blockIdx.x;
    // hardware places workgroup wg on XCD wg % 8: give each XCD a contiguous
    // range of logical ids
    int tile = (nwg & 7) == 0 ? (wg & 7) * (nwg >> 3) + (wg >> 3) : wg;
    if (tile >= ntiles) return;

    // One stream of stages over all of the workgroup's tiles: the last stage
    // of a tile loads stage 0 of the next one, so no tile starts cold.
    Pipe<FMT> P;
    Target cur = tile_target<FMT>(p, tile, 0);
#pragma unroll
    for (int q = 0; q < 8; ++q) load_piece<FMT, ALIGNED>(P, lds, 0, cur, p, c, q);
    commit_stage<FMT, ALIGNED>(P, lds, 0, c);
    __syncthreads();

    int g = 0;   // stages done by this workgroup: ring slot = g & 1
    for (;;) {
        const int next = tile + nwg;
        Target nt = tile_target<FMT>(p, next < ntiles ? next : tile, 0);
        if (next >= ntiles) nt.inval = kOOB;

        f32x16 acc[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
        // the "previous stage" of a tile's first stage contributes nothing
        P.F1 = Frags<FMT>{};
#pragma unroll
        for (int i = 0; i < 4; ++i) P.F1.sa[i] = P.F1.sb[i] = 127u;

        for (int s = 0; s < p.nk; ++s, ++g) {
            Target tg = cur;
            tg.s = s + 1;
            if (s + 1 == p.nk) tg = nt;
            Target pf = cur;
            pf.s = s + kPrefetch;
            if (pf.s >= p.nk) pf.inval = kOOB;
            stage<FMT, ALIGNED>(P, acc, lds, g & 1, p, c, tg, pf);
        }
        phase<FMT, ALIGNED>(acc, P, P.F1, P.F0, lds, p, c, false, 0, 0, nullptr, 0);

        int tm, tn;
        tile_coords(tile, p, tm, tn);
        store_tile(acc, p, tm * kTileM, tn * kTileN, c);
        if (next >= ntiles) break;
        tile = next;
        cur = nt;
    }
}

template <int FMT>
hipError_t launch_fmt(const Params &p, int grid, hipStream_t stream)
{
    const dim3 g(grid), b(kThreads);
    if (FMT == kBF16 || FMT == kNVFP4 || p.scales_aligned)
        hipLaunchKernelGGL((gemm_kernel<FMT, true>), g, b, 0, stream, p);
    else
        hipLaunchKernelGGL((gemm_kernel<FMT, false>), g, b, 0, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(int fmt, const Params &p, int grid, hipStream_t stream)
{
    switch (fmt) {
    case kBF16: return launch_fmt<kBF16>(p, grid, stream);
    case kMXFP8: return launch_fmt<kMXFP8>(p, grid, stream);
    case kMXFP4: return launch_fmt<kMXFP4>(p, grid, stream);
    case kNVFP4: return launch_fmt<kNVFP4>(p, grid, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace dbs
