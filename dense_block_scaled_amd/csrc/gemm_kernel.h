// gemm_kernel.h -- gfx950 (MI355X, CDNA4) kernels for the block-scaled GEMM
//
//     D[m, n] = bf16( alpha * sum_k dA[m, k] * dB[n, k] ),   fp32 accumulation
//
// One persistent kernel template serves the four formats (and the mixed MX
// element pairs) and two tile shapes; the gemm_*.hip units instantiate it.  Design (and where it departs from the Blackwell kernels the pages
// describe):
//
// * Scheduling.  A persistent grid of at most one workgroup per CU walks the
//   output tiles (cf. the persistent tile loop in "ThunderKittens Now on
//   NVIDIA Vera Rubin NVL72", Blackwell GEMM recap, and the static persistent
//   scheduler in "Dissecting ThunderKittens").  Workgroups are dispatched
//   round-robin over the 8 XCDs, so workgroup ids are remapped to give every
//   XCD a contiguous run of tile ids, and tile ids are rastered in groups of
//   `group_m` tile rows: the tiles one XCD runs at the same time share A and
//   B panels in that XCD's L2 (the locality concern of the "ThunderKittens
//   2.0" notes, section 6, and the raster-order tuning of the Vera Rubin
//   post, final optimisations).
// * Tile shapes (chosen by the host).  Square: 256 x 256 output tiles, 8
//   waves (two per SIMD), each owning 128 x 64 as 4 x 2 MFMA blocks of 32 x
//   32.  Skinny (when 256 x 256 tiles cannot fill the CUs, e.g. M = 256):
//   256 x 64 tiles, 8 waves of 32 x 64 on a three-slot ring, or 4 waves of
//   64 x 64 (raw NVFP4, and where stages pass through registers).  Two waves per SIMD matter on
//   gfx950: a wave that issues a global or LDS load stalls its own MFMA
//   stream for tens of cycles, and the second wave's MFMAs fill that gap
//   (the role split the pages obtain from dedicated producer warps).
// * Staging.  Each stage moves a tile-rows x 128-byte slab of A and of B into
//   one slot of a two-slot (skinny: up to three-slot) LDS ring (cf. the stage-count discussion of
//   "Async Tensor Core: Hopper wgmma -> Blackwell tcgen05", sections 3.1 and
//   4.3).  BF16/E4M3/E2M1 slabs go straight from HBM to LDS (buffer_load
//   ... lds), so staging costs no VGPRs and no LDS-write instructions; the
//   loads for stage s+1 are issued during stage s, spread between MFMAs.
//   Each lane fetches the global chunk that belongs at its fixed LDS
//   position under an XOR swizzle of the 16-byte chunks, which keeps
//   fragment reads bank-conflict-free.  Buffer loads return zero for rows
//   past M or N and for K columns past K (ragged shapes).  One barrier per
//   stage and no fences (cf. "ThunderKittens 2.0", section 1).
// * Scales.  MX scale bytes ride the same stage as their operand slab
//   (direct-to-LDS dword loads), and each lane feeds its E8M0 byte to the
//   scaled MFMA as the per-lane scale operand (the gfx950 counterpart of
//   issuing the scale copy from the same thread as the MMA, "ThunderKittens
//   2.0", section 2.1).
// * Math.  Each wave reuses every A fragment for all of its B blocks and
//   every B fragment for all of its A blocks from VGPRs (cf. dual
//   accumulation, "ThunderKittens 2.0", section 2.2).  Fragments are
//   double-buffered in VGPRs: the reads for k-step kk+1 are in flight while
//   the MFMAs of kk issue, and the MFMAs of a stage's last k-step are issued
//   after the barrier, behind the next stage's first reads.  BF16:
//   v_mfma_f32_32x32x16_bf16.  MXFP8/MXFP4: v_mfma_scale_f32_32x32x64_f8f6f4,
//   whose per-operand format codes also take E5M2 and, beside an 8-bit
//   operand, packed E2M1 (FP8 x FP4: the E2M1 operand in a ring of its own,
//   see F4Pos).  NVFP4: gfx950's scaled MFMA takes only E8M0 per 32, so
//   E2M1 x E4M3 is decoded exactly into fp16 (a product of 2- and 4-bit
//   significands with magnitude in [2^-10, 2688]) and multiplied on
//   v_mfma_f32_32x32x16_f16, tA*tB applied in the epilogue.  Where the packed
//   rows allow it (kNVFP4R) the codes and scales are staged as they are and
//   decoded in registers after the fragment read; otherwise the loader
//   decodes into LDS on the way in.
// * Epilogue.  alpha * acc -> bf16 (round to nearest even) -> global with
//   non-temporal buffer stores (out-of-range rows and columns dropped), in
//   the same kernel.
// * Operand layouts.  A and B may each be stored MN-major; such slots are
//   read with gfx950's transposed LDS reads (see Mn).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "launch.h"

namespace dbs {

// Launchers of the translation units (gemm_*.hip); launch_gemm (gemm.hip)
// picks one by format.
hipError_t launch_gemm_bf16(int shape, const Params &p, int grid, hipStream_t stream);
hipError_t launch_gemm_mxfp8(int shape, const Params &p, int grid, hipStream_t stream);
hipError_t launch_gemm_mx8_e5m2(int shape, const Params &p, int grid, hipStream_t stream);
hipError_t launch_gemm_mx8_fp4(int shape, const Params &p, int grid, hipStream_t stream);   // E2M1 or FP6 beside 8-bit
hipError_t launch_gemm_mxfp4(int shape, const Params &p, int grid, hipStream_t stream);
hipError_t launch_gemm_nvfp4(int shape, const Params &p, int grid, hipStream_t stream);
hipError_t launch_gemm_nvfp4_raw(int shape, const Params &p, int grid, hipStream_t stream);
// FP6 x FP6 at the FP6 rate on 256 x 256 tiles (gemm_mxfp6.hip).
hipError_t launch_gemm_mxfp6(const Params &p, int grid, hipStream_t stream);
// BF16 with decoupled A / B rings, A's slot released early or at the
// stage's end (gemm_bf16_ea.hip).
hipError_t launch_gemm_bf16_ea(const Params &p, bool early, int grid, hipStream_t stream);

namespace {

typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;
typedef __attribute__((ext_vector_type(2))) int i32x2;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((address_space(3))) void lds_void;

constexpr uint32_t kOOB = 0x80000000u;         // beyond every num_records we set
// Cache policy of the output stores: non-temporal.  D is written once and
// never read by the kernel; streaming it keeps more of A and B in the caches
// (BF16 8192^3: 1.5% in an A/B run; the other formats unchanged).
constexpr int kStoreNT = 2;

#define DBS_FENCE() __builtin_amdgcn_sched_barrier(0)

// Debug builds with DBS_LDS_POISON=1 (a separate library, libdbs_poison.so)
// fill the LDS destination of every direct-to-LDS load with 0xFF bytes before
// issuing it: NaN as bf16, E4M3, E5M2, E8M0 and as an NVFP4 scale, -6 and -7.5
// as E2M1 and E2M3 codes.  A fragment or scale read that ran ahead of its
// load's wait would then see poison instead of the data of an older stage,
// and the debug build's results would differ from the product build's.
#ifndef DBS_LDS_POISON
#define DBS_LDS_POISON 0
#endif

// Buffer resource over [base, base + bytes): loads at offsets >= bytes return
// zero, stores there are dropped.  Word 3 = 0x00020000 is the gfx9-family
// raw-buffer configuration (32-bit data format, no swizzle, no stride).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// Direct-to-LDS load of BYTES (4, 12 or 16) per lane into the wave's block
// at `dst` (lane i's bytes at dst + 4 i for dword loads, in a 16-byte cell
// dst + 16 i otherwise).  In the poison build the lane first fills that cell
// with 0xFF and waits for the write, so the load's data lands after it; every
// poisoned cell is rewritten by the same lane's load, which the stage's
// barrier waits for.
template <int BYTES>
__device__ __forceinline__ void lds_dma(__amdgpu_buffer_rsrc_t rsrc, uint8_t *dst, uint32_t voff)
{
    static_assert(BYTES == 4 || BYTES == 12 || BYTES == 16, "dword, dwordx3 or dwordx4 loads");
#if DBS_LDS_POISON
    const uint32_t lane = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    if constexpr (BYTES == 4)
        *reinterpret_cast<uint32_t *>(dst + 4 * lane) = ~0u;
    else
        *reinterpret_cast<i32x4 *>(dst + 16 * lane) = i32x4{-1, -1, -1, -1};
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#endif
    // (the builtin takes its size as a literal)
    if constexpr (BYTES == 4)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void *)dst, 4, voff, 0, 0, 0);
    else if constexpr (BYTES == 12)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void *)dst, 12, voff, 0, 0, 0);
    else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void *)dst, 16, voff, 0, 0, 0);
}

constexpr int kRowBytes = 128;                 // bytes of one tile row per stage

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

// Where output tile `tile` of a TM x TN tiling lies: rows m0 .. mend-1 of A
// and D (mend: the end of its group, or M), columns n0 .. of D, its group's
// B and sB blocks at byte offsets boff and sboff, and its output scale.
struct TileRef {
    int m0, mend, n0;
    int64_t boff, sboff;
    float alpha;
};

template <int TM, int TN>
__device__ __forceinline__ TileRef tile_ref(int tile, const Params &p)
{
    TileRef r;
    if (p.ngroups == 0) {
        int tm, tn;
        tile_coords(tile, p, tm, tn);
        r.m0 = tm * TM;
        r.mend = p.M;
        r.n0 = tn * TN;
        r.boff = r.sboff = 0;
        r.alpha = p.alpha;
        return r;
    }
    // the group holding the tile: the last g with gtiles[g] <= tile (binary
    // search over the uniform table; empty groups have equal neighbours)
    int lo = 0, hi = p.ngroups;          // gtiles[lo] <= tile < gtiles[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (p.gtiles[mid] <= tile) lo = mid; else hi = mid;
    }
    const int g = lo;
    const int rows = p.goff[g + 1] - p.goff[g];
    const int tmg = (rows + TM - 1) / TM;
    const int local = tile - p.gtiles[g];
    r.m0 = p.goff[g] + (local % tmg) * TM;
    r.mend = p.goff[g + 1];
    r.n0 = (local / tmg) * TN;
    r.boff = (int64_t)g * p.N * p.lda;
    r.sboff = (int64_t)g * p.N * p.sld;
    r.alpha = p.galpha[g];
    return r;
}

// ------------------------------------------------------------- tile shapes

// TM x TN output tile (TM rows of A, TN rows of B per stage) computed by a
// WM x WN grid of waves, each owning MB x NB MFMA blocks of 32 x 32, over an
// NS-slot LDS ring.  A stage moves (TM + TN) / 8 wave-loads of 1 KiB (8 rows
// x 128 bytes); wave w issues QA of A and QB of B.  LDS: A slots 0..NS-1 | B
// slots 0..NS-1 | scale slots (MX formats) SA 0..NS-1 | SB 0..NS-1 of rows x
// BPS bytes.  LAY: bit 0 set if A is stored MN-major (K x M), bit 1 if B is
// (K x N); a slot of an MN-major operand holds the same bytes as a K-major
// one, arranged as the stage's K-rows (see Mn below).  EC: the 8-bit MX
// element formats as gfx950's f8f6f4 MFMA codes, A in bits 0..2 and B in
// bits 3..5 (0 = E4M3, 1 = E5M2, 4 = E2M1 packed: see F4Pos); E4M3 and E5M2
// take the same bytes and fragments, only the MFMA's format fields differ.
// CV (8-bit MX kernels): the source element of an operand that arrives as
// E2M1 or FP6 (E2M3, E3M2) and is widened on its way into LDS (see load_cv)
// to the 8-bit format holding all its values exactly (E2M1, E2M3 -> E4M3;
// E3M2 -> E5M2), which is what the MFMAs then see.
constexpr int pow2_at_least(int n) { return n <= 1 ? 1 : 2 * pow2_at_least((n + 1) / 2); }

template <int TM_, int TN_, int WM_, int WN_, int NS_ = 2, int LAY_ = 0, int EC_ = 0, int CV_ = 0>
struct Shape {
    static constexpr int TM = TM_, TN = TN_, WM = WM_, WN = WN_, NS = NS_, LAY = LAY_, EC = EC_, CV = CV_;
    static constexpr bool AMN = (LAY & 1) != 0, BMN = (LAY & 2) != 0;
    // widened operands: source element of A (bits 0..1) and B (bits 2..3):
    // 0 none, 1 E2M1, 2 E2M3, 3 E3M2
    static constexpr int ASRC = CV & 3, BSRC = (CV >> 2) & 3;
    static constexpr bool ACV = ASRC != 0, BCV = BSRC != 0;
    static constexpr int CA = EC & 7, CB = (EC >> 3) & 7;
    // an E2M1 operand (code 4) of an 8-bit kernel, staged as packed codes
    static constexpr bool AF4 = CA == 4, BF4 = CB == 4;
    // the format whose staging operand A / B follows in a kernel of format F
    template <int F>
    static constexpr int fa() { return AF4 ? 2 : F; }      // 2: kMXFP4
    template <int F>
    static constexpr int fb() { return BF4 ? 2 : F; }
    static constexpr int NW = WM * WN;
    static constexpr int kThreads = 64 * NW;
    static constexpr int MB = TM / WM / 32, NB = TN / WN / 32;
    static constexpr int RPL = 1024 / kRowBytes;   // rows per 1 KiB wave-load
    static constexpr int QA = TM / RPL / NW, QB = TN / RPL / NW;
    static constexpr int kSlotA = TM * kRowBytes, kSlotB = TN * kRowBytes;
    static constexpr int kLdsA = 0, kLdsB = NS * kSlotA, kLdsS = NS * (kSlotA + kSlotB);
    static_assert(MB * 32 * WM == TM && NB * 32 * WN == TN, "waves must tile the output tile");
    static_assert(QA * RPL * NW == TM && QB * RPL * NW == TN && QB > 0, "wave-loads must split evenly");
    static_assert(TM % 64 == 0 && TN % 64 == 0, "row groups must be whole waves");
    static_assert(NS >= 2, "the ring needs two slots");
    // slot offsets only touch bits above every in-slot address (see read_frag)
    static_assert((kSlotA & (kSlotA - 1)) == 0 && (kSlotB & (kSlotB - 1)) == 0 &&
                      kLdsB % (pow2_at_least(NS) * kSlotB) == 0,
                  "slot offsets must be OR-able");
};
using Square = Shape<kSquareTM, kSquareTN, 2, 4>;
// Skinny tiles hold 40 KiB per slot: formats whose stages arrive entirely by
// direct-to-LDS loads use a three-slot ring (loads get two stages to land)
// and 8 waves of 32 x 64 (two per SIMD); register-staged ones (NVFP4,
// unaligned MX scales) keep two slots and 4 waves of 64 x 64.
using Skinny = Shape<kSkinnyTM, kSkinnyTN, 4, 1>;
using SkinnyDeep = Shape<kSkinnyTM, kSkinnyTN, 8, 1, 3>;
// Square tiles for MX scales whose rows are not whole dwords (K % 128 != 0):
// the register-staged scale bytes do not fit beside two waves per SIMD, so
// this variant runs one wave per SIMD, each owning 128 x 128.
using SquareW4 = Shape<kSquareTM, kSquareTN, 2, 2>;
// 256 x 64 tiles with 8 waves of 32 x 64 on a two-slot ring: FP6 operands,
// widened through registers, with two waves per SIMD to hide their loads.
using SkinnyW8 = Shape<kSkinnyTM, kSkinnyTN, 8, 1>;
// 256 x 64 tiles for raw NVFP4 with K-major operands: 4 waves of 64 x 64 (one
// per SIMD, accumulators in AGPRs) decode 4 fragments per 4 MFMAs, a third
// less VALU work per MFMA than 8 waves of 32 x 64; a three-slot ring.
using SkinnyW4Deep = Shape<kSkinnyTM, kSkinnyTN, 4, 1, 3>;

// Shape S with operand layouts LAY, 8-bit MX element codes EC and widened
// E2M1 operands CV.
template <class S, int LAY, int EC = S::EC, int CV = S::CV>
using WithLayout = Shape<S::TM, S::TN, S::WM, S::WN, S::NS, LAY, EC, CV>;

// ------------------------------------------------------------ format traits

template <int FMT>
struct Fmt;
template <>
struct Fmt<kBF16> {
    static constexpr int KSB = 32;         // row bytes per MFMA k-step (16 K)
    static constexpr int BPS = 0;          // MX scale bytes per row per stage
    using Frag = bf16x8;
};
template <>
struct Fmt<kNVFP4> {
    static constexpr int KSB = 32;         // fp16 in LDS, same geometry as bf16
    static constexpr int BPS = 0;
    using Frag = f16x8;
};
template <>
struct Fmt<kMXFP8> {
    static constexpr int KSB = 64;         // 64 K per k-step, 32 bytes per lane
    static constexpr int BPS = 4;          // 2 blocks of 32 per k-step
    using Frag = i32x8;
};
template <>
struct Fmt<kMXFP4> {
    static constexpr int KSB = 32;         // 64 K per k-step, 16 bytes per lane
    static constexpr int BPS = 8;
    using Frag = i32x4;
};
template <>
struct Fmt<kNVFP4R> {
    static constexpr int KSB = 32;         // staged like E2M1 MX: 64 K per k-step
    static constexpr int BPS = 16;         // E4M3 scale bytes per row per stage (one per 16 K)
    using Frag = i32x4;
};

// MX scales: E8M0 per 32, fed to the scaled MFMA
template <int FMT>
constexpr bool mx_scales() { return FMT == kMXFP8 || FMT == kMXFP4; }

// MFMA k-steps per stage
template <int FMT, class S>
constexpr int kk_of() { return kRowBytes / Fmt<FMT>::KSB; }

// MN-major operands (A stored K x M, B stored K x N; FP4 packs two elements
// of consecutive rows of the tile, i.e. consecutive M or N, per byte, low
// nibble first).  A slot of such an operand holds the stage's KS = 8 *
// kRowBytes / EB K-rows, each the T elements of the tile's rows of that
// operand (RB = T * EB / 8 bytes), as RB / 16 chunks of 16 bytes under an
// XOR swizzle f(row).  The MFMA fragments come out of it through gfx950's
// transposed LDS reads (ds_read_b64_tr_b16 / _b8 / _b4).  Within each group
// of 16 lanes such a read takes a block of 4 (b16), 8 (b8) or 16 (b4) K-rows
// x 16 columns, every lane giving the address of 8 bytes of one K-row (rows
// in lane order, 4, 2 or 1 lanes per row), and returns to lane j the column
// j of the block, i.e. 4, 8 or 16 consecutive K values of one output row or
// column, packed like a K-major fragment (established with a one-wave
// probe).  A 32-column fragment of one k-step takes 2 (BF16, E2M1) or 4
// (E4M3) such reads, lane group g covering columns 16 (g % 2) .. +15 and
// lane half g / 2 its half of the k-step.
//
// The reads of one instruction cover W = 2 * EB / 8 chunks of each of
// 16 / W K-rows per half-wave (32 columns): the swizzle moves consecutive
// K-rows to different banks.  Rows of RB < 256 bytes share a 256-byte bank
// line (P = 16 / CPR of them), so f only has to separate rows P apart.
template <int FMT, int T>
struct Mn {
    static constexpr int EB = FMT == kBF16 ? 16 : FMT == kMXFP8 ? 8 : 4;   // element bits
    static constexpr int RB = T * EB / 8;                                  // bytes per K-row
    static constexpr int KS = 8 * kRowBytes / EB;                          // K-rows per stage
    static constexpr int CPR = RB / 16;
    static constexpr int CPRM = CPR < 16 ? CPR : 16;
    static constexpr int P = 16 / CPRM;
    static constexpr int W = 2 * EB / 8;
    static constexpr int NF = CPRM / W;                  // distinct swizzle values
    static constexpr int PERIOD = P * NF;                // f(r + PERIOD) = f(r)
    static constexpr int RPL = 1024 / RB;                // K-rows per 1 KiB wave-load
    static constexpr int KSTEP = FMT == kBF16 ? 16 : 64; // K-rows per MFMA k-step
    static constexpr int QSTEP = FMT == kBF16 ? 4 : FMT == kMXFP8 ? 8 : 16;   // K-rows between sub-reads
    __device__ static constexpr int f(int r) { return W * ((r / P) % NF); }
    static_assert(FMT != kNVFP4, "MN-major NVFP4 operands are staged raw (kNVFP4R)");
    static_assert(NF >= 1 && RB <= 1024 && KS * RB == T * kRowBytes, "slot geometry");
    // the K-rows one lane reads lie whole periods apart: one swizzle value per lane
    static_assert(KSTEP % PERIOD == 0 && QSTEP % PERIOD == 0, "one swizzle value per lane");
    // the K-rows of wave-load L depend on L at most through its parity
    static_assert(RPL % PERIOD == 0 || 2 * RPL == PERIOD, "wave-load swizzle");
};

// How MX scales reach LDS (the kernels' SM parameter):
//  kScalesRegs:  any row stride; thread-owned byte loads through registers
//                into NS per-stage slots of (TM + TN) rows x BPS bytes;
//  kScalesStage: rows of whole dwords; per-stage direct-to-LDS dword loads
//                into the same per-stage slots;
//  kScalesChunk: rows of whole dwords, two-slot rings with a whole number of
//                chunks per tile; the scales of kScaleChunk / BPS consecutive
//                stages (16 bytes per row: E4M3 4 stages, E2M1 2) form a
//                chunk, kept in two alternating buffers of (TM + TN) rows x
//                16 bytes.  During each stage of a chunk the next chunk's
//                rows are loaded a portion at a time, four lanes per row, so
//                a row costs one memory request per chunk instead of one per
//                stage (a per-stage fetch of 4 or 8 bytes from each of the
//                tile's 512 scale rows costs as many L2 requests as the
//                stage's operand slabs).
//  kScalesRows16: raw NVFP4 only (16 scale bytes per row per stage), scale
//                rows of whole 16-byte pieces on 16-byte boundaries: the
//                per-stage slots filled by 16-byte direct-to-LDS loads, one
//                row per lane (a quarter of the dword loads' instructions).
constexpr int kScalesRegs = 0, kScalesStage = 1, kScalesChunk = 2, kScalesRows16 = 4;
constexpr int kScaleChunk = 16;
// NVFP4 has no MX scales; its SM parameter says whether K ends on a whole
// 32-element half-row (kNvWhole) or halfway through one (kNvHalf: K % 32 ==
// 16, which the format allows).  Then packed rows (K/2 bytes) start on
// 8-byte boundaries only and scale rows (K/16 bytes) on byte boundaries, so
// the loader fetches each half-row as two 8-byte pieces and its two scales
// as single bytes, and the past-K piece of a row's last half reads zero
// codes and a zero scale.
constexpr int kNvWhole = 1, kNvHalf = 3;

template <int FMT>
constexpr int scale_spc() { return Fmt<FMT>::BPS > 0 ? kScaleChunk / Fmt<FMT>::BPS : 1; }

template <int FMT, class S, int SM>
constexpr int lds_bytes()
{
    return Fmt<FMT>::BPS == 0     ? S::kLdsS
           : SM == kScalesChunk ? S::kLdsS + 2 * (S::TM + S::TN) * kScaleChunk
                                : S::kLdsS + S::NS * (S::TM + S::TN) * Fmt<FMT>::BPS;
}

// E4M3 fragments are 8 VGPRs: with 8 waves (256 VGPRs per wave) two full
// sets do not fit beside the accumulators, so A fragments are single-buffered
// and each is re-read as soon as its last MFMA of the k-step has issued.
template <int FMT, class S>
constexpr bool rolling() { return FMT == kMXFP8 && S::MB * S::NB >= 8; }

// NVFP4 with one wave per column of the wave grid (the skinny tiles): every
// A row is used by a single wave, so each wave decodes its own A rows
// straight into MFMA fragments and only B goes through LDS.  Within a stage
// (64 K elements) lane half h then takes elements [32h, 32h+32): k-step kk
// uses elements 32h + 8kk .. +7 of A and of B (the same permutation of K on
// both operands leaves the dot products unchanged).
template <int FMT, class S>
constexpr bool adirect() { return FMT == kNVFP4 && S::WN == 1; }

// Per-lane constants of one workgroup.  w, wm, wn are wave-uniform.
template <class S>
struct Ctx {
    int t, lane, h, lr;
    int w, wm, wn;
    uint32_t fa, fb;                 // LDS address of the lane's fragment read, block 0, k-step 0, slot 0
    uint32_t sa, sb;                 // LDS address of the lane's MX scale row, block 0, slot 0
    uint32_t r8lda;                  // the lane's row within a wave-load times the row stride
    uint32_t x4;                     // the lane's chunk within a wave-load, swizzle applied, << 4
    uint32_t ma[2], mb[2];           // MN-major A / B: the lane's global offset in a wave-load of parity 0 / 1
};

// Whose stages a load fetches: the tile whose operand and scale rows start
// at the four buffer resources.  A workgroup with nothing left loads from
// empty resources, so every load reads zero.
struct Target {
    __amdgpu_buffer_rsrc_t ra, rb, rsa, rsb;
};

// The packed E2M1 operand of an 8-bit kernel (S::AF4 / S::BF4) has a ring of
// its own: a slot holds 256 K of every row (128-byte rows, staged as MXFP4
// stages them) and serves two 8-bit stages of 128 K.  Stage s of a tile
// reads half s % 2 of slot rs (its MXFP4 k-steps 2 (s % 2), 2 (s % 2) + 1)
// and loads the same half of the slot's wave-loads of 256-K stage ks (from
// resource r) into slot ls = rs ^ 1, which the two stages before last read.
struct F4Pos {
    int rs, half, ls, ks;
    __amdgpu_buffer_rsrc_t r;
};

template <int FMT, class S>
struct Frags {
    // a packed E2M1 operand of an 8-bit kernel holds MXFP4 fragments
    typename std::conditional<S::AF4, i32x4, typename Fmt<FMT>::Frag>::type a[S::MB];
    typename std::conditional<S::BF4, i32x4, typename Fmt<FMT>::Frag>::type b[S::NB];
    // raw NVFP4: the two E4M3 scales of each fragment's 32 elements (lane half
    // h holds K 32h .. 32h+31 of the k-step, two 16-element blocks)
    uint32_t sa[FMT == kNVFP4R ? S::MB : 1], sb[FMT == kNVFP4R ? S::NB : 1];
};

// MX scales of one stage for the lane's row of each row block, one dword per
// block: the byte the scaled MFMA takes for k-step kk sits at byte
// scale_sel<FMT>(kk), which the instruction's op_sel picks (established with
// a one-instruction probe: op_sel k selects byte k of the scale register).
template <class S>
struct Scales {
    uint32_t a[S::MB][2], b[S::NB][2];   // [0]: the op_sel-ready dword; [1]: raw high dword (E2M1)
};

template <int FMT>
constexpr int scale_sel(int kk) { return FMT == kMXFP8 ? 2 * kk : kk; }

template <typename V>
__device__ __forceinline__ V lds_read(const uint8_t *lds, uint32_t addr)
{
    return *reinterpret_cast<const V *>(lds + addr);
}

// Fragment read for k-step kk at LDS address fbase of slot 0; `sel` is the
// slot's byte offset (a power of two above every bit of fbase, so adding it
// equals OR-ing it in).  16-bit formats: lane l holds the 8 elements of chunk
// 2 kk + l/32 of its row.  E2M1: 32 elements, chunk 2 kk + l/32.  E4M3: in
// the 32x32x64 scaled MFMA with 8-bit elements, lane half h holds K
// positions [16h, 16h+16) in bytes 0..15 and [32+16h, 48+16h) in bytes
// 16..31, and its scale applies to K block h, i.e. bytes 16h..16h+15 of both
// halves (established with a one-instruction probe); so lane half h reads
// chunks 4 kk + h and 4 kk + 2 + h.  With the XOR swizzle, chunk 2 kk + h of
// a row sits at fbase ^ (kk << 5) and chunk 4 kk + h at fbase ^ (kk << 6).
// The whole address is one XOR of fbase with a wave-uniform value, computed
// at the read so that no per-k-step address stays live in a VGPR.  Row block
// i (rows r + 32 i) differs from block 0 only by 32 i rows (an immediate
// offset of 4096 i bytes) and by bit 2 of the swizzle when i is odd
// (((r + 32 i) >> 3) & 7 = ((r >> 3) + 4 i) & 7), i.e. by address bit 6.
template <int FMT, int KSH = 5>
__device__ __forceinline__ typename Fmt<FMT>::Frag read_frag(const uint8_t *lds, uint32_t fbase, uint32_t sel, int kk,
                                                             int blk)
{
    const uint32_t flip = (uint32_t)(64 * (blk & 1)), off = (uint32_t)(32 * kRowBytes * blk);
    if constexpr (FMT == kMXFP8) {
        const uint32_t x = fbase ^ (sel | ((uint32_t)(kk << 6) ^ flip));
        const i32x4 v0 = lds_read<i32x4>(lds, x + off), v1 = lds_read<i32x4>(lds, (x ^ 32u) + off);
        return i32x8{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
    } else {
        return lds_read<typename Fmt<FMT>::Frag>(lds, (fbase ^ (sel | ((uint32_t)(kk << KSH) ^ flip))) + off);
    }
}

// MN-major fragment of block `blk` (32 columns), k-step kk: the transposed
// reads of the lane's K-rows (see Mn).  fbase is the lane's address for block
// 0, k-step 0, slot 0 with the swizzle applied (mn_base); block and slot
// offsets occupy bits no other term uses, so they enter by XOR, and the
// k-step and sub-read rows are whole swizzle periods further down, so they
// enter as immediate offsets.
template <int FMT, int T>
__device__ __forceinline__ typename Fmt<FMT>::Frag read_frag_mn(const uint8_t *lds, uint32_t fbase, uint32_t sel,
                                                                int kk, int blk)
{
    using G = Mn<FMT, T>;
    typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    const uint32_t x = fbase ^ (sel | (uint32_t)(blk * 4 * G::EB));
    auto rd = [&](int dr) -> i32x2 {
        const uint8_t *ptr = lds + x + dr * G::RB;
        if constexpr (FMT == kBF16)
            return __builtin_bit_cast(i32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)ptr));
        else if constexpr (FMT == kMXFP8)
            return __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2 *)ptr);
        else
            return __builtin_amdgcn_ds_read_tr4_b64_v2i32((lds_i32x2 *)ptr);
    };
    const int r = kk * G::KSTEP;
    if constexpr (FMT == kMXFP8) {
        // bytes 0..15: K 16h .. 16h+15; bytes 16..31: K 32+16h .. (see read_frag)
        const i32x2 v0 = rd(r), v1 = rd(r + 8), v2 = rd(r + 32), v3 = rd(r + 40);
        return i32x8{v0[0], v0[1], v1[0], v1[1], v2[0], v2[1], v3[0], v3[1]};
    } else {
        const i32x2 v0 = rd(r), v1 = rd(r + G::QSTEP);
        return __builtin_bit_cast(typename Fmt<FMT>::Frag, i32x4{v0[0], v0[1], v1[0], v1[1]});
    }
}

// The lane's fragment-read address (block 0, k-step 0, slot 0) in an
// MN-major operand region whose wave owns columns wc ..: lane 16 g + j
// addresses K-row r0 of its read block (lane half g / 2 taking the second
// half of each k-step) at the 8 bytes of columns 16 (g % 2) + .. that its
// position in the group stands for.
template <int FMT, int T>
__device__ __forceinline__ uint32_t mn_base(int lane, int wc, int region)
{
    using G = Mn<FMT, T>;
    const int g = lane >> 4, j = lane & 15;
    int r0, cb;
    if constexpr (FMT == kBF16) {
        r0 = 8 * (g >> 1) + (j >> 2);                        // 4 lanes per K-row, 4 columns each
        cb = 2 * (wc + 16 * (g & 1) + 4 * (j & 3));
    } else if constexpr (FMT == kMXFP8) {
        r0 = 16 * (g >> 1) + (j >> 1);                       // 2 lanes per K-row, 8 columns each
        cb = wc + 16 * (g & 1) + 8 * (j & 1);
    } else {
        r0 = 32 * (g >> 1) + j;                              // 1 lane per K-row, 16 columns
        cb = wc / 2 + 8 * (g & 1);
    }
    return (uint32_t)(region + r0 * G::RB + (cb ^ (G::f(r0) << 4)));
}

// The lane's global offset within an MN-major wave-load of parity `par`
// (relative to the operand's first column of the tile; row stride ldx
// bytes): it lands on slot byte 1024 L + 16 lane, i.e. K-row L RPL + r and
// physical chunk pc, and fetches the logical chunk the swizzle puts there.
template <int FMT, int T>
__device__ __forceinline__ uint32_t mn_dma_lane(int lane, int par, int ldx)
{
    using G = Mn<FMT, T>;
    const int r = (16 * lane) / G::RB, pc = ((16 * lane) % G::RB) >> 4;
    return (uint32_t)(r * ldx + ((pc ^ G::f(r + par * G::RPL)) << 4));
}

// MX scales: lane l of a 32x32x64 scaled MFMA supplies the E8M0 scale of K
// block l/32 of row l%32; for k-step kk that is byte 2 kk + l/32 of the row's
// stage scales.  One read per row block and stage: E4M3 rows hold 4 bytes
// (kk = 0, 1), shifted right by 8 (l/32) so k-step kk's byte is byte 2 kk;
// E2M1 rows hold 8 bytes (kk = 0..3), of which bytes l/32, 2 + l/32,
// 4 + l/32, 6 + l/32 are packed into bytes 0..3.
// The stage's scale rows are read raw at the start of the stage and made
// op_sel-ready where first needed (adjust_scales), so the adjustment does not
// wait on reads that were just issued.
template <int FMT>
__device__ __forceinline__ void read_scale_row(uint32_t (&r)[2], const uint8_t *lds, uint32_t addr)
{
    if constexpr (FMT == kMXFP8) {
        r[0] = lds_read<uint32_t>(lds, addr);
    } else {
        const u32x2 v = lds_read<u32x2>(lds, addr);
        r[0] = v[0];
        r[1] = v[1];
    }
}

template <int FMT>
__device__ __forceinline__ void adjust_scale_row(uint32_t (&r)[2], int h)
{
    if constexpr (FMT == kMXFP8)
        r[0] >>= 8 * h;
    else
        r[0] = __builtin_amdgcn_perm(r[1], r[0], 0x06040200u + 0x01010101u * (uint32_t)h);
}

template <int FMT, class S>
__device__ __forceinline__ void read_scales(Scales<S> &sc, const uint8_t *lds, int slot, const Ctx<S> &c)
{
    constexpr int BPS = Fmt<FMT>::BPS;
#pragma unroll
    for (int i = 0; i < S::MB; ++i)
        read_scale_row<FMT>(sc.a[i], lds, c.sa + (uint32_t)(slot * S::TM * BPS + i * 32 * BPS));
#pragma unroll
    for (int j = 0; j < S::NB; ++j)
        read_scale_row<FMT>(sc.b[j], lds, c.sb + (uint32_t)(slot * S::TN * BPS + j * 32 * BPS));
}

// Chunked layout: a row's 16 chunk bytes hold dword d at position
// d ^ chunk_swz(row), row = the row's index in the concatenated list (see
// dma_scale_portion).  The 32 rows one scale read covers lie 16 bytes apart:
// rows 8 apart are 128 bytes apart and rows 16 apart 256, so without the
// swizzle they would meet in one bank whether the LDS serves a read 128 or
// 256 bytes at a time.  Dword reads (E4M3; 32 lanes) take position
// d ^ ((row / 8) % 4), so rows r, r + 8, r + 16, r + 24 use four different
// dwords; 8-byte reads (E2M1; a stage's two dwords stay together) swap the
// row's two halves by bit 3 ^ bit 4 of the row, which separates rows 8 apart
// (16 lanes a pass) and rows 16 apart (32 lanes a pass).  c.sa and c.sb carry
// 4 chunk_swz in their (otherwise zero) bits 2-3, so the stage's byte offset
// enters by XOR.
template <int FMT>
__device__ __forceinline__ constexpr int chunk_swz(int row)
{
    return Fmt<FMT>::BPS == 4 ? (row >> 3) & 3 : 2 * (((row >> 3) ^ (row >> 4)) & 1);
}

template <int FMT, class S>
__device__ __forceinline__ void read_scales_chunk(Scales<S> &sc, const uint8_t *lds, int par, int j, const Ctx<S> &c)
{
    constexpr int BPS = Fmt<FMT>::BPS;
    const uint32_t o = (uint32_t)(par * (S::TM + S::TN) * kScaleChunk);
    const uint32_t jb = (uint32_t)(j * BPS);
#pragma unroll
    for (int i = 0; i < S::MB; ++i)
        read_scale_row<FMT>(sc.a[i], lds, (c.sa ^ jb) + o + (uint32_t)(i * 32 * kScaleChunk));
#pragma unroll
    for (int jj = 0; jj < S::NB; ++jj)
        read_scale_row<FMT>(sc.b[jj], lds, (c.sb ^ jb) + o + (uint32_t)(jj * 32 * kScaleChunk));
}

template <int FMT, class S>
__device__ __forceinline__ void adjust_scales(Scales<S> &sc, const Ctx<S> &c)
{
#pragma unroll
    for (int i = 0; i < S::MB; ++i) adjust_scale_row<FMT>(sc.a[i], c.h);
#pragma unroll
    for (int j = 0; j < S::NB; ++j) adjust_scale_row<FMT>(sc.b[j], c.h);
}

template <int FMT, class S>
__device__ __forceinline__ void read_a(Frags<FMT, S> &f, int i, const uint8_t *lds, int slot, int kk,
                                       const Ctx<S> &c)
{
    if constexpr (S::AMN)
        f.a[i] = read_frag_mn<FMT, S::TM>(lds, c.fa, (uint32_t)(slot * S::kSlotA), kk, i);
    else
        f.a[i] = read_frag<FMT>(lds, c.fa, (uint32_t)(slot * S::kSlotA), kk, i);
    if constexpr (FMT == kNVFP4R)
        f.sa[i] = lds_read<uint16_t>(lds, (c.sa ^ (uint32_t)(4 * kk)) + (uint32_t)(slot * S::TM * 16 + i * 32 * 16 + 2 * c.h));
}

template <int FMT, class S>
__device__ __forceinline__ void read_b(Frags<FMT, S> &f, int j, const uint8_t *lds, int slot, int kk,
                                       const Ctx<S> &c)
{
    // with A decoded in registers, B's k-step kk is chunk 4h + kk of the row
    constexpr int KSH = adirect<FMT, S>() ? 4 : 5;
    if constexpr (S::BMN)
        f.b[j] = read_frag_mn<FMT, S::TN>(lds, c.fb, (uint32_t)(slot * S::kSlotB), kk, j);
    else
        f.b[j] = read_frag<FMT, KSH>(lds, c.fb, (uint32_t)(slot * S::kSlotB), kk, j);
    if constexpr (FMT == kNVFP4R)
        f.sb[j] = lds_read<uint16_t>(lds, (c.sb ^ (uint32_t)(4 * kk)) + (uint32_t)(slot * S::TN * 16 + j * 32 * 16 + 2 * c.h));
}

// Fragments of a packed E2M1 operand of an 8-bit kernel: MXFP4 k-step
// 2 half + kk of its ring slot (lane half h: K 32h .. 32h + 31 of the 8-bit
// k-step kk, the layout the f8f6f4 MFMA takes for E2M1).
template <int FMT, class S>
__device__ __forceinline__ void read_a_f4(Frags<FMT, S> &f, int i, const uint8_t *lds, const F4Pos &fp, int kk,
                                          const Ctx<S> &c)
{
    if constexpr (S::AMN)
        f.a[i] = read_frag_mn<kMXFP4, S::TM>(lds, c.fa, (uint32_t)(fp.rs * S::kSlotA), 2 * fp.half + kk, i);
    else
        f.a[i] = read_frag<kMXFP4>(lds, c.fa, (uint32_t)(fp.rs * S::kSlotA), 2 * fp.half + kk, i);
}

template <int FMT, class S>
__device__ __forceinline__ void read_b_f4(Frags<FMT, S> &f, int j, const uint8_t *lds, const F4Pos &fp, int kk,
                                          const Ctx<S> &c)
{
    if constexpr (S::BMN)
        f.b[j] = read_frag_mn<kMXFP4, S::TN>(lds, c.fb, (uint32_t)(fp.rs * S::kSlotB), 2 * fp.half + kk, j);
    else
        f.b[j] = read_frag<kMXFP4>(lds, c.fb, (uint32_t)(fp.rs * S::kSlotB), 2 * fp.half + kk, j);
}

// ------------------------------------------------------------------ scales

// MX scales of the target stage go to scale slot `slot`: TM (A) and TN (B)
// rows of BPS bytes, i.e. TM*BPS/4 + TN*BPS/4 dwords, stored densely.
//
// Rows whose stage scales are whole dwords (row stride K/32 a multiple of 4):
// direct-to-LDS dword wave-loads.  Wave-load n of an operand writes its
// dwords 64n .. 64n+63 (LDS bytes 256n ..); dword d is word d % (BPS/4) of
// row d / (BPS/4).  Wave w issues wave-loads w, w + NW, ... of the
// concatenated list (A then B).  A dword past the row's last block (partial
// last stage) reads zero.
template <int FMT, class S>
__device__ __forceinline__ void dma_scales(uint8_t *lds, int slot, const Target &tg, int ks, const Ctx<S> &c, int sld)
{
    constexpr int BPS = Fmt<FMT>::BPS, WPR = BPS / 4;
    constexpr int NSA = S::TM * BPS / 256, NSB = S::TN * BPS / 256, NS = NSA + NSB;
    // Every wave issues the same number of loads, with no branch: when the
    // wave count does not divide the load count, the spare loads repeat
    // earlier ones (same bytes to the same place).  A branch here would split
    // the stage's code and let the compiler gather the MFMAs after it.
#pragma unroll
    for (int k = 0; k < (NS + S::NW - 1) / S::NW; ++k) {
        const int n = (c.w + k * S::NW) % NS;      // wave-uniform
        const bool is_a = n < NSA;
        const int nn = is_a ? n : n - NSA;
        const int d = nn * 64 + c.lane;
        const int row = d / WPR, word = d % WPR;
        // raw NVFP4 (16-byte rows): position `word` of the row holds its
        // dword word ^ ((row / 8) % 4) (see the kernel's scale addresses)
        const int o = ks * BPS + 4 * (BPS == 16 ? word ^ ((row >> 3) & 3) : word);
        const uint32_t off = (uint32_t)(row * sld + o) | (o < sld ? 0u : kOOB);
        const int dst = S::kLdsS + (is_a ? slot * S::TM * BPS : S::NS * S::TM * BPS + slot * S::TN * BPS) + nn * 256;
        lds_dma<4>(is_a ? tg.rsa : tg.rsb, lds + dst, off);
    }
}

// kScalesRows16: lane i of wave-load n of the concatenated row list (A rows,
// then B rows) fetches the 16 stage bytes of row 64 n + i.  Spare loads
// repeat earlier ones, as in dma_scales.
template <int FMT, class S>
__device__ __forceinline__ void dma_scale_rows16(uint8_t *lds, int slot, const Target &tg, int ks, const Ctx<S> &c,
                                                 int sld)
{
    static_assert(Fmt<FMT>::BPS == 16, "one 16-byte piece per row and stage");
    constexpr int NSA = S::TM / 64, NSB = S::TN / 64, NL = NSA + NSB;
#pragma unroll
    for (int k = 0; k < (NL + S::NW - 1) / S::NW; ++k) {
        const int n = (c.w + k * S::NW) % NL;      // wave-uniform
        const bool is_a = n < NSA;
        const int nn = is_a ? n : n - NSA;
        const int o = ks * 16;
        const uint32_t off = (uint32_t)((nn * 64 + c.lane) * sld + o) | (o < sld ? 0u : kOOB);
        const int dst = S::kLdsS + (is_a ? slot * S::TM * 16 : S::NS * S::TM * 16 + slot * S::TN * 16) + nn * 1024;
        lds_dma<16>(is_a ? tg.rsa : tg.rsb, lds + dst, off);
    }
}

// Chunked scales: portion u (0 .. scale_spc - 1) of chunk `chunk` (bytes
// 16 chunk .. 16 chunk + 15 of every row) into chunk buffer `par`: rows
// u R .. (u + 1) R - 1 of the concatenated row list (A rows, then B rows;
// R = (TM + TN) / scale_spc), 16 rows per dword wave-load: lane i lands on
// dword position i % 4 of row i / 4 and fetches the row's dword
// (i % 4) ^ chunk_swz(row) (see read_scales_chunk).  Dwords past a row's end
// read zero.
template <int FMT, class S>
__device__ __forceinline__ void dma_scale_portion(uint8_t *lds, int par, const Target &stg, int chunk, int u,
                                                  const Ctx<S> &c, int sld)
{
    constexpr int R = (S::TM + S::TN) / scale_spc<FMT>(), NLP = R / 16;
    static_assert(NLP % S::NW == 0 && S::TM % 32 == 0, "portions split evenly over the waves; B rows keep bit 4");
#pragma unroll
    for (int k = 0; k < NLP / S::NW; ++k) {
        const int row0 = u * R + (c.w + k * S::NW) * 16;      // wave-uniform
        const int o = chunk * kScaleChunk + 4 * ((c.lane & 3) ^ chunk_swz<FMT>(row0 + (c.lane >> 2)));
        const bool is_a = row0 < S::TM;
        const int r = (is_a ? row0 : row0 - S::TM) + (c.lane >> 2);
        const uint32_t off = (uint32_t)(r * sld + o) | (o < sld ? 0u : kOOB);
        const int dst = S::kLdsS + par * (S::TM + S::TN) * kScaleChunk + row0 * kScaleChunk;
        lds_dma<4>(is_a ? stg.rsa : stg.rsb, lds + dst, off);
    }
}

// Any other row stride: thread t fetches the BPS bytes of rows t, t + threads,
// ... of the concatenated row list (A rows then B rows) one by one (bytes
// past the row's last block read zero) and writes them to LDS before the
// stage's barrier.
template <class S>
constexpr int scale_units() { return (S::TM + S::TN + S::kThreads - 1) / S::kThreads; }

template <int FMT, class S>
struct ScaleBytes {
    static constexpr int BPS = Fmt<FMT>::BPS > 0 ? Fmt<FMT>::BPS : 1;
    uint32_t v[scale_units<S>()][BPS];
};

template <int FMT, class S>
__device__ __forceinline__ void load_scale_bytes(ScaleBytes<FMT, S> &r, const Target &tg, int ks, const Ctx<S> &c,
                                                 int sld)
{
    constexpr int BPS = Fmt<FMT>::BPS;
#pragma unroll
    for (int k = 0; k < scale_units<S>(); ++k) {
        const int u0 = c.w * 64 + k * S::kThreads;   // wave-uniform: TM, TN are multiples of 64
        if (u0 < S::TM + S::TN) {
            const bool is_a = u0 < S::TM;
            const int row = u0 + c.lane - (is_a ? 0 : S::TM);
#pragma unroll
            for (int b = 0; b < BPS; ++b) {
                const int o = ks * BPS + b;
                const uint32_t off = (uint32_t)(row * sld + o) | (o < sld ? 0u : kOOB);
                r.v[k][b] = __builtin_amdgcn_raw_buffer_load_b8(is_a ? tg.rsa : tg.rsb, off, 0, 0);
            }
        }
    }
}

template <int FMT, class S>
__device__ __forceinline__ void store_scale_bytes(const ScaleBytes<FMT, S> &r, uint8_t *lds, int slot, const Ctx<S> &c)
{
    constexpr int BPS = Fmt<FMT>::BPS;
#pragma unroll
    for (int k = 0; k < scale_units<S>(); ++k) {
        const int u0 = c.w * 64 + k * S::kThreads;   // wave-uniform: TM, TN are multiples of 64
        if (u0 < S::TM + S::TN) {
            const bool is_a = u0 < S::TM;
            const int row = u0 + c.lane - (is_a ? 0 : S::TM);
            uint8_t *dst = lds + S::kLdsS + (is_a ? slot * S::TM * BPS : S::NS * S::TM * BPS + slot * S::TN * BPS) +
                           row * BPS;
#pragma unroll
            for (int b = 0; b < BPS; ++b) dst[b] = (uint8_t)r.v[k][b];
        }
    }
}

// ------------------------------------------------------------------- math

// One 32x32 block for one k-step.  The MFMA's first operand is the B
// fragment, so each lane ends up holding 4 consecutive output columns.
// MX: the scale operands are the blocks' stage scale dwords, of which op_sel
// SEL picks the byte of this k-step.
// For 8-bit MX elements CA and CB are the format codes of A and B (the
// instruction's second and first operand).
__device__ __forceinline__ i32x8 widen_frag(const i32x8 &v) { return v; }
__device__ __forceinline__ i32x8 widen_frag(const i32x4 &v) { return i32x8{v[0], v[1], v[2], v[3], 0, 0, 0, 0}; }

template <int FMT, int SEL, int CA = 0, int CB = 0, class FA, class FB>
__device__ __forceinline__ void mma1(f32x16 &acc, const FA &a, uint32_t sa, const FB &b, uint32_t sb)
{
    if constexpr (FMT == kBF16) {
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, acc, 0, 0, 0);
    } else if constexpr (FMT == kNVFP4) {
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(b, a, acc, 0, 0, 0);
    } else if constexpr (FMT == kMXFP8) {
        // (an E2M1 operand, code 4, takes the low four dwords)
        acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(widen_frag(b), widen_frag(a), acc, CB, CA, SEL, (int)sb,
                                                              SEL, (int)sa);
    } else {
        const i32x8 bb = {b[0], b[1], b[2], b[3], 0, 0, 0, 0};
        const i32x8 aa = {a[0], a[1], a[2], a[3], 0, 0, 0, 0};
        acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bb, aa, acc, 4, 4, SEL, (int)sb, SEL, (int)sa);
    }
}

// ------------------------------------------------------ direct-to-LDS loads

// Wave-load L of an operand of the target stage into ring slot `slot`.  It
// writes 64 lanes x 16 bytes to consecutive LDS bytes, i.e. rows 8L .. 8L+7
// x 8 chunks, so lane i lands on row 8L + i/8, physical chunk i%8, and
// fetches the logical chunk the swizzle places there:
// (i%8) ^ swz(8L + i/8) = (i%8) ^ (i/8) ^ (L%8).  Chunks past the row end (a
// partial last stage) read zeros.
template <class S>
__device__ __forceinline__ void dma_op(uint8_t *lds, int dst, __amdgpu_buffer_rsrc_t rsrc, int ks, const Ctx<S> &c,
                                       int L, int lda, uint32_t r8)
{
    const int k0 = ks * kRowBytes;
    const uint32_t kc = c.x4 ^ (uint32_t)((L & 7) << 4);
    const uint32_t off = (r8 + kc + (uint32_t)(L * 8 * lda + k0)) | (kc < (uint32_t)(lda - k0) ? 0u : kOOB);
    lds_dma<16>(rsrc, lds + dst + L * 1024, off);
}

// Wave-load L of an MN-major operand (T columns per tile) of stage ks into
// slot bytes dst + 1024 L ..: K-rows ks KS + L RPL + .. of the operand,
// whose rows are ldx bytes apart; `lo` holds the lane's offsets for even
// and odd L (see mn_dma_lane).  K-rows past K lie past the end of the
// resource (it ends with the operand) and read zero; columns past M or N
// read the start of the next K-row, which only reaches outputs that are
// never stored.
template <int FMT, int T>
__device__ __forceinline__ void dma_mn(uint8_t *lds, int dst, __amdgpu_buffer_rsrc_t rsrc, int ks,
                                       const uint32_t (&lo)[2], int L, int q, int ldx)
{
    using G = Mn<FMT, T>;
    // with 2 RPL = PERIOD the parity of L = w Q + q is that of q (Q even)
    const int par = G::RPL % G::PERIOD == 0 ? 0 : (q & 1);
    const uint32_t row = (uint32_t)(ks * G::KS + L * G::RPL) * (uint32_t)ldx;   // wave-uniform
    lds_dma<16>(rsrc, lds + dst + L * 1024, lo[par] + row);
}

// Wave w issues wave-loads w*Q + q, q < Q, of each operand.
template <class S>
__device__ __forceinline__ void dma_a(uint8_t *lds, int slot, const Target &tg, int ks, const Ctx<S> &c, int q,
                                      int lda)
{
    dma_op(lds, S::kLdsA + slot * S::kSlotA, tg.ra, ks, c, c.w * S::QA + q, lda, c.r8lda);
}

template <class S>
__device__ __forceinline__ void dma_b(uint8_t *lds, int slot, const Target &tg, int ks, const Ctx<S> &c, int q,
                                      int lda)
{
    dma_op(lds, S::kLdsB + slot * S::kSlotB, tg.rb, ks, c, c.w * S::QB + q, lda, c.r8lda);
}

// Packed E2M1 operand of an 8-bit kernel (rows of ldc = K / 2 bytes): wave
// w issues wave-loads w 2Q + half Q + q, q < Q, of 256-K stage fp.ks into
// slot fp.ls of the operand's ring, Q = QA / 2 (A) or QB / 2 (B).
template <class S, bool IS_A>
constexpr int f4_q() { return (IS_A ? S::QA : S::QB) / 2; }

template <class S, bool IS_A>
__device__ __forceinline__ void dma_f4(uint8_t *lds, int slot, __amdgpu_buffer_rsrc_t r, int ks, int half,
                                       const Ctx<S> &c, int q, int ldc, int ldm)
{
    constexpr int Q = f4_q<S, IS_A>();
    static_assert(2 * Q == (IS_A ? S::QA : S::QB), "a 256-K stage splits into two halves");
    const int dst = IS_A ? S::kLdsA + slot * S::kSlotA : S::kLdsB + slot * S::kSlotB;
    const int L = c.w * 2 * Q + half * Q + q;
    if constexpr (IS_A ? S::AMN : S::BMN) {
        // MN-major (K-rows of ldm bytes): the parity of L is that of half Q + q
        constexpr int T = IS_A ? S::TM : S::TN;
        dma_mn<kMXFP4, T>(lds, dst, r, ks, IS_A ? c.ma : c.mb, L, half * Q + q, ldm);
    } else {
        dma_op(lds, dst, r, ks, c, L, ldc, (uint32_t)((c.lane >> 3) * ldc));
    }
}

// ---------------------------------------------------------- NVFP4 staging

// A stage covers 64 K elements = 32 packed bytes per row, i.e. two halves of
// 16 bytes (32 elements) with two E4M3 scales each.  The concatenated list
// of half-rows (A then B) is split over the threads: thread t takes units
// t, t + threads, ...; each unit expands to 64 bytes of fp16 (4 LDS chunks).
// With A decoded in registers (adirect) the list holds the B half-rows only.
template <class S, bool AD>
constexpr int fp4_rows() { return AD ? S::TN : S::TM + S::TN; }

template <class S, bool AD>
constexpr int fp4_units() { return (2 * fp4_rows<S, AD>() + S::kThreads - 1) / S::kThreads; }

template <class S, bool AD>
struct Fp4Regs {
    i32x4 v[fp4_units<S, AD>()];
    uint32_t s[fp4_units<S, AD>()];
};

// Packed bytes ks*32 + hoff .. +15 of a row (hoff = 16 * half) and its two
// scale bytes ks*4 + hoff/8 .. +1.  kNvWhole: each half is all in or all out
// (the two halves of a last stage can differ).  kNvHalf: the two 8-byte
// pieces of the half (and their scales) are in or out separately.  The
// out-of-range flag rides in the vector offset; the scalar offset carries
// only the in-range stage offset.
template <int SM>
__device__ __forceinline__ void load_fp4_half(i32x4 &v, uint32_t &sc, __amdgpu_buffer_rsrc_t rs,
                                              __amdgpu_buffer_rsrc_t rss, int row, int hoff, int ks, int lda, int sld)
{
    const int hb = ks * 32 + hoff;                     // the half's first byte in the row
    const uint32_t pad = hb < lda ? 0u : kOOB;
    if constexpr (SM == kNvHalf) {
        const uint32_t pad1 = hb + 8 < lda ? 0u : kOOB;
        const u32x2 lo = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(
                                                       rs, (uint32_t)(row * lda + hoff) | pad, (uint32_t)(ks * 32), 0));
        const u32x2 hi = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(
                                                       rs, (uint32_t)(row * lda + hoff + 8) | pad1, (uint32_t)(ks * 32), 0));
        v = i32x4{(int)lo[0], (int)lo[1], (int)hi[0], (int)hi[1]};
        const uint32_t s0 = __builtin_amdgcn_raw_buffer_load_b8(rss, (uint32_t)(row * sld + hoff / 8) | pad,
                                                                 (uint32_t)(ks * 4), 0);
        const uint32_t s1 = __builtin_amdgcn_raw_buffer_load_b8(rss, (uint32_t)(row * sld + hoff / 8 + 1) | pad1,
                                                                 (uint32_t)(ks * 4), 0);
        sc = s0 | (s1 << 8);
    } else {
        v = __builtin_amdgcn_raw_buffer_load_b128(rs, (uint32_t)(row * lda + hoff) | pad, (uint32_t)(ks * 32), 0);
        sc = __builtin_amdgcn_raw_buffer_load_b16(rss, (uint32_t)(row * sld + hoff / 8) | pad, (uint32_t)(ks * 4), 0);
    }
}

template <int SM, class S, bool AD>
__device__ __forceinline__ void load_fp4(Fp4Regs<S, AD> &r, const Target &tg, int ks, const Ctx<S> &c, int lda,
                                         int sld)
{
    constexpr int TA = AD ? 0 : S::TM;   // A rows in the list
#pragma unroll
    for (int k = 0; k < fp4_units<S, AD>(); ++k) {
        const int u0 = c.w * 64 + k * S::kThreads;   // wave-uniform
        if (u0 < 2 * fp4_rows<S, AD>()) {
            const bool is_a = u0 < 2 * TA;
            const int hr = u0 + c.lane - (is_a ? 0 : 2 * TA);
            const int row = hr >> 1, half = hr & 1;
            load_fp4_half<SM>(r.v[k], r.s[k], is_a ? tg.ra : tg.rb, is_a ? tg.rsa : tg.rsb, row, half * 16, ks, lda,
                              sld);
        }
    }
}

// E4M3 scale byte -> fp16 (exact: E4M3 values lie inside fp16's normal range).
__device__ __forceinline__ f16x2 e4m3_pair(uint32_t byte)
{
    const _Float16 v = (_Float16)__builtin_amdgcn_cvt_f32_fp8((int)byte, 0);
    return f16x2{v, v};
}

// The two E4M3 bytes in bits 0..15 -> two fp16 (exact, unit scale).
__device__ __forceinline__ f16x2 e4m3_two(uint32_t bytes)
{
    return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(bytes, 1.0f, false);
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

template <class S, bool AD>
__device__ __forceinline__ void store_fp4(const Fp4Regs<S, AD> &r, uint8_t *lds, int slot, const Ctx<S> &c)
{
    constexpr int TA = AD ? 0 : S::TM;
#pragma unroll
    for (int k = 0; k < fp4_units<S, AD>(); ++k) {
        const int u0 = c.w * 64 + k * S::kThreads;   // wave-uniform
        if (u0 < 2 * fp4_rows<S, AD>()) {
            const bool is_a = u0 < 2 * TA;
            const int hr = u0 + c.lane - (is_a ? 0 : 2 * TA);
            const int row = hr >> 1, half = hr & 1;
            uint8_t *base = lds + (is_a ? S::kLdsA + slot * S::kSlotA : S::kLdsB + slot * S::kSlotB);
            const f16x2 lo = e4m3_pair(r.s[k] & 0xFF), hi = e4m3_pair((r.s[k] >> 8) & 0xFF);
#pragma unroll
            for (int d = 0; d < 4; ++d)
                *reinterpret_cast<i32x4 *>(base + lds_off(row, half * 4 + d)) =
                    expand8((uint32_t)r.v[k][d], d < 2 ? lo : hi);
        }
    }
}

// A rows decoded in registers: the lane loads the 16 packed bytes (32
// elements) of half h of its row in each of the wave's row blocks, with their
// two E4M3 scales, and decodes dword kk into the fragment of k-step kk.
template <class S>
struct Fp4A {
    i32x4 v[S::MB];
    uint32_t s[S::MB];
};

template <int SM, class S>
__device__ __forceinline__ void load_fp4_a(Fp4A<S> &r, const Target &tg, int ks, const Ctx<S> &c, int lda, int sld)
{
#pragma unroll
    for (int i = 0; i < S::MB; ++i) {
        const int row = c.wm * (S::TM / S::WM) + i * 32 + c.lr;
        load_fp4_half<SM>(r.v[i], r.s[i], tg.ra, tg.rsa, row, c.h * 16, ks, lda, sld);
    }
}

template <class S>
__device__ __forceinline__ void decode_fp4_a(f16x8 (&a)[S::MB][4], const Fp4A<S> &r)
{
#pragma unroll
    for (int i = 0; i < S::MB; ++i) {
        const f16x2 lo = e4m3_pair(r.s[i] & 0xFF), hi = e4m3_pair((r.s[i] >> 8) & 0xFF);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            a[i][kk] = __builtin_bit_cast(f16x8, expand8((uint32_t)r.v[i][kk], kk < 2 ? lo : hi));
    }
}

// ------------------------------------------- E2M1 operands of 8-bit GEMMs

// An E2M1 or FP6 operand paired with an E4M3 / E5M2 one (or FP6 with FP6): a
// 128-element stage row is four pieces of 32 elements (one E8M0 block each):
// 16 packed bytes (E2M1) or 24 (FP6, four elements per three bytes).  The
// concatenated piece list (the widened operands' rows, A's first) is split
// over the threads, thread t taking pieces t, t + threads, ...  Each piece is
// loaded into registers and written to LDS as the 32 codes of the same
// values in the 8-bit format that holds them all exactly (E2M1 and E2M3 in
// E4M3, E3M2 in E5M2), so the MX scales stay as they are -- into logical
// chunks 2p and 2p + 1 of its row of the 8-bit slot.
template <class S>
constexpr int cv_rows() { return (S::ACV ? S::TM : 0) + (S::BCV ? S::TN : 0); }

template <class S>
constexpr int cv_units() { return (4 * cv_rows<S>() + S::kThreads - 1) / S::kThreads; }

// first unit of phase group g of a stage with KK phases
template <class S, int KK>
constexpr int cv_group(int g) { return g >= KK ? cv_units<S>() : g * ((cv_units<S>() + KK - 1) / KK) < cv_units<S>() ? g * ((cv_units<S>() + KK - 1) / KK) : cv_units<S>(); }

// dwords per piece: 4 (E2M1) or 6 (FP6); both widened operands of an FP6 x
// FP6 kernel have FP6 pieces
template <class S>
constexpr int cv_words() { return (S::ASRC >= 2 || S::BSRC >= 2) ? 6 : 4; }

// The 8-wave 256 x 64 tile has the registers for all of a stage's pieces at
// once: loaded at the stage's start, written to LDS at its end.
template <class S>
constexpr bool cv_early() { return S::NW == 8 && S::TN == 64; }

template <class S>
struct CvRegs {
    uint32_t v[cv_units<S>() > 0 ? cv_units<S>() : 1][cv_words<S>()];
};

// Units K0 .. K1-1 of the thread's pieces (a stage's pieces go in groups, one
// per k-step phase: loaded at the start of a phase, written to LDS at the
// start of the next, so only a group's registers are live at a time).
template <class S, int K0, int K1>
__device__ __forceinline__ void load_cv(CvRegs<S> &r, const Target &tg, int ks, const Ctx<S> &c, int ldc)
{
    constexpr int TA = S::ACV ? S::TM : 0;   // A rows in the list
    constexpr int W = cv_words<S>(), PB = 4 * W;  // dwords and bytes per piece
#pragma unroll
    for (int k = K0; k < K1; ++k) {
        const int u0 = c.w * 64 + k * S::kThreads;   // wave-uniform: 4 TM is a multiple of 64
        if (u0 < 4 * cv_rows<S>()) {
            const bool is_a = u0 < 4 * TA;
            const int pu = u0 + c.lane - (is_a ? 0 : 4 * TA);
            const int row = pu >> 2, piece = pu & 3;
            // rows are K PB / 32 bytes, K % 32 == 0: a piece is all in or all out
            const uint32_t pad = ks * 4 * PB + piece * PB < ldc ? 0u : kOOB;
            const uint32_t off = (uint32_t)(row * ldc + piece * PB) | pad;
            const __amdgpu_buffer_rsrc_t rs = is_a ? tg.ra : tg.rb;
            if constexpr (W == 4) {
                const i32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, off, (uint32_t)(ks * 4 * PB), 0);
#pragma unroll
                for (int q = 0; q < 4; ++q) r.v[k][q] = (uint32_t)v[q];
            } else {
                // three 8-byte loads (pieces start on 8-byte boundaries)
#pragma unroll
                for (int q = 0; q < 3; ++q) {
                    const u32x2 v = __builtin_bit_cast(
                        u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, off + 8u * q, (uint32_t)(ks * 4 * PB), 0));
                    r.v[k][2 * q] = v[0];
                    r.v[k][2 * q + 1] = v[1];
                }
            }
        }
    }
}

// 8 E2M1 codes (one dword, low nibble first) -> their 8 E4M3 codes: exact
// decode, then the hardware's E4M3 encoding of an E4M3 value (no rounding).
__device__ __forceinline__ u32x2 widen8(uint32_t w)
{
    typedef __attribute__((ext_vector_type(2))) float f32x2;
    const f32x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
    const f32x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
    const f32x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
    const f32x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
    int lo = __builtin_amdgcn_cvt_pk_fp8_f32(p0[0], p0[1], 0, false);
    lo = __builtin_amdgcn_cvt_pk_fp8_f32(p1[0], p1[1], lo, true);
    int hi = __builtin_amdgcn_cvt_pk_fp8_f32(p2[0], p2[1], 0, false);
    hi = __builtin_amdgcn_cvt_pk_fp8_f32(p3[0], p3[1], hi, true);
    return u32x2{(uint32_t)lo, (uint32_t)hi};
}

// 32 FP6 codes (six dwords, element j at bits 6j..) -> their 32 codes in
// E4M3 (SRC 2: E2M3) or E5M2 (SRC 3: E3M2): the hardware's exact decode to
// fp16, then its 8-bit encoding of values the 8-bit format holds exactly.
template <int SRC>
__device__ __forceinline__ void widen32_fp6(const uint32_t (&w)[6], uint32_t (&out)[8])
{
    typedef __attribute__((ext_vector_type(6))) unsigned int u32x6;
    typedef __attribute__((ext_vector_type(32))) _Float16 f16x32;
    typedef __attribute__((ext_vector_type(2))) short i16x2;
    const u32x6 src = {w[0], w[1], w[2], w[3], w[4], w[5]};
    f16x32 h;
    if constexpr (SRC == 2)
        h = __builtin_amdgcn_cvt_scalef32_pk32_f16_fp6(src, 1.0f);
    else
        h = __builtin_amdgcn_cvt_scalef32_pk32_f16_bf6(src, 1.0f);
#pragma unroll
    for (int d = 0; d < 8; ++d) {
        i16x2 r = {0, 0};
        if constexpr (SRC == 2) {
            r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(r, f16x2{h[4 * d], h[4 * d + 1]}, 1.0f, false);
            r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(r, f16x2{h[4 * d + 2], h[4 * d + 3]}, 1.0f, true);
        } else {
            r = __builtin_amdgcn_cvt_scalef32_pk_bf8_f16(r, f16x2{h[4 * d], h[4 * d + 1]}, 1.0f, false);
            r = __builtin_amdgcn_cvt_scalef32_pk_bf8_f16(r, f16x2{h[4 * d + 2], h[4 * d + 3]}, 1.0f, true);
        }
        out[d] = __builtin_bit_cast(uint32_t, r);
    }
}

template <class S, int K0, int K1>
__device__ __forceinline__ void store_cv(const CvRegs<S> &r, uint8_t *lds, int slot, const Ctx<S> &c)
{
    constexpr int TA = S::ACV ? S::TM : 0;
#pragma unroll
    for (int k = K0; k < K1; ++k) {
        const int u0 = c.w * 64 + k * S::kThreads;   // wave-uniform
        if (u0 < 4 * cv_rows<S>()) {
            const bool is_a = u0 < 4 * TA;
            const int pu = u0 + c.lane - (is_a ? 0 : 4 * TA);
            const int row = pu >> 2, piece = pu & 3;
            uint8_t *base = lds + (is_a ? S::kLdsA + slot * S::kSlotA : S::kLdsB + slot * S::kSlotB);
            uint32_t e[8];
            if constexpr (cv_words<S>() == 4) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const u32x2 t = widen8(r.v[k][q]);
                    e[2 * q] = t[0];
                    e[2 * q + 1] = t[1];
                }
            } else if constexpr (S::ASRC == S::BSRC || !S::ACV || !S::BCV) {
                widen32_fp6<S::ACV ? S::ASRC : S::BSRC>(r.v[k], e);
            } else {
                // E2M3 on one side, E3M2 on the other (wave-uniform choice)
                if (is_a) widen32_fp6<S::ASRC>(r.v[k], e);
                else widen32_fp6<S::BSRC>(r.v[k], e);
            }
            *reinterpret_cast<i32x4 *>(base + lds_off(row, 2 * piece)) =
                i32x4{(int)e[0], (int)e[1], (int)e[2], (int)e[3]};
            *reinterpret_cast<i32x4 *>(base + lds_off(row, 2 * piece + 1)) =
                i32x4{(int)e[4], (int)e[5], (int)e[6], (int)e[7]};
        }
    }
}

// --------------------------------------------------------------- epilogue

// acc[i][j] holds, for output row m = wm*TM/WM + 32 i + lane%32, the columns
// n = wn*TN/WN + 32 j + 8 g + 4 (lane/32) + q in register 4 g + q.  Each
// 32-row block is stored through its own buffer resource, so rows past M
// and columns past N are dropped by the hardware range check.
__device__ __forceinline__ uint32_t pack_bf16(float x, float y)
{
    typedef __attribute__((ext_vector_type(2))) float f32x2;
    typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x, y}, bf16x2));
}

template <class S>
__device__ __forceinline__ void store_tile(const f32x16 (&acc)[S::MB][S::NB], const Params &p, const TileRef &tr,
                                           const Ctx<S> &c)
{
    const int m0 = tr.m0, n0 = tr.n0;
    const float alpha = tr.alpha;
#pragma unroll
    for (int i = 0; i < S::MB; ++i) {
        const int r0 = m0 + c.wm * (S::TM / S::WM) + i * 32;
        const uint32_t bytes = __builtin_amdgcn_readfirstlane((uint32_t)max(0, min(32, tr.mend - r0)) * (uint32_t)p.N * 2u);
        const __amdgpu_buffer_rsrc_t rd = make_rsrc(p.D + (int64_t)r0 * p.N, bytes);
#pragma unroll
        for (int j = 0; j < S::NB; ++j) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int n = n0 + c.wn * (S::TN / S::WN) + j * 32 + g * 8 + c.h * 4;
                const f32x16 &a = acc[i][j];
                const uint32_t lo = pack_bf16(a[4 * g] * alpha, a[4 * g + 1] * alpha);
                const uint32_t hi = pack_bf16(a[4 * g + 2] * alpha, a[4 * g + 3] * alpha);
                const uint32_t base = (uint32_t)(c.lr * p.N + n) * 2u;
                if (p.vec_store) {
                    // N % 4 == 0 and n % 4 == 0: the 4 columns are all in or all out
                    __builtin_amdgcn_raw_buffer_store_b64(u32x2{lo, hi}, rd, n < p.N ? base : kOOB, 0, kStoreNT);
                } else {
                    const uint16_t v[4] = {(uint16_t)lo, (uint16_t)(lo >> 16), (uint16_t)hi, (uint16_t)(hi >> 16)};
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        __builtin_amdgcn_raw_buffer_store_b16(v[q], rd, n + q < p.N ? base + 2 * q : kOOB, 0, kStoreNT);
                }
            }
        }
    }
}

// Epilogue through LDS (when N % 8 == 0 and D is 16-byte aligned): each wave
// writes one 32-row block-row of its bf16 results into its own 32 x (NB*64)
// byte buffer in the just-consumed ring slot `xslot` (its A part, or A and B
// parts for half of the waves each when the A part is too small; 16-byte
// chunks XOR-swizzled by row), reads it back row-major (CPR lanes per row)
// and stores whole 16-byte chunks, so one store instruction covers 64/CPR
// full rows of the wave's columns instead of 32 rows x 16 bytes.  The same
// wave's LDS writes and reads execute in order; the caller meets a barrier
// before the slot is refilled.
// The wave's staging buffer holds 32 rows of NB * 64 bytes.
template <class S>
constexpr int epilogue_wave_bytes() { return 32 * S::NB * 64; }

template <class S>
__device__ __forceinline__ void store_tile_lds_at(const f32x16 (&acc)[S::MB][S::NB], uint8_t *buf, const Params &p,
                                                  const TileRef &tr, const Ctx<S> &c)
{
    const int m0 = tr.m0, n0 = tr.n0;
    const float alpha = tr.alpha;
    constexpr int RB = S::NB * 64;          // bytes per staged row
    constexpr int CPR = RB / 16;            // 16-byte chunks per staged row
    constexpr int RPI = 64 / CPR;           // rows per read instruction
    const int nc = n0 + c.wn * (S::TN / S::WN);
#pragma unroll
    for (int i = 0; i < S::MB; ++i) {
#pragma unroll
        for (int j = 0; j < S::NB; ++j) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const f32x16 &a = acc[i][j];
                const uint32_t lo = pack_bf16(a[4 * g] * alpha, a[4 * g + 1] * alpha);
                const uint32_t hi = pack_bf16(a[4 * g + 2] * alpha, a[4 * g + 3] * alpha);
                const int ch = (4 * j + g) ^ (c.lr & (CPR - 1));
                *reinterpret_cast<u32x2 *>(buf + c.lr * RB + 16 * ch + 8 * c.h) = u32x2{lo, hi};
            }
        }
        const int r0 = m0 + c.wm * (S::TM / S::WM) + i * 32;
        const uint32_t bytes = __builtin_amdgcn_readfirstlane((uint32_t)max(0, min(32, tr.mend - r0)) * (uint32_t)p.N * 2u);
        const __amdgpu_buffer_rsrc_t rd = make_rsrc(p.D + (int64_t)r0 * p.N, bytes);
#pragma unroll
        for (int q = 0; q < 32 / RPI; ++q) {
            const int r = q * RPI + c.lane / CPR, ch = c.lane % CPR;
            const i32x4 v = *reinterpret_cast<const i32x4 *>(buf + r * RB + 16 * (ch ^ (r & (CPR - 1))));
            const int n = nc + ch * 8;
            // N % 8 == 0 and n % 8 == 0: the 8 columns are all in or all out
            __builtin_amdgcn_raw_buffer_store_b128(v, rd, n < p.N ? (uint32_t)(r * p.N + n) * 2u : kOOB, 0, kStoreNT);
        }
    }
}

template <class S>
__device__ __forceinline__ void store_tile_lds(const f32x16 (&acc)[S::MB][S::NB], uint8_t *lds, int xslot,
                                               const Params &p, const TileRef &tr, const Ctx<S> &c)
{
    constexpr int WB = epilogue_wave_bytes<S>();
    constexpr bool SPLIT = S::NW * WB > S::kSlotA;
    static_assert(!SPLIT || (S::NW / 2 * WB <= S::kSlotA && S::NW / 2 * WB <= S::kSlotB),
                  "epilogue buffers must fit in one ring slot");
    uint8_t *buf = !SPLIT           ? lds + S::kLdsA + xslot * S::kSlotA + c.w * WB
                   : c.w < S::NW / 2 ? lds + S::kLdsA + xslot * S::kSlotA + c.w * WB
                                     : lds + S::kLdsB + xslot * S::kSlotB + (c.w - S::NW / 2) * WB;
    store_tile_lds_at<S>(acc, buf, p, tr, c);
}

// ------------------------------------------------------------------ kernel

// End of a stage: this wave's LDS reads and writes are done and all but its
// newest `newer` memory operations have completed; then all waves meet.
// Memory operations complete in order, so with the loads of the last NS-2
// stages left in flight the next stage's slot (loaded NS-2 stages before
// them) has landed for every wave: after the barrier it may be read, and the
// slot just read may be refilled.
template <int NEWER>
__device__ __forceinline__ void stage_barrier()
{
    DBS_FENCE();
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"i"(NEWER) : "memory");
    DBS_FENCE();
}

// Loads each wave issues per stage on the direct-to-LDS path (operand
// wave-loads plus an equal share of the MX scale wave-loads); only that path
// uses rings deeper than two slots.
template <int FMT, class S, int SM>
constexpr int stage_loads_min()
{
    constexpr int NSC = Fmt<FMT>::BPS == 0 ? 0
                        : SM == kScalesRows16 ? (S::TM + S::TN) / 64
                                              : (S::TM + S::TN) * Fmt<FMT>::BPS / 256;
    return S::QA + S::QB + (NSC + S::NW - 1) / S::NW;
}

// Raw NVFP4: the fp16 fragments of one element group (one MFMA k-step) of
// the k-step whose MFMAs come next, decoded while the current ones issue.
template <class S>
struct NvDec {
    f16x8 a[S::MB], b[S::NB];
};

// State threaded through the stage function.
template <int FMT, class S>
struct Pipe {
    Frags<FMT, S> F0, F1;                    // k-step fragments, double-buffered
    NvDec<S> dec;                            // raw NVFP4: the next element group, decoded
    Scales<S> sprev, scur;                   // MX scales of the previous and of this stage
    Fp4Regs<S, adirect<FMT, S>()> fp4;
    Fp4A<S> fp4a;                            // adirect: the wave's packed A rows of the next stage
    f16x8 acur[S::MB][4];                    // adirect: this stage's A fragments per k-step
    f16x8 aprev[S::MB];                      // adirect: the previous stage's last k-step
    ScaleBytes<FMT, S> sbytes;
    CvRegs<S> cv;                            // widened E2M1 operands: the next stage's packed pieces
};

// Load pieces of a stage.  Direct-to-LDS formats: piece q issues wave-load q
// of A (q < QA) and of B (q < QB); the MX scale loads go with the last piece.
// NVFP4: one piece with all of the thread's register-staged loads.
template <int FMT, class S>
constexpr int npieces() { return FMT == kNVFP4 ? 1 : (S::QA > S::QB ? S::QA : S::QB); }

// Where a stage stands in the chunked-scale sequence: it reads stage j of
// the chunk in buffer pc and loads portion j of chunk `lchunk` of the tile
// whose scale rows start at stg (the next chunk) into buffer pc ^ 1.
struct ChunkPos {
    int pc, j, lchunk;
};

template <int FMT, class S, int SM>
__device__ __forceinline__ void load_piece(Pipe<FMT, S> &P, uint8_t *lds, int slot, const Target &tg, int ks,
                                           const Params &p, const Ctx<S> &c, int q, const Target &stg,
                                           const ChunkPos &cp, const F4Pos &fp)
{
    if constexpr (FMT == kNVFP4) {
        load_fp4<SM>(P.fp4, tg, ks, c, p.lda, p.sld);
        if constexpr (adirect<FMT, S>()) load_fp4_a<SM>(P.fp4a, tg, ks, c, p.lda, p.sld);
    } else {
        if constexpr (S::AF4) {
            if (q < f4_q<S, true>()) dma_f4<S, true>(lds, fp.ls, fp.r, fp.ks, fp.half, c, q, p.ldc, p.ldam);
        } else if (q < S::QA && !S::ACV) {
            if constexpr (S::AMN) {
                static_assert(Mn<FMT, S::TM>::RPL % Mn<FMT, S::TM>::PERIOD == 0 || S::QA % 2 == 0, "parity");
                dma_mn<FMT, S::TM>(lds, S::kLdsA + slot * S::kSlotA, tg.ra, ks, c.ma, c.w * S::QA + q, q, p.ldam);
            } else {
                dma_a(lds, slot, tg, ks, c, q, p.lda);
            }
        }
        if constexpr (S::BF4) {
            if (q < f4_q<S, false>()) dma_f4<S, false>(lds, fp.ls, fp.r, fp.ks, fp.half, c, q, p.ldc, p.ldbm);
        } else if (q < S::QB && !S::BCV) {
            if constexpr (S::BMN) {
                static_assert(Mn<FMT, S::TN>::RPL % Mn<FMT, S::TN>::PERIOD == 0 || S::QB % 2 == 0, "parity");
                dma_mn<FMT, S::TN>(lds, S::kLdsB + slot * S::kSlotB, tg.rb, ks, c.mb, c.w * S::QB + q, q, p.ldbm);
            } else {
                dma_b(lds, slot, tg, ks, c, q, p.lda);
            }
        }
        if constexpr (FMT == kMXFP8 || FMT == kMXFP4 || FMT == kNVFP4R) {
            if (q == npieces<FMT, S>() - 1) {
                if constexpr (SM == kScalesStage)
                    dma_scales<FMT>(lds, slot, tg, ks, c, p.sld);
                else if constexpr (SM == kScalesRows16)
                    dma_scale_rows16<FMT>(lds, slot, tg, ks, c, p.sld);
                else if constexpr (SM == kScalesChunk)
                    dma_scale_portion<FMT>(lds, cp.pc ^ 1, stg, cp.lchunk, cp.j, c, p.sld);
                else
                    load_scale_bytes(P.sbytes, tg, ks, c, p.sld);
            }
        }
    }
}

// Register-staged parts of a stage (NVFP4 data, unaligned MX scales) go to
// LDS before the stage's barrier.
template <int FMT, class S, int SM, bool ALL = false>
__device__ __forceinline__ void commit_stage(Pipe<FMT, S> &P, uint8_t *lds, int slot, const Ctx<S> &c)
{
    if constexpr (FMT == kNVFP4) store_fp4(P.fp4, lds, slot, c);
    if constexpr (adirect<FMT, S>()) {
        // the stage ending now keeps its last k-step for the next stage's
        // first phase; the loaded stage becomes the current one
#pragma unroll
        for (int i = 0; i < S::MB; ++i) P.aprev[i] = P.acur[i][3];
        decode_fp4_a<S>(P.acur, P.fp4a);
    }
    if constexpr ((FMT == kMXFP8 || FMT == kMXFP4 || FMT == kNVFP4R) && SM == kScalesRegs)
        store_scale_bytes(P.sbytes, lds, slot, c);
    if constexpr (S::ACV || S::BCV) {
        // the last phase group (ALL: every group, loaded together in the prologue)
        constexpr int KK = kk_of<FMT, S>();
        store_cv<S, (ALL || cv_early<S>()) ? 0 : cv_group<S, KK>(KK - 1), cv_units<S>()>(P.cv, lds, slot, c);
    }
}

// Raw NVFP4 k-step: fragment element groups d = 0..3 (K 32h + 8d .. +7 for
// lane half h) are decoded exactly into fp16 with their block's E4M3 scale
// (groups 0, 1: the first 16-element block, 2, 3: the second) and each group
// feeds one v_mfma_f32_32x32x16_f16.  A and B fragments are decoded alike, so
// the MFMAs see the same permutation of K on both sides.
template <class S>
__device__ __forceinline__ void nv_decode(NvDec<S> &o, const Frags<kNVFP4R, S> &f, int d)
{
#pragma unroll
    for (int i = 0; i < S::MB; ++i) {
        const f16x2 s2 = e4m3_two(f.sa[i]);
        o.a[i] = __builtin_bit_cast(f16x8, expand8((uint32_t)f.a[i][d], d < 2 ? f16x2{s2[0], s2[0]}
                                                                              : f16x2{s2[1], s2[1]}));
    }
#pragma unroll
    for (int j = 0; j < S::NB; ++j) {
        const f16x2 s2 = e4m3_two(f.sb[j]);
        o.b[j] = __builtin_bit_cast(f16x8, expand8((uint32_t)f.b[j][d], d < 2 ? f16x2{s2[0], s2[0]}
                                                                              : f16x2{s2[1], s2[1]}));
    }
}

// The MFMAs of k-step `cur`, software-pipelined over its element groups: dec
// holds group 0, already decoded; the MFMAs of group d issue while group d + 1
// is decoded (the VALU work then runs beside the matrix core instead of ahead
// of it), and during the last group's MFMAs group 0 of the next k-step (`nxt`,
// read from LDS in this phase) is decoded into dec (NEXT; the tile's last
// phase has no next k-step).  The 8-wave square tiles (8 MFMAs a group)
// alternate one MFMA with six VALU instructions; the other shapes keep the
// compiler's order (measured better on the skinny tiles).
template <class S, bool NEXT>
__device__ __forceinline__ void nv_raw_mma(f32x16 (&acc)[S::MB][S::NB], NvDec<S> &dec,
                                           const Frags<kNVFP4R, S> &cur, const Frags<kNVFP4R, S> &nxt)
{
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        NvDec<S> nd;
        if (d < 3) nv_decode<S>(nd, cur, d + 1);
        else if constexpr (NEXT) nv_decode<S>(nd, nxt, 0);
#pragma unroll
        for (int i = 0; i < S::MB; ++i)
#pragma unroll
            for (int j = 0; j < S::NB; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(dec.b[j], dec.a[i], acc[i][j], 0, 0, 0);
        if (d < 3 || NEXT) dec = nd;
    }
    if constexpr (S::NW == 8 && S::MB * S::NB >= 8) {
#pragma unroll
        for (int q = 0; q < 4 * S::MB * S::NB; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);   // six VALU
        }
    }
}

// Phase PH of a stage (PH = 0 .. KK-1): the MB x NB MFMAs of one k-step —
// the previous stage's last k-step (set F1) for PH = 0, k-step PH-1 of this
// stage (set (PH-1) & 1) otherwise — while k-step PH of slot `rslot` is read
// into the other set (if RD).  With LOADS, the stage's load pieces are issued
// between MFMAs: piece q after MFMA number q of the stage.  Rolling formats
// keep A in F0 only: each A fragment is re-read right after its last MFMA.
template <int FMT, class S, int SM, int PH, bool RD, bool LOADS>
__device__ __forceinline__ void phase(f32x16 (&acc)[S::MB][S::NB], Pipe<FMT, S> &P, uint8_t *lds, const Params &p,
                                      const Ctx<S> &c, int rslot, const Target &tg, int ks, int lslot,
                                      const Target &stg, const ChunkPos &cp, const F4Pos &fp)
{
    auto rda = [&](Frags<FMT, S> &f, int i) {
        if constexpr (S::AF4) read_a_f4(f, i, lds, fp, PH, c);
        else read_a(f, i, lds, rslot, PH, c);
    };
    auto rdb = [&](Frags<FMT, S> &f, int j) {
        if constexpr (S::BF4) read_b_f4(f, j, lds, fp, PH, c);
        else read_b(f, j, lds, rslot, PH, c);
    };
    constexpr int MB = S::MB, NB = S::NB;
    constexpr bool CUR1 = PH == 0 || ((PH - 1) & 1);
    Frags<FMT, S> &cur = CUR1 ? P.F1 : P.F0;
    Frags<FMT, S> &nxt = CUR1 ? P.F0 : P.F1;
    constexpr bool ROLL = rolling<FMT, S>();
    Frags<FMT, S> &fa = ROLL ? P.F0 : cur;      // where this phase's A fragments are
    constexpr int T = kk_of<FMT, S>() * MB * NB, NP = npieces<FMT, S>();
    // pieces go out right after the first MFMAs of the stage, so that they
    // have the longest time to land before the stage's barrier
    constexpr int SP = 1;
    static_assert(NP <= T, "every piece needs an MFMA slot");

    // the k-step these MFMAs consume and its stage's scales
    constexpr int KC = PH == 0 ? kk_of<FMT, S>() - 1 : PH - 1;
    const Scales<S> &sc = PH == 0 ? P.sprev : P.scur;

    if constexpr (RD) {
        // the stage's scale rows first: LDS reads complete in order, so the
        // adjustment in the next phase then waits for them alone and not for
        // the fragment reads issued after them
        if constexpr (mx_scales<FMT>() && PH == 0) {
            if constexpr (SM == kScalesChunk)
                read_scales_chunk<FMT, S>(P.scur, lds, cp.pc, cp.j, c);
            else
                read_scales<FMT>(P.scur, lds, rslot, c);
        }
        if constexpr (ROLL) {
#pragma unroll
            for (int j = 0; j < NB; ++j) rdb(nxt, j);
        } else {
            if constexpr (!adirect<FMT, S>()) {
#pragma unroll
                for (int i = 0; i < MB; ++i) rda(nxt, i);
            }
#pragma unroll
            for (int j = 0; j < NB; ++j) rdb(nxt, j);
        }
    }
    if constexpr (mx_scales<FMT>() && PH == 1) adjust_scales<FMT>(P.scur, c);
    if constexpr ((S::ACV || S::BCV) && LOADS) {
        constexpr int KK = kk_of<FMT, S>();
        if constexpr (cv_early<S>()) {
            // every piece of the next stage from memory now, all to LDS at
            // the stage's end: a whole stage for the loads to land
            if constexpr (PH == 0) load_cv<S, 0, cv_units<S>()>(P.cv, tg, ks, c, p.ldc);
        } else {
            // widened pieces: the previous group to LDS, this phase's group from memory
            if constexpr (PH > 0) store_cv<S, cv_group<S, KK>(PH - 1), cv_group<S, KK>(PH)>(P.cv, lds, lslot, c);
            load_cv<S, cv_group<S, KK>(PH), cv_group<S, KK>(PH + 1)>(P.cv, tg, ks, c, p.ldc);
        }
    }
    DBS_FENCE();
    if constexpr (FMT == kNVFP4R) {
        nv_raw_mma<S, RD>(acc, P.dec, cur, nxt);
        if constexpr (LOADS) {
#pragma unroll
            for (int q = 0; q < NP; ++q) {
                DBS_FENCE();
                if (PH == 0) load_piece<FMT, S, SM>(P, lds, lslot, tg, ks, p, c, q, stg, cp, fp);
                DBS_FENCE();
            }
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < MB; ++i) {
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            if constexpr (adirect<FMT, S>())
                mma1<FMT, 0>(acc[i][j], PH == 0 ? P.aprev[i] : P.acur[i][KC], 0u, cur.b[j], 0u);
            else
                mma1<FMT, scale_sel<FMT>(KC), S::CA, S::CB>(acc[i][j], fa.a[i], sc.a[i][0], cur.b[j], sc.b[j][0]);
            if constexpr (LOADS) {
                constexpr int base = PH * MB * NB;
                const int pos = base + i * NB + j;   // compile-time after unrolling
                if ((pos + 1) % SP == 0 && (pos + 1) / SP - 1 < NP) {
                    DBS_FENCE();
                    load_piece<FMT, S, SM>(P, lds, lslot, tg, ks, p, c, (pos + 1) / SP - 1, stg, cp, fp);
                    DBS_FENCE();
                }
            }
        }
        if constexpr (ROLL && RD) {
            DBS_FENCE();
            rda(P.F0, i);
            DBS_FENCE();
        }
    }
}

// One stage read from ring slot `slot` while stage ks of target tg is loaded
// into slot `nxt` (the slot read by the previous stage).  On entry F1 holds the last k-step of the previous
// stage (zeros at a tile's first stage): its MFMAs form the first phase,
// interleaved with the loads and with the reads of k-step 0 of this stage.
// The per-lane constants are re-declared opaque at every stage: addresses
// derived from them are then recomputed where they are used instead of being
// hoisted out of the stage loop into registers the accumulators need.
template <class S>
__device__ __forceinline__ void opaque(Ctx<S> &c)
{
    asm volatile("" : "+v"(c.t), "+v"(c.lane), "+v"(c.sa), "+v"(c.sb));
    if constexpr (!S::AMN || !S::BMN) asm volatile("" : "+v"(c.r8lda), "+v"(c.x4));
    asm volatile("" : "+v"(c.fa), "+v"(c.fb));
    if constexpr (S::AMN) asm volatile("" : "+v"(c.ma[0]), "+v"(c.ma[1]));
    if constexpr (S::BMN) asm volatile("" : "+v"(c.mb[0]), "+v"(c.mb[1]));
}

template <int FMT, class S, int SM>
__device__ __forceinline__ void stage(Pipe<FMT, S> &P, f32x16 (&acc)[S::MB][S::NB], uint8_t *lds, int slot,
                                      int nxt, const Params &p, Ctx<S> &c, const Target &tg, int ks, const Target &stg,
                                      const ChunkPos &cp, const F4Pos &fp)
{
    constexpr int KK = kk_of<FMT, S>();
    static_assert(S::NS == 2 || (FMT != kNVFP4 && SM != kScalesRegs && !S::ACV && !S::BCV),
                  "deeper rings need direct-to-LDS stages");
    static_assert(!(S::ACV || S::BCV) || (FMT == kMXFP8 && S::LAY == 0), "widened E2M1: 8-bit MX, K-major");
    static_assert(!(S::AF4 || S::BF4) || (FMT == kMXFP8 && S::NS == 2 && !S::ACV && !S::BCV && !(S::AF4 && S::BF4)),
                  "packed E2M1 beside 8-bit elements: two-slot rings");
    static_assert(SM != kScalesChunk || S::NS == 2, "chunked scales run on two-slot rings");
    static_assert(KK == 2 || KK == 4, "stages hold 2 or 4 k-steps");
    opaque(c);
    phase<FMT, S, SM, 0, true, true>(acc, P, lds, p, c, slot, tg, ks, nxt, stg, cp, fp);
    phase<FMT, S, SM, 1, true, true>(acc, P, lds, p, c, slot, tg, ks, nxt, stg, cp, fp);
    if constexpr (KK > 2) {
        phase<FMT, S, SM, 2, true, true>(acc, P, lds, p, c, slot, tg, ks, nxt, stg, cp, fp);
        phase<FMT, S, SM, 3, true, true>(acc, P, lds, p, c, slot, tg, ks, nxt, stg, cp, fp);
    }
    commit_stage<FMT, S, SM>(P, lds, nxt, c);
    if constexpr (mx_scales<FMT>()) {
#pragma unroll
        for (int i = 0; i < S::MB; ++i) P.sprev.a[i][0] = P.scur.a[i][0];
#pragma unroll
        for (int j = 0; j < S::NB; ++j) P.sprev.b[j][0] = P.scur.b[j][0];
    }
    stage_barrier<(S::NS - 2) * stage_loads_min<FMT, S, SM>()>();
}

// Buffer resources of output tile `tile`: A/B rows and their scale rows.
template <int FMT, class S>
__device__ __forceinline__ Target tile_target(const Params &p, int tile)
{
    const TileRef r = tile_ref<S::TM, S::TN>(tile, p);
    const int rows_a = min(r.mend - r.m0, S::TM), rows_b = min(p.N - r.n0, S::TN);
    Target t;
    if constexpr (S::AMN) {
        // from the tile's first column to the end of the K x M operand
        constexpr int EB = Mn<S::template fa<FMT>(), S::TM>::EB;
        const int64_t c0 = (int64_t)r.m0 * EB / 8;
        t.ra = make_rsrc(p.A + c0, (uint32_t)((int64_t)p.K * p.ldam - c0));
    } else if constexpr (S::ACV || S::AF4) {
        t.ra = make_rsrc(p.A + (int64_t)r.m0 * p.ldc, (uint32_t)(rows_a * p.ldc));
    } else {
        t.ra = make_rsrc(p.A + (int64_t)r.m0 * p.lda, (uint32_t)(rows_a * p.lda));
    }
    if constexpr (S::BMN) {
        constexpr int EB = Mn<S::template fb<FMT>(), S::TN>::EB;
        const int64_t c0 = (int64_t)r.n0 * EB / 8;
        t.rb = make_rsrc(p.B + c0, (uint32_t)((int64_t)p.K * p.ldbm - c0));
    } else if constexpr (S::BCV || S::BF4) {
        t.rb = make_rsrc(p.B + r.boff + (int64_t)r.n0 * p.ldc, (uint32_t)(rows_b * p.ldc));
    } else {
        t.rb = make_rsrc(p.B + r.boff + (int64_t)r.n0 * p.lda, (uint32_t)(rows_b * p.lda));
    }
    t.rsa = t.ra;
    t.rsb = t.rb;
    if constexpr (FMT != kBF16) {
        t.rsa = make_rsrc(p.sA + (int64_t)r.m0 * p.sld, (uint32_t)(rows_a * p.sld));
        t.rsb = make_rsrc(p.sB + r.sboff + (int64_t)r.n0 * p.sld, (uint32_t)(rows_b * p.sld));
    }
    return t;
}

__device__ __forceinline__ Target null_target()
{
    Target t;
    t.ra = t.rb = t.rsa = t.rsb = make_rsrc(nullptr, 0);
    return t;
}

template <int FMT, class S, int SM>
__global__ __launch_bounds__(S::kThreads, 1) void gemm_kernel(Params p)
{
    __shared__ __attribute__((aligned(1024))) uint8_t lds[lds_bytes<FMT, S, SM>()];
    constexpr int BPS = Fmt<FMT>::BPS;
    constexpr int MB = S::MB, NB = S::NB;

    Ctx<S> c;
    c.t = threadIdx.x;
    c.lane = c.t & 63;
    c.h = c.lane >> 5;
    c.lr = c.lane & 31;
    c.w = __builtin_amdgcn_readfirstlane(c.t >> 6);
    c.wm = c.w / S::WN;
    c.wn = c.w % S::WN;
    const int ra0 = c.wm * (S::TM / S::WM) + c.lr, rb0 = c.wn * (S::TN / S::WN) + c.lr;
    // (block offsets stay below the slot bits: row + 32 i < rows per slot)
    c.fa = (uint32_t)(S::kLdsA + ra0 * kRowBytes + ((c.h ^ swz(ra0)) << 4));
    c.fb = (uint32_t)(S::kLdsB + rb0 * kRowBytes + (((adirect<FMT, S>() ? 4 * c.h : c.h) ^ swz(rb0)) << 4));
    if constexpr (SM == kScalesChunk) {
        // bits 3-4 of the row index swizzle the row's dwords
        // (read_scales_chunk); rows 32 i further down keep them
        c.sa = (uint32_t)(S::kLdsS + ra0 * kScaleChunk) | (uint32_t)(4 * chunk_swz<FMT>(ra0));
        c.sb = (uint32_t)(S::kLdsS + (S::TM + rb0) * kScaleChunk) | (uint32_t)(4 * chunk_swz<FMT>(S::TM + rb0));
    } else if constexpr (FMT == kNVFP4R && SM == kScalesStage) {
        // raw NVFP4 scale rows of 16 bytes read 2 bytes of one dword per
        // lane: rows 8 and 16 apart (128 and 256 bytes) would meet in one
        // bank, so dword d of a row sits at position d ^ ((row / 8) % 4)
        // (dma_scales), carried here in bits 2-3 for the k-step's XOR;
        // rows 32 i further down keep them
        c.sa = (uint32_t)(S::kLdsS + ra0 * BPS) | (uint32_t)(4 * ((ra0 >> 3) & 3));
        c.sb = (uint32_t)(S::kLdsS + S::NS * S::TM * BPS + rb0 * BPS) | (uint32_t)(4 * ((rb0 >> 3) & 3));
    } else {
        c.sa = (uint32_t)(S::kLdsS + ra0 * BPS);
        c.sb = (uint32_t)(S::kLdsS + S::NS * S::TM * BPS + rb0 * BPS);
    }
    c.r8lda = (uint32_t)((c.lane >> 3) * p.lda);
    c.x4 = (uint32_t)(((c.lane & 7) ^ (c.lane >> 3)) << 4);
    if constexpr (S::AMN) {
        constexpr int FA = S::template fa<FMT>();
        c.fa = mn_base<FA, S::TM>(c.lane, c.wm * (S::TM / S::WM), S::kLdsA);
        c.ma[0] = mn_dma_lane<FA, S::TM>(c.lane, 0, p.ldam);
        c.ma[1] = mn_dma_lane<FA, S::TM>(c.lane, 1, p.ldam);
    }
    if constexpr (S::BMN) {
        constexpr int FB = S::template fb<FMT>();
        c.fb = mn_base<FB, S::TN>(c.lane, c.wn * (S::TN / S::WN), S::kLdsB);
        c.mb[0] = mn_dma_lane<FB, S::TN>(c.lane, 0, p.ldbm);
        c.mb[1] = mn_dma_lane<FB, S::TN>(c.lane, 1, p.ldbm);
    }

    const int ntiles = p.tiles_m * p.tiles_n;
    const int nwg = gridDim.x, wg = blockIdx.x;
    // hardware places workgroup wg on XCD wg % 8: give each XCD a contiguous
    // range of logical ids
    int tile = (nwg & 7) == 0 ? (wg & 7) * (nwg >> 3) + (wg >> 3) : wg;
    if (tile >= ntiles) return;

    // One stream of stages over all of the workgroup's tiles: the last stage
    // of a tile loads stage 0 of the next one, so no tile starts cold.
    Pipe<FMT, S> P;
    if constexpr (adirect<FMT, S>()) {
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) P.acur[i][kk] = f16x8{};
    }
    // The load stream runs NS-1 stages ahead of the stage being computed,
    // across the workgroup's tiles (a tile has at least NS-1 stages: the host
    // picks a shallower ring otherwise); ld holds the resources of the tile
    // it loads from (empty past the last tile).
    Target ld = tile_target<FMT, S>(p, tile);
    // chunked scales: stg holds the scale rows the portion loads read from,
    // which move to the next tile a chunk ahead of the operand loads; the
    // first tile's chunk 0 goes to buffer 0 now
    constexpr int SPC = scale_spc<FMT>();
    Target stg = ld;
    ChunkPos cp{0, 0, 0};
    // a packed E2M1 operand: its first 256-K stage goes to slot 0 of its ring
    constexpr bool F4 = S::AF4 || S::BF4;
    __amdgpu_buffer_rsrc_t f4r = S::AF4 ? ld.ra : ld.rb;
    int f4s = 0;   // the E2M1 ring slot the next stage reads
    F4Pos fp{0, 0, 0, 0, f4r};
#pragma unroll
    for (int f = 0; f < S::NS - 1; ++f) {
#pragma unroll
        for (int q = 0; q < npieces<FMT, S>(); ++q) load_piece<FMT, S, SM>(P, lds, f, ld, f, p, c, q, stg, cp, fp);
        if constexpr (S::ACV || S::BCV) load_cv<S, 0, cv_units<S>()>(P.cv, ld, f, c, p.ldc);
        commit_stage<FMT, S, SM, true>(P, lds, f, c);
    }
    if constexpr (F4) {
#pragma unroll
        for (int q = 0; q < f4_q<S, S::AF4>(); ++q)
            dma_f4<S, S::AF4>(lds, 0, f4r, 0, 1, c, q, p.ldc, S::AF4 ? p.ldam : p.ldbm);
    }
    if constexpr (SM == kScalesChunk) {
#pragma unroll
        for (int u = 0; u < SPC; ++u) dma_scale_portion<FMT>(lds, 0, ld, 0, u, c, p.sld);
    }
    __syncthreads();
    int pc = 0;   // chunk buffer of the stage being computed

    int rs = 0;   // ring slot the next stage reads
    int xs = 0;   // ring slot the last stage read
    for (;;) {
        f32x16 acc[MB][NB];
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int j = 0; j < NB; ++j) acc[i][j] = f32x16{};
        // the "previous stage" of a tile's first stage contributes nothing
        P.F1 = Frags<FMT, S>{};
        if constexpr (FMT == kNVFP4R) P.dec = NvDec<S>{};   // its group 0, decoded
        if constexpr (adirect<FMT, S>()) {
#pragma unroll
            for (int i = 0; i < MB; ++i) P.aprev[i] = f16x8{};
        }
        if constexpr (rolling<FMT, S>()) {
#pragma unroll
            for (int i = 0; i < MB; ++i) P.F0.a[i] = {};
        }
        if constexpr (mx_scales<FMT>()) {
            // unit E8M0 scales (finite) for those zero fragments
#pragma unroll
            for (int i = 0; i < MB; ++i) P.sprev.a[i][0] = 0x7F7F7F7Fu;
#pragma unroll
            for (int j = 0; j < NB; ++j) P.sprev.b[j][0] = 0x7F7F7F7Fu;
        }

        const int next = tile + nwg;
        for (int s = 0; s < p.nk; ++s) {
            // stage s loads stage s+NS-1 of the stream into the slot the
            // previous stage read
            int ks = s + S::NS - 1;
            if (ks >= p.nk) {
                ks -= p.nk;
                if (ks == 0) ld = next < ntiles ? tile_target<FMT, S>(p, next) : null_target();
            }
            const int ls = rs == 0 ? S::NS - 1 : rs - 1;
            if constexpr (SM == kScalesChunk) {
                // a tile holds a whole number of chunks; stage s loads
                // portion s % SPC of the next chunk, which past the tile's
                // last chunk is the next tile's first
                cp.pc = pc;
                cp.j = s % SPC;
                cp.lchunk = s / SPC + 1;
                if (cp.lchunk * SPC == p.nk) {
                    cp.lchunk = 0;
                    if (cp.j == 0) stg = next < ntiles ? tile_target<FMT, S>(p, next) : null_target();
                }
            }
            if constexpr (F4) {
                // stages s, s + 1 (s even) load the two halves of the
                // operand's next 256-K stage: this tile's s / 2 + 1, or the
                // next tile's first
                fp = F4Pos{f4s, s & 1, f4s ^ 1, s / 2 + 1, f4r};
                if (s + 2 >= p.nk) {
                    if (s + 2 == p.nk) {
                        const Target t = next < ntiles ? tile_target<FMT, S>(p, next) : null_target();
                        f4r = S::AF4 ? t.ra : t.rb;
                    }
                    fp.ks = 0;
                    fp.r = f4r;
                }
            }
            stage<FMT, S, SM>(P, acc, lds, rs, ls, p, c, ld, ks, stg, cp, fp);
            if constexpr (F4) f4s ^= s & 1;
            if constexpr (SM == kScalesChunk) pc ^= cp.j == SPC - 1 ? 1 : 0;
            xs = rs;
            rs = rs + 1 == S::NS ? 0 : rs + 1;
        }
        phase<FMT, S, SM, 0, false, false>(acc, P, lds, p, c, 0, ld, 0, 0, stg, cp, fp);

        const TileRef tr = tile_ref<S::TM, S::TN>(tile, p);
        // (the one-wave-per-SIMD variant has no registers to spare for the
        // staged epilogue)
        if (S::NW == 8 || S::NB <= 2) {
            if (p.vec16) {
                // the slot the last stage read is free until the next
                // tile's first stage refills it
                // (a packed E2M1 A: the slot of its ring the tile read last)
                store_tile_lds<S>(acc, lds, S::AF4 ? (f4s ^ 1) : xs, p, tr, c);
                asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
            } else {
                store_tile<S>(acc, p, tr, c);
            }
        } else {
            store_tile<S>(acc, p, tr, c);
        }
        if (next >= ntiles) break;
        tile = next;
    }
}

template <class S>
constexpr int shape_id() { return std::is_same<S, Square>::value ? kShapeSquare : kShapeSkinny; }

// Shape dispatch of a translation unit's launcher: F(S) for the chosen shape.
template <class F>
hipError_t by_shape(int shape, F &&f)
{
    if (shape == kShapeSquare) return f(Square{});
    if (shape == kShapeSkinny) return f(Skinny{});
    return hipErrorInvalidValue;
}

// K elements per stage of kernel (FMT, S)
template <int FMT, class S>
constexpr int stage_elems()
{
    return FMT == kBF16 || FMT == kNVFP4 ? kRowBytes / 2 : FMT == kMXFP8 ? kRowBytes : 2 * kRowBytes;
}

// 8-bit MX kernels with E5M2 on either side (element codes ec: 1 A, 8 B, 9
// both), in each operand layout.
template <int EC, int SM, class S0>
hipError_t launch_ec_lay(const Params &p, int grid, hipStream_t stream)
{
    switch (p.lay) {
    case 0: hipLaunchKernelGGL((gemm_kernel<kMXFP8, WithLayout<S0, 0, EC>, SM>), dim3(grid), dim3(S0::kThreads), 0, stream, p); break;
    case 1: hipLaunchKernelGGL((gemm_kernel<kMXFP8, WithLayout<S0, 1, EC>, SM>), dim3(grid), dim3(S0::kThreads), 0, stream, p); break;
    case 2: hipLaunchKernelGGL((gemm_kernel<kMXFP8, WithLayout<S0, 2, EC>, SM>), dim3(grid), dim3(S0::kThreads), 0, stream, p); break;
    case 3: hipLaunchKernelGGL((gemm_kernel<kMXFP8, WithLayout<S0, 3, EC>, SM>), dim3(grid), dim3(S0::kThreads), 0, stream, p); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int SM, class S0>
hipError_t launch_ec(const Params &p, int grid, hipStream_t stream)
{
    switch (p.ec) {
    case 1: return launch_ec_lay<1, SM, S0>(p, grid, stream);
    case 8: return launch_ec_lay<8, SM, S0>(p, grid, stream);
    case 9: return launch_ec_lay<9, SM, S0>(p, grid, stream);
    default: return hipErrorInvalidValue;
    }
}

// E5: the 8-bit MX kernels with E5M2 on either side (their own translation
// unit); otherwise E4M3 on both sides.
template <int FMT, int SM, class S0, bool E5 = false>
hipError_t launch_one(const Params &p0, int grid, hipStream_t stream)
{
    Params p = p0;
    p.nk = (p.K + stage_elems<FMT, S0>() - 1) / stage_elems<FMT, S0>();
    if constexpr (FMT == kNVFP4) {
        if (p.lay != 0) return hipErrorInvalidValue;   // MN-major NVFP4 runs on the raw kernels
        hipLaunchKernelGGL((gemm_kernel<FMT, S0, SM>), dim3(grid), dim3(S0::kThreads), 0, stream, p);
    } else {
        if constexpr (FMT == kMXFP8) {
            if (p.cv != 0) return hipErrorInvalidValue;    // launch_cv's and launch_f4's
            if constexpr (E5) {
                // E5M2 on either side: the same staging as E4M3 in every
                // layout, other MFMA format fields
                if (p.ec != 1 && p.ec != 8 && p.ec != 9) return hipErrorInvalidValue;
                return launch_ec<SM, S0>(p, grid, stream);
            } else {
                if (p.ec != 0) return hipErrorInvalidValue;
            }
        }
        // raw NVFP4 with K-major operands: the 8-wave square tiles and the
        // 4-wave skinny ones with 16-byte scale pieces only
        constexpr bool K0 = FMT != kNVFP4R || (std::is_same<S0, Square>::value && SM != kScalesRegs) ||
                            (std::is_same<S0, SkinnyW4Deep>::value && SM == kScalesRows16);
        if (!K0 && p.lay == 0) return hipErrorInvalidValue;
        switch (p.lay) {
        case 0:
            if constexpr (K0)
                hipLaunchKernelGGL((gemm_kernel<FMT, WithLayout<S0, 0>, SM>), dim3(grid), dim3(S0::kThreads), 0, stream, p);
            break;
        case 1: hipLaunchKernelGGL((gemm_kernel<FMT, WithLayout<S0, 1>, SM>), dim3(grid), dim3(S0::kThreads), 0, stream, p); break;
        case 2: hipLaunchKernelGGL((gemm_kernel<FMT, WithLayout<S0, 2>, SM>), dim3(grid), dim3(S0::kThreads), 0, stream, p); break;
        case 3: hipLaunchKernelGGL((gemm_kernel<FMT, WithLayout<S0, 3>, SM>), dim3(grid), dim3(S0::kThreads), 0, stream, p); break;
        default: return hipErrorInvalidValue;
        }
    }
    return hipGetLastError();
}

template <int FMT, class S>
constexpr int stages_of(int K) { return (K + stage_elems<FMT, S>() - 1) / stage_elems<FMT, S>(); }

// 8-bit MX GEMMs with a widened E2M1 or FP6 operand (K-major; cv names the
// sources, see Shape).  The register-staged pieces do not fit beside the
// 8-wave square kernel's fragments (the compiler spills 160+ registers
// there): E2M1 runs square problems on the one-wave-per-SIMD tiles, FP6
// (whose pieces spill even there) only on 256 x 64 tiles, which the host
// picks for it.  Scale rows take the register-staged path on the square tiles
// and on unaligned skinny problems.
template <int SM, class S0>
hipError_t launch_cv(const Params &p0, int grid, hipStream_t stream)
{
    static_assert(S0::NS == 2, "register-staged operands use two-slot rings");
    Params p = p0;
    p.nk = (p.K + stage_elems<kMXFP8, S0>() - 1) / stage_elems<kMXFP8, S0>();
    if (p.lay != 0) return hipErrorInvalidValue;
#define DBS_CV(CVV, ECV) \
    case (CVV) * 64 + (ECV): \
        hipLaunchKernelGGL((gemm_kernel<kMXFP8, WithLayout<S0, 0, ECV, CVV>, SM>), dim3(grid), dim3(S0::kThreads), 0, \
                           stream, p); \
        break;
    if constexpr (std::is_same<S0, SquareW4>::value) {
        // (FP6 operands run on 256 x 64 tiles: the host picks them)
        switch (p.cv * 64 + p.ec) {
            // E2M1 beside E4M3 / E5M2
            DBS_CV(1, 0) DBS_CV(1, 8) DBS_CV(4, 0) DBS_CV(4, 1)
        default: return hipErrorInvalidValue;
        }
    } else if constexpr (std::is_same<S0, SkinnyW8>::value) {
        // FP6 only (E2M1 widens on the 4-wave 256 x 64 tile)
        switch (p.cv * 64 + p.ec) {
            // E2M3 (widened to E4M3) / E3M2 (to E5M2) beside E4M3 / E5M2
            DBS_CV(2, 0) DBS_CV(2, 8) DBS_CV(3, 1) DBS_CV(3, 9)
            DBS_CV(8, 0) DBS_CV(8, 1) DBS_CV(12, 8) DBS_CV(12, 9)
            // FP6 x FP6
            DBS_CV(10, 0) DBS_CV(14, 8) DBS_CV(11, 1) DBS_CV(15, 9)
        default: return hipErrorInvalidValue;
        }
    } else {
        switch (p.cv * 64 + p.ec) {
            DBS_CV(1, 0) DBS_CV(1, 8) DBS_CV(4, 0) DBS_CV(4, 1)
        default: return hipErrorInvalidValue;
        }
    }
#undef DBS_CV
    return hipGetLastError();
}

// 8-bit MX GEMMs with an E2M1 operand staged as packed codes (K % 256 == 0,
// K-major): the element codes with 4 on the E2M1 side.
template <int SM, class S0>
hipError_t launch_f4(const Params &p0, int grid, hipStream_t stream)
{
    static_assert(S0::NS == 2, "the E2M1 ring pairs with a two-slot ring");
    Params p = p0;
    p.nk = p.K / stage_elems<kMXFP8, S0>();
    if (p.K % 256 != 0) return hipErrorInvalidValue;
    const int ca = p.cv == 1 ? 4 : p.ec & 7, cb = p.cv == 4 ? 4 : (p.ec >> 3) & 7;
    switch (ca | (cb << 3)) {
    case 4: return launch_ec_lay<4, SM, S0>(p, grid, stream);
    case 12: return launch_ec_lay<12, SM, S0>(p, grid, stream);
    case 32: return launch_ec_lay<32, SM, S0>(p, grid, stream);
    case 33: return launch_ec_lay<33, SM, S0>(p, grid, stream);
    default: return hipErrorInvalidValue;
    }
}

// 8-bit MX GEMMs with an E2M1 or FP6 operand (cv != 0): E2M1 takes the
// packed path when K % 256 == 0, everything else the widening path.
template <class S>
hipError_t launch_fp8_fp4(const Params &p, int grid, hipStream_t stream)
{
    const bool e2m1 = p.cv == 1 || p.cv == 4;   // (an FP6 operand is always widened)
    if (e2m1 && p.K % 256 == 0) {
        // FP8 x FP4 on the MFMA's mixed formats: the E2M1 operand in its
        // own ring of packed 256-K stages
        if (!p.scales_aligned) {
            using U = typename std::conditional<std::is_same<S, Square>::value, SquareW4, S>::type;
            return launch_f4<kScalesRegs, U>(p, grid, stream);
        }
        if constexpr (std::is_same<S, Square>::value) {
            if (stages_of<kMXFP8, S>(p.K) % scale_spc<kMXFP8>() == 0)
                return launch_f4<kScalesChunk, S>(p, grid, stream);
        }
        return launch_f4<kScalesStage, S>(p, grid, stream);
    }
    if (p.cv != 0) {
        if constexpr (std::is_same<S, Square>::value) {
            // widened FP6 has 256 x 64 kernels only (the host routes it there)
            if (!e2m1) return hipErrorNotSupported;
            return launch_cv<kScalesRegs, SquareW4>(p, grid, stream);
        } else {
            if (!e2m1) {
                // FP6 (the host puts it on these tiles)
                if (p.scales_aligned) return launch_cv<kScalesStage, SkinnyW8>(p, grid, stream);
                return launch_cv<kScalesRegs, SkinnyW8>(p, grid, stream);
            }
            if (p.scales_aligned) return launch_cv<kScalesStage, S>(p, grid, stream);
            return launch_cv<kScalesRegs, S>(p, grid, stream);
        }
    }
    return hipErrorInvalidValue;
}

template <int FMT, class S, bool E5 = false>
hipError_t launch_fmt(const Params &p, int grid, hipStream_t stream)
{
    if constexpr (FMT == kMXFP8 && !E5) {
        // E2M1 beside E4M3/E5M2, and E5M2 pairs: their own translation units
        if (p.cv != 0) return launch_gemm_mx8_fp4(shape_id<S>(), p, grid, stream);
        if (p.ec != 0) return launch_gemm_mx8_e5m2(shape_id<S>(), p, grid, stream);
    }
    if constexpr (FMT == kMXFP8 || FMT == kMXFP4) {
        if (!p.scales_aligned) {
            using U = typename std::conditional<std::is_same<S, Square>::value, SquareW4, S>::type;
            return launch_one<FMT, kScalesRegs, U, E5>(p, grid, stream);
        }
    }
    if constexpr (FMT == kNVFP4) {
        if (p.K % 32) return launch_one<FMT, kNvHalf, S>(p, grid, stream);
        return launch_one<FMT, kNvWhole, S>(p, grid, stream);
    }

    // stages that arrive entirely by direct-to-LDS loads get a deeper ring
    // when every tile has enough stages to fill it
    if constexpr (std::is_same<S, Skinny>::value && FMT != kNVFP4) {
        if (p.cv == 0 && stages_of<FMT, SkinnyDeep>(p.K) >= SkinnyDeep::NS - 1)
            return launch_one<FMT, kScalesStage, SkinnyDeep, E5>(p, grid, stream);
    }
    // MX scales in chunks when a tile's stages split into whole chunks (and
    // a chunk's portions into whole wave-loads per wave)
    if constexpr ((FMT == kMXFP8 || FMT == kMXFP4) && S::NS == 2 &&
                  ((S::TM + S::TN) / scale_spc<FMT>() / 16) % S::NW == 0) {
        if (stages_of<FMT, S>(p.K) % scale_spc<FMT>() == 0)
            return launch_one<FMT, kScalesChunk, S, E5>(p, grid, stream);
    }
    return launch_one<FMT, kScalesStage, S, E5>(p, grid, stream);
}

// Raw NVFP4 (K % 32 == 0, or an MN-major operand).  Square tiles: the 8-wave
// kernel when the scale rows take dword loads (K-major or not: it beats
// decoding into LDS by about a fifth at 8192^3); otherwise the register-staged
// scale bytes need the one-wave-per-SIMD tiles, and K-major operands go back
// to the NVFP4 kernels.  Skinny tiles: K-major operands keep the NVFP4
// kernels (the raw-ring kernel), MN-major ones take the deeper ring when
// every tile has the stages to fill it.
template <class S>
hipError_t launch_nvfp4_raw(const Params &p, int grid, hipStream_t stream)
{
    // scale rows of whole 16-byte stage pieces on 16-byte boundaries
    const bool r16 = p.scales_aligned && p.K % 256 == 0 &&
                     ((reinterpret_cast<uintptr_t>(p.sA) | reinterpret_cast<uintptr_t>(p.sB)) & 15) == 0;
    if constexpr (std::is_same<S, Square>::value) {
        if (p.scales_aligned) return launch_one<kNVFP4R, kScalesStage, Square>(p, grid, stream);
        if (p.lay == 0) return launch_fmt<kNVFP4, S>(p, grid, stream);
        return launch_one<kNVFP4R, kScalesRegs, SquareW4>(p, grid, stream);
    } else {
        if (p.lay == 0 && r16 && stages_of<kNVFP4R, SkinnyW4Deep>(p.K) >= SkinnyW4Deep::NS - 1)
            return launch_one<kNVFP4R, kScalesRows16, SkinnyW4Deep>(p, grid, stream);
        if (p.lay == 0) return launch_fmt<kNVFP4, S>(p, grid, stream);
        if (p.scales_aligned && stages_of<kNVFP4R, SkinnyDeep>(p.K) >= SkinnyDeep::NS - 1) {
            if (r16) return launch_one<kNVFP4R, kScalesRows16, SkinnyDeep>(p, grid, stream);
            return launch_one<kNVFP4R, kScalesStage, SkinnyDeep>(p, grid, stream);
        }
        if (p.scales_aligned) return launch_one<kNVFP4R, kScalesStage, S>(p, grid, stream);
        return launch_one<kNVFP4R, kScalesRegs, S>(p, grid, stream);
    }
}

}  // namespace
}  // namespace dbs
