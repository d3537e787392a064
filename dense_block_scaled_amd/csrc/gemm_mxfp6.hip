// gemm_mxfp6.hip -- MXFP6 GEMM (E2M3 / E3M2 on both sides) at the MFMA's
// native FP6 rate
//
// gfx950's scaled MFMA (v_mfma_scale_f32_32x32x64_f8f6f4) takes FP6 operands
// directly: format codes 2 (E2M3) and 3 (E3M2), six VGPRs per lane, lane half
// h of a 64-K step holding K 32h .. 32h+31 as 24 packed bytes in the order the
// rows store them (element j at bits 6j .. 6j+5; established with a one-wave
// probe against random codes, as for the other formats), and its E8M0 scale
// applying to those 32 elements.  An FP6 x FP6 product runs at the FP4 rate,
// twice the 8-bit one.  ("Dissecting ThunderKittens", tile abstractions: one
// element type per operand tile.)
//
// Tiles and waves are those of the 8-wave square kernels (gemm_kernel.h):
// 256 x 256 output tiles, persistent workgroups with the XCD-aware raster, 8
// waves of 128 x 64 (4 x 2 MFMA blocks of 32 x 32), fp32 accumulators, the
// LDS-staged bf16 epilogue, a two-slot ring.  What differs is the staging of
// the 24-byte fragments:
//
// * A stage is 128 K elements: 96 bytes of every A and B row of the tile, as
//   eight 12-byte pieces of 16 elements.  They arrive by direct-to-LDS buffer
//   loads of 12 bytes per lane (buffer_load_dwordx3 ... lds), which write
//   lane i's bytes at 16 i (established with a one-wave probe: the last four
//   bytes of each 16-byte cell stay untouched).  So a slot row is eight
//   16-byte cells, each holding one piece, like an MXFP8 row of eight 16-byte
//   chunks of 16 elements, and takes the same XOR swizzle of the cells
//   (cell ^ ((row ^ row / 8) % 8)): a wave-load fills rows 8L .. 8L+7, each
//   lane fetching the piece that belongs at its fixed cell.
// * The fragment of k-step kk for lane half h is pieces 4 kk + 2 h and
//   4 kk + 2 h + 1 of its row: two ds_read_b96 of 16-byte-aligned cells.
// * E8M0 scales: 4 bytes (blocks 0..3 of the stage) per row, read once per
//   stage per row block and fed to the MFMA with op_sel picking the k-step's
//   byte, as for MXFP8.  When a tile's stages come in whole chunks of four
//   (K % 512 == 0) a row's scales arrive 16 bytes (four stages) at a time
//   into two alternating chunk buffers, a quarter of the next chunk's rows
//   per stage, so a scale row costs one memory request per four stages (a
//   per-stage dword of each of the tile's 512 rows costs as many requests as
//   the stage's operand rows); else one dword wave-load per wave and stage
//   into per-stage slots.
//
// * Stage-blocked operands (Params::blk6, the FP4-rate NVFP4 path, whose
//   workspace this library lays out itself): the 96 bytes of a stage of eight
//   consecutive rows 8g .. 8g+7 lie together, 768 contiguous bytes at
//   (g nk + ks) 768 + 96 (row % 8) for nk stages a row, so a wave-load
//   (eight rows of one stage) reads six whole 128-byte lines where eight
//   96-byte row pieces of the row-major layout touch twelve on average
//   (a piece straddles two lines half of the time).  Row group g starts
//   where row 8g of the row-major layout would, so the tile's rows start
//   at the same offset; operand rows are padded to a multiple of 8 (the
//   padding rows only feed outputs that are never stored).
//
// Problems this kernel takes (the host checks): FP6 on both operands,
// K-major, K a multiple of 128 (whole stages; rows of whole dwords of
// scales), scale rows on 4-byte boundaries, and enough 256 x 256 tiles to
// occupy a quarter of the CUs.
#include "gemm_kernel.h"

namespace dbs {

namespace {
namespace f6 {

using S = Shape<kSquareTM, kSquareTN, 2, 4>;
constexpr int kRow = 128;                              // LDS bytes of a tile row per stage: 8 cells of 16
constexpr int kGRow = 96;                              // global bytes of a row per stage
constexpr int kKs = 128;                               // K elements per stage
constexpr int kOp = S::TM * kRow;                      // one operand's part of a slot
constexpr int kSlot = 2 * kOp;                         // A rows, then B rows
constexpr int NS = 2;
constexpr int kScaleSlot = (S::TM + S::TN) * 4;        // A rows, then B rows, 4 bytes each
constexpr int kChunk = 16;                             // chunked scales: bytes per row per chunk
constexpr int kSpc = kChunk / 4;                       // stages per chunk
constexpr int kChunkBuf = (S::TM + S::TN) * kChunk;    // one chunk buffer: A rows, then B rows
constexpr int kLdsS = NS * kSlot;
template <bool CH>
constexpr int lds_bytes() { return kLdsS + (CH ? 2 * kChunkBuf : NS * kScaleSlot); }
constexpr int kLoadsOp = S::TM / 8 / S::NW;            // wave-loads per wave, operand and stage
constexpr int kLoads = 2 * kLoadsOp + 1;               // and one scale wave-load
static_assert(lds_bytes<false>() <= 160 * 1024 && lds_bytes<true>() <= 160 * 1024, "LDS budget");
static_assert((S::TM + S::TN) / kSpc == 16 * S::NW && S::TM % ((S::TM + S::TN) / kSpc) == 0,
              "a chunk portion is one 16-row dword wave-load per wave, all of one operand");
static_assert(S::TM == S::TN && S::MB == 4 && S::NB == 2, "square tiles, 128 x 64 per wave");
static_assert(S::NW * epilogue_wave_bytes<S>() <= kSlot, "epilogue staging fits in a ring slot");
static_assert((S::TM + S::TN) * 4 == S::NW * 256, "one scale wave-load per wave");
static_assert((kOp & (kOp - 1)) == 0 && (kSlot & (kSlot - 1)) == 0, "slot offsets are OR-able");

// 24 bytes of one row's unit: a lane's FP6 fragment of one k-step (one
// vector value, so that it stays in registers)
typedef __attribute__((ext_vector_type(6))) int Frag6;

// A fragments are single-buffered: each is re-read for the next k-step right
// after its last MFMA of the current one.  B fragments are double-buffered.
struct Frags6 {
    Frag6 a[S::MB];
    Frag6 b[2][S::NB];
};

struct Sc6 {
    uint32_t a[S::MB], b[S::NB];
};

struct Lane {
    int lane, h, lr, w, wm, wn;
    uint32_t fa, fb;        // LDS address of the lane's first cell: block 0, k-step 0, slot 0, swizzle applied
    uint32_t r8;            // the lane's row within a wave-load: (lane / 8) * lda, or (lane / 8) * 96 stage-blocked
    uint32_t kst;           // bytes from one stage of a row to the next: 96, or 768 stage-blocked
    uint32_t x;             // (lane % 8) ^ (lane / 8): the lane's cell within a wave-load, before (L % 8)
    uint32_t sa, sb;        // chunked scales: LDS address of the lane's A / B row in chunk buffer 0, with
                            // 4 ((row / 8) % 4) in bits 2-3
};

// Where the chunked scales of a stage come from and go: the stage reads
// dword j of chunk buffer pc and loads portion j of chunk lchunk, from the
// scale rows sa / sb, into buffer pc ^ 1.
struct Chunk6 {
    int pc, j, lchunk;
    __amdgpu_buffer_rsrc_t sa, sb;
};

typedef __attribute__((ext_vector_type(3))) int i32x3;

// The MFMA operand: six dwords, the other two unused for FP6 formats.
__device__ __forceinline__ i32x8 frag_op(const Frag6 &f) { return __builtin_shufflevector(f, f, 0, 1, 2, 3, 4, 5, -1, -1); }

// Fragment of k-step kk, row block blk, in the slot at byte `sel` (a power of
// two above every in-slot bit): cells 4 kk + 2 h (+1) of the lane's row.
// fbase holds the row, the swizzle and 2 h; block blk adds 32 rows (4096
// bytes) and flips swizzle bit 2 when odd (((r + 32 blk) / 8) % 8 = (r / 8 +
// 4 blk) % 8), i.e. address bit 6, as does kk.
__device__ __forceinline__ Frag6 read_frag6(const uint8_t *lds, uint32_t fbase, uint32_t sel, int kk, int blk)
{
    const uint32_t x = (fbase | sel) ^ (uint32_t)(64 * (kk ^ (blk & 1)));
    const uint32_t off = (uint32_t)(blk * 32 * kRow);
    const i32x3 p0 = *reinterpret_cast<const i32x3 *>(__builtin_assume_aligned(lds + x + off, 16));
    const i32x3 p1 = *reinterpret_cast<const i32x3 *>(__builtin_assume_aligned(lds + (x ^ 16u) + off, 16));
    return __builtin_shufflevector(p0, p1, 0, 1, 2, 3, 4, 5);
}

__device__ __forceinline__ Frag6 read_a(const uint8_t *lds, int slot, int kk, int i, const Lane &c)
{
    return read_frag6(lds, c.fa, (uint32_t)(slot * kSlot), kk, i);
}

__device__ __forceinline__ Frag6 read_b(const uint8_t *lds, int slot, int kk, int j, const Lane &c)
{
    return read_frag6(lds, c.fb, (uint32_t)(slot * kSlot), kk, j);
}

__device__ __forceinline__ void read_scales(Sc6 &sc, const uint8_t *lds, int slot, const Lane &c)
{
    const uint32_t base = (uint32_t)(kLdsS + slot * kScaleSlot);
#pragma unroll
    for (int i = 0; i < S::MB; ++i)
        sc.a[i] = lds_read<uint32_t>(lds, base + (uint32_t)((c.wm * 128 + 32 * i + c.lr) * 4));
#pragma unroll
    for (int j = 0; j < S::NB; ++j)
        sc.b[j] = lds_read<uint32_t>(lds, base + (uint32_t)((S::TM + c.wn * 64 + 32 * j + c.lr) * 4));
}

// Chunked layout: a row's 16 bytes hold dword d (one per stage) at position
// d ^ ((row / 8) % 4), row = the row's index in the concatenated list: the
// 32 rows one read covers are 16 bytes apart, so rows 8 and 16 apart (128
// and 256 bytes) would meet in one bank, and the swizzle gives rows r,
// r + 8, r + 16, r + 24 four different dwords.
__device__ __forceinline__ void read_scales_chunk(Sc6 &sc, const uint8_t *lds, int pc, int j, const Lane &c)
{
    const uint32_t o = (uint32_t)(pc * kChunkBuf), jb = (uint32_t)(4 * j);
#pragma unroll
    for (int i = 0; i < S::MB; ++i) sc.a[i] = lds_read<uint32_t>(lds, (c.sa ^ jb) + o + (uint32_t)(i * 32 * kChunk));
#pragma unroll
    for (int jj = 0; jj < S::NB; ++jj)
        sc.b[jj] = lds_read<uint32_t>(lds, (c.sb ^ jb) + o + (uint32_t)(jj * 32 * kChunk));
}

// Lane half h takes blocks 2 kk + h of the stage: byte 2 kk after a shift by 8 h.
__device__ __forceinline__ void adjust(Sc6 &sc, const Lane &c)
{
#pragma unroll
    for (int i = 0; i < S::MB; ++i) sc.a[i] >>= 8 * c.h;
#pragma unroll
    for (int j = 0; j < S::NB; ++j) sc.b[j] >>= 8 * c.h;
}

// Wave-load q (0 .. kLoadsOp-1) of operand X of stage ks into slot `slot`:
// slot rows 8L .. 8L+7 with L = w kLoadsOp + q; lane i lands on cell i % 8
// of row 8L + i / 8, whose swizzle is (i / 8) ^ (L % 8), and fetches the
// 12-byte piece (i % 8) ^ (i / 8) ^ (L % 8) of that row's stage.  Rows past
// the operand's end lie past the buffer resource and read zero (stage-blocked:
// the resource ends with the last row's group of 8, padding rows included).
template <bool IS_A>
__device__ __forceinline__ void load_op(uint8_t *lds, int slot, __amdgpu_buffer_rsrc_t r, int ks, int q,
                                        const Lane &c, int lda)
{
    const int L = c.w * kLoadsOp + q;
    const uint32_t piece = c.x ^ (uint32_t)(L & 7);
    const uint32_t off = c.r8 + (uint32_t)(L * 8 * lda) + (uint32_t)ks * c.kst + 12u * piece;
    const int dst = slot * kSlot + (IS_A ? 0 : kOp) + L * 1024;
    lds_dma<12>(r, lds + dst, off);
}

// The stage's scales: wave w fetches the dword of rows 64 (w % 4) + lane of
// A (w < 4) or B, i.e. bytes 4 ks .. 4 ks + 3 of the row (blocks 4 ks ..).
__device__ __forceinline__ void load_scales(uint8_t *lds, int slot, const Target &tg, int ks, const Lane &c, int sld)
{
    const bool is_a = c.w < 4;
    const uint32_t off = (uint32_t)((64 * (c.w & 3) + c.lane) * sld + 4 * ks);
    const int dst = kLdsS + slot * kScaleSlot + c.w * 256;
    lds_dma<4>(is_a ? tg.rsa : tg.rsb, lds + dst, off);
}

// Chunked scales: portion u (0 .. 3) of chunk `chunk` (bytes 16 chunk ..
// 16 chunk + 15 of every scale row) into chunk buffer `pc`: rows 128 u ..
// 128 u + 127 of the concatenated list (A rows, then B rows), wave w taking
// rows 128 u + 16 w .. + 15: lane i lands on dword position i % 4 of row
// i / 4 and fetches the row's dword (i % 4) ^ ((row / 8) % 4) (see
// read_scales_chunk).  Dwords past a row's end and rows past the operand's
// read zero.
__device__ __forceinline__ void load_scale_portion(uint8_t *lds, int pc, __amdgpu_buffer_rsrc_t sa,
                                                   __amdgpu_buffer_rsrc_t sb, int chunk, int u, const Lane &c, int sld)
{
    const int row0 = u * ((S::TM + S::TN) / kSpc) + c.w * 16;     // wave-uniform
    const bool is_a = row0 < S::TM;
    const int r = (is_a ? row0 : row0 - S::TM) + (c.lane >> 2);
    const int o = chunk * kChunk + 4 * ((c.lane & 3) ^ (((row0 + (c.lane >> 2)) >> 3) & 3));
    const uint32_t off = (uint32_t)(r * sld + o) | (o < sld ? 0u : kOOB);
    const int dst = kLdsS + pc * kChunkBuf + row0 * kChunk;
    lds_dma<4>(is_a ? sa : sb, lds + dst, off);
}

// Load n (0 .. kLoads-1) of the wave's share of a stage: operand rows, then
// the stage's scales (per stage) or a portion of the next chunk (CH).
// Buffer resources of a tile: those of the 8-bit kernels, with the operand
// resources extended to whole groups of 8 rows when stage-blocked.
__device__ __forceinline__ Target target6(const Params &p, int tile)
{
    Target t = tile_target<kMXFP8, S>(p, tile);
    if (p.blk6) {
        const TileRef r = tile_ref<S::TM, S::TN>(tile, p);
        const int ra = (min(r.mend - r.m0, S::TM) + 7) & ~7, rb = (min(p.N - r.n0, S::TN) + 7) & ~7;
        t.ra = make_rsrc(p.A + (int64_t)r.m0 * p.lda, (uint32_t)(ra * p.lda));
        t.rb = make_rsrc(p.B + r.boff + (int64_t)r.n0 * p.lda, (uint32_t)(rb * p.lda));
    }
    return t;
}

template <bool CH>
__device__ __forceinline__ void load_piece(uint8_t *lds, int slot, const Target &tg, int ks, int n, const Lane &c,
                                           const Params &p, const Chunk6 &cp)
{
    if (n < kLoadsOp)
        load_op<true>(lds, slot, tg.ra, ks, n, c, p.lda);
    else if (n < 2 * kLoadsOp)
        load_op<false>(lds, slot, tg.rb, ks, n - kLoadsOp, c, p.lda);
    else if constexpr (CH)
        load_scale_portion(lds, cp.pc ^ 1, cp.sa, cp.sb, cp.lchunk, cp.j, c, p.sld);
    else
        load_scales(lds, slot, tg, ks, c, p.sld);
}

template <int CA, int CB, int SEL>
__device__ __forceinline__ void mma(f32x16 &acc, const Frag6 &a, uint32_t sa, const Frag6 &b, uint32_t sb)
{
    acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(frag_op(b), frag_op(a), acc, CB, CA, SEL, (int)sb, SEL,
                                                          (int)sa);
}

// The MB x NB MFMAs of one k-step, on A fragments F.a and B fragments
// F.b[CUR], with scale op_sel SEL.  With RD, k-step rk of slot rs is read
// meanwhile: B first (into the other buffer), then each A fragment right
// after its last MFMA.  With LOADS, the wave's load pieces of stage ks go
// out one after each MFMA (the ninth after the last).
template <int CA, int CB, int SEL, int CUR, bool RD, bool LOADS, bool CH>
__device__ __forceinline__ void mfmas(f32x16 (&acc)[S::MB][S::NB], Frags6 &F, const Sc6 &sc, uint8_t *lds, int rs,
                                      int rk, int lslot, const Target &tg, int ks, const Lane &c, const Params &p,
                                      const Chunk6 &cp)
{
    if constexpr (RD) {
#pragma unroll
        for (int j = 0; j < S::NB; ++j) F.b[CUR ^ 1][j] = read_b(lds, rs, rk, j, c);
    }
#pragma unroll
    for (int i = 0; i < S::MB; ++i) {
#pragma unroll
        for (int j = 0; j < S::NB; ++j) {
            mma<CA, CB, SEL>(acc[i][j], F.a[i], sc.a[i], F.b[CUR][j], sc.b[j]);
            if constexpr (LOADS) {
                constexpr int per = S::MB * S::NB;           // 8 MFMAs, 9 loads: two after the last
                const int m = i * S::NB + j;
                DBS_FENCE();
                load_piece<CH>(lds, lslot, tg, ks, m, c, p, cp);
                if (m == per - 1) load_piece<CH>(lds, lslot, tg, ks, per, c, p, cp);
                DBS_FENCE();
            }
        }
        if constexpr (RD) {
            DBS_FENCE();
            F.a[i] = read_a(lds, rs, rk, i, c);
            DBS_FENCE();
        }
    }
}

// One stage read from slot rs while stage ks of target tg loads into the
// other slot.  On entry F holds the previous stage's last k-step (A, and B
// in buffer 1; zeros and unit scales at a tile's first stage): its MFMAs go
// first, behind the reads of this stage's scales and first k-step.
template <int CA, int CB, bool CH>
__device__ __forceinline__ void stage(f32x16 (&acc)[S::MB][S::NB], Frags6 &F, Sc6 &sprev, Sc6 &scur, uint8_t *lds,
                                      int rs, const Target &tg, int ks, const Lane &c, const Params &p,
                                      const Chunk6 &cp)
{
    if constexpr (CH)
        read_scales_chunk(scur, lds, cp.pc, cp.j, c);
    else
        read_scales(scur, lds, rs, c);
    DBS_FENCE();
    mfmas<CA, CB, 2, 1, true, true, CH>(acc, F, sprev, lds, rs, 0, rs ^ 1, tg, ks, c, p, cp);
    DBS_FENCE();
    adjust(scur, c);
    mfmas<CA, CB, 0, 0, true, false, CH>(acc, F, scur, lds, rs, 1, rs ^ 1, tg, ks, c, p, cp);
    sprev = scur;
    // this wave's loads have landed and its reads of slot rs are done; after
    // the barrier every wave's have: the next stage may read the other slot
    // and the one after it refill this one
    stage_barrier<0>();
}

}  // namespace f6

template <int CA, int CB, bool CH>
__global__ __launch_bounds__(512, 1) void gemm_mxfp6_kernel(Params p)
{
    using namespace f6;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[lds_bytes<CH>()];
    Lane c;
    const int t = threadIdx.x;
    c.lane = t & 63;
    c.h = c.lane >> 5;
    c.lr = c.lane & 31;
    c.w = __builtin_amdgcn_readfirstlane(t >> 6);
    c.wm = c.w / S::WN;
    c.wn = c.w % S::WN;
    // rows wm*128 + lr (A), wn*64 + lr (B): the swizzle of both is that of
    // row lr, ((lr % 8) ^ (lr / 8)) % 8; lane half h reads cells 2h, 2h + 1
    // of its k-step's four
    const uint32_t sw = (uint32_t)(((c.lr & 7) ^ (c.lr >> 3)) & 7);
    c.fa = (uint32_t)((c.wm * 128 + c.lr) * kRow) | ((sw << 4) ^ (uint32_t)(32 * c.h));
    c.fb = (uint32_t)(kOp + (c.wn * 64 + c.lr) * kRow) | ((sw << 4) ^ (uint32_t)(32 * c.h));
    c.r8 = (uint32_t)((c.lane >> 3) * (p.blk6 ? kGRow : p.lda));
    c.kst = (uint32_t)(p.blk6 ? 8 * kGRow : kGRow);
    c.x = (uint32_t)((c.lane & 7) ^ (c.lane >> 3));
    // chunk rows wm*128 + lr (A), TM + wn*64 + lr (B): bits 3-4 of either are those of lr
    const uint32_t s4 = (uint32_t)(4 * ((c.lr >> 3) & 3));
    c.sa = (uint32_t)(kLdsS + (c.wm * 128 + c.lr) * kChunk) | s4;
    c.sb = (uint32_t)(kLdsS + (S::TM + c.wn * 64 + c.lr) * kChunk) | s4;

    const int ntiles = p.tiles_m * p.tiles_n;
    const int nwg = gridDim.x, wg = blockIdx.x;
    int tile = (nwg & 7) == 0 ? (wg & 7) * (nwg >> 3) + (wg >> 3) : wg;
    if (tile >= ntiles) return;

    // the first stage of the first tile; the stage stream then runs one
    // stage ahead across the workgroup's tiles
    Target ld = target6(p, tile);
    Chunk6 cp{0, 0, 0, ld.rsa, ld.rsb};
    if constexpr (CH) {
#pragma unroll
        for (int n = 0; n < 2 * kLoadsOp; ++n) load_piece<CH>(lds, 0, ld, 0, n, c, p, cp);
#pragma unroll
        for (int u = 0; u < kSpc; ++u) load_scale_portion(lds, 0, cp.sa, cp.sb, 0, u, c, p.sld);
    } else {
#pragma unroll
        for (int n = 0; n < kLoads; ++n) load_piece<CH>(lds, 0, ld, 0, n, c, p, cp);
    }
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");

    Frags6 F;
    Sc6 sprev, scur;
    int rs = 0;     // slot the next stage reads
    int xs = 0;     // slot the last stage read
    for (;;) {
        f32x16 acc[S::MB][S::NB];
#pragma unroll
        for (int i = 0; i < S::MB; ++i)
#pragma unroll
            for (int j = 0; j < S::NB; ++j) acc[i][j] = f32x16{};
#pragma unroll
        for (int i = 0; i < S::MB; ++i) F.a[i] = Frag6{};
#pragma unroll
        for (int j = 0; j < S::NB; ++j) F.b[1][j] = Frag6{};
#pragma unroll
        for (int i = 0; i < S::MB; ++i) sprev.a[i] = 0x7F7F7F7Fu;
#pragma unroll
        for (int j = 0; j < S::NB; ++j) sprev.b[j] = 0x7F7F7F7Fu;

        const int next = tile + nwg;
        if constexpr (CH) {
            // the chunk stream runs one chunk ahead: the tile's last chunk
            // loads the next tile's first (cp.sa / cp.sb switch to its scale
            // rows there; ld, the operand rows, at the tile's last stage)
            const int nch = p.nk / kSpc;
            for (int s = 0; s < p.nk; ++s) {
                int ks = s + 1;
                if (ks == p.nk) {
                    ks = 0;
                    ld = next < ntiles ? target6(p, next) : null_target();
                }
                cp.j = s & (kSpc - 1);
                cp.lchunk = s / kSpc + 1;
                if (cp.lchunk == nch) {
                    cp.lchunk = 0;
                    if (cp.j == 0) {
                        const Target nt = next < ntiles ? target6(p, next) : null_target();
                        cp.sa = nt.rsa;
                        cp.sb = nt.rsb;
                    }
                }
                stage<CA, CB, CH>(acc, F, sprev, scur, lds, rs, ld, ks, c, p, cp);
                if (cp.j == kSpc - 1) cp.pc ^= 1;
                xs = rs;
                rs ^= 1;
            }
        } else {
            for (int s = 0; s < p.nk; ++s) {
                // stage s loads the next one of the stream: this tile's s + 1,
                // or the next tile's first
                int ks = s + 1;
                if (ks == p.nk) {
                    ks = 0;
                    ld = next < ntiles ? target6(p, next) : null_target();
                }
                stage<CA, CB, CH>(acc, F, sprev, scur, lds, rs, ld, ks, c, p, cp);
                xs = rs;
                rs ^= 1;
            }
        }
        // the last k-step
        mfmas<CA, CB, 2, 1, false, false, CH>(acc, F, sprev, lds, 0, 0, 0, ld, 0, c, p, cp);

        // epilogue through the slot the last stage read (refilled only by the
        // stage after the next barrier)
        Ctx<S> e;
        e.lane = c.lane;
        e.h = c.h;
        e.lr = c.lr;
        e.w = c.w;
        e.wm = c.wm;
        e.wn = c.wn;
        const TileRef tr = tile_ref<S::TM, S::TN>(tile, p);
        if (p.vec16) {
            store_tile_lds_at<S>(acc, lds + xs * kSlot + c.w * epilogue_wave_bytes<S>(), p, tr, e);
            asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        } else {
            store_tile<S>(acc, p, tr, e);
        }
        if (next >= ntiles) break;
        tile = next;
    }
}

}  // namespace

hipError_t launch_gemm_mxfp6(const Params &p0, int grid, hipStream_t stream)
{
    Params p = p0;
    p.nk = p.K / f6::kKs;
    if (p.K % f6::kKs || p.nk < 1 || !p.scales_aligned || p.lay != 0) return hipErrorInvalidValue;
    const int ca = p.ec & 7, cb = (p.ec >> 3) & 7;
    // chunked scales when every tile's stages come in whole chunks
    const bool ch = p.nk % f6::kSpc == 0;
#define DBS_F6(A_, B_) \
    case (A_) | ((B_) << 3): \
        if (ch) \
            hipLaunchKernelGGL((gemm_mxfp6_kernel<A_, B_, true>), dim3(grid), dim3(512), 0, stream, p); \
        else \
            hipLaunchKernelGGL((gemm_mxfp6_kernel<A_, B_, false>), dim3(grid), dim3(512), 0, stream, p); \
        break;
    switch (ca | (cb << 3)) {
        DBS_F6(2, 2) DBS_F6(2, 3) DBS_F6(3, 2) DBS_F6(3, 3)
    default: return hipErrorInvalidValue;
    }
#undef DBS_F6
    return hipGetLastError();
}

}  // namespace dbs
