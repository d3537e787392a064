// gemm_bf16_ea.hip -- BF16 GEMM with decoupled A and B rings and early
// release of A's stage (or, for comparison, release at the stage's end)
//
// The schedule is the one the "ThunderKittens Now on NVIDIA Vera Rubin NVL72"
// post describes among its new features (item 5): once every consumer has
// read a stage's A tile, A's slot is handed back to the loader before the
// stage's MMAs are done with B, so the next A tile gets more time to land.
// On gfx950 the MFMAs read their operands from registers, so "has read A"
// means "holds the stage's A fragments in VGPRs"; that takes 64 VGPRs per
// wave for a 64-K BF16 stage of 128 rows, which fits only beside
// accumulators kept in AGPRs, i.e. one wave per SIMD:
//
// * 256 x 256 output tiles, 4 waves of 128 x 128 (4 x 4 MFMA blocks of
//   32 x 32, v_mfma_f32_32x32x16_bf16), persistent workgroups with the
//   XCD-aware raster, the LDS-staged bf16 epilogue of the other kernels.
// * A and B each have a two-slot ring of 64-K stages (256 rows x 128 bytes,
//   the chunk swizzle and direct-to-LDS wave-loads of gemm_kernel.h).  The
//   A stream runs one stage ahead of the B stream.
// * Stage g: read A(g)'s four k-steps and B(g)'s first into registers,
//   issuing meanwhile the deferred MFMAs of stage g-1's last k-step and
//   B(g+1)'s loads; wait for the reads and meet the other waves (A's slot is
//   free now: every wave holds A(g)); issue A(g+2)'s loads into it while the
//   MFMAs of k-steps 0..2 run; then wait for A(g+1) and B(g+1) (not A(g+2))
//   and meet again (B's slot is free).  A's loads get about a stage and a
//   half to land instead of one.
// * EARLY = false is the same kernel with A's slot handed back at the
//   stage's end, as B's is: A(g+1) loads at the start of stage g, beside
//   B(g+1), into the slot stage g-1 read (as early as that slot allows), no
//   barrier between the A reads and the MFMAs, and every load of the stage
//   lands before its closing barrier.
//
// Problems this kernel takes (the host checks): K-major BF16, K % 8 == 0,
// at least two stages (K > 64).
#include "gemm_kernel.h"

namespace dbs {

namespace {
namespace ea {

using S = SquareW4;                                     // 256 x 256, 4 waves of 128 x 128
constexpr int KK = kRowBytes / Fmt<kBF16>::KSB;         // k-steps per stage: 4
constexpr int kSlot = S::TM * kRowBytes;                // 32 KiB
constexpr int kLdsA = 0, kLdsB = 2 * kSlot;
constexpr int kLds = 4 * kSlot;
constexpr int kLoads = S::QA;                           // wave-loads per wave, operand and stage: 8
static_assert(S::TM == S::TN && S::MB == 4 && S::NB == 4 && S::QA == S::QB, "square tiles, 128 x 128 per wave");
static_assert(S::NW * epilogue_wave_bytes<S>() <= kSlot, "epilogue staging fits in one B slot");
static_assert((kSlot & (kSlot - 1)) == 0 && kLdsB % (2 * kSlot) == 0, "slot offsets are OR-able");
static_assert(kLds <= 160 * 1024, "LDS budget");

struct EaFrags {
    bf16x8 a[KK][S::MB];        // the stage's A fragments, all k-steps
    bf16x8 b[2][S::NB];         // B fragments, double-buffered over k-steps
};

__device__ __forceinline__ bf16x8 rd(const uint8_t *lds, uint32_t fbase, uint32_t sel, int kk, int blk)
{
    return read_frag<kBF16>(lds, fbase, sel, kk, blk);
}

__device__ __forceinline__ void mma(f32x16 &acc, const bf16x8 &a, const bf16x8 &b)
{
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, acc, 0, 0, 0);
}

// The 16 MFMAs of one k-step on A fragments fa and B fragments fb.
__device__ __forceinline__ void mfmas(f32x16 (&acc)[S::MB][S::NB], const bf16x8 (&fa)[S::MB],
                                      const bf16x8 (&fb)[S::NB])
{
#pragma unroll
    for (int i = 0; i < S::MB; ++i)
#pragma unroll
        for (int j = 0; j < S::NB; ++j) mma(acc[i][j], fa[i], fb[j]);
}

// Wave-load q of A (IS_A) or B stage ks of the rows at `r` into ring slot
// `slot` (rows 8L .. 8L+7, L = w QA + q; see dma_op).
template <bool IS_A>
__device__ __forceinline__ void load(uint8_t *lds, int slot, __amdgpu_buffer_rsrc_t r, int ks, int q,
                                     const Ctx<S> &c, int lda)
{
    dma_op(lds, (IS_A ? kLdsA : kLdsB) + slot * kSlot, r, ks, c, c.w * kLoads + q, lda, c.r8lda);
}

}  // namespace ea

template <bool EARLY>
__global__ __launch_bounds__(256, 1) void gemm_bf16_ea_kernel(Params p)
{
    using namespace ea;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[kLds];
    Ctx<S> c;
    c.t = threadIdx.x;
    c.lane = c.t & 63;
    c.h = c.lane >> 5;
    c.lr = c.lane & 31;
    c.w = __builtin_amdgcn_readfirstlane(c.t >> 6);
    c.wm = c.w / S::WN;
    c.wn = c.w % S::WN;
    const int ra0 = c.wm * (S::TM / S::WM) + c.lr, rb0 = c.wn * (S::TN / S::WN) + c.lr;
    c.fa = (uint32_t)(kLdsA + ra0 * kRowBytes + ((c.h ^ swz(ra0)) << 4));
    c.fb = (uint32_t)(kLdsB + rb0 * kRowBytes + ((c.h ^ swz(rb0)) << 4));
    c.r8lda = (uint32_t)((c.lane >> 3) * p.lda);
    c.x4 = (uint32_t)(((c.lane & 7) ^ (c.lane >> 3)) << 4);

    const int ntiles = p.tiles_m * p.tiles_n;
    const int nwg = gridDim.x, wg = blockIdx.x;
    int tile = (nwg & 7) == 0 ? (wg & 7) * (nwg >> 3) + (wg >> 3) : wg;
    if (tile >= ntiles) return;

    // Prologue: A(0), A(1) (EARLY) and B(0) of the first tile.  The A
    // stream then runs two stages (EARLY; else one) ahead of the stage being
    // computed, the B stream one.
    Target ta = tile_target<kBF16, S>(p, tile);     // whose rows the A loads fetch
    Target tb = ta;                                  // whose rows the B loads fetch
#pragma unroll
    for (int q = 0; q < kLoads; ++q) load<true>(lds, 0, ta.ra, 0, q, c, p.lda);
    if constexpr (EARLY) {
#pragma unroll
        for (int q = 0; q < kLoads; ++q) load<true>(lds, 1, ta.ra, 1, q, c, p.lda);
    }
#pragma unroll
    for (int q = 0; q < kLoads; ++q) load<false>(lds, 0, tb.rb, 0, q, c, p.lda);
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");

    EaFrags F;
    int g = 0;          // stream stage: slots g & 1 hold A(g) and B(g)
    // the A stream: the next A loads fetch stage ka of tile ta_tile (two
    // stages past the one being computed: with two stages a tile, the next
    // tile's first)
    int ka = EARLY ? 2 : 1, ta_tile = tile;
    if (ka >= p.nk) {
        ka -= p.nk;
        ta_tile += nwg;
        ta = ta_tile < ntiles ? tile_target<kBF16, S>(p, ta_tile) : null_target();
    }
    for (;;) {
        f32x16 acc[S::MB][S::NB];
#pragma unroll
        for (int i = 0; i < S::MB; ++i)
#pragma unroll
            for (int j = 0; j < S::NB; ++j) acc[i][j] = f32x16{};
        // the deferred k-step of the stage before the tile's first: zeros
#pragma unroll
        for (int i = 0; i < S::MB; ++i) F.a[KK - 1][i] = bf16x8{};
#pragma unroll
        for (int j = 0; j < S::NB; ++j) F.b[1][j] = bf16x8{};
        const int next = tile + nwg;
        for (int s = 0; s < p.nk; ++s, ++g) {
            // per-lane bases re-declared each stage, so that nothing derived
            // from them is hoisted out of the loop into registers
            opaque(c);
            const uint32_t sel = (uint32_t)((g & 1) * kSlot);
            // B(s + 1) of this tile, or the next tile's B(0)
            int kb = s + 1;
            if (kb == p.nk) {
                kb = 0;
                tb = next < ntiles ? tile_target<kBF16, S>(p, next) : null_target();
            }
            // reads of A(s) k-steps 0..2 and B(s) k-step 0, B(s+1)'s loads,
            // then the previous stage's last k-step (its fragments are in
            // F.a[KK-1] and F.b[1]), then A(s) k-step KK-1
#pragma unroll
            for (int kk = 0; kk < KK - 1; ++kk)
#pragma unroll
                for (int i = 0; i < S::MB; ++i) F.a[kk][i] = rd(lds, c.fa, sel, kk, i);
            DBS_FENCE();
#pragma unroll
            for (int q = 0; q < kLoads; ++q) load<false>(lds, (g + 1) & 1, tb.rb, kb, q, c, p.lda);
            if constexpr (!EARLY) {
                // A(s+1) into the slot stage s-1 read, as early as that allows
#pragma unroll
                for (int q = 0; q < kLoads; ++q) load<true>(lds, (g + 1) & 1, ta.ra, ka, q, c, p.lda);
            }
            mfmas(acc, F.a[KK - 1], F.b[1]);
            DBS_FENCE();
#pragma unroll
            for (int j = 0; j < S::NB; ++j) F.b[0][j] = rd(lds, c.fb, sel, 0, j);
#pragma unroll
            for (int i = 0; i < S::MB; ++i) F.a[KK - 1][i] = rd(lds, c.fa, sel, KK - 1, i);
            // every wave holds A(s): its slot may be refilled
            DBS_FENCE();
            if constexpr (EARLY) asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
            DBS_FENCE();
            // (EARLY) A(s+2)'s loads go into the slot just released
            // k-steps 0 .. KK-2, each reading B's next k-step; A(s+2)'s
            // loads go out two per k-step
#pragma unroll
            for (int kk = 0; kk < KK - 1; ++kk) {
#pragma unroll
                for (int j = 0; j < S::NB; ++j) F.b[(kk + 1) & 1][j] = rd(lds, c.fb, sel, kk + 1, j);
#pragma unroll
                for (int i = 0; i < S::MB; ++i) {
#pragma unroll
                    for (int j = 0; j < S::NB; ++j) {
                        mma(acc[i][j], F.a[kk][i], F.b[kk & 1][j]);
                        if (EARLY && j == S::NB - 1 && (i & 1)) {
                            // wave-loads 0 .. 5 over k-steps 0 .. 2
                            DBS_FENCE();
                            load<true>(lds, g & 1, ta.ra, ka, 2 * kk + (i >> 1), c, p.lda);
                            DBS_FENCE();
                        }
                    }
                }
            }
            if constexpr (EARLY) {
#pragma unroll
                for (int q = 2 * (KK - 1); q < kLoads; ++q) load<true>(lds, g & 1, ta.ra, ka, q, c, p.lda);
            }
            // the A stream moves on, to the following tile past the last stage
            if (++ka == p.nk) {
                ka = 0;
                ta_tile += nwg;
                ta = ta_tile < ntiles ? tile_target<kBF16, S>(p, ta_tile) : null_target();
            }
            // A(s+1) and B(s+1) have landed for this wave (memory operations
            // complete in order; with EARLY A(s+2)'s kLoads stay in flight)
            // and its reads of B(s) are done; after the barrier, for every
            // wave.  At a tile's last stage the compiler may read the
            // accumulators right after the barrier (moving them between
            // registers), and it counts the barrier's inline assembly as wait
            // states it does not emit: five explicit ones keep every such read
            // at least 11 (an 8-pass MFMA's) after the last MFMA.
            DBS_FENCE();
            asm volatile("s_nop 4");
            DBS_FENCE();
            asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"i"(EARLY ? kLoads : 0) : "memory");
            DBS_FENCE();
        }
        // the last k-step
        mfmas(acc, F.a[KK - 1], F.b[1]);

        // epilogue through the B slot the last stage read: B's next loads
        // (the next tile's B(1)) go there only after the barrier below
        const TileRef tr = tile_ref<S::TM, S::TN>(tile, p);
        if (p.vec16) {
            store_tile_lds_at<S>(acc, lds + kLdsB + ((g - 1) & 1) * kSlot + c.w * epilogue_wave_bytes<S>(), p, tr, c);
            asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        } else {
            store_tile<S>(acc, p, tr, c);
        }
        if (next >= ntiles) break;
        tile = next;
    }
    // the A stream's last loads (into the ring, for tiles that do not exist:
    // they read nothing) must not be in flight when the workgroup ends
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

}  // namespace

hipError_t launch_gemm_bf16_ea(const Params &p0, bool early, int grid, hipStream_t stream)
{
    Params p = p0;
    p.nk = (p.K + 63) / 64;
    if (p.nk < 2 || p.lay != 0 || p.ngroups != 0) return hipErrorInvalidValue;
    if (early)
        hipLaunchKernelGGL(gemm_bf16_ea_kernel<true>, dim3(grid), dim3(256), 0, stream, p);
    else
        hipLaunchKernelGGL(gemm_bf16_ea_kernel<false>, dim3(grid), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace dbs
