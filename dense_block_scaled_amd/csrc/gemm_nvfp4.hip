// gemm_nvfp4.hip -- NVFP4 GEMM kernels: decoded into LDS, the raw-ring skinny kernel, and the raw-staged kernels
// (instantiations of the kernel template in gemm_kernel.h; one translation
// unit per group of formats so that the library builds in parallel)
#include "gemm_kernel.h"

namespace dbs {

namespace {

// --------------------------------------------- NVFP4, skinny tiles, raw ring

// Grouped NVFP4 on 256 x 64 tiles when K % 256 == 0 and the scale rows start
// on 16-byte boundaries (a single GEMM under these conditions runs on the
// 4-wave raw kernel of gemm_kernel.h, which measured faster).  The packed E2M1 rows and their E4M3 scales arrive by
// direct-to-LDS loads, unchanged, into a ring of kRawSlots raw slots; a raw
// stage covers 256 K elements, i.e. one 128-byte line of every packed row and
// 16 bytes of every scale row, so each row costs one memory request per
// stage.  The MFMAs run on sub-stages of 64 K elements (four per raw stage),
// software-pipelined over the 8 waves (32 x 64 of the tile each): during
// sub-stage u a wave issues the MFMAs of u from registers, reads the B
// fragments of u + 1 from the decoded-B ring, decodes its own 32 A rows of
// u + 1 straight into fp16 MFMA fragments, and decodes an eighth of B of
// u + 2 into the three-slot ring of decoded fp16 B sub-slots (exact: see
// expand8).  One barrier per sub-stage; raw stage t + 2 is loaded during raw
// stage t.
namespace nv {
using S = Shape<256, 64, 8, 1, 2>;
constexpr int kRawSlots = 3, kDecSlots = 3;
constexpr int kRawA = S::TM * 128, kRawB = S::TN * 128, kRawSA = S::TM * 16, kRawSB = S::TN * 16;
constexpr int kRaw = kRawA + kRawB + kRawSA + kRawSB;           // bytes per raw slot
constexpr int kDec = S::TN * kRowBytes;                         // decoded B sub-slot: 64 rows x 64 fp16
constexpr int kLdsDec = 0, kLdsRaw = kDecSlots * kDec;          // decoded sub-slots first (slot bits OR-able)
constexpr int kLds = kLdsRaw + kRawSlots * kRaw;
static_assert(kLds <= 160 * 1024, "LDS budget");
static_assert(kDec == S::kSlotB, "read_b addresses decoded sub-slots like B slots");

// 16-byte chunks of a 128-byte raw row: 16 consecutive rows reading the same
// logical chunk hit distinct bank groups.
__device__ __forceinline__ int swz_raw(int row) { return (row >> 1) & 7; }

// The six wave-loads of a raw stage a wave issues (k = 0..5): k < 4: A rows
// 8(w + 8k) .. +7; k = 4: B rows 8w .. 8w+7; k = 5: A scale rows 64w .. +63
// (w < 4) or the B scale rows (w >= 4; waves 5..7 repeat wave 4's load, same
// bytes to the same place).  Lane i of an operand wave-load lands on row
// 8n + i/8, physical chunk i%8, and fetches the logical chunk the raw swizzle
// puts there.  Offsets past a row's end carry the out-of-range flag (the
// whole 16 bytes are in or out: lda and sld are multiples of 16).  The
// operand of every load is known at compile time or picked by a two-way
// select, never by an index (which would put the resources in memory).
template <int K>
__device__ __forceinline__ void raw_load(uint8_t *lds, int slot, const Target &tg, int kr, const Ctx<S> &c,
                                         const Params &p)
{
    const int base = kLdsRaw + slot * kRaw;
    if constexpr (K < 5) {
        constexpr bool is_a = K < 4;
        const int nn = is_a ? c.w + 8 * K : c.w;
        const int row = 8 * nn + (c.lane >> 3);
        const int o = kr * 128 + (((c.lane & 7) ^ swz_raw(row)) << 4);
        const uint32_t off = (uint32_t)(row * p.lda + o) | (o < p.lda ? 0u : kOOB);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(is_a ? tg.ra : tg.rb,
                                                 (lds_void *)(lds + base + (is_a ? 0 : kRawA) + nn * 1024), 16, off, 0,
                                                 0, 0);
    } else {
        const bool is_a = c.w < 4;
        const int nn = is_a ? c.w : 0;
        const int o = kr * 16;
        const uint32_t off = (uint32_t)((64 * nn + c.lane) * p.sld + o) | (o < p.sld ? 0u : kOOB);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(is_a ? tg.rsa : tg.rsb,
                                                 (lds_void *)(lds + base + kRawA + kRawB + (is_a ? 0 : kRawSA) + nn * 1024),
                                                 16, off, 0, 0, 0);
    }
}
static_assert(kRawA / 1024 == 4 * S::NW && kRawB / 1024 == S::NW && kRawSA / 1024 == 4 && kRawSB / 1024 == 1,
              "raw_load's split of a raw stage over the waves");

// The wave's loads K0 .. K1-1 of raw stage kr.
template <int K0, int K1>
__device__ __forceinline__ void raw_pieces(uint8_t *lds, int slot, const Target &tg, int kr, const Ctx<S> &c,
                                           const Params &p)
{
    if constexpr (K0 < K1) {
        raw_load<K0>(lds, slot, tg, kr, c, p);
        raw_pieces<K0 + 1, K1>(lds, slot, tg, kr, c, p);
    }
}

// Raw bytes of one sub-stage a thread decodes: the 16 packed bytes and two
// scale bytes of its A row half (lane half h takes elements [32h, 32h+32) of
// the sub-stage; k-step kk uses 32h + 8kk .. +7, and B's decoded fragments
// follow the same permutation of K, see adirect), and one packed dword and
// scale byte of its B unit (row t/8, elements 8(t%8) .. +7).
struct RawA {
    i32x4 v;
    uint32_t sc;
};
struct RawB {
    uint32_t v, sc;
};

__device__ __forceinline__ void read_raw_a(RawA &r, const uint8_t *lds, int slot, int u, const Ctx<S> &c)
{
    const int base = kLdsRaw + slot * kRaw;
    const int row = c.w * 32 + c.lr;
    const int lc = 2 * u + c.h;
    r.v = lds_read<i32x4>(lds, (uint32_t)(base + row * 128 + ((lc ^ swz_raw(row)) << 4)));
    r.sc = lds_read<uint16_t>(lds, (uint32_t)(base + kRawA + kRawB + row * 16 + 4 * u + 2 * c.h));
}

__device__ __forceinline__ void read_raw_b(RawB &r, const uint8_t *lds, int slot, int u, const Ctx<S> &c)
{
    const int base = kLdsRaw + slot * kRaw;
    const int row = c.t >> 3, c8 = c.t & 7;
    const int lc = 2 * u + (c8 >> 2);
    r.v = lds_read<uint32_t>(lds, (uint32_t)(base + kRawA + row * 128 + ((lc ^ swz_raw(row)) << 4) + 4 * (c8 & 3)));
    r.sc = lds_read<uint8_t>(lds, (uint32_t)(base + kRawA + kRawB + kRawSA + row * 16 + 4 * u + (c8 >> 1)));
}

__device__ __forceinline__ void decode_a(f16x8 (&a)[4], const RawA &r)
{
    const f16x2 s2 = e4m3_two(r.sc);
    const f16x2 lo = {s2[0], s2[0]}, hi = {s2[1], s2[1]};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) a[kk] = __builtin_bit_cast(f16x8, expand8((uint32_t)r.v[kk], kk < 2 ? lo : hi));
}

__device__ __forceinline__ void decode_b(uint8_t *lds, const RawB &r, int ds, const Ctx<S> &c)
{
    const int row = c.t >> 3, c8 = c.t & 7;
    const f16x2 s2 = e4m3_two(r.sc);
    *reinterpret_cast<i32x4 *>(lds + kLdsDec + ds * kDec + lds_off(row, c8)) = expand8(r.v, f16x2{s2[0], s2[0]});
}

// B fragments of a sub-stage from decoded sub-slot ds.
__device__ __forceinline__ void read_bfrags(Frags<kNVFP4, S> (&b)[4], const uint8_t *lds, int ds, const Ctx<S> &c)
{
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        read_b(b[kk], 0, lds, ds, kk, c);
        read_b(b[kk], 1, lds, ds, kk, c);
    }
}

template <int NEWER>
__device__ __forceinline__ void sub_barrier()
{
    DBS_FENCE();
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"i"(NEWER) : "memory");
    DBS_FENCE();
}

// Sub-stage U of raw stage t (raw slot `slot`; raw stage t + 1 in `nslot`),
// with d = the sub-stage's index mod 3: MFMAs on (acur, bcur); B fragments
// of the next sub-stage (decoded sub-slot d + 1) into bnext; decode of the
// wave's A rows of the next sub-stage (from racur, read one sub-stage
// earlier) into anext, and of the thread's B unit two sub-stages ahead (from
// rbcur) into decoded sub-slot d + 2; raw reads for the decodes of the next
// sub-stage (A two ahead into ranext, B three ahead into rbnext); the wave's
// loads of raw stage t + 2 (three in each of the first two sub-stages; target
// tg, tile-relative kr2) into raw slot `lslot`.  Raw stage t + 1 is first
// read in sub-stage 1: the barrier closing sub-stage 0 waits for every load
// but the three issued since.
template <int U>
__device__ __forceinline__ void sub_stage(f32x16 (&acc)[1][2], const f16x8 (&acur)[4], f16x8 (&anext)[4],
                                          const Frags<kNVFP4, S> (&bcur)[4], Frags<kNVFP4, S> (&bnext)[4],
                                          const RawA &racur, RawA &ranext, const RawB &rbcur, RawB &rbnext,
                                          uint8_t *lds, int slot, int nslot, int lslot, int d, const Target &tg,
                                          int kr2, const Ctx<S> &c, const Params &p)
{
    const int d1 = d == 2 ? 0 : d + 1, d2 = d1 == 2 ? 0 : d1 + 1;
    read_bfrags(bnext, lds, d1, c);
    if constexpr (U == 0) raw_pieces<0, 3>(lds, lslot, tg, kr2, c, p);
    if constexpr (U == 1) raw_pieces<3, 6>(lds, lslot, tg, kr2, c, p);
    read_raw_a(ranext, lds, U >= 2 ? nslot : slot, (U + 2) & 3, c);
    read_raw_b(rbnext, lds, U >= 1 ? nslot : slot, (U + 3) & 3, c);
    decode_a(anext, racur);
    decode_b(lds, rbcur, d2, c);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bcur[kk].b[0], acur[kk], acc[0][0], 0, 0, 0);
        acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bcur[kk].b[1], acur[kk], acc[0][1], 0, 0, 0);
    }
    if constexpr (U == 0)
        sub_barrier<3>();
    else
        sub_barrier<63>();
}
}  // namespace nv

__global__ __launch_bounds__(512, 1) void gemm_nvfp4_raw_kernel(Params p)
{
    using S = nv::S;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[nv::kLds];
    Ctx<S> c;
    c.t = threadIdx.x;
    c.lane = c.t & 63;
    c.h = c.lane >> 5;
    c.lr = c.lane & 31;
    c.w = __builtin_amdgcn_readfirstlane(c.t >> 6);
    c.wm = c.w;
    c.wn = 0;
    // decoded B fragments: rows lr (+32), chunk 4h + kk (see adirect)
    c.fa = 0;
    c.fb = (uint32_t)(nv::kLdsDec + c.lr * kRowBytes + (((4 * c.h) ^ swz(c.lr)) << 4));
    c.sa = c.sb = 0;
    c.r8lda = 0;
    c.x4 = 0;

    const int ntiles = p.tiles_m * p.tiles_n;
    const int nwg = gridDim.x, wg = blockIdx.x;
    int tile = (nwg & 7) == 0 ? (wg & 7) * (nwg >> 3) + (wg >> 3) : wg;
    if (tile >= ntiles) return;

    // raw stages of a tile: p.nk >= 2 (the host checks); the streams of raw
    // stages and sub-stages run across the workgroup's tiles
    Target ld = tile_target<kNVFP4, S>(p, tile);
    nv::raw_pieces<0, 6>(lds, 0, ld, 0, c, p);
    nv::raw_pieces<0, 6>(lds, 1, ld, 1, c, p);
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    // fill the pipeline: A of sub-stage 0 decoded, B of sub-stages 0 and 1
    // decoded (sub-slots 0, 1) and B of 0 read; raw bytes of A of 1 and of B
    // of 2 in registers
    f16x8 a0[4], a1[4];
    Frags<kNVFP4, S> b0[4], b1[4];
    nv::RawA ra0, ra1;
    nv::RawB rb0, rb1;
    nv::read_raw_a(ra0, lds, 0, 0, c);
    nv::decode_a(a0, ra0);
    nv::read_raw_b(rb0, lds, 0, 0, c);
    nv::decode_b(lds, rb0, 0, c);
    nv::read_raw_b(rb0, lds, 0, 1, c);
    nv::decode_b(lds, rb0, 1, c);
    nv::read_raw_a(ra0, lds, 0, 1, c);
    nv::read_raw_b(rb0, lds, 0, 2, c);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    nv::read_bfrags(b0, lds, 0, c);

    int rs = 0;      // raw slot of the raw stage being computed
    int d = 0;       // sub-stage index mod 3 (decoded-B ring)
    for (;;) {
        f32x16 acc[1][2];
        acc[0][0] = f32x16{};
        acc[0][1] = f32x16{};
        const int next = tile + nwg;
        for (int t = 0; t < p.nk; ++t) {
            int kr2 = t + 2;
            if (kr2 >= p.nk) {
                kr2 -= p.nk;
                if (kr2 == 0) ld = next < ntiles ? tile_target<kNVFP4, S>(p, next) : null_target();
            }
            const int ns = rs == nv::kRawSlots - 1 ? 0 : rs + 1;
            const int ls = ns == nv::kRawSlots - 1 ? 0 : ns + 1;
            const int d1 = d == 2 ? 0 : d + 1, d2 = d1 == 2 ? 0 : d1 + 1;   // d + 1, d + 2 (mod 3); d + 3 = d
            nv::sub_stage<0>(acc, a0, a1, b0, b1, ra0, ra1, rb0, rb1, lds, rs, ns, ls, d, ld, kr2, c, p);
            nv::sub_stage<1>(acc, a1, a0, b1, b0, ra1, ra0, rb1, rb0, lds, rs, ns, ls, d1, ld, kr2, c, p);
            nv::sub_stage<2>(acc, a0, a1, b0, b1, ra0, ra1, rb0, rb1, lds, rs, ns, ls, d2, ld, kr2, c, p);
            nv::sub_stage<3>(acc, a1, a0, b1, b0, ra1, ra0, rb1, rb0, lds, rs, ns, ls, d, ld, kr2, c, p);
            d = d1;      // four sub-stages advance the index by 4 = 1 (mod 3)
            rs = ns;
        }
        store_tile<S>(acc, p, tile_ref<S::TM, S::TN>(tile, p), c);
        // the raw-stage waits count loads; keep the stores out of them
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        if (next >= ntiles) break;
        tile = next;
    }
}

}  // namespace

hipError_t launch_nvfp4_ring(const Params &p, int grid, hipStream_t stream)
{
    Params q = p;
    q.nk = p.K / 256;
    hipLaunchKernelGGL(gemm_nvfp4_raw_kernel, dim3(grid), dim3(nv::S::kThreads), 0, stream, q);
    return hipGetLastError();
}

hipError_t launch_gemm_nvfp4(int shape, const Params &p, int grid, hipStream_t stream)
{
    return by_shape(shape, [&](auto s) { return launch_fmt<kNVFP4, decltype(s)>(p, grid, stream); });
}

hipError_t launch_gemm_nvfp4_raw(int shape, const Params &p, int grid, hipStream_t stream)
{
    return by_shape(shape, [&](auto s) { return launch_nvfp4_raw<decltype(s)>(p, grid, stream); });
}
}  // namespace dbs
