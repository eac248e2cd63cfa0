// decode_wide.hip -- paged MLA decode for 128-row query tiles (h_q * s_q of
// 48 rows or more), where QK^T and PV are dense enough to be MFMA-bound.
//
// Same operation as decode.hip: softmax(scale * Q K^T) V per query row over
// the 64-token paged latent cache (FlashMLA, "DeepSeek publica FlashMLA como
// codigo abierto", release bullets), K = the 576-wide row, V its first 512
// dims.  Here one workgroup carries 128 query rows over a scheduler part, so
// every cache byte it stages feeds 128 rows of MFMA work.
//
// gfx950 mapping:
//  * 4 waves; wave w owns query rows [32w, 32w + 32) of the tile over all
//    512 value dims (O^T: 16 blocks of 32x32 fp32 = 256 accumulator
//    registers) and keeps its Q^T fragments in registers (36 k-steps of 16
//    dims), so no cross-wave merge is ever needed.  When h_q * s_q is not a
//    multiple of 128 the last tile is partly empty: a wave without rows only
//    fetches its share of each tile, rows past the end read zero queries and
//    are not written.  The cache is still streamed once per 128 rows, which
//    beats one pass per 16-row tile from 48 rows on.
//  * The cache streams through LDS in 32-token tiles (36,864 B) held in four
//    stages: while tile t is multiplied by Q, tile t - 1 is still read for
//    the value product and tiles t + 1, t + 2 are in flight.  Tiles arrive by
//    direct global->LDS DMA (buffer_load ... lds, 16 B per lane); tokens
//    outside the part read as zeros through the buffer descriptor's range
//    check.  A tile never crosses a page (tiles are 32-token aligned).  The
//    LDS layout of a tile (blocks of 8 rows x 8 chunks, swizzled) is the one
//    in tile_layout.h; wave w fetches row group w.  Page numbers come from a
//    64-entry window of the block table held one per lane.
//  * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (A = K from LDS with
//    ds_read_b128, B = Q^T from registers).  Its accumulator layout holds 16
//    keys of one query row per lane, which is directly the P^T operand of the
//    value product (keys mapped consistently on both sides).
//  * O^T += V^T P^T on the same MFMA; V^T fragments come from LDS through
//    ds_read_b64_tr_b16 (two 4-key reads per 8-key operand).
//  * Software pipeline, one wave per SIMD: iteration t issues the QK^T chain
//    of tile t with the DMA of tile t + 2 threaded through it, then the
//    softmax of tile t interleaved with the value product of tile t - 1, so
//    the matrix pipe has independent work while the wave does vector math.
//  * Online softmax in fp32, log2 domain, with an exact sum (lse) and one
//    over the weights as fed.  Each weight goes to the value product as two
//    bf16 terms, its rounding and the rounding residual (exact in fp32), on
//    two MFMAs over the same V^T fragment, so the product sees it to about
//    2^-16 relative; one term (2^-8) lets rows whose weight sits on a few
//    keys with far-apart value rows miss 1e-2.  The second term doubles the
//    value MFMAs (68 -> 100 per wave and tile).  O is never rescaled inside the tile loop (it lives in
//    the 256 accumulator registers, and any VALU rescale would force copies
//    of all of them through VGPRs): a row's first visible key sets its
//    exponent origin, and if a later score exceeds the origin by more than
//    64 (weights stay below 2^64, far from fp32 overflow) the workgroup
//    redoes the segment once, with each row's maximum score over the segment
//    as its origin, which no score can exceed: at most two passes.  Real
//    attention scores never grow like that after the first key, so the redo
//    is a correctness path.
//  * Results go out as bf16 rows (a sequence the schedule did not cut) or
//    fp32 partials with their lse.  Lane swaps 32 and 16 lanes apart first
//    gather four lanes per output row, so a store instruction writes 16 rows
//    x 64 contiguous bytes rather than 32 rows x 16 or 32.
//
// The QK^T chains and the DMA are inline assembly (below); everything they
// touch is passed as operands, M0 -- which the LDS DMA takes its
// destination from -- is set inside each block before use (no other code in
// this kernel uses M0), and the blocks that add scalar offsets declare SCC
// clobbered.  The cache DMA is marked non-temporal (nt): each cache row is
// read once per row tile, and streaming it past the caches leaves them to
// the split partials the merge reads back right after the call.
#include "mla_device.h"
#include "kernels.h"
#include "stamps.h"
#include "tile_layout.h"

namespace mla {

constexpr int kWWaves = 4;
constexpr int kWThreads = kWWaves * 64;
constexpr int kWRows = 32 * kWWaves;                 // 128 query rows per workgroup
static_assert(kWRows == kWideRows, "row tile of the wide kernel");
constexpr int kStages = 4;
constexpr int kKSteps = kDqk / 16;                   // 36
constexpr int kDBlocks = kDv / 32;                   // 16
constexpr float kWOriginSlack = 64.0f;   // log2 units
constexpr int kPvAhead = 2;              // value fragments (pairs of reads) read ahead

#if MLA_STAMPS
// Instrumented build only: the record buffer of stamps.h, or null.
__device__ uint64_t *g_stamps_wide;
hipError_t set_stamps_wide(uint64_t *buf)
{
    return hipMemcpyToSymbol(HIP_SYMBOL(g_stamps_wide), &buf, sizeof(buf));
}
#endif

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// One wave's DMA of one tile: rows 8 wave .. 8 wave + 7, all 72 chunks, as
// nine 1 KB blocks.  Lane l fetches row 8 wave + l / 8, chunk
// 8 j + ((l % 8) ^ swz(row)) into block position l of block j.
struct TileDma {
    u32x4_t rsrc;   // buffer descriptor of the tile's page
    int voff;       // lane's byte offset in the page (0x40000000 = outside: zeros)
    int soff;       // page offset of this wave's row group
    int m0;         // LDS address of this wave's block of chunk group 0
};

__device__ __forceinline__ TileDma tile_dma(const uint16_t *kv, int page, int T, int kbeg,
                                            int kend, int wave, int trow, int lane_off,
                                            int stage_addr)
{
    const uint64_t base = reinterpret_cast<uint64_t>(kv) + (uint64_t)page * kPageBytes;
    TileDma a;
    a.rsrc = u32x4_t{(uint32_t)base, (uint32_t)(base >> 32) & 0xFFFFu, (uint32_t)kPageBytes,
                     0x00020000u};
    const int key = T * kTileKeys + trow;
    a.voff = (key >= kbeg && key < kend) ? lane_off : 0x40000000;
    a.soff = ((T & 1) * kTileKeys + 8 * wave) * kRowBytes;
    a.m0 = stage_addr + 1024 * wave;
    return a;
}

__device__ __forceinline__ void dma_issue(const TileDma &a)
{
    int tmp;
    asm volatile(
        "s_mov_b32 m0, %4\n"
        "s_nop 0\n"
        "buffer_load_dwordx4 %2, %1, %3 offen nt lds\n"
        "s_add_u32 m0, %4, 4096\n"
        "s_add_u32 %0, %3, 128\n"
        "s_nop 0\n"
        "buffer_load_dwordx4 %2, %1, %0 offen nt lds\n"
        "s_add_u32 m0, %4, 8192\n"
        "s_add_u32 %0, %3, 256\n"
        "s_nop 0\n"
        "buffer_load_dwordx4 %2, %1, %0 offen nt lds\n"
        "s_add_u32 m0, %4, 12288\n"
        "s_add_u32 %0, %3, 384\n"
        "s_nop 0\n"
        "buffer_load_dwordx4 %2, %1, %0 offen nt lds\n"
        "s_add_u32 m0, %4, 16384\n"
        "s_add_u32 %0, %3, 512\n"
        "s_nop 0\n"
        "buffer_load_dwordx4 %2, %1, %0 offen nt lds\n"
        "s_add_u32 m0, %4, 20480\n"
        "s_add_u32 %0, %3, 640\n"
        "s_nop 0\n"
        "buffer_load_dwordx4 %2, %1, %0 offen nt lds\n"
        "s_add_u32 m0, %4, 24576\n"
        "s_add_u32 %0, %3, 768\n"
        "s_nop 0\n"
        "buffer_load_dwordx4 %2, %1, %0 offen nt lds\n"
        "s_add_u32 m0, %4, 28672\n"
        "s_add_u32 %0, %3, 896\n"
        "s_nop 0\n"
        "buffer_load_dwordx4 %2, %1, %0 offen nt lds\n"
        "s_add_u32 m0, %4, 32768\n"
        "s_add_u32 %0, %3, 1024\n"
        "s_nop 0\n"
        "buffer_load_dwordx4 %2, %1, %0 offen nt lds\n"
        : "=&s"(tmp)
        : "s"(a.rsrc), "v"(a.voff), "s"(a.soff), "s"(a.m0)
        : "memory", "scc");
}

// S^T[32 keys][32 rows] = K Q^T over the 576 dims of one 32-token tile: 36
// v_mfma_f32_32x32x16_bf16 with A = K rows from LDS (ds_read_b128, four in
// flight; k-step kk reads kb[kk % 4] + 4096 (kk / 4)) and B = Q^T from
// registers.  The chain is written out here so that its accumulator lives
// in VGPRs while the value accumulators occupy all 256 AGPRs.  Hazards the
// compiler cannot see inside the block are covered in it: each MFMA waits
// for its own K fragment (LDS returns in order; earlier outstanding LDS or
// scalar loads only make the counts stricter), chained MFMAs accumulate
// into exactly the same registers (forwarded back to back), a DMA waits one
// state after writing M0 (its immediate offset stays 0: on an LDS DMA it
// would move the LDS destination too), and 24 wait states after the last MFMA cover the
// longest XDL-write -> VALU-access requirement (12 on gfx950) before the
// caller reads S.  The DMA variant threads the next tile's nine DMA
// instructions through the chain so their issue overlaps the matrix work.
#define MLA_QF(i) "v"(qf[i])
__device__ __forceinline__ void qk_tile(f32x16_t &s, const int kb[4], const bf16x8_t qf[kKSteps])
{
    bf16x8_t k0, k1, k2, k3;
    asm volatile(
        "ds_read_b128 %1, %5\n"
        "ds_read_b128 %2, %6\n"
        "ds_read_b128 %3, %7\n"
        "ds_read_b128 %4, %8\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %1, %9, 0\n"
        "ds_read_b128 %1, %5 offset:4096\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %2, %10, %0\n"
        "ds_read_b128 %2, %6 offset:4096\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %3, %11, %0\n"
        "ds_read_b128 %3, %7 offset:4096\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %4, %12, %0\n"
        "ds_read_b128 %4, %8 offset:4096\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %1, %13, %0\n"
        "ds_read_b128 %1, %5 offset:8192\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %2, %14, %0\n"
        "ds_read_b128 %2, %6 offset:8192\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %3, %15, %0\n"
        "ds_read_b128 %3, %7 offset:8192\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %4, %16, %0\n"
        "ds_read_b128 %4, %8 offset:8192\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %1, %17, %0\n"
        "ds_read_b128 %1, %5 offset:12288\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %2, %18, %0\n"
        "ds_read_b128 %2, %6 offset:12288\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %3, %19, %0\n"
        "ds_read_b128 %3, %7 offset:12288\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %4, %20, %0\n"
        "ds_read_b128 %4, %8 offset:12288\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %1, %21, %0\n"
        "ds_read_b128 %1, %5 offset:16384\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %2, %22, %0\n"
        "ds_read_b128 %2, %6 offset:16384\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %3, %23, %0\n"
        "ds_read_b128 %3, %7 offset:16384\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %4, %24, %0\n"
        "ds_read_b128 %4, %8 offset:16384\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %1, %25, %0\n"
        "ds_read_b128 %1, %5 offset:20480\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %2, %26, %0\n"
        "ds_read_b128 %2, %6 offset:20480\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %3, %27, %0\n"
        "ds_read_b128 %3, %7 offset:20480\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %4, %28, %0\n"
        "ds_read_b128 %4, %8 offset:20480\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %1, %29, %0\n"
        "ds_read_b128 %1, %5 offset:24576\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %2, %30, %0\n"
        "ds_read_b128 %2, %6 offset:24576\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %3, %31, %0\n"
        "ds_read_b128 %3, %7 offset:24576\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %4, %32, %0\n"
        "ds_read_b128 %4, %8 offset:24576\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %1, %33, %0\n"
        "ds_read_b128 %1, %5 offset:28672\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %2, %34, %0\n"
        "ds_read_b128 %2, %6 offset:28672\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %3, %35, %0\n"
        "ds_read_b128 %3, %7 offset:28672\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %4, %36, %0\n"
        "ds_read_b128 %4, %8 offset:28672\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %1, %37, %0\n"
        "ds_read_b128 %1, %5 offset:32768\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %2, %38, %0\n"
        "ds_read_b128 %2, %6 offset:32768\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %3, %39, %0\n"
        "ds_read_b128 %3, %7 offset:32768\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %4, %40, %0\n"
        "ds_read_b128 %4, %8 offset:32768\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %1, %41, %0\n"
        "s_waitcnt lgkmcnt(2)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %2, %42, %0\n"
        "s_waitcnt lgkmcnt(1)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %3, %43, %0\n"
        "s_waitcnt lgkmcnt(0)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %4, %44, %0\n"
        "s_nop 7\n"
        "s_nop 7\n"
        "s_nop 7\n"
        : "=&v"(s), "=&v"(k0), "=&v"(k1), "=&v"(k2), "=&v"(k3)
        : "v"(kb[0]), "v"(kb[1]), "v"(kb[2]), "v"(kb[3]),
          MLA_QF(0), MLA_QF(1), MLA_QF(2), MLA_QF(3), MLA_QF(4), MLA_QF(5), MLA_QF(6),
          MLA_QF(7), MLA_QF(8), MLA_QF(9), MLA_QF(10), MLA_QF(11), MLA_QF(12), MLA_QF(13),
          MLA_QF(14), MLA_QF(15), MLA_QF(16), MLA_QF(17), MLA_QF(18), MLA_QF(19), MLA_QF(20),
          MLA_QF(21), MLA_QF(22), MLA_QF(23), MLA_QF(24), MLA_QF(25), MLA_QF(26), MLA_QF(27),
          MLA_QF(28), MLA_QF(29), MLA_QF(30), MLA_QF(31), MLA_QF(32), MLA_QF(33), MLA_QF(34),
          MLA_QF(35)
        : "memory");
}

__device__ __forceinline__ void qk_tile_dma(f32x16_t &s, const int kb[4],
                                            const bf16x8_t qf[kKSteps], const TileDma &a)
{
    bf16x8_t k0, k1, k2, k3;
    int tmp;
    asm volatile(
        "ds_read_b128 %1, %6\n"
        "ds_read_b128 %2, %7\n"
        "ds_read_b128 %3, %8\n"
        "ds_read_b128 %4, %9\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %1, %10, 0\n"
        "ds_read_b128 %1, %6 offset:4096\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %2, %11, %0\n"
        "ds_read_b128 %2, %7 offset:4096\n"
        "s_mov_b32 m0, %49\n"
        "s_nop 0\n"
        "buffer_load_dwordx4 %47, %46, %48 offen nt lds\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %3, %12, %0\n"
        "ds_read_b128 %3, %8 offset:4096\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %4, %13, %0\n"
        "ds_read_b128 %4, %9 offset:4096\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %1, %14, %0\n"
        "ds_read_b128 %1, %6 offset:8192\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %2, %15, %0\n"
        "ds_read_b128 %2, %7 offset:8192\n"
        "s_add_u32 m0, %49, 4096\n"
        "s_add_u32 %5, %48, 128\n"
        "s_nop 0\n"
        "buffer_load_dwordx4 %47, %46, %5 offen nt lds\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %3, %16, %0\n"
        "ds_read_b128 %3, %8 offset:8192\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %4, %17, %0\n"
        "ds_read_b128 %4, %9 offset:8192\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %1, %18, %0\n"
        "ds_read_b128 %1, %6 offset:12288\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %2, %19, %0\n"
        "ds_read_b128 %2, %7 offset:12288\n"
        "s_add_u32 m0, %49, 8192\n"
        "s_add_u32 %5, %48, 256\n"
        "s_nop 0\n"
        "buffer_load_dwordx4 %47, %46, %5 offen nt lds\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %3, %20, %0\n"
        "ds_read_b128 %3, %8 offset:12288\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %4, %21, %0\n"
        "ds_read_b128 %4, %9 offset:12288\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %1, %22, %0\n"
        "ds_read_b128 %1, %6 offset:16384\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %2, %23, %0\n"
        "ds_read_b128 %2, %7 offset:16384\n"
        "s_add_u32 m0, %49, 12288\n"
        "s_add_u32 %5, %48, 384\n"
        "s_nop 0\n"
        "buffer_load_dwordx4 %47, %46, %5 offen nt lds\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %3, %24, %0\n"
        "ds_read_b128 %3, %8 offset:16384\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %4, %25, %0\n"
        "ds_read_b128 %4, %9 offset:16384\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %1, %26, %0\n"
        "ds_read_b128 %1, %6 offset:20480\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %2, %27, %0\n"
        "ds_read_b128 %2, %7 offset:20480\n"
        "s_add_u32 m0, %49, 16384\n"
        "s_add_u32 %5, %48, 512\n"
        "s_nop 0\n"
        "buffer_load_dwordx4 %47, %46, %5 offen nt lds\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %3, %28, %0\n"
        "ds_read_b128 %3, %8 offset:20480\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %4, %29, %0\n"
        "ds_read_b128 %4, %9 offset:20480\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %1, %30, %0\n"
        "ds_read_b128 %1, %6 offset:24576\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %2, %31, %0\n"
        "ds_read_b128 %2, %7 offset:24576\n"
        "s_add_u32 m0, %49, 20480\n"
        "s_add_u32 %5, %48, 640\n"
        "s_nop 0\n"
        "buffer_load_dwordx4 %47, %46, %5 offen nt lds\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %3, %32, %0\n"
        "ds_read_b128 %3, %8 offset:24576\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %4, %33, %0\n"
        "ds_read_b128 %4, %9 offset:24576\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %1, %34, %0\n"
        "ds_read_b128 %1, %6 offset:28672\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %2, %35, %0\n"
        "ds_read_b128 %2, %7 offset:28672\n"
        "s_add_u32 m0, %49, 24576\n"
        "s_add_u32 %5, %48, 768\n"
        "s_nop 0\n"
        "buffer_load_dwordx4 %47, %46, %5 offen nt lds\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %3, %36, %0\n"
        "ds_read_b128 %3, %8 offset:28672\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %4, %37, %0\n"
        "ds_read_b128 %4, %9 offset:28672\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %1, %38, %0\n"
        "ds_read_b128 %1, %6 offset:32768\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %2, %39, %0\n"
        "ds_read_b128 %2, %7 offset:32768\n"
        "s_add_u32 m0, %49, 28672\n"
        "s_add_u32 %5, %48, 896\n"
        "s_nop 0\n"
        "buffer_load_dwordx4 %47, %46, %5 offen nt lds\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %3, %40, %0\n"
        "ds_read_b128 %3, %8 offset:32768\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %4, %41, %0\n"
        "ds_read_b128 %4, %9 offset:32768\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %1, %42, %0\n"
        "s_waitcnt lgkmcnt(2)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %2, %43, %0\n"
        "s_add_u32 m0, %49, 32768\n"
        "s_add_u32 %5, %48, 1024\n"
        "s_nop 0\n"
        "buffer_load_dwordx4 %47, %46, %5 offen nt lds\n"
        "s_waitcnt lgkmcnt(1)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %3, %44, %0\n"
        "s_waitcnt lgkmcnt(0)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %4, %45, %0\n"
        "s_nop 7\n"
        "s_nop 7\n"
        "s_nop 7\n"
        : "=&v"(s), "=&v"(k0), "=&v"(k1), "=&v"(k2), "=&v"(k3), "=&s"(tmp)
        : "v"(kb[0]), "v"(kb[1]), "v"(kb[2]), "v"(kb[3]),
          MLA_QF(0), MLA_QF(1), MLA_QF(2), MLA_QF(3), MLA_QF(4), MLA_QF(5), MLA_QF(6),
          MLA_QF(7), MLA_QF(8), MLA_QF(9), MLA_QF(10), MLA_QF(11), MLA_QF(12), MLA_QF(13),
          MLA_QF(14), MLA_QF(15), MLA_QF(16), MLA_QF(17), MLA_QF(18), MLA_QF(19), MLA_QF(20),
          MLA_QF(21), MLA_QF(22), MLA_QF(23), MLA_QF(24), MLA_QF(25), MLA_QF(26), MLA_QF(27),
          MLA_QF(28), MLA_QF(29), MLA_QF(30), MLA_QF(31), MLA_QF(32), MLA_QF(33), MLA_QF(34),
          MLA_QF(35),
          "s"(a.rsrc), "v"(a.voff), "s"(a.soff), "s"(a.m0)
        : "memory", "scc");
}
#undef MLA_QF

// Value-product step j (of 32): dim block and k-step, ordered so consecutive
// steps accumulate into different blocks
__device__ __forceinline__ constexpr int pv_block(int j) { return 2 * (j >> 2) + (j & 1); }
__device__ __forceinline__ constexpr int pv_kstep(int j) { return (j >> 1) & 1; }
// the two 4-key transposed reads of (dim block d, k-step kk)
__device__ __forceinline__ void pv_read(const int vb[2][2], int d, int kk, i16x4_t &lo, i16x4_t &hi)
{
    const int off = 2048 * kk + 4096 * (d >> 1);
    lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (i16x4_t __attribute__((address_space(3))) *)(uintptr_t)(vb[0][d & 1] + off));
    hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (i16x4_t __attribute__((address_space(3))) *)(uintptr_t)(vb[1][d & 1] + off));
}

// O^T[dims][32 rows] += V^T P^T for one tile, each weight as two terms
// (pf + rf), over kBlocks dim blocks of 32: 4 kBlocks MFMAs, V^T fragments
// of (dim block d, k-step kk) at vb[read][d % 2] + 2048 kk + 4096 (d / 2)
// (keys 16 apart are two row groups apart with the same swizzle; a wave
// that starts at a later dim block has that offset in vb)
template <int kBlocks>
__device__ __forceinline__ void pv_tile(f32x16_t o[kBlocks], const int vb[2][2], bf16x8_t pf0,
                                        bf16x8_t pf1, bf16x8_t rf0, bf16x8_t rf1)
{
    i16x4_t vlo[kPvAhead], vhi[kPvAhead];
#pragma unroll
    for (int j = 0; j < kPvAhead; ++j) {
        const int d = j >> 1, kk = j & 1, off = 2048 * kk + 4096 * (d >> 1);
        vlo[j] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (i16x4_t __attribute__((address_space(3))) *)(uintptr_t)(vb[0][d & 1] + off));
        vhi[j] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (i16x4_t __attribute__((address_space(3))) *)(uintptr_t)(vb[1][d & 1] + off));
    }
#pragma unroll
    for (int j = 0; j < 2 * kBlocks; ++j) {
        const int lb = j >> 1, kk = j & 1;
        const i16x4_t lo = vlo[j % kPvAhead], hi = vhi[j % kPvAhead];
        const i16x8_t a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        o[lb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                        kk ? pf1 : pf0, o[lb], 0, 0, 0);
        o[lb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                        kk ? rf1 : rf0, o[lb], 0, 0, 0);
        const int nj = j + kPvAhead;
        if (nj < 2 * kBlocks) {
            const int nd = nj >> 1, nkk = nj & 1, off = 2048 * nkk + 4096 * (nd >> 1);
            vlo[j % kPvAhead] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (i16x4_t __attribute__((address_space(3))) *)(uintptr_t)(vb[0][nd & 1] + off));
            vhi[j % kPvAhead] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (i16x4_t __attribute__((address_space(3))) *)(uintptr_t)(vb[1][nd & 1] + off));
        }
    }
}

struct WideRow {
    float m;    // exponent origin (log2 units), -inf before the first visible key
    float l;    // this lane's share of sum 2^(s - m) (gives the lse)
    float lr;   // the same over the weights as fed (normalizes the output)
};

// the value of x in the other half of the wave (lane ^ 32), summed or maxed
__device__ __forceinline__ float half_max(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// kQuad = false: wave w owns query rows [32 w, 32 w + 32) of a 128-row tile
// over all 512 value dims.  kQuad = true: a 32-row tile whose rows all four
// waves share, wave w owning value dims [128 w, 128 w + 128): every wave runs
// the same score chain and softmax (the same LDS tile, no extra HBM bytes),
// each multiplies a quarter of the value dims, and no cross-wave merge is
// needed.  That serves 32 query rows from one pass over the cache.
template <bool kQuad>
__device__ __forceinline__ void decode_wide_body(DecodeParams p, const int32_t *__restrict__ bt,
                                                 const int32_t *__restrict__ seqlens,
                                                 const int32_t *__restrict__ meta)
{
    constexpr int kTileRows = kQuad ? 32 : kWRows;          // query rows per workgroup
    constexpr int kBlocks = kQuad ? kDBlocks / kWWaves : kDBlocks;   // dim blocks per wave
    constexpr int kPvSteps = 2 * kBlocks;                   // value MFMA pairs per tile
    constexpr int kSteps = kPvSteps > 20 ? kPvSteps : 20;   // softmax needs 20 slices
    __shared__ __attribute__((aligned(1024))) char tiles[kStages * kTileBytes];
    // set by any wave whose rows need the segment redone; read by all after a
    // barrier that follows every write, cleared after a second barrier
    __shared__ int redo;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n32 = lane & 31;        // query row of this lane inside the wave's block
    const int g = lane >> 5;          // half: keys 4g.. of each 8-key group
    const int part = blockIdx.x;
    const int rt = blockIdx.y;
    const int R = p.s_q * p.h_q;

    MLA_STAMP_BEGIN();
    const int32_t *rec = meta + part * kPartInts;
    const int s0 = rec[0];
    if (s0 < 0) {
        MLA_STAMP_END(g_stamps_wide);
        return;
    }
    const int t0 = rec[1], s1 = rec[2], t1 = rec[3], slot0 = rec[4];
    const int32_t *split_off = meta + p.num_parts * kPartInts;
    const int lds_addr = (int)(uintptr_t)(lds_char_t *)tiles;
    if (threadIdx.x == 0) redo = 0;
    // the stage the first iteration's (zero-weight) value product reads must
    // hold finite values: clear it once
    {
        char *z = tiles + (kStages - 1) * kTileBytes;
        for (int i = threadIdx.x; i < kTileBytes / 16; i += kWThreads)
            *reinterpret_cast<u32x4_t *>(z + 16 * i) = u32x4_t{0u, 0u, 0u, 0u};
    }

    // DMA: this lane's tile row and its in-page offset without tile and group terms
    const int trow = 8 * wave + (lane >> 3);
    const int lane_off = dma_lane_offset(wave, lane);
    const int row0 = rt * kTileRows + (kQuad ? 0 : 32 * wave);   // the wave's first row
    const int row = row0 + n32;
    // the wave's first dim block, kept in a vector register: the kernel has
    // no scalar register to spare for it
    int d_base = kQuad ? kBlocks * wave : 0;
    if constexpr (kQuad) asm volatile("" : "+v"(d_base));
    // a row count that is not a multiple of 128 leaves the last tile partly
    // empty: waves without rows only fetch their share of each tile
    const bool has_rows = row0 < R;   // uniform
    const bool row_ok = row < R;

    for (int seq = s0; seq <= s1; ++seq) {
        const int n = min(seqlens[seq], kMaxSeqLen);
        const int ks = seq == s0 ? t0 : 0;
        const int ke = seq == s1 ? t1 : n;
        if (ks >= ke) continue;
        MLA_STAMP_SEGMENT();
        const int nsplit = split_off[seq + 1] - split_off[seq];
        const int slot = seq == s0 ? slot0 : split_off[seq];
        const int32_t *bt_row = bt + (int64_t)seq * p.bt_stride;
        const int T0 = ks / kTileKeys;
        const int ntiles = (ke + kTileKeys - 1) / kTileKeys - T0;
        // block-table window: lane i holds the page of page slot pw_base + i
        const int pg_last = (ke - 1) / kPage;
        int pw_base = -1, pwin = 0;
        auto window_at = [&](int base) {
            pw_base = base;
            // columns past the table's width repeat its last one; entries
            // outside the cache are clamped into it (negative ones too)
            const int64_t col = min((int64_t)(base + lane), p.bt_stride - 1);
            pwin = base + lane <= pg_last ? (int)min((uint32_t)bt_row[col], p.page_max) : 0;
        };
        auto page_of = [&](int T) {
            const int i = (T >> 1) - pw_base;
            if (i >= 64) {   // uniform: move the window (every 4096 tokens)
                window_at(pw_base + 64);
                return __builtin_amdgcn_readlane(pwin, i - 64);
            }
            return __builtin_amdgcn_readlane(pwin, i);
        };

        int limit = ke;
        if (p.causal) limit = min(ke, n - p.s_q + 1 + row / p.h_q);
        // keys below this bound are visible to every row of the wave (lane 0
        // holds its first row, whose causal bound is the lowest)
        const int lim_min = __builtin_amdgcn_readfirstlane(limit);

        bf16x8_t qf[kKSteps];
        float m_hint = -INFINITY;     // origin of the second pass (segment maximum)
        WideRow st;
        f32x16_t o[kBlocks];
        for (int attempt = 0;; ++attempt) {
            if (pw_base != ks / kPage) window_at(ks / kPage);
            // start the first two tiles' DMA (and, once per segment, the Q^T loads)
#pragma unroll
            for (int sg = 0; sg < 2; ++sg)
                if (sg < ntiles)
                    dma_issue(tile_dma(p.kv, page_of(T0 + sg), T0 + sg, ks, ke, wave, trow,
                                       lane_off, lds_addr + sg * kTileBytes));
            if (attempt == 0) {
                const uint16_t *qrow = p.q + ((int64_t)seq * R + (row_ok ? row : 0)) * kDqk + 8 * g;
#pragma unroll
                for (int kk = 0; kk < kKSteps; ++kk)
                    qf[kk] = row_ok ? *reinterpret_cast<const bf16x8_t *>(qrow + 16 * kk)
                                    : bf16x8_t{};
            }
            st = WideRow{m_hint, 0.f, 0.f};
#pragma unroll
            for (int d = 0; d < kBlocks; ++d) o[d] = f32x16_t{};

            // fragment addresses: K of tile t (stage t % 4), V of tile t - 1
            int kb[4], vb[2][2];
            {
                int ln = lane;
                asm volatile("" : "+v"(ln));   // derived here, not kept across attempts
                const int r32 = ln & 31, gg = ln >> 5;
#pragma unroll
                for (int j = 0; j < 4; ++j) kb[j] = lds_addr + tile_off(r32, 2 * j + gg);
                // lane 16G + 4e + c (G: g' = G >> 1, h = G & 1) points at key
                // 16 kk + 4 g' + e (+8), dims 32d + 16h + 4c .. +3: chunk
                // 8 (d / 2) + (4 (d % 2) + 2h + c/2), half c % 2
                const int trG = ln >> 4;
                const int tg = trG >> 1, th = trG & 1;
                const int te = (ln >> 2) & 3, tc = ln & 3;
#pragma unroll
                for (int rd = 0; rd < 2; ++rd) {
                    const int key = 4 * tg + te + 8 * rd;
#pragma unroll
                    for (int par = 0; par < 2; ++par)
                        vb[rd][par] = lds_addr + (kStages - 1) * kTileBytes +
                                      tile_off(key, 4 * par + 2 * th + (tc >> 1)) + 8 * (tc & 1) +
                                      4096 * (d_base >> 1);   // d_base is even
                }
            }

            // P^T operands of the previous tile (zero before the first: that
            // iteration's value product adds nothing)
            bf16x8_t pp0 = {}, pp1 = {}, rp0 = {}, rp1 = {};
            bool low_any = false;         // some row of the wave outgrew its origin
            float mrun = -INFINITY;       // running maximum of the row's scores
            MLA_STAMP_PHASE(0);
            for (int t = 0; t < ntiles; ++t) {
                const int T = T0 + t;
                // this wave's part of tile t has landed (tile t + 1 may still be
                // in flight); the barrier makes the tile visible and guarantees
                // every wave is done with iteration t - 1, i.e. with tile t - 2,
                // whose stage the DMA for tile t + 2 reuses
                if (t + 1 < ntiles)
                    asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
                else
                    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                __syncthreads();

                if (!has_rows) {
                    if (t + 2 < ntiles)
                        dma_issue(tile_dma(p.kv, page_of(T + 2), T + 2, ks, ke, wave, trow,
                                           lane_off, lds_addr + ((t + 2) & 3) * kTileBytes));
                } else {
                    // ---- S^T[32 keys][32 rows] = K Q^T (+ DMA of tile t + 2) ----
                    f32x16_t s;
                    if (t + 2 < ntiles)
                        qk_tile_dma(s, kb, qf,
                                    tile_dma(p.kv, page_of(T + 2), T + 2, ks, ke, wave, trow,
                                             lane_off, lds_addr + ((t + 2) & 3) * kTileBytes));
                    else
                        qk_tile(s, kb, qf);

                    // ---- softmax of tile t (lane: row n32, keys 8(r/4) + 4g + r%4),
                    //      interleaved with the value product of tile t - 1 ----
                    if (!(T * kTileKeys >= ks && T * kTileKeys + kTileKeys <= lim_min)) {
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int key = T * kTileKeys + 8 * (r >> 2) + 4 * g + (r & 3);
                            if (!(key >= ks && key < limit)) s[r] = -INFINITY;
                        }
                    }
                    // The value product's 32 MFMAs go out one per step, in an order
                    // where consecutive ones accumulate into different blocks; after
                    // each, a slice of the softmax runs on the vector unit while the
                    // matrix unit works.  The schedule barriers keep that order.
                    float tmax = -INFINITY, m_use = 0.f;
                    float ex[16];
                    uint32_t pw[8], pr[8];
                    i16x4_t vlo[kPvAhead], vhi[kPvAhead];
#pragma unroll
                    for (int j = 0; j < kPvAhead; ++j)
                        pv_read(vb, pv_block(j), pv_kstep(j), vlo[j], vhi[j]);
#pragma unroll
                    for (int j = 0; j < kSteps; ++j) {
                        if (j < kPvSteps) {
                            const int lb = pv_block(j), kk = pv_kstep(j);
                            const i16x4_t lo = vlo[j % kPvAhead], hi = vhi[j % kPvAhead];
                            const i16x8_t a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                            o[lb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                                __builtin_bit_cast(bf16x8_t, a), kk ? pp1 : pp0, o[lb], 0, 0, 0);
                            o[lb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                                __builtin_bit_cast(bf16x8_t, a), kk ? rp1 : rp0, o[lb], 0, 0, 0);
                            if (j + kPvAhead < kPvSteps)
                                pv_read(vb, pv_block(j + kPvAhead), pv_kstep(j + kPvAhead),
                                        vlo[j % kPvAhead], vhi[j % kPvAhead]);
                        }
                        __builtin_amdgcn_sched_barrier(0);
                        // ---- softmax slice j of tile t (lane: row n32, keys
                        //      8(r/4) + 4g + r%4) ----
                        if (j < 3) {
#pragma unroll
                            for (int r = 6 * j; r < 6 * j + 6 && r < 16; ++r) tmax = fmaxf(tmax, s[r]);
                        } else if (j == 3) {
                            tmax = half_max(tmax) * p.scale_log2;
                            if (st.m == -INFINITY) st.m = tmax;   // first visible key: O, l still 0
                            mrun = fmaxf(mrun, tmax);
                            // origin too low: redo (never in the second pass, whose
                            // origin is the segment maximum)
                            low_any |= __builtin_amdgcn_ballot_w64(tmax > st.m + kWOriginSlack) != 0;
                            m_use = st.m == -INFINITY ? 0.f : st.m;
                        } else if (j < 20 && (j & 1) == 0) {
                            const int r = j - 4;
                            ex[r] = fast_exp2(__builtin_fmaf(s[r], p.scale_log2, -m_use));
                            ex[r + 1] = fast_exp2(__builtin_fmaf(s[r + 1], p.scale_log2, -m_use));
                        } else if (j < 20) {
                            const int r = j - 5;
                            st.l += ex[r] + ex[r + 1];
                            const uint32_t w = pack_bf16x2(ex[r], ex[r + 1]);
                            pw[r >> 1] = w;
                            st.lr = __builtin_amdgcn_fdot2_f32_bf16(
                                __builtin_bit_cast(bf16x2_t, w),
                                __builtin_bit_cast(bf16x2_t, 0x3F803F80u), st.lr, false);
                            // the rounding residual, exact in fp32, as the second term
                            const uint32_t q = pack_bf16x2(ex[r] - bf16_lo(w), ex[r + 1] - bf16_hi(w));
                            pr[r >> 1] = q;
                            st.lr = __builtin_amdgcn_fdot2_f32_bf16(
                                __builtin_bit_cast(bf16x2_t, q),
                                __builtin_bit_cast(bf16x2_t, 0x3F803F80u), st.lr, false);
                        }
                        __builtin_amdgcn_sched_barrier(0);
                    }
                    pp0 = __builtin_bit_cast(bf16x8_t, u32x4_t{pw[0], pw[1], pw[2], pw[3]});
                    pp1 = __builtin_bit_cast(bf16x8_t, u32x4_t{pw[4], pw[5], pw[6], pw[7]});
                    rp0 = __builtin_bit_cast(bf16x8_t, u32x4_t{pr[0], pr[1], pr[2], pr[3]});
                    rp1 = __builtin_bit_cast(bf16x8_t, u32x4_t{pr[4], pr[5], pr[6], pr[7]});
                }

                // next stages: K moves to tile t + 1, V to tile t
                const int kstep = (t & 3) == 3 ? -3 * kTileBytes : kTileBytes;
                const int vstep = ((t - 1) & 3) == 3 ? -3 * kTileBytes : kTileBytes;
#pragma unroll
                for (int j = 0; j < 4; ++j) kb[j] += kstep;
#pragma unroll
                for (int j = 0; j < 4; ++j) vb[j >> 1][j & 1] += vstep;
            }
            // the last tile's value product (its softmax ran in the last iteration)
            if (has_rows) pv_tile<kBlocks>(o, vb, pp0, pp1, rp0, rp1);
            if (low_any) redo = 1;
            // drain the DMA pipeline; every wave sees the same redo flag
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            const int again = redo;
            __syncthreads();
            MLA_STAMP_PHASE(1);
            if (!again || attempt > 0) break;
            if (threadIdx.x == 0) redo = 0;
            m_hint = mrun;   // both halves of a row hold the same maximum
        }

        // ---- epilogue: this wave's 32 rows (its dims of them with kQuad),
        //      no cross-wave merge ----
        st.l = half_sum(st.l);
        st.lr = half_sum(st.lr);
        const float inv = st.lr > 0.f ? 1.f / st.lr : 0.f;
        const float lse_v = st.l > 0.f ? (st.m + fast_log2(st.l)) * kLn2 : -INFINITY;
        // Result stores.  Lane (row n, g) holds dims 8 q4 + 4g .. + 4 of each
        // 32-dim block.  Swapping words between lane halves (32 apart) and
        // between 16-lane rows (16 apart) gathers four lanes per output row,
        // so a store instruction writes 16 rows x 64 contiguous bytes instead
        // of 32 rows x 16 or 32.  After the swaps lane l holds a piece of row
        // (l & 15) (first register) or 16 + (l & 15) (second register) at
        // column offset 8 pc + 4g (fp32) or 16 pc + 8g (bf16), pc = (l >> 4) & 1.
        // Every lane takes part in the swaps; only the stores skip rows >= R.
        if (has_rows) {
            // lane < 32 writes its row's lse; derived here, not a lane mask
            // held in scalar registers across the key loop
            int ll = lane;
            asm volatile("" : "+v"(ll));
            const bool lse_ok = ll < 32 && row0 + ll < R && (!kQuad || d_base == 0);
            const int pc = (lane >> 4) & 1;
            const int row_x = row0 + (lane & 15);
            const bool ok_x = row_x < R, ok_y = row_x + 16 < R;
            if (nsplit == 1) {
                uint16_t *dst = p.out + ((int64_t)seq * R + row_x) * kDv + 32 * d_base + 16 * pc + 8 * g;
#pragma unroll
                for (int d = 0; d < kBlocks; ++d) {
                    u32x4_t w[2];
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        // q4 = 2h: o[d][8h + 0..3], q4 = 2h + 1: o[d][8h + 4..7]; after
                        // the half swap lane (n, g) holds dims 16 h + 8g .. + 8
                        const int b = 8 * h;
                        const auto lo = __builtin_amdgcn_permlane32_swap(
                            pack_bf16x2(o[d][b] * inv, o[d][b + 1] * inv),
                            pack_bf16x2(o[d][b + 4] * inv, o[d][b + 5] * inv), false, false);
                        const auto hi = __builtin_amdgcn_permlane32_swap(
                            pack_bf16x2(o[d][b + 2] * inv, o[d][b + 3] * inv),
                            pack_bf16x2(o[d][b + 6] * inv, o[d][b + 7] * inv), false, false);
                        w[h] = u32x4_t{lo[0], hi[0], lo[1], hi[1]};
                    }
                    u32x4_t x, y;
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const auto sw = __builtin_amdgcn_permlane16_swap(w[0][k], w[1][k], false, false);
                        x[k] = sw[0];
                        y[k] = sw[1];
                    }
                    if (ok_x) *reinterpret_cast<u32x4_t *>(dst + 32 * d) = x;
                    if (ok_y) *reinterpret_cast<u32x4_t *>(dst + 16 * kDv + 32 * d) = y;
                }
                if (lse_ok) p.lse[(int64_t)seq * R + row] = lse_v;
            } else {
                float *dst = p.o_part + ((int64_t)slot * R + row_x) * kDv + 32 * d_base + 8 * pc + 4 * g;
#pragma unroll
                for (int d = 0; d < kBlocks; ++d)
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const int b = 8 * h;   // q4 = 2h and 2h + 1
                        f32x4_t x, y;
#pragma unroll
                        for (int k = 0; k < 4; ++k) {
                            const auto sw = __builtin_amdgcn_permlane16_swap(
                                __float_as_uint(o[d][b + k] * inv), __float_as_uint(o[d][b + 4 + k] * inv),
                                false, false);
                            x[k] = __uint_as_float(sw[0]);
                            y[k] = __uint_as_float(sw[1]);
                        }
                        if (ok_x) *reinterpret_cast<f32x4_t *>(dst + 32 * d + 16 * h) = x;
                        if (ok_y) *reinterpret_cast<f32x4_t *>(dst + 16 * kDv + 32 * d + 16 * h) = y;
                    }
                if (lse_ok) p.lse_part[(int64_t)slot * R + row] = lse_v;
            }
        }
        MLA_STAMP_PHASE(2);
    }
    MLA_STAMP_END(g_stamps_wide);
}

// The int tables are separate restrict arguments: with no aliasing store the
// compiler can read them through the scalar cache (wave-uniform indices).
__global__ __launch_bounds__(kWThreads, 1) void decode_wide_kernel(
    DecodeParams p, const int32_t *__restrict__ bt, const int32_t *__restrict__ seqlens,
    const int32_t *__restrict__ meta)
{
    decode_wide_body<false>(p, bt, seqlens, meta);
}

__global__ __launch_bounds__(kWThreads, 1) void decode_wide32_kernel(
    DecodeParams p, const int32_t *__restrict__ bt, const int32_t *__restrict__ seqlens,
    const int32_t *__restrict__ meta)
{
    decode_wide_body<true>(p, bt, seqlens, meta);
}

hipError_t launch_decode_wide(const DecodeParams &p, int num_parts, int row_tiles,
                              hipStream_t stream)
{
    hipLaunchKernelGGL(decode_wide_kernel, dim3(num_parts, row_tiles), dim3(kWThreads), 0,
                       stream, p, p.block_table, p.seqlens, p.meta);
    return hipGetLastError();
}

hipError_t launch_decode_wide32(const DecodeParams &p, int num_parts, int row_tiles,
                                hipStream_t stream)
{
    hipLaunchKernelGGL(decode_wide32_kernel, dim3(num_parts, row_tiles), dim3(kWThreads), 0,
                       stream, p, p.block_table, p.seqlens, p.meta);
    return hipGetLastError();
}

}  // namespace mla
