// tile_layout.h -- the LDS layout of a 32-token tile of the paged latent
// cache, shared by the decode kernels that stream tiles through LDS.
//
// A tile (32 rows of 576 bf16 = 72 chunks of 16 B per row, 36,864 B) is
// stored as 36 blocks of 8 rows x 8 chunks; block (row group i, chunk group
// j) sits at byte (4 j + i) * 1024.  Inside a block, row r's chunk c (mod 8)
// is at position c ^ swz(r).  One direct global->LDS DMA instruction
// (64 lanes x 16 B) fills one block, so the wave that fetches row group i
// gives every lane the same in-page offset in all nine of its instructions
// and only scalar offsets change.  swz() makes both fragment read patterns
// of the kernels -- 16 B per lane along a row (MFMA A operand of K) and the
// 8 B transposed reads of V -- land on distinct LDS banks.
#pragma once

#include "mla_device.h"

namespace mla {

constexpr int kTileKeys = 32;
constexpr int kRowChunks = kDqk / 8;                     // 72
constexpr int kTileBytes = kTileKeys * kRowChunks * 16;  // 36864

typedef char __attribute__((address_space(3))) lds_char_t;

__device__ __forceinline__ int swz(int r) { return ((2 * (r & 7)) ^ ((r >> 2) & 3)) & 7; }

// LDS byte offset (within a tile) of tile row r, chunk c
__device__ __forceinline__ int tile_off(int r, int c)
{
    return 1024 * (4 * (c >> 3) + (r >> 3)) + 128 * (r & 7) + 16 * ((c & 7) ^ swz(r));
}

// This lane's part of a tile DMA: tile row 8 * group + lane / 8 and, in
// every chunk group j, chunk 8 j + ((lane % 8) ^ swz(row)); its byte offset
// within a page, without the tile's and the row group's offset.
__device__ __forceinline__ int dma_lane_offset(int group, int lane)
{
    return (lane >> 3) * kRowBytes + 16 * ((lane & 7) ^ swz(8 * group + (lane >> 3)));
}

// DMA of one row group (8 rows x 72 chunks) of tile T of a sequence into the
// tile buffer at `stage`: nine 1 KB blocks.  Rows outside [kbeg, kend) read
// as zero (buffer range check).  The LDS-DMA immediate offset is left 0: it
// would move the LDS destination as well.
__device__ __forceinline__ void dma_row_group(lds_char_t *stage, const uint16_t *kv, int page,
                                              int T, int kbeg, int kend, int group, int lane,
                                              int lane_off)
{
    const __amdgpu_buffer_rsrc_t rsrc =
        make_rsrc(reinterpret_cast<const char *>(kv) + (int64_t)page * kPageBytes, kPageBytes);
    const int key = T * kTileKeys + 8 * group + (lane >> 3);
    const int voff = (key >= kbeg && key < kend) ? lane_off : 0x40000000;
    int soff = ((T & 1) * kTileKeys + 8 * group) * kRowBytes;
    int base = (int)(uintptr_t)stage + 1024 * group;
    // keep the nine scalar offsets derived here rather than precomputed and held
    asm volatile("" : "+s"(soff), "+s"(base));
#pragma unroll
    for (int j = 0; j < kRowChunks / 8; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rsrc, (void __attribute__((address_space(3))) *)(uintptr_t)(base + 4096 * j), 16,
            voff, soff + 128 * j, 0, 0);
}

}  // namespace mla
