// kernels.h -- internal launch interface between the C ABI (abi.cpp) and the
// gfx950 kernels.  Not part of the public header.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

struct DecodeParams {
    const uint16_t *q;
    const uint16_t *kv;
    const int32_t *block_table;
    int64_t bt_stride;
    uint32_t page_max;   // num_pages - 1: block-table entries are clamped to [0, page_max]
    const int32_t *seqlens;
    const int32_t *meta;
    int num_parts;
    int s_q;
    int h_q;
    int causal;
    float scale_log2;   // scale * log2(e)
    float *o_part;
    float *lse_part;
    uint16_t *out;
    float *lse;
};

struct CombineParams {
    const float *o_part;
    const float *lse_part;
    const int32_t *split_off;   // [batch + 1]
    // sliced merge of heavily split sequences inside a decode call: extra
    // workgroups before each sequence [batch + 1] (null: the standalone merge)
    const int32_t *extra_off;
    int rows;                   // s_q * h_q
    int skip_single;            // rows of single-split sequences are already final
    uint16_t *out;
    float *lse;
};


struct AbsorbParams {
    const uint16_t *x;
    int64_t x_sb, x_sh;
    const uint16_t *w;      // bf16 weights, or null when w8 is set
    const uint8_t *w8;      // E4M3 weights [heads][K][N]
    const float *wscale;    // their scales [heads][ceil(K/128)][ceil(N/128)]
    int K, N;
    uint16_t *y;
    int64_t y_sb, y_sh;
    int batch;
    int heads;
};

// Sequences split more than kFewSplits ways are "heavy": inside a decode
// call each row of one is merged by heavy_slices(k) workgroups, one per slice
// of 512 / heavy_slices(k) output dims (see combine.hip).
constexpr int kFewSplits = 32;
constexpr int kCombineRows = 4;                 // rows per combine workgroup
// dim slices for a heavy sequence with k slots: 2 for 33..63, 4 from 64, 8
// from 128, 16 from 256; so its kCombineRows * slices workgroups per row
// group are at most k / 4
__host__ __device__ constexpr int heavy_slices(int k)
{
    return k >= 256 ? 16 : k >= 128 ? 8 : k >= 64 ? 4 : 2;
}

constexpr int kPartInts = 8;          // ints per scheduler-part record
constexpr int kMetaMaxBatch = 8192;
// Sequence lengths are capped at 2^21 tokens on the device, which keeps the
// scheduler's chunk and cost sums (8192 sequences of 2^17 chunks, plus the
// leads) inside int32.
constexpr int kMaxSeqLen = 1 << 21;
constexpr int kMaxParts = 65536;

// Offsets (in int32) of the metadata sections for batch B and P parts:
// part records, split offsets [B + 1], total chunks, and the extra combine
// workgroups before each sequence [B + 1].
struct MetaLayout {
    int64_t B, P;
    __host__ __device__ int64_t split_off() const { return kPartInts * P; }
    __host__ __device__ int64_t total_chunks() const { return split_off() + B + 1; }
    __host__ __device__ int64_t extra_off() const { return total_chunks() + 1; }
    __host__ __device__ int64_t ints() const { return extra_off() + B + 1; }
    // extra combine workgroups per row group: a heavy sequence with k slots
    // has kCombineRows * heavy_slices(k) - 1 <= k / 4, and the slots of all
    // sequences number fewer than B + P
    __host__ __device__ int64_t extra_max() const { return (B + P) / 4 + 1; }
};

// seg_cost: the schedule's price of one sequence segment, in chunks, also
// its lead; choose: pick the lead per call between 0 and seg_cost (see
// metadata.hip)
hipError_t launch_metadata(const int32_t *seqlens, int batch, int num_parts, int seg_cost,
                           bool choose, int32_t *meta, hipStream_t stream);
hipError_t launch_decode_r16(const DecodeParams &p, int num_parts, int row_tiles,
                             hipStream_t stream);
// query rows per workgroup of the wide decode kernel (used when s_q*h_q is a
// multiple of it)
constexpr int kWideRows = 128;
// The 128-row kernel serves multiples of 128 rows and, with a partly empty
// last tile, any row count from 48 on (it streams the cache once per 128
// rows instead of once per 16); the 16-row kernel serves 16 and 32 rows.
constexpr int kWideMinRows = 48;
constexpr bool use_wide(int rows) { return rows % kWideRows == 0 || rows >= kWideMinRows; }
// 32 rows run on the shared-row variant of the 128-row kernel (one pass over
// the cache instead of two 16-row passes); 16 rows on the 16-row kernel.
constexpr bool use_wide32(int rows) { return rows == 32; }
constexpr int decode_row_tiles(int rows)
{
    return use_wide(rows) ? (rows + kWideRows - 1) / kWideRows
                          : use_wide32(rows) ? 1 : (rows + 15) / 16;
}
// The schedule's price of one sequence segment (query load, pipeline fill,
// result write), in chunks, for the kernel serving s_q * h_q rows: 16 for
// the 16-row kernel, 24 for the 128-row kernel (measured per-segment
// overheads; metadata.hip picks each call's lead with it).
constexpr int segment_cost(int rows) { return use_wide(rows) ? 24 : 16; }
hipError_t launch_decode_wide(const DecodeParams &p, int num_parts, int row_tiles,
                              hipStream_t stream);
hipError_t launch_decode_wide32(const DecodeParams &p, int num_parts, int row_tiles,
                                hipStream_t stream);
// `extra_wgs`: upper bound on the extra workgroups of heavily split sequences
hipError_t launch_combine(const CombineParams &p, int batch, int extra_wgs, hipStream_t stream);
hipError_t launch_absorb(const AbsorbParams &p, int heads, hipStream_t stream);
// Where mla_decode's partial results go: the caller's workspace (ptr, bytes),
// or, when `resolve` is set, a buffer of `bytes` that resolve() returns for
// the current device (the library's own scratch array).
struct WorkspaceSource {
    void *ptr = nullptr;
    size_t bytes = 0;
    int (*resolve)(void **ptr) = nullptr;
    bool debug_checks = true;   // honour MLA_DEBUG_CHECKS (host copies and a sync)
};

// The validated decode call behind mla_decode and mla_decode_noalloc (abi.cpp).
int decode_call(const uint16_t *q, const uint16_t *kv_cache, int64_t num_pages,
                const int32_t *block_table, int64_t bt_stride, const int32_t *seqlens, int batch,
                int s_q, int h_q, int d_qk, int d_v, int page_size, float scale, int causal,
                const int32_t *metadata, int num_parts, const WorkspaceSource &ws, uint16_t *out,
                float *lse, void *stream);
// Record a failure reason for mla_last_error(); returns `status`.
int set_error(int status, const char *fmt, ...);

hipError_t launch_probe_read(const void *buf, int64_t bytes, int workgroups, uint32_t *sink,
                             hipStream_t stream);
hipError_t launch_probe_mfma(int iters, int workgroups, float *sink, hipStream_t stream);
#if MLA_STAMPS
hipError_t set_stamps_r16(uint64_t *buf);
hipError_t set_stamps_wide(uint64_t *buf);
#endif
hipError_t launch_probe_lds(int waves, int depth, int iters, int workgroups, uint32_t *ticks,
                            uint32_t *sink, hipStream_t stream);

}  // namespace mla
