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
    int rows;                   // s_q * h_q
    int skip_single;            // rows of single-split sequences are already final
    uint16_t *out;
    float *lse;
};

struct AbsorbParams {
    const uint16_t *x;
    int64_t x_sb, x_sh;
    const uint16_t *w;
    int K, N;
    uint16_t *y;
    int64_t y_sb, y_sh;
    int batch;
};

constexpr int kPartInts = 8;          // ints per scheduler-part record
constexpr int kMetaMaxBatch = 8192;
constexpr int kMaxParts = 65536;

hipError_t launch_metadata(const int32_t *seqlens, int batch, int num_parts, int lead,
                           int32_t *meta, hipStream_t stream);
hipError_t launch_decode_r16(const DecodeParams &p, int num_parts, int row_tiles,
                             hipStream_t stream);
// query rows per workgroup of the wide decode kernel (used when s_q*h_q is a
// multiple of it)
constexpr int kWideRows = 128;
// schedule cost of starting a sequence, in chunks, for the kernel that
// serves s_q * h_q rows (see metadata.hip)
constexpr int schedule_lead(int rows) { return rows % kWideRows == 0 ? 8 : 16; }
hipError_t launch_decode_wide(const DecodeParams &p, int num_parts, int row_tiles,
                              hipStream_t stream);
hipError_t launch_combine(const CombineParams &p, int batch, hipStream_t stream);
hipError_t launch_absorb(const AbsorbParams &p, int heads, hipStream_t stream);

}  // namespace mla
