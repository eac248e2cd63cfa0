// metadata.hip -- variable-length split scheduling for paged MLA decode.
//
// The FlashMLA release ("DeepSeek publica FlashMLA como codigo abierto",
// release bullets) targets serving batches whose sequences differ in length.
// Here every sequence is a run of 16-token chunks; the concatenation of all
// runs is cut into `num_parts` contiguous ranges whose sizes differ by at most
// one chunk, so a long sequence is spread over many workgroups and short ones
// share a workgroup.  With T chunks and P' = min(num_parts, T) used parts,
// part p < P' covers chunks [floor(p*T/P'), floor((p+1)*T/P')) (never empty)
// and the part owning chunk f is floor(((f+1)*P' - 1) / T); parts >= P' are
// empty.  A sequence touched by k parts gets k partial-result slots (k = 1:
// written in place by the decode kernel).
//
// One workgroup of 1024 threads; lengths are read on the device, so a
// serving loop needs no host synchronization.  Layout of the output is
// documented with mla_metadata_ints() in the public header.
#include "mla_device.h"
#include "kernels.h"

namespace mla {

constexpr int kMetaThreads = 1024;

// Exclusive scan over the workgroup: shuffle scan inside each wave, then
// every thread adds the totals of the waves before it (two barriers).
__device__ int block_exclusive_scan(int v, int *wave_tot, int &total)
{
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    int inc = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int up = __shfl_up(inc, off);
        if (lane >= off) inc += up;
    }
    if (lane == 63) wave_tot[wave] = inc;
    __syncthreads();
    int before = 0;
    total = 0;
#pragma unroll
    for (int w = 0; w < kMetaThreads / 64; ++w) {
        const int tw = wave_tot[w];
        if (w < wave) before += tw;
        total += tw;
    }
    __syncthreads();   // wave_tot may be rewritten by the next scan
    return before + inc - v;
}

__device__ __forceinline__ int part_of_chunk(int64_t f, int64_t parts, int64_t total)
{
    return (int)(((f + 1) * parts - 1) / total);
}

// largest b in [0, batch) with prefix[b] <= f (prefix nondecreasing, prefix[0] = 0)
__device__ __forceinline__ int find_seq(const int *prefix, int batch, int f)
{
    int lo = 0, hi = batch - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (prefix[mid] <= f) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

__global__ __launch_bounds__(kMetaThreads) void metadata_kernel(const int32_t *seqlens, int batch,
                                                               int num_parts, int32_t *meta)
{
    __shared__ int prefix[kMetaMaxBatch + 1];   // chunk offsets of the sequences
    __shared__ int splits[kMetaMaxBatch + 1];   // partial-slot offsets
    __shared__ int scratch[kMetaThreads / 64];
    const int t = threadIdx.x;
    const int per = (batch + kMetaThreads - 1) / kMetaThreads;
    const int b0 = min(batch, t * per);
    const int b1 = min(batch, b0 + per);

    int local = 0;
    for (int b = b0; b < b1; ++b) {
        const int ch = (max(seqlens[b], 0) + kChunk - 1) / kChunk;
        prefix[b] = ch;
        local += ch;
    }
    int total = 0;
    int run = block_exclusive_scan(local, scratch, total);
    for (int b = b0; b < b1; ++b) {
        const int ch = prefix[b];
        prefix[b] = run;
        run += ch;
    }
    if (t == 0) prefix[batch] = total;
    __syncthreads();
    const int used = min(num_parts, total);   // every used part gets >= 1 chunk

    local = 0;
    for (int b = b0; b < b1; ++b) {
        const int ch = prefix[b + 1] - prefix[b];
        const int ns = ch == 0 ? 0
                               : part_of_chunk(prefix[b] + ch - 1, used, total) -
                                     part_of_chunk(prefix[b], used, total) + 1;
        splits[b] = ns;
        local += ns;
    }
    int total_splits = 0;
    run = block_exclusive_scan(local, scratch, total_splits);
    for (int b = b0; b < b1; ++b) {
        const int ns = splits[b];
        splits[b] = run;
        run += ns;
    }
    if (t == 0) splits[batch] = total_splits;
    __syncthreads();

    int32_t *split_off = meta + num_parts * kPartInts;
    for (int b = t; b <= batch; b += kMetaThreads) split_off[b] = splits[b];
    if (t == 0) split_off[batch + 1] = total;

    for (int part = t; part < num_parts; part += kMetaThreads) {
        int32_t *rec = meta + part * kPartInts;
        int r[kPartInts] = {-1, 0, -1, 0, 0, 0, 0, 0};
        if (part < used) {
            const int f0 = (int)((int64_t)part * total / used);
            const int f1 = (int)((int64_t)(part + 1) * total / used);
            const int s0 = find_seq(prefix, batch, f0);
            const int s1 = find_seq(prefix, batch, f1 - 1);
            r[0] = s0;
            r[1] = (f0 - prefix[s0]) * kChunk;
            r[2] = s1;
            r[3] = min((f1 - prefix[s1]) * kChunk, max(seqlens[s1], 0));
            r[4] = splits[s0] + (part - part_of_chunk(prefix[s0], used, total));
        }
#pragma unroll
        for (int i = 0; i < kPartInts; ++i) rec[i] = r[i];
    }
}

hipError_t launch_metadata(const int32_t *seqlens, int batch, int num_parts, int32_t *meta,
                           hipStream_t stream)
{
    hipLaunchKernelGGL(metadata_kernel, dim3(1), dim3(kMetaThreads), 0, stream, seqlens, batch,
                       num_parts, meta);
    return hipGetLastError();
}

}  // namespace mla
