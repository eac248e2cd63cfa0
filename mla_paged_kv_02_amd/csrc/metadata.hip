// metadata.hip -- variable-length split scheduling for paged MLA decode.
//
// The FlashMLA release ("DeepSeek publica FlashMLA como codigo abierto",
// release bullets) targets serving batches whose sequences differ in length.
// Here every sequence is a run of 16-token chunks, and a workgroup pays a
// fixed extra cost (query load, pipeline fill, result write) for every
// sequence segment it runs.  The schedule works on cost units: sequence b
// with ch_b > 0 chunks is C lead-in units followed by its ch_b chunk units.
// The concatenation of all sequences' units (TC in total) is cut into
// U = min(num_parts, TC) ranges, part p < U covering units
// [floor(p*TC/U), floor((p+1)*TC/U)); a part holds the chunks whose units
// fall in its range (a range of lead-in units only makes an empty part), so a
// part that starts a sequence gets C fewer chunks.  The lead C is the
// segment price S (segment_cost in kernels.h: 16 chunks for the 16-row
// kernel, 24 for the 128-row kernel) or, for the 128-row kernel, 0 when that
// prices lower: each part costs its chunks plus S per segment, and the lead
// whose largest part is smaller wins (equal-length sequences split evenly
// want no lead; mixed lengths, whose parts straddle sequences, want S).
// Chunk i of sequence b sits at unit cpre[b] + C + i, and the part owning
// unit x is floor(((x+1)*U - 1) / TC).  A sequence touched by k parts gets k
// partial-result slots (k = 1: written in place by the decode kernel).
// A sequence with more than kFewSplits slots is "heavy": the decode call's
// merge gives it kCombineRows * heavy_slices(k) workgroups per row group, the
// extra ones numbered after all sequences (extra_off).
//
// One workgroup of 256 threads; lengths are read on the device once (the
// per-sequence data lives in LDS), so a serving loop needs no host
// synchronization.  Layout of the output is documented with
// mla_metadata_ints() in the public header.
#include "mla_device.h"
#include "kernels.h"

namespace mla {

constexpr int kMetaThreads = 256;

// Exclusive scans of two values at once over the workgroup: shuffle scans
// inside each wave, then every thread adds the totals of the waves before it
// (one barrier; the caller's next scan waits on its own barrier before it
// rewrites wave_tot, so each call alternates between two halves).
__device__ void block_exclusive_scan2(int v0, int v1, int *wave_tot, int &run0, int &run1,
                                      int &total0, int &total1)
{
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    int a = v0, b = v1;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int ua = __shfl_up(a, off), ub = __shfl_up(b, off);
        if (lane >= off) {
            a += ua;
            b += ub;
        }
    }
    constexpr int kW = kMetaThreads / 64;
    if (lane == 63) {
        wave_tot[wave] = a;
        wave_tot[kW + wave] = b;
    }
    __syncthreads();
    int before0 = 0, before1 = 0;
    total0 = total1 = 0;
#pragma unroll
    for (int w = 0; w < kW; ++w) {
        const int t0 = wave_tot[w], t1 = wave_tot[kW + w];
        if (w < wave) {
            before0 += t0;
            before1 += t1;
        }
        total0 += t0;
        total1 += t1;
    }
    run0 = before0 + a - v0;
    run1 = before1 + b - v1;
}

// floor(a * b / c) for a, b, c >= 0 (c > 0); 32-bit arithmetic when the
// product fits (the usual case), else 64-bit
__device__ __forceinline__ int muldiv(int a, int b, int c, bool small)
{
    if (small) return (int)((uint32_t)a * (uint32_t)b / (uint32_t)c);
    return (int)((int64_t)a * b / c);
}

__device__ __forceinline__ int part_of_chunk(int f, int parts, int total, bool small)
{
    return small ? (int)(((uint32_t)f * (uint32_t)parts + (uint32_t)parts - 1) / (uint32_t)total)
                 : (int)(((int64_t)(f + 1) * parts - 1) / total);
}

// largest b in [0, batch) with a[b] <= x (a nondecreasing, a[0] = 0)
__device__ __forceinline__ int find_last_le(const int *a, int batch, int x)
{
    int lo = 0, hi = batch - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (a[mid] <= x) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

// Cost-unit offset of sequence b for lead L: its chunk offset plus L for
// every non-empty sequence before it.
__device__ __forceinline__ int unit_of(const int *prefix, const int *nepre, int lead, int b)
{
    return prefix[b] + lead * nepre[b];
}

// largest b in [0, batch) with unit_of(b) <= x
__device__ __forceinline__ int find_last_unit_le(const int *prefix, const int *nepre, int lead,
                                                 int batch, int x)
{
    int lo = 0, hi = batch - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (unit_of(prefix, nepre, lead, mid) <= x) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

// The chunks [f0, f1) of part `part` < used under lead L (empty when
// f0 >= f1): its units [x0, x1) hold the chunks whose units lie in them.
// f0 lies in sequence s0, f1 - 1 in s1 (both non-empty).
struct PartRange {
    int s0, f0, s1, f1;
};
__device__ __forceinline__ PartRange part_range(int part, int lead, int tc, int used, bool small,
                                                const int *prefix, const int *nepre, int batch)
{
    const int x0 = muldiv(part, tc, used, small);
    const int x1 = muldiv(part + 1, tc, used, small);
    // first chunk at unit >= x0, one past the last chunk at unit < x1
    const int ba = find_last_unit_le(prefix, nepre, lead, batch, x0);
    const int f0 = prefix[ba] + max(0, x0 - unit_of(prefix, nepre, lead, ba) - lead);
    const int bz = find_last_unit_le(prefix, nepre, lead, batch, x1 - 1);
    const int iz = x1 - 1 - unit_of(prefix, nepre, lead, bz) - lead;
    const int f1 = iz >= 0 ? prefix[bz] + iz + 1 : prefix[bz];
    // the range ends in bz's lead units: its last chunk is in the last
    // non-empty sequence before bz
    const int s1 = iz >= 0 || f0 >= f1 ? bz : find_last_le(prefix, batch, f1 - 1);
    return PartRange{ba, f0, s1, f1};
}

// A part's price under lead L: its chunks plus seg_cost per sequence it
// touches (0 for an empty part).
__device__ __forceinline__ int part_cost(int part, int lead, int tc, int used, bool small,
                                                  const int *prefix, const int *nepre, int batch,
                                                  int seg_cost)
{
    const int x0 = muldiv(part, tc, used, small);
    const int x1 = muldiv(part + 1, tc, used, small);
    const int ba = find_last_unit_le(prefix, nepre, lead, batch, x0);
    const int bz = find_last_unit_le(prefix, nepre, lead, batch, x1 - 1);
    const int f0 = prefix[ba] + max(0, x0 - unit_of(prefix, nepre, lead, ba) - lead);
    const int iz = x1 - 1 - unit_of(prefix, nepre, lead, bz) - lead;
    const int f1 = iz >= 0 ? prefix[bz] + iz + 1 : prefix[bz];
    // sequences ba..bz hold the part's chunks, less bz when the range ends
    // in its lead units (ba is non-empty)
    const int segs = nepre[bz] - nepre[ba] + (iz >= 0 ? 1 : 0);
    return f0 < f1 ? f1 - f0 + seg_cost * segs : 0;
}

// The leads the schedule tries when it chooses (see mla_get_metadata in the
// public header): 0 and the segment cost.
constexpr int kLeadCands = 2;
static_assert(kMetaThreads % (64 * kLeadCands) == 0, "each candidate gets whole waves");

__global__ __launch_bounds__(kMetaThreads) void metadata_kernel(const int32_t *seqlens, int batch,
                                                               int num_parts, int seg_cost,
                                                               int choose, int32_t *meta)
{
    __shared__ int prefix[kMetaMaxBatch + 1];        // chunk offsets of the sequences
    __shared__ int nepre[kMetaMaxBatch + 1];         // non-empty sequences before b
    __shared__ int splits[kMetaMaxBatch + 1];        // partial-slot offsets
    __shared__ unsigned char tail[kMetaMaxBatch];    // tokens in a sequence's last chunk
    __shared__ int scratch[3][2 * kMetaThreads / 64];   // one per scan: no reuse race
    __shared__ int lead_max[kMetaThreads / 64];         // per wave: its candidate's largest part
    const int t = threadIdx.x;
    const int per = (batch + kMetaThreads - 1) / kMetaThreads;
    const int b0 = min(batch, t * per);
    const int b1 = min(batch, b0 + per);

    // chunk counts and non-empty sequences, scanned together
    int local = 0, local_ne = 0;
    for (int b = b0; b < b1; ++b) {
        const int n = min(max(seqlens[b], 0), kMaxSeqLen);
        const int ch = (n + kChunk - 1) / kChunk;
        prefix[b] = ch;
        tail[b] = (unsigned char)(n - kChunk * (ch - 1));   // 1..16 (unused when ch == 0)
        local += ch;
        local_ne += ch > 0;
    }
    int total = 0, total_ne = 0, run = 0, run_ne = 0;
    block_exclusive_scan2(local, local_ne, scratch[0], run, run_ne, total, total_ne);
    for (int b = b0; b < b1; ++b) {
        const int ch = prefix[b];
        prefix[b] = run;
        nepre[b] = run_ne;
        run += ch;
        run_ne += ch > 0;
    }
    if (t == 0) {
        prefix[batch] = total;
        nepre[batch] = total_ne;
    }
    __syncthreads();

    // the lead: seg_cost, or (when choosing) whichever of 0 and seg_cost
    // cuts the batch with the smaller largest part, every segment priced at
    // seg_cost chunks (ties: seg_cost)
    int lead = seg_cost;
    if (choose) {
        // the two candidates are priced at once, each by half of the threads
        constexpr int kHalf = kMetaThreads / kLeadCands;
        const int i = t / kHalf;   // wave-uniform
        const int ld = i == 0 ? 0 : seg_cost;
        const int tci = total + ld * total_ne;
        const int usedi = min(num_parts, tci);
        const bool smalli = (int64_t)(tci + 1) * usedi < 0x7FFFFFFF;
        int m = 0;
        for (int part = t % kHalf; part < usedi; part += kHalf)
            m = max(m, part_cost(part, ld, tci, usedi, smalli, prefix, nepre, batch, seg_cost));
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) m = max(m, __shfl_xor(m, off));
        if ((t & 63) == 0) lead_max[t >> 6] = m;
        __syncthreads();
        int m0 = 0, m1 = 0;
        for (int w = 0; w < kMetaThreads / 64; ++w) {
            if (w < kHalf / 64) m0 = max(m0, lead_max[w]);
            else m1 = max(m1, lead_max[w]);
        }
        if (m0 < m1) lead = 0;
    }
    const int tc = total + lead * total_ne;
    const int used = min(num_parts, tc);
    const bool small = (int64_t)(tc + 1) * used < 0x7FFFFFFF;

    local = 0;
    for (int b = b0; b < b1; ++b) {
        const int ch = prefix[b + 1] - prefix[b];
        const int x = unit_of(prefix, nepre, lead, b) + lead;   // unit of the first chunk
        const int ns = ch == 0 ? 0
                               : part_of_chunk(x + ch - 1, used, tc, small) -
                                     part_of_chunk(x, used, tc, small) + 1;
        splits[b] = ns;
        local += ns;
    }
    int total_splits = 0, unused_run = 0, unused_total = 0;
    block_exclusive_scan2(local, 0, scratch[1], run, unused_run, total_splits, unused_total);
    for (int b = b0; b < b1; ++b) {
        const int ns = splits[b];
        splits[b] = run;
        run += ns;
    }
    if (t == 0) splits[batch] = total_splits;
    __syncthreads();

    const MetaLayout L{batch, num_parts};
    int32_t *split_off = meta + L.split_off();
    for (int b = t; b <= batch; b += kMetaThreads) split_off[b] = splits[b];
    if (t == 0) meta[L.total_chunks()] = total;

    // heavy sequences: extra merge workgroups
    int local_x = 0;
    for (int b = b0; b < b1; ++b) {
        const int ns = splits[b + 1] - splits[b];
        if (ns > kFewSplits) local_x += kCombineRows * heavy_slices(ns) - 1;
    }
    int total_x = 0, run_x = 0, unused_run2 = 0, unused_total2 = 0;
    block_exclusive_scan2(local_x, 0, scratch[2], run_x, unused_run2, total_x, unused_total2);
    int32_t *extra_off = meta + L.extra_off();
    for (int b = b0; b < b1; ++b) {
        const int ns = splits[b + 1] - splits[b];
        extra_off[b] = run_x;
        if (ns > kFewSplits) run_x += kCombineRows * heavy_slices(ns) - 1;
    }
    if (t == 0) extra_off[batch] = total_x;

    for (int part = t; part < num_parts; part += kMetaThreads) {
        int32_t *rec = meta + part * kPartInts;
        int r[kPartInts] = {-1, 0, -1, 0, 0, 0, 0, 0};
        if (part < used) {
            const PartRange pr = part_range(part, lead, tc, used, small, prefix, nepre, batch);
            if (pr.f0 < pr.f1) {
                const int s0 = pr.s0, s1 = pr.s1, f0 = pr.f0, f1 = pr.f1;
                r[0] = s0;
                r[1] = (f0 - prefix[s0]) * kChunk;
                r[2] = s1;
                // ends at a chunk boundary, or at the length if it takes s1's last chunk
                r[3] = f1 == prefix[s1 + 1] ? (f1 - 1 - prefix[s1]) * kChunk + tail[s1]
                                            : (f1 - prefix[s1]) * kChunk;
                r[4] = splits[s0] + (part - part_of_chunk(unit_of(prefix, nepre, lead, s0) + lead,
                                                          used, tc, small));
            }
        }
        *reinterpret_cast<int4 *>(rec) = make_int4(r[0], r[1], r[2], r[3]);
        *reinterpret_cast<int4 *>(rec + 4) = make_int4(r[4], r[5], r[6], r[7]);
    }
}

hipError_t launch_metadata(const int32_t *seqlens, int batch, int num_parts, int seg_cost,
                           bool choose, int32_t *meta, hipStream_t stream)
{
    hipLaunchKernelGGL(metadata_kernel, dim3(1), dim3(kMetaThreads), 0, stream, seqlens, batch,
                       num_parts, seg_cost, choose ? 1 : 0, meta);
    return hipGetLastError();
}

}  // namespace mla
