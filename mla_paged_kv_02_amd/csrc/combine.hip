// combine.hip -- split-KV merge of partial decode results.
//
// Each split s of a row carries a normalized partial output o_s and the
// natural-log sum-exp lse_s of its key range.  With M = max_s lse_s the
// merged row is lse = M + ln sum_s exp(lse_s - M) and
// out = sum_s exp(lse_s - lse) o_s (the log-sum-exp weights of FlashAttention-
// style split decoding, a lineage the FlashMLA release bullets name).
//
// A workgroup (4 waves) merges 4 rows of one sequence.  The common case, a
// sequence cut into at most kFewSplits parts, gives each wave one row: lane i
// reads split i's lse, one wave reduction gives M and the sum, and each lane
// accumulates 8 of the 512 dims with up to 8 splits' loads in flight -- one
// memory round trip for the usual two to eight splits, no LDS, no barrier.
//
// A sequence cut into more parts (one very long sequence among short ones)
// would leave a few workgroups with hundreds of round trips.  Inside a decode
// call it is merged in two levels: workgroup z of a row group merges splits
// [16 z, 16 z + 16) the same way and writes the result over split 16 z (no
// other workgroup reads that range); then, after a release fence, it counts
// itself done on the row group's counter, and the workgroup that completes
// the count acquires and merges the ceil(k / 16) level-one results (the same
// formula: a merge of merges is the merge of the union) and resets the
// counter.  The standalone entry point, whose inputs are read-only, merges
// such sequences with all four waves on each row instead.
#include "mla_device.h"
#include "kernels.h"

namespace mla {

constexpr int kCombineWaves = kCombineRows;
constexpr int kCombineThreads = kCombineWaves * 64;
constexpr int kCombineInflight = 8;

__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
    return v;
}

__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    return v;
}

__device__ __forceinline__ void store_row(const CombineParams &p, int b, int row, int lane,
                                          const float acc[8], float lse_v)
{
    uint16_t *dst = p.out + ((int64_t)b * p.rows + row) * kDv + 8 * lane;
    u32x4_t v;
    v[0] = pack_bf16x2(acc[0], acc[1]);
    v[1] = pack_bf16x2(acc[2], acc[3]);
    v[2] = pack_bf16x2(acc[4], acc[5]);
    v[3] = pack_bf16x2(acc[6], acc[7]);
    *reinterpret_cast<u32x4_t *>(dst) = v;
    if (lane == 0) p.lse[(int64_t)b * p.rows + row] = lse_v;
}

// acc += sum over this wave's splits s = s_begin, s_begin + stride, ... < ns
// of w(s) * o_part[s][row][8 lane .. 8 lane + 7], up to 8 loads in flight
template <typename W>
__device__ __forceinline__ void accumulate(const float *o_row, int64_t split_stride, int s_begin,
                                           int stride, int ns, int lane, W weight, float acc[8])
{
    for (int s0 = s_begin; s0 < ns; s0 += stride * kCombineInflight) {
        f32x4_t a[kCombineInflight], c[kCombineInflight];
        float w[kCombineInflight];
#pragma unroll
        for (int u = 0; u < kCombineInflight; ++u) {
            const int s = s0 + u * stride;   // uniform
            w[u] = 0.f;                      // stays 0 for absent splits
            a[u] = c[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            if (s < ns) {
                w[u] = weight(s);            // 0 for an empty split
                const float *src = o_row + s * split_stride + 8 * lane;
                a[u] = *reinterpret_cast<const f32x4_t *>(src);
                c[u] = *reinterpret_cast<const f32x4_t *>(src + 4);
            }
        }
#pragma unroll
        for (int u = 0; u < kCombineInflight; ++u) {
            if (w[u] == 0.f) continue;   // an empty split's o is not used
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc[e] += w[u] * a[u][e];
                acc[e + 4] += w[u] * c[u][e];
            }
        }
    }
}

// One wave merges one row over `count` slots: slot k is at o_row +
// k * slot_stride floats and lse_col[k * lse_stride]; count <= 64.
__device__ __forceinline__ void merge_row_wave(const float *o_row, int64_t slot_stride,
                                               const float *lse_col, int64_t lse_stride, int count,
                                               int lane, float acc[8], float &lse_v)
{
    if (count <= kCombineInflight) {
        // few slots: their rows are requested together with the lse values
        // (one memory round trip); a row of an empty slot gets weight 0
        f32x4_t a[kCombineInflight], c[kCombineInflight];
#pragma unroll
        for (int u = 0; u < kCombineInflight; ++u) {
            a[u] = c[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            if (u < count) {   // uniform
                const float *src = o_row + u * slot_stride + 8 * lane;
                a[u] = *reinterpret_cast<const f32x4_t *>(src);
                c[u] = *reinterpret_cast<const f32x4_t *>(src + 4);
            }
        }
        const float ls = lane < count ? lse_col[(int64_t)lane * lse_stride] : -INFINITY;
        const float M = wave_max(ls);
        lse_v = -INFINITY;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = 0.f;
        if (M == -INFINITY) return;
        const float e = fast_exp2((ls - M) * kLog2e);
        const float total = wave_sum(e);
        lse_v = M + fast_log2(total) * kLn2;
        const float wl = e / total;
#pragma unroll
        for (int u = 0; u < kCombineInflight; ++u) {
            if (u >= count) break;   // uniform
            const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), u));
            if (w == 0.f) continue;   // an empty split's row is not used
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                acc[q] += w * a[u][q];
                acc[q + 4] += w * c[u][q];
            }
        }
        return;
    }
    const float ls = lane < count ? lse_col[(int64_t)lane * lse_stride] : -INFINITY;
    const float M = wave_max(ls);
    lse_v = -INFINITY;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    if (M == -INFINITY) return;
    const float e = fast_exp2((ls - M) * kLog2e);   // 0 for absent or empty slots
    const float total = wave_sum(e);
    lse_v = M + fast_log2(total) * kLn2;
    const float wl = e / total;                   // lane k holds slot k's weight
    accumulate(o_row, slot_stride, 0, 1, count, lane,
               [&](int k) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), k)); },
               acc);
}

// Index of the sequence whose extra workgroups include number e (extra_off
// is an exclusive prefix, nondecreasing): the largest b with extra_off[b] <= e.
__device__ __forceinline__ int extra_owner(const int32_t *extra_off, int batch, int e)
{
    int lo = 0, hi = batch - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (extra_off[mid] <= e) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

__global__ __launch_bounds__(kCombineThreads) void combine_kernel(CombineParams p, int batch)
{
    __shared__ float red[kCombineWaves];
    __shared__ __attribute__((aligned(16))) float part_sum[kCombineWaves - 1][kDv];
    __shared__ int last;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    // workgroup y < batch: sequence y, chunk 0; later ones: extra chunks of
    // heavy sequences
    int b = blockIdx.y, z = 0;
    if (b >= batch) {
        if (p.extra_off == nullptr) return;
        const int e = b - batch;
        if (e >= p.extra_off[batch]) return;   // unused (the grid is an upper bound)
        b = extra_owner(p.extra_off, batch, e);
        z = e - p.extra_off[b] + 1;
    }
    const int first = p.split_off[b];
    const int ns = p.split_off[b + 1] - first;
    if (p.skip_single && ns == 1) return;
    const int64_t split_stride = (int64_t)p.rows * kDv;   // floats between a row's splits
    const int row = blockIdx.x * kCombineWaves + wave;
    const float *o_row = p.o_part + ((int64_t)first * p.rows + row) * kDv;
    const float *lse_col = p.lse_part + (int64_t)first * p.rows + row;

    if (ns <= kFewSplits) {
        // one wave per row
        if (row >= p.rows) return;
        float acc[8], lse_v;
        merge_row_wave(o_row, split_stride, lse_col, p.rows, ns, lane, acc, lse_v);
        store_row(p, b, row, lane, acc, lse_v);
        return;
    }

    if (p.counters != nullptr) {
        // two levels; level one: splits [16 z, 16 z + 16) -> over split 16 z
        const int nz = (ns + kHeavyChunk - 1) / kHeavyChunk;
        const int s0 = kHeavyChunk * z;
        if (row < p.rows) {
            float acc[8], lse_v;
            merge_row_wave(o_row + s0 * split_stride, split_stride, lse_col + (int64_t)s0 * p.rows,
                           p.rows, min(kHeavyChunk, ns - s0), lane, acc, lse_v);
            float *dst = p.o_part + ((int64_t)(first + s0) * p.rows + row) * kDv + 8 * lane;
            *reinterpret_cast<f32x4_t *>(dst) = f32x4_t{acc[0], acc[1], acc[2], acc[3]};
            *reinterpret_cast<f32x4_t *>(dst + 4) = f32x4_t{acc[4], acc[5], acc[6], acc[7]};
            if (lane == 0) p.lse_part[(int64_t)(first + s0) * p.rows + row] = lse_v;
        }
        __syncthreads();   // every wave's results issued
        int32_t *counter = p.counters + (int64_t)p.heavy_rank[b] * kRowGroupsMax + blockIdx.x;
        if (threadIdx.x == 0) {
            __threadfence();   // release this workgroup's level-one results
            last = atomicAdd(counter, 1) == nz - 1;
        }
        __syncthreads();
        if (!last) return;
        __threadfence();   // acquire the other workgroups' results
        if (row < p.rows) {
            // level two: the nz results sit at splits 0, 16, 32, ...
            float acc[8], lse_v;
            if (nz <= 64) {
                merge_row_wave(o_row, kHeavyChunk * split_stride, lse_col,
                               (int64_t)kHeavyChunk * p.rows, nz, lane, acc, lse_v);
            } else {
                float m = -INFINITY;
                for (int k = lane; k < nz; k += 64)
                    m = fmaxf(m, lse_col[(int64_t)k * kHeavyChunk * p.rows]);
                m = wave_max(m);
                lse_v = -INFINITY;
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[e] = 0.f;
                if (m != -INFINITY) {
                    float t = 0.f;
                    for (int k = lane; k < nz; k += 64)
                        t += fast_exp2((lse_col[(int64_t)k * kHeavyChunk * p.rows] - m) * kLog2e);
                    lse_v = m + fast_log2(wave_sum(t)) * kLn2;
                    accumulate(o_row, kHeavyChunk * split_stride, 0, 1, nz, lane,
                               [&](int k) {
                                   return fast_exp2(
                                       (lse_col[(int64_t)k * kHeavyChunk * p.rows] - lse_v) * kLog2e);
                               },
                               acc);
                }
            }
            store_row(p, b, row, lane, acc, lse_v);
        }
        if (threadIdx.x == 0) *counter = 0;   // ready for the next call
        return;
    }

    // many splits, one level: the four waves merge each of the block's rows
    // together
    for (int r = 0; r < kCombineWaves; ++r) {
        const int row = blockIdx.x * kCombineWaves + r;
        if (row >= p.rows) break;   // uniform
        const float *lse_col = p.lse_part + (int64_t)first * p.rows + row;
        float m = -INFINITY;
        for (int s = threadIdx.x; s < ns; s += kCombineThreads)
            m = fmaxf(m, lse_col[(int64_t)s * p.rows]);
        m = wave_max(m);
        if (lane == 0) red[wave] = m;
        __syncthreads();
        float M = red[0];
#pragma unroll
        for (int w = 1; w < kCombineWaves; ++w) M = fmaxf(M, red[w]);
        __syncthreads();

        float lse_v = -INFINITY;
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (M != -INFINITY) {
            float t = 0.f;
            for (int s = threadIdx.x; s < ns; s += kCombineThreads)
                t += fast_exp2((lse_col[(int64_t)s * p.rows] - M) * kLog2e);
            t = wave_sum(t);
            if (lane == 0) red[wave] = t;
            __syncthreads();
            float total = 0.f;
#pragma unroll
            for (int w = 0; w < kCombineWaves; ++w) total += red[w];
            lse_v = M + fast_log2(total) * kLn2;
            const float *o_row = p.o_part + ((int64_t)first * p.rows + row) * kDv;
            accumulate(o_row, split_stride, wave, kCombineWaves, ns, lane,
                       [&](int s) {
                           return fast_exp2((lse_col[(int64_t)s * p.rows] - lse_v) * kLog2e);
                       },
                       acc);
        }
        // the four waves' sums meet in LDS; wave 0 writes the row
        if (wave > 0) {
            *reinterpret_cast<f32x4_t *>(&part_sum[wave - 1][8 * lane]) =
                f32x4_t{acc[0], acc[1], acc[2], acc[3]};
            *reinterpret_cast<f32x4_t *>(&part_sum[wave - 1][8 * lane + 4]) =
                f32x4_t{acc[4], acc[5], acc[6], acc[7]};
        }
        __syncthreads();
        if (wave == 0) {
#pragma unroll
            for (int w = 0; w < kCombineWaves - 1; ++w)
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[e] += part_sum[w][8 * lane + e];
            store_row(p, b, row, lane, acc, lse_v);
        }
        __syncthreads();   // red and part_sum are reused by the next row
    }
}

hipError_t launch_combine(const CombineParams &p, int batch, int extra_wgs, hipStream_t stream)
{
    hipLaunchKernelGGL(combine_kernel,
                       dim3((p.rows + kCombineWaves - 1) / kCombineWaves, batch + extra_wgs),
                       dim3(kCombineThreads), 0, stream, p, batch);
    return hipGetLastError();
}

}  // namespace mla
