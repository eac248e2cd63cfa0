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
// A sequence cut into more parts (one very long sequence among short ones)
// is merged row by row by all four waves together, each taking every 4th
// split, with the partial sums meeting in LDS.
#include "mla_device.h"
#include "kernels.h"

namespace mla {

constexpr int kCombineThreads = 256;
constexpr int kCombineWaves = kCombineThreads / 64;
constexpr int kCombineInflight = 8;
constexpr int kFewSplits = 32;

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

__global__ __launch_bounds__(kCombineThreads) void combine_kernel(CombineParams p)
{
    __shared__ float red[kCombineWaves];
    __shared__ __attribute__((aligned(16))) float part_sum[kCombineWaves - 1][kDv];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int b = blockIdx.y;
    const int first = p.split_off[b];
    const int ns = p.split_off[b + 1] - first;
    if (p.skip_single && ns == 1) return;
    const int64_t split_stride = (int64_t)p.rows * kDv;   // floats between a row's splits

    if (ns <= kFewSplits) {
        // one wave per row
        const int row = blockIdx.x * kCombineWaves + wave;
        if (row >= p.rows) return;
        const float *lse_col = p.lse_part + (int64_t)first * p.rows + row;
        const float ls = lane < ns ? lse_col[(int64_t)lane * p.rows] : -INFINITY;
        const float M = wave_max(ls);
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        float lse_v = -INFINITY;
        if (M != -INFINITY) {
            const float e = fast_exp2((ls - M) * kLog2e);   // 0 for absent splits
            const float total = wave_sum(e);
            lse_v = M + fast_log2(total) * kLn2;
            const float wl = e / total;                   // lane s holds split s's weight
            const float *o_row = p.o_part + ((int64_t)first * p.rows + row) * kDv;
            accumulate(o_row, split_stride, 0, 1, ns, lane,
                       [&](int s) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), s)); },
                       acc);
        }
        store_row(p, b, row, lane, acc, lse_v);
        return;
    }

    // many splits: the four waves merge each of the block's rows together
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

hipError_t launch_combine(const CombineParams &p, int batch, hipStream_t stream)
{
    hipLaunchKernelGGL(combine_kernel, dim3((p.rows + kCombineWaves - 1) / kCombineWaves, batch),
                       dim3(kCombineThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace mla
