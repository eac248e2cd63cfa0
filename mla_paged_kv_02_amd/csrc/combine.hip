// combine.hip -- split-KV merge of partial decode results.
//
// Each split s of a row carries a normalized partial output o_s and the
// natural-log sum-exp lse_s of its key range.  With M = max_s lse_s the
// merged row is lse = M + ln sum_s exp(lse_s - M) and
// out = sum_s exp(lse_s - lse) o_s (the log-sum-exp weights of FlashAttention-
// style split decoding, a lineage the FlashMLA release bullets name).
//
// One workgroup (4 waves) per output row.  All 256 threads first read the
// row's lse values (256 splits per round trip) and reduce max and sum; then
// the waves take every 4th split, each lane accumulating 8 of the 512 dims
// with up to 8 splits' loads in flight, and the four partial sums meet in
// LDS.  A sequence cut into hundreds of parts (one very long sequence among
// short ones) is merged in a few round trips instead of one per split.
#include "mla_device.h"
#include "kernels.h"

namespace mla {

constexpr int kCombineThreads = 256;
constexpr int kCombineWaves = kCombineThreads / 64;
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

__global__ __launch_bounds__(kCombineThreads) void combine_kernel(CombineParams p)
{
    __shared__ float red[kCombineWaves];
    __shared__ __attribute__((aligned(16))) float part_sum[kCombineWaves - 1][kDv];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int row = blockIdx.x;
    const int b = blockIdx.y;
    const int first = p.split_off[b];
    const int ns = p.split_off[b + 1] - first;
    if (p.skip_single && ns == 1) return;
    const float *lse_col = p.lse_part + (int64_t)first * p.rows + row;

    // max over splits
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

        // this wave's splits: wave, wave + 4, ...; up to 8 in flight
        for (int s0 = wave; s0 < ns; s0 += kCombineWaves * kCombineInflight) {
            f32x4_t a[kCombineInflight], c[kCombineInflight];
            float w[kCombineInflight];
#pragma unroll
            for (int u = 0; u < kCombineInflight; ++u) {
                const int s = s0 + u * kCombineWaves;
                const int sc = s < ns ? s : s0;      // a valid split for the load
                const float ls = lse_col[(int64_t)sc * p.rows];
                w[u] = s < ns ? fast_exp2((ls - lse_v) * kLog2e) : 0.f;   // 0 for empty splits
                const float *src = p.o_part + ((int64_t)(first + sc) * p.rows + row) * kDv + 8 * lane;
                a[u] = *reinterpret_cast<const f32x4_t *>(src);
                c[u] = *reinterpret_cast<const f32x4_t *>(src + 4);
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
    // the four waves' sums meet in LDS; wave 0 writes the row
    if (wave > 0) {
        *reinterpret_cast<f32x4_t *>(&part_sum[wave - 1][8 * lane]) =
            f32x4_t{acc[0], acc[1], acc[2], acc[3]};
        *reinterpret_cast<f32x4_t *>(&part_sum[wave - 1][8 * lane + 4]) =
            f32x4_t{acc[4], acc[5], acc[6], acc[7]};
    }
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int w = 0; w < kCombineWaves - 1; ++w)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += part_sum[w][8 * lane + e];
    uint16_t *dst = p.out + ((int64_t)b * p.rows + row) * kDv + 8 * lane;
    u32x4_t v;
    v[0] = pack_bf16x2(acc[0], acc[1]);
    v[1] = pack_bf16x2(acc[2], acc[3]);
    v[2] = pack_bf16x2(acc[4], acc[5]);
    v[3] = pack_bf16x2(acc[6], acc[7]);
    *reinterpret_cast<u32x4_t *>(dst) = v;
    if (lane == 0) p.lse[(int64_t)b * p.rows + row] = lse_v;
}

hipError_t launch_combine(const CombineParams &p, int batch, hipStream_t stream)
{
    hipLaunchKernelGGL(combine_kernel, dim3(p.rows, batch), dim3(kCombineThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace mla
