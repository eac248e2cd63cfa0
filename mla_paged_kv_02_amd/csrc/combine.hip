// combine.hip -- split-KV merge of partial decode results.
//
// Each split s of a row carries a normalized partial output o_s and the
// natural-log sum-exp lse_s of its key range.  With M = max_s lse_s the
// merged row is lse = M + ln sum_s exp(lse_s - M) and
// out = sum_s exp(lse_s - lse) o_s (the log-sum-exp weights of FlashAttention-
// style split decoding, a lineage the FlashMLA release bullets name).
//
// One wave per output row.  Lane s first loads lse_s of split s (all splits
// of the row in one round trip), the wave reduces max and sum with cross-lane
// operations, and then every lane accumulates its 8 of the 512 dims over the
// splits; those loads are independent, so they are all in flight together.
#include "mla_device.h"
#include "kernels.h"

namespace mla {

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

__global__ __launch_bounds__(256) void combine_kernel(CombineParams p)
{
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int b = blockIdx.y;
    if (row >= p.rows) return;
    const int first = p.split_off[b];
    const int ns = p.split_off[b + 1] - first;
    if (p.skip_single && ns == 1) return;

    // pass 1: the row's lse over all splits (64 splits per round)
    float M = -INFINITY;
    for (int s0 = 0; s0 < ns; s0 += 64) {
        const float ls = s0 + lane < ns ? p.lse_part[(int64_t)(first + s0 + lane) * p.rows + row]
                                        : -INFINITY;
        M = fmaxf(M, wave_max(ls));
    }
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float lse_v = -INFINITY;
    if (M != -INFINITY) {
        float total = 0.f;
        for (int s0 = 0; s0 < ns; s0 += 64) {
            const float ls = s0 + lane < ns
                                 ? p.lse_part[(int64_t)(first + s0 + lane) * p.rows + row]
                                 : -INFINITY;
            total += wave_sum(fast_exp2((ls - M) * kLog2e));
        }
        lse_v = M + fast_log2(total) * kLn2;
        // pass 2: weighted sum of the partial outputs, 4 splits in flight
        for (int s0 = 0; s0 < ns; s0 += 64) {
            const float ls = s0 + lane < ns
                                 ? p.lse_part[(int64_t)(first + s0 + lane) * p.rows + row]
                                 : -INFINITY;
            const float w_lane = fast_exp2((ls - lse_v) * kLog2e);   // 0 for empty splits
            const int cnt = min(64, ns - s0);
            for (int s = 0; s < cnt; s += 4) {
                f32x4_t a[4], c[4];
                float w[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int su = min(s + u, cnt - 1);
                    w[u] = s + u < cnt ? __shfl(w_lane, su) : 0.f;
                    const float *src =
                        p.o_part + ((int64_t)(first + s0 + su) * p.rows + row) * kDv + 8 * lane;
                    a[u] = *reinterpret_cast<const f32x4_t *>(src);
                    c[u] = *reinterpret_cast<const f32x4_t *>(src + 4);
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    if (w[u] == 0.f) continue;   // empty split (its o is ignored)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        acc[e] += w[u] * a[u][e];
                        acc[e + 4] += w[u] * c[u][e];
                    }
                }
            }
        }
    }
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
    hipLaunchKernelGGL(combine_kernel, dim3((p.rows + 3) / 4, batch), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace mla
