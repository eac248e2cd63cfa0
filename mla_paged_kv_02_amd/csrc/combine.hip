// combine.hip -- split-KV merge of partial decode results.
//
// Each split s of a row carries a normalized partial output o_s and the
// natural-log sum-exp lse_s of its key range.  With M = max_s lse_s the
// merged row is lse = M + ln sum_s exp(lse_s - M) and
// out = sum_s exp(lse_s - lse) o_s (the log-sum-exp weights of FlashAttention-
// style split decoding, a lineage the FlashMLA release bullets name).
// One wave per output row; every lane owns 8 of the 512 dims, so each split
// is read as two coalesced 16-byte loads per lane.
#include "mla_device.h"
#include "kernels.h"

namespace mla {


__global__ __launch_bounds__(256) void combine_kernel(CombineParams p)
{
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int b = blockIdx.y;
    if (row >= p.rows) return;
    const int first = p.split_off[b];
    const int ns = p.split_off[b + 1] - first;
    if (p.skip_single && ns == 1) return;

    float M = -INFINITY;
    for (int s = 0; s < ns; ++s) M = fmaxf(M, p.lse_part[(int64_t)(first + s) * p.rows + row]);

    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float lse_v = -INFINITY;
    if (M != -INFINITY) {
        float total = 0.f;
        for (int s = 0; s < ns; ++s)
            total += fast_exp2((p.lse_part[(int64_t)(first + s) * p.rows + row] - M) * kLog2e);
        lse_v = M + fast_log2(total) * kLn2;
        for (int s = 0; s < ns; ++s) {
            const float ls = p.lse_part[(int64_t)(first + s) * p.rows + row];
            if (ls == -INFINITY) continue;
            const float w = fast_exp2((ls - lse_v) * kLog2e);
            const float *src = p.o_part + ((int64_t)(first + s) * p.rows + row) * kDv + 8 * lane;
            const f32x4_t a = *reinterpret_cast<const f32x4_t *>(src);
            const f32x4_t c = *reinterpret_cast<const f32x4_t *>(src + 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc[e] += w * a[e];
                acc[e + 4] += w * c[e];
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
