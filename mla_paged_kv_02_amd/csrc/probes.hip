// probes.hip -- the achievable peaks that the decode's roofline fractions are
// also quoted against: a streaming HBM read and a dense bf16 MFMA loop.
//
// read_probe_kernel: a workgroup reads 16 KB contiguous per pass (each
// thread four 16-byte words, 4 KB apart, all in flight together), passes
// striding over the grid; the words fold into an XOR that is stored only if
// it equals a value no input produces in practice (so the loads stay live and
// nothing else is written).
//
// mfma_probe_kernel: every wave keeps eight independent 32x32 fp32
// accumulators and issues iters x 8 v_mfma_f32_32x32x16_bf16 (32768 flops
// each) from register operands; the sum of the accumulators goes to
// sink[global wave] so the chain is live.  Four waves per workgroup, one per
// SIMD.
#include "mla_device.h"
#include "kernels.h"

namespace mla {

constexpr int kProbeThreads = 256;
constexpr int kReadUnroll = 4;

__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const u32x4_t *__restrict__ buf,
                                                                   int64_t n16, uint32_t *sink)
{
    constexpr int64_t kPass = (int64_t)kProbeThreads * kReadUnroll;   // words per workgroup pass
    u32x4_t acc = {0u, 0u, 0u, 0u};
    for (int64_t base = (int64_t)blockIdx.x * kPass + threadIdx.x; base < n16;
         base += (int64_t)gridDim.x * kPass) {
        u32x4_t v[kReadUnroll];
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u) {
            const int64_t i = base + (int64_t)u * kProbeThreads;
            v[u] = i < n16 ? buf[i] : u32x4_t{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u];
    }
    const uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
    if (x == 0x9E3779B9u && acc.x == 0x7F4A7C15u) sink[0] = x;
}

__global__ __launch_bounds__(kProbeThreads) void mfma_probe_kernel(int iters, float *sink)
{
    const int lane = threadIdx.x & 63;
    bf16x8_t a, b;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        a[j] = (__bf16)(0.001f * (float)(lane + j));
        b[j] = (__bf16)(0.002f * (float)(lane - j));
    }
    f32x16_t c[8];
#pragma unroll
    for (int k = 0; k < 8; ++k)
#pragma unroll
        for (int r = 0; r < 16; ++r) c[k][r] = 0.0f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int k = 0; k < 8; ++k) c[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[k], 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += c[k][r];
    if (lane == 0) sink[blockIdx.x * (kProbeThreads / 64) + (threadIdx.x >> 6)] = s;
}

hipError_t launch_probe_read(const void *buf, int64_t bytes, int workgroups, uint32_t *sink,
                             hipStream_t stream)
{
    hipLaunchKernelGGL(read_probe_kernel, dim3(workgroups), dim3(kProbeThreads), 0, stream,
                       static_cast<const u32x4_t *>(buf), bytes / 16, sink);
    return hipGetLastError();
}

hipError_t launch_probe_mfma(int iters, int workgroups, float *sink, hipStream_t stream)
{
    hipLaunchKernelGGL(mfma_probe_kernel, dim3(workgroups), dim3(kProbeThreads), 0, stream, iters,
                       sink);
    return hipGetLastError();
}

}  // namespace mla
