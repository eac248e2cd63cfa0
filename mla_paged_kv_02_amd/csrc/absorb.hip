// absorb.hip -- per-head batched matmul for non-materialized MLA absorption.
//
// "[Attention] MLA get rid of materialization" (PR description) keeps W_UK
// and W_UV separate and applies them as sequential matmuls around the latent
// attention: q_lat = q_nope . W_UK[h] before it, y = o_lat . W_UV[h] after it.
// Each is y[b, h, :] = x[b, h, :] . W[h] with W[h] a K x N bf16 matrix.
//
// gfx950 mapping: a workgroup computes a 64 (batch) x 64 (columns) tile of
// one head as y^T = W^T x^T on v_mfma_f32_16x16x32_bf16.  W's K x 64 column
// slab goes through LDS and is read back transposed with ds_read_b64_tr_b16
// (the A operand needs 8 consecutive k per lane, which are 2N bytes apart in
// memory); x rows are already k-contiguous and feed the B operand straight
// from global memory.  The op is HBM-bound (37.7 MB per call at 128 heads x
// 128 x 512), so every thread issues the loads of G 32-row slabs of k at
// once -- G = 4 for K = 128, 16 for K = 512, 8 otherwise -- and the
// workgroup pays one memory round trip per G slabs instead of one per slab.
// The accumulator layout puts 4 consecutive output columns in each lane, so
// stores are 8 bytes.  Consecutive workgroup numbers go to the eight XCDs in
// turn, and each XCD has its own L2: the grid is numbered so that all tiles
// of a head share an XCD (number L -> XCD L % 8, head L % 8 + 8 ((L / 8) /
// tiles per head)), which keeps a head's x rows and W slabs in one L2
// instead of fetching them from HBM once per XCD.
#include "mla_device.h"
#include "kernels.h"

namespace mla {

constexpr int kAbsThreads = 256;
constexpr int kAbsBM = 64;              // batch rows per workgroup (16 per wave)
constexpr int kAbsBN = 64;              // output columns per workgroup
constexpr int kAbsKSlab = 32;           // k rows per slab (one 16-byte load per thread)
constexpr int kWStride = kAbsBN + 8;    // bf16 per staged row (144 B)


template <int G>
__global__ __launch_bounds__(kAbsThreads) void absorb_kernel(AbsorbParams p)
{
    __shared__ __attribute__((aligned(16))) short wt[G * kAbsKSlab * kWStride];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int r16 = lane & 15;
    const int g = lane >> 4;
    const int ntn = p.N / kAbsBN;
    const int tiles = ntn * ((p.batch + kAbsBM - 1) / kAbsBM);   // per head
    const int k8 = blockIdx.x >> 3;
    const int h = (blockIdx.x & 7) + 8 * (k8 / tiles);
    if (h >= p.heads) return;   // padding of the head count to a multiple of 8 (uniform)
    const int t = k8 % tiles;
    const int n0 = (t % ntn) * kAbsBN;
    const int m0 = (t / ntn) * kAbsBM;

    const uint16_t *wh = p.w + (int64_t)h * p.K * p.N;
    const int brow = m0 + wave * 16 + r16;               // batch row of this lane (B operand)
    const bool row_ok = brow < p.batch;
    const uint16_t *xrow = p.x + (int64_t)(row_ok ? brow : 0) * p.x_sb + (int64_t)h * p.x_sh;

    // staging: thread t copies 16 bytes of each slab: row t / 8, columns 8 * (t % 8)
    const int srow = threadIdx.x >> 3;
    const int scol = 8 * (threadIdx.x & 7);

    f32x4_t acc[4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) acc[mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // transposed-read address: lane 16g + 4e + c -> slab row 8g + e, column 4c
    const int tr_row = 8 * g + (r16 >> 2);
    const int tr_col = 4 * (r16 & 3);

    for (int kg = 0; kg < p.K; kg += G * kAbsKSlab) {
        const int ns = min(G, (p.K - kg) / kAbsKSlab);   // slabs in this group (uniform)
        u32x4_t wv[G], xv[G];
#pragma unroll
        for (int s = 0; s < G; ++s) {
            wv[s] = u32x4_t{0u, 0u, 0u, 0u};
            xv[s] = u32x4_t{0u, 0u, 0u, 0u};
            if (s < ns) {
                const int k0 = kg + s * kAbsKSlab;
                wv[s] = *reinterpret_cast<const u32x4_t *>(wh + (int64_t)(k0 + srow) * p.N + n0 +
                                                           scol);
                if (row_ok) xv[s] = *reinterpret_cast<const u32x4_t *>(xrow + k0 + 8 * g);
            }
        }
        __syncthreads();   // the previous group fully consumed
#pragma unroll
        for (int s = 0; s < G; ++s)
            if (s < ns)
                *reinterpret_cast<u32x4_t *>(wt + (s * kAbsKSlab + srow) * kWStride + scol) = wv[s];
        __syncthreads();
#pragma unroll
        for (int s = 0; s < G; ++s) {
            if (s < ns) {
#pragma unroll
                for (int mb = 0; mb < 4; ++mb) {
                    const short *base = wt + (s * kAbsKSlab + tr_row) * kWStride + 16 * mb + tr_col;
                    const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (i16x4_t __attribute__((address_space(3))) *)(base));
                    const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (i16x4_t __attribute__((address_space(3))) *)(base + 4 * kWStride));
                    const i16x8_t a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                    acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, xv[s]),
                        acc[mb], 0, 0, 0);
                }
            }
        }
    }

    if (!row_ok) return;
    uint16_t *yrow = p.y + (int64_t)brow * p.y_sb + (int64_t)h * p.y_sh + n0;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
        u32x2_t v;
        v[0] = pack_bf16x2(acc[mb][0], acc[mb][1]);
        v[1] = pack_bf16x2(acc[mb][2], acc[mb][3]);
        *reinterpret_cast<u32x2_t *>(yrow + 16 * mb + 4 * g) = v;
    }
}

hipError_t launch_absorb(const AbsorbParams &p, int heads, hipStream_t stream)
{
    const int tiles = (p.N / kAbsBN) * ((p.batch + kAbsBM - 1) / kAbsBM);
    const dim3 grid((unsigned)((heads + 7) / 8 * 8) * (unsigned)tiles);
    if (p.K == 4 * kAbsKSlab)
        hipLaunchKernelGGL(absorb_kernel<4>, grid, dim3(kAbsThreads), 0, stream, p);
    else if (p.K == 16 * kAbsKSlab)
        hipLaunchKernelGGL(absorb_kernel<16>, grid, dim3(kAbsThreads), 0, stream, p);
    else
        hipLaunchKernelGGL(absorb_kernel<8>, grid, dim3(kAbsThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace mla
