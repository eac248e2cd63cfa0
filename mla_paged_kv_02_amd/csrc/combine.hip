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
// call each of its rows is cut into S = heavy_slices(k) slices of 512 / S
// dims, and one workgroup merges one row's slice: its 256 lanes are groups
// of 128 / S lanes, one 16-byte load each per split, and group g takes splits
// g, g + G, g + 2G, ... (G groups), loading their lse values and partial
// rows together, up to 16 of each per lane in flight -- one memory round trip
// for up to 16 G splits (S is chosen so that covers 33..511 splits).  Each
// lane keeps a running maximum, sum and weighted sum of its own splits, which
// the lanes of a wave and then the four waves fold together through LDS.
// The extra workgroups (numbered after the sequences) come from the
// schedule; nothing is written but the merged rows.  The standalone entry
// point merges such sequences with all four waves on each row instead.
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

// A lane's 8 dims of a row: acc[0..3] = dims 4 lane .. + 3 and acc[4..7] =
// dims 256 + 4 lane .. + 3, so each load or store instruction of a wave
// covers one contiguous half row.
constexpr int kHalfDv = kDv / 2;

__device__ __forceinline__ void store_row(const CombineParams &p, int b, int row, int lane,
                                          const float acc[8], float lse_v)
{
    uint16_t *dst = p.out + ((int64_t)b * p.rows + row) * kDv + 4 * lane;
    *reinterpret_cast<u32x2_t *>(dst) = u32x2_t{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
    *reinterpret_cast<u32x2_t *>(dst + kHalfDv) =
        u32x2_t{pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7])};
    if (lane == 0) p.lse[(int64_t)b * p.rows + row] = lse_v;
}

// acc += sum over this wave's splits s = s_begin, s_begin + stride, ... < ns
// of w(s) * o_part[s][row][the lane's 8 dims], up to 8 loads in flight
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
                const float *src = o_row + s * split_stride + 4 * lane;
                a[u] = *reinterpret_cast<const f32x4_t *>(src);
                c[u] = *reinterpret_cast<const f32x4_t *>(src + kHalfDv);
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
                const float *src = o_row + u * slot_stride + 4 * lane;
                a[u] = *reinterpret_cast<const f32x4_t *>(src);
                c[u] = *reinterpret_cast<const f32x4_t *>(src + kHalfDv);
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

// Running log-sum-exp state of a set of splits: the maximum m of their lse
// values, l = sum exp(lse_s - m) and acc = sum exp(lse_s - m) o_s over 4 dims
// (m = -inf, l = 0, acc = 0 for none).  fold() adds another such state.
struct MergeState {
    float m, l;
    f32x4_t acc;
    __device__ __forceinline__ void fold(float m2, float l2, const f32x4_t &acc2)
    {
        const float M = fmaxf(m, m2);
        const float c1 = m == -INFINITY ? 0.f : fast_exp2((m - M) * kLog2e);
        const float c2 = m2 == -INFINITY ? 0.f : fast_exp2((m2 - M) * kLog2e);
        l = l * c1 + l2 * c2;
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = acc[e] * c1 + acc2[e] * c2;
        m = M;
    }
};

constexpr int kHeavyInflight = 16;

// One workgroup of a heavy sequence's merge inside a decode call: item z of
// the row group blockIdx.x is row (z % 4) of the group, dim slice z / 4.
__device__ __forceinline__ void merge_heavy_slice(const CombineParams &p, int b, int z, int first,
                                                  int ns, int lane, int wave, float *lds_f,
                                                  float *red)
{
    const int row = blockIdx.x * kCombineRows + z % kCombineRows;
    if (row >= p.rows) return;                         // uniform over the workgroup
    const int S = heavy_slices(ns);
    const int width = kDv / S;                         // dims of the slice: 256 .. 32
    const int lanes = width / 4;                       // lanes per split: 64 .. 8
    const int groups = kCombineThreads / lanes;        // G: 4 .. 32
    const int g = (int)threadIdx.x / lanes;
    const int d = (z / kCombineRows) * width + 4 * (lane % lanes);
    const int64_t split_stride = (int64_t)p.rows * kDv;
    const float *o_row = p.o_part + ((int64_t)first * p.rows + row) * kDv + d;
    const float *lse_col = p.lse_part + (int64_t)first * p.rows + row;

    MergeState st{-INFINITY, 0.f, f32x4_t{0.f, 0.f, 0.f, 0.f}};
    for (int base = 0; base < ns; base += groups * kHeavyInflight) {   // uniform
        float ls[kHeavyInflight];
        f32x4_t o[kHeavyInflight];
#pragma unroll
        for (int u = 0; u < kHeavyInflight; ++u) {
            const int s = base + g + groups * u;
            ls[u] = -INFINITY;
            if (s < ns) {
                ls[u] = lse_col[(int64_t)s * p.rows];
                o[u] = *reinterpret_cast<const f32x4_t *>(o_row + s * split_stride);
            }
        }
        float mb = st.m;
#pragma unroll
        for (int u = 0; u < kHeavyInflight; ++u) mb = fmaxf(mb, ls[u]);
        if (mb == -INFINITY) continue;                 // no non-empty split yet
        const float c = fast_exp2((st.m - mb) * kLog2e);   // 0 while st.m = -inf
        st.l *= c;
#pragma unroll
        for (int e = 0; e < 4; ++e) st.acc[e] *= c;
#pragma unroll
        for (int u = 0; u < kHeavyInflight; ++u) {
            if (ls[u] == -INFINITY) continue;          // absent or empty: its o is not used
            const float w = fast_exp2((ls[u] - mb) * kLog2e);
            st.l += w;
#pragma unroll
            for (int e = 0; e < 4; ++e) st.acc[e] += w * o[u][e];
        }
        st.m = mb;
    }
    // the wave's groups (lanes lanes apart), then the four waves
    for (int off = lanes; off < 64; off <<= 1) {
        f32x4_t a2;
#pragma unroll
        for (int e = 0; e < 4; ++e) a2[e] = __shfl_xor(st.acc[e], off);
        st.fold(__shfl_xor(st.m, off), __shfl_xor(st.l, off), a2);
    }
    if (wave > 0 && lane < lanes) {
        *reinterpret_cast<f32x4_t *>(lds_f + (wave - 1) * kDv + 4 * lane) = st.acc;
        if (lane == 0) {
            red[2 * wave] = st.m;
            red[2 * wave + 1] = st.l;
        }
    }
    __syncthreads();
    if (wave > 0 || lane >= lanes) return;
#pragma unroll
    for (int w = 1; w < kCombineWaves; ++w)
        st.fold(red[2 * w], red[2 * w + 1],
                *reinterpret_cast<const f32x4_t *>(lds_f + (w - 1) * kDv + 4 * lane));
    const int64_t out_row = (int64_t)b * p.rows + row;
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    float lse_v = -INFINITY;
    if (st.m != -INFINITY) {
        const float inv = 1.f / st.l;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = st.acc[e] * inv;
        lse_v = st.m + fast_log2(st.l) * kLn2;
    }
    uint2 packed;
    packed.x = pack_bf16x2(v[0], v[1]);
    packed.y = pack_bf16x2(v[2], v[3]);
    *reinterpret_cast<uint2 *>(p.out + out_row * kDv + d) = packed;
    if (d == 0) p.lse[out_row] = lse_v;
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

// The standalone merge of a heavy sequence: the four waves merge each of the
// block's rows together.
__device__ __forceinline__ void merge_heavy_rows(const CombineParams &p, int b, int first, int ns,
                                                 int lane, int wave, float *lds_f, float *red)
{
    const int64_t split_stride = (int64_t)p.rows * kDv;
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
            float *dst = lds_f + (wave - 1) * kDv + 8 * lane;
            *reinterpret_cast<f32x4_t *>(dst) = f32x4_t{acc[0], acc[1], acc[2], acc[3]};
            *reinterpret_cast<f32x4_t *>(dst + 4) = f32x4_t{acc[4], acc[5], acc[6], acc[7]};
        }
        __syncthreads();
        if (wave == 0) {
#pragma unroll
            for (int w = 0; w < kCombineWaves - 1; ++w)
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[e] += lds_f[w * kDv + 8 * lane + e];
            store_row(p, b, row, lane, acc, lse_v);
        }
        __syncthreads();   // red and lds_f are reused by the next row
    }
}

// kSliced: inside a decode call (heavy sequences merged in dim slices by the
// schedule's extra workgroups); otherwise the standalone merge (four waves
// per row of a heavy sequence).  Two instantiations, so that the decode's
// merge does not carry the register needs of the standalone path.
template <bool kSliced>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(CombineParams p, int batch)
{
    __shared__ float red[2 * kCombineWaves];
    __shared__ __attribute__((aligned(16))) float lds_f[(kCombineWaves - 1) * kDv];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    // workgroup y < batch: sequence y, chunk 0; later ones: extra chunks of
    // heavy sequences
    int b = blockIdx.y, z = 0;
    if (b >= batch) {
        if (!kSliced) return;
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

    if constexpr (kSliced) {
        merge_heavy_slice(p, b, z, first, ns, lane, wave, lds_f, red);
    } else {
        merge_heavy_rows(p, b, first, ns, lane, wave, lds_f, red);
    }
}

hipError_t launch_combine(const CombineParams &p, int batch, int extra_wgs, hipStream_t stream)
{
    const dim3 grid((p.rows + kCombineWaves - 1) / kCombineWaves, batch + extra_wgs);
    if (p.extra_off != nullptr)
        hipLaunchKernelGGL(combine_kernel<true>, grid, dim3(kCombineThreads), 0, stream, p, batch);
    else
        hipLaunchKernelGGL(combine_kernel<false>, grid, dim3(kCombineThreads), 0, stream, p,
                           batch);
    return hipGetLastError();
}

}  // namespace mla
