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
// The accumulator layout puts 4 consecutive output columns in each lane;
// two lane swaps regroup them so that stores are 16 bytes.  Consecutive
// workgroup numbers go to the eight XCDs in turn, and each XCD has its own
// L2: the grid is numbered so that all tiles of a head share an XCD (number
// L -> XCD L % 8, head L % 8 + 8 ((L / 8) / tiles per head)), which keeps a
// head's x rows and W slabs in one L2 instead of fetching them from HBM once
// per XCD.  With fewer than 8 heads (one head with the heads folded into K
// is a plain matmul) the tiles are numbered in order instead, so that all
// XCDs share the work.
//
// The same PR stores the weights in fp8 and decompresses them to 16-bit
// floats for the bmm.  With fp8 weights (OCP E4M3 codes, one fp32 scale per
// 128 x 128 block) each thread loads 8 codes per slab instead of 8 bf16
// (half the weight bytes) and decompresses them in registers before the LDS
// stage; the rest of the kernel is the bf16 one.
#include <algorithm>

#include "mla_device.h"
#include "kernels.h"

namespace mla {

constexpr int kAbsThreads = 256;
constexpr int kAbsBM = 64;              // batch rows per workgroup (16 per wave)
constexpr int kAbsBN = 64;              // output columns per workgroup
constexpr int kAbsKSlab = 32;           // k rows per slab (one 16-byte load per thread)
constexpr int kWStride = kAbsBN + 8;    // bf16 per staged row (144 B)
constexpr int kFp8Block = 128;          // scale block of fp8 weights (k and n)

// fp8 weights: gfx950 decodes OCP E4M3 codes to fp32 exactly
// (v_cvt_pk_f32_fp8).  The weight is bf16(code * scale), the exact product
// rounded once to nearest even.  The fp32 product p = RN(code * scale) cannot
// step over a bf16 rounding midpoint (midpoints are fp32 values), so
// rounding p to bf16 (v_cvt_pk_bf16_f32, nearest even) is already right
// unless p lies exactly on a midpoint while the exact product does not;
// there the product's rounding error (exact, by fma) picks the side.
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t round_scaled_bf16x2(float v0, float v1, float scale)
{
    const float p0 = v0 * scale, p1 = v1 * scale;
    uint32_t r = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{p0, p1}, bf16x2_v));
    const uint32_t u0 = __float_as_uint(p0), u1 = __float_as_uint(p1);
    if (__builtin_expect(((u0 & 0xFFFFu) == 0x8000u) | ((u1 & 0xFFFFu) == 0x8000u), 0)) {
        const float e0 = __builtin_fmaf(v0, scale, -p0), e1 = __builtin_fmaf(v1, scale, -p1);
        if ((u0 & 0xFFFFu) == 0x8000u && e0 != 0.f)
            r = (r & 0xFFFF0000u) | ((((e0 > 0.f) == (p0 > 0.f)) ? u0 + 0x8000u : u0) >> 16);
        if ((u1 & 0xFFFFu) == 0x8000u && e1 != 0.f)
            r = (r & 0xFFFFu) | ((((e1 > 0.f) == (p1 > 0.f)) ? u1 + 0x8000u : u1) & 0xFFFF0000u);
    }
    return r;
}
// One (head, 64 x 64 output tile) work item: item number idx -> head and
// tile.  With 8 heads or more, item idx lands on head (idx % 8) + 8 ((idx /
// 8) / tiles): a persistent grid whose size is a multiple of 8 keeps item
// idx on the XCD of workgroup idx % 8, so all tiles of a head share one L2.
// With fewer heads (one head with the heads folded into K is a plain matmul)
// items are numbered in order, so that every XCD gets work.
struct AbsItem {
    int h, n0, m0;
};

__device__ __forceinline__ AbsItem abs_item(const AbsorbParams &p, int idx, int tiles, int ntn)
{
    int h, t;
    if (p.heads >= 8) {
        const int k8 = idx >> 3;
        h = (idx & 7) + 8 * (k8 / tiles);
        t = k8 % tiles;
    } else {
        h = idx / tiles;
        t = idx % tiles;
    }
    return AbsItem{h, (t % ntn) * kAbsBN, (t / ntn) * kAbsBM};
}

// The registers one step loads: G 32-row slabs of W's 64-column slab (bf16,
// or fp8 codes and their block scale) and of this lane's x row.
template <int G>
struct AbsRegs {
    u32x4_t wv[G], xv[G];
    u32x2_t wq[G];
    float wsc[G];
};

// A workgroup walks its items (idx = blockIdx.x, + gridDim.x, ...) and, in
// each, the groups of G slabs along K.  Every step issues the next step's
// global loads before it stages and multiplies the current one, so one
// step's loads are always in flight behind the matrix work; W's slab goes
// through one of two LDS buffers (one barrier per step: a buffer is written
// again only two steps later, after every wave has passed the barrier that
// follows its last reads).
template <int G, bool kFp8>
__global__ __launch_bounds__(kAbsThreads, 2) void absorb_kernel(AbsorbParams p, int total_items)
{
    __shared__ __attribute__((aligned(16))) short wt[2][G * kAbsKSlab * kWStride];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int r16 = lane & 15;
    const int g = lane >> 4;
    const int ntn = p.N / kAbsBN;
    const int tiles = ntn * ((p.batch + kAbsBM - 1) / kAbsBM);   // per head
    const int ngroups = (p.K + G * kAbsKSlab - 1) / (G * kAbsKSlab);
    const int kblocks = (p.K + kFp8Block - 1) / kFp8Block;
    const int nblocks = (p.N + kFp8Block - 1) / kFp8Block;
    // staging: thread t copies 16 bytes of each slab: row t / 8, columns 8 * (t % 8)
    const int srow = threadIdx.x >> 3;
    const int scol = 8 * (threadIdx.x & 7);
    // transposed-read address: lane 16g + 4e + c -> slab row 8g + e, column 4c
    const int tr_row = 8 * g + (r16 >> 2);
    const int tr_col = 4 * (r16 & 3);

    // the next item of this workgroup at or after idx (padding heads skipped)
    auto next_item = [&](int idx) {
        while (idx < total_items && abs_item(p, idx, tiles, ntn).h >= p.heads) idx += gridDim.x;
        return idx;
    };
    // Every step issues the same number of global loads, without branches
    // and without touching their results (slabs past K re-read the group's
    // last slab and are not used; rows past the batch read row 0, which only
    // feeds output rows that are never stored), so the wait before a step's
    // staging can leave the next step's loads in flight.
    auto load = [&](AbsRegs<G> &r, const AbsItem &it, int grp) {
        const int kg = grp * G * kAbsKSlab;
        const int ns = min(G, (p.K - kg) / kAbsKSlab);   // slabs in this group (uniform)
        const int brow = it.m0 + wave * 16 + r16;
        const uint16_t *xrow =
            p.x + (int64_t)(brow < p.batch ? brow : 0) * p.x_sb + (int64_t)it.h * p.x_sh;
        const uint16_t *wh = p.w + (int64_t)it.h * p.K * p.N;
        const uint8_t *w8h = p.w8 + (int64_t)it.h * p.K * p.N;
        // a 64-column tile lies inside one 128-column scale block
        const float *sch = p.wscale + ((int64_t)it.h * kblocks) * nblocks + it.n0 / kFp8Block;
#pragma unroll
        for (int s = 0; s < G; ++s) {
            const int k0 = kg + min(s, ns - 1) * kAbsKSlab;
            // the weights are read once per call: non-temporal, so that the
            // caches keep the x rows the head's other column tiles re-read
            if (kFp8) {
                r.wq[s] = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t *>(
                    w8h + (int64_t)(k0 + srow) * p.N + it.n0 + scol));
                r.wsc[s] = sch[(k0 / kFp8Block) * nblocks];
            } else {
                r.wv[s] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(
                    wh + (int64_t)(k0 + srow) * p.N + it.n0 + scol));
            }
            r.xv[s] = *reinterpret_cast<const u32x4_t *>(xrow + k0 + 8 * g);
        }
    };

    int idx = next_item(blockIdx.x);
    if (idx >= total_items) return;   // uniform
    AbsItem cur = abs_item(p, idx, tiles, ntn);
    int grp = 0, buf = 0;
    f32x4_t acc[4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) acc[mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // one step: prefetch the next step into `nx`, then stage and multiply `cr`;
    // false when this was the workgroup's last step
    auto step = [&](AbsRegs<G> &cr, AbsRegs<G> &nx) {
        int nidx = idx, ngrp = grp + 1;
        if (ngrp == ngroups) {
            ngrp = 0;
            nidx = next_item(idx + gridDim.x);
        }
        const bool more = nidx < total_items;
        const AbsItem nit = more ? abs_item(p, nidx, tiles, ntn) : cur;
        // the last step re-reads its own group (unused), keeping the load count fixed
        load(nx, nit, more ? ngrp : grp);
        __builtin_amdgcn_sched_barrier(0);   // the next loads go out before this step's work

        const int ns = min(G, (p.K - grp * G * kAbsKSlab) / kAbsKSlab);
        if (kFp8) {
            // decompress to bf16 in registers, in the layout of the bf16 path
            // (byte i of a word is code i; the pair form decodes bytes 0-1 or 2-3)
#pragma unroll
            for (int s = 0; s < G; ++s)
#pragma unroll
                for (int jw = 0; jw < 2; ++jw) {
                    const f32x2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)cr.wq[s][jw], false);
                    const f32x2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)cr.wq[s][jw], true);
                    cr.wv[s][2 * jw] = round_scaled_bf16x2(lo[0], lo[1], cr.wsc[s]);
                    cr.wv[s][2 * jw + 1] = round_scaled_bf16x2(hi[0], hi[1], cr.wsc[s]);
                }
        }
        short *wb = wt[buf];
#pragma unroll
        for (int s = 0; s < G; ++s)
            if (s < ns)
                *reinterpret_cast<u32x4_t *>(wb + (s * kAbsKSlab + srow) * kWStride + scol) =
                    cr.wv[s];
        __syncthreads();
#pragma unroll
        for (int s = 0; s < G; ++s) {
            if (s < ns) {
#pragma unroll
                for (int mb = 0; mb < 4; ++mb) {
                    const short *base = wb + (s * kAbsKSlab + tr_row) * kWStride + 16 * mb + tr_col;
                    const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (i16x4_t __attribute__((address_space(3))) *)(base));
                    const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (i16x4_t __attribute__((address_space(3))) *)(base + 4 * kWStride));
                    const i16x8_t a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                    acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, cr.xv[s]),
                        acc[mb], 0, 0, 0);
                }
            }
        }
        if (grp == ngroups - 1) {
            // the item is complete: its 64 x 64 tile goes out.  Lane (r16, g)
            // holds columns 16 mb + 4g .. + 4 of row r16; a swap 32 lanes apart
            // and one 16 lanes apart (all four lanes of a row take part) leave
            // lane (r16, g) columns 32 i + 8g .. + 8 in pair i, so each store
            // writes 16 bytes and a row's four lanes 64 contiguous bytes
            const int brow = cur.m0 + wave * 16 + r16;
            if (brow < p.batch) {
                uint16_t *yrow = p.y + (int64_t)brow * p.y_sb + (int64_t)cur.h * p.y_sh + cur.n0;
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    uint32_t x[2], z[2];
#pragma unroll
                    for (int k = 0; k < 2; ++k) {
                        const auto a = __builtin_amdgcn_permlane32_swap(
                            pack_bf16x2(acc[2 * i][2 * k], acc[2 * i][2 * k + 1]),
                            pack_bf16x2(acc[2 * i + 1][2 * k], acc[2 * i + 1][2 * k + 1]), false, false);
                        const auto b = __builtin_amdgcn_permlane16_swap(a[0], a[1], false, false);
                        x[k] = b[0];
                        z[k] = b[1];
                    }
                    *reinterpret_cast<u32x4_t *>(yrow + 32 * i + 8 * g) = u32x4_t{x[0], x[1], z[0], z[1]};
                }
            }
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) acc[mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
        idx = nidx;
        grp = ngrp;
        cur = nit;
        buf ^= 1;
        return more;
    };

    AbsRegs<G> ra, rb;
    load(ra, cur, 0);
    // two steps per trip, so the register sets alternate without copies
    while (step(ra, rb) && step(rb, ra)) {
    }
}

int absorb_grid_cap()
{
    // two workgroups per CU of the current device (cached per device)
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 512;
    if (cached[dev] == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            cus < 1)
            cus = 256;
        cached[dev] = 2 * cus;
    }
    return cached[dev];
}

template <int G>
void launch_group(const AbsorbParams &p, int total_items, hipStream_t stream)
{
    int grid = std::min(total_items, absorb_grid_cap());
    if (grid >= 8) grid -= grid % 8;   // keeps each item on the XCD of workgroup idx % 8
    if (p.w8 != nullptr)
        hipLaunchKernelGGL((absorb_kernel<G, true>), dim3(grid), dim3(kAbsThreads), 0, stream, p,
                           total_items);
    else
        hipLaunchKernelGGL((absorb_kernel<G, false>), dim3(grid), dim3(kAbsThreads), 0, stream, p,
                           total_items);
}

hipError_t launch_absorb(const AbsorbParams &p, int heads, hipStream_t stream)
{
    const int tiles = (p.N / kAbsBN) * ((p.batch + kAbsBM - 1) / kAbsBM);
    const int total = (heads >= 8 ? (heads + 7) / 8 * 8 : heads) * tiles;
    if (p.K == 4 * kAbsKSlab) launch_group<4>(p, total, stream);
    else launch_group<8>(p, total, stream);
    return hipGetLastError();
}

}  // namespace mla
