// decode_wide.hip -- paged MLA decode for 128-row query tiles (h_q * s_q a
// multiple of 128), where QK^T and PV are dense enough to be MFMA-bound.
//
// Same operation as decode.hip: softmax(scale * Q K^T) V per query row over
// the 64-token paged latent cache (FlashMLA, "DeepSeek publica FlashMLA como
// codigo abierto", release bullets), K = the 576-wide row, V its first 512
// dims.  Here one workgroup carries 128 query rows over a scheduler part, so
// every cache byte it stages feeds 128 rows of MFMA work.
//
// gfx950 mapping:
//  * 4 waves; wave w owns query rows [32w, 32w + 32) of the tile over all
//    512 value dims (O^T: 16 blocks of 32x32 fp32 = 256 accumulator
//    registers) and keeps its Q^T fragments in registers (36 k-steps of 16
//    dims), so no cross-wave merge is ever needed.
//  * The cache streams through LDS in 32-token tiles (36,864 B), filled by
//    direct global->LDS DMA (buffer_load ... lds, 16 B per lane) three tiles
//    ahead; tokens outside the part arrive as zeros through the buffer
//    descriptor's range check.  A tile never crosses a page (tiles are
//    32-token aligned).  The 16-byte chunk index is XOR-swizzled per row so
//    both read patterns below are free of bank conflicts.
//  * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (A = K from LDS with
//    ds_read_b128, B = Q^T from registers).  Its accumulator layout holds 16
//    keys of one query row per lane, which is directly the P^T operand of the
//    value product (keys mapped consistently on both sides).
//  * O^T += V^T P^T on the same MFMA; V^T fragments come from LDS through
//    ds_read_b64_tr_b16 (two 4-key reads per 8-key operand).
//  * Online softmax in fp32, log2 domain, with exact and bf16-rounded sums as
//    in decode.hip.  O is never rescaled inside the tile loop (it lives in
//    the 256 accumulator registers, and any VALU rescale would force copies
//    of all of them through VGPRs): a row's first visible key sets its
//    exponent origin, and if a later score exceeds the origin by more than
//    64 (weights stay below 2^64, far from fp32 overflow) the workgroup
//    redoes the segment with the larger origin.  Real attention scores never
//    grow like that after the first key, so the redo is a correctness path.
#include "mla_device.h"
#include "kernels.h"

namespace mla {

constexpr int kWWaves = 4;
constexpr int kWThreads = kWWaves * 64;
constexpr int kWRows = 32 * kWWaves;                 // 128 query rows per workgroup
static_assert(kWRows == kWideRows, "row tile of the wide kernel");
constexpr int kTileKeys = 32;
constexpr int kRowChunks = kDqk / 8;                 // 72 chunks of 16 B per cache row
constexpr int kTileChunks = kTileKeys * kRowChunks;  // 2304
constexpr int kTileBytes = kTileChunks * 16;         // 36864
constexpr int kStages = 3;                           // tiles in LDS (two in flight)
constexpr int kDmaPerWave = kTileChunks / 64 / kWWaves;   // 9 instructions of 1 KB
constexpr int kKSteps = kDqk / 16;                   // 36
constexpr int kDBlocks = kDv / 32;                   // 16
constexpr float kWOriginSlack = 64.0f;   // log2 units
constexpr int kPvAhead = 2;              // value fragments (pairs of reads) read ahead

typedef char __attribute__((address_space(3))) lds_char_t;

// chunk swizzle: row r's 16-byte chunk c lives at slot 72 r + (c ^ swz(r))
__device__ __forceinline__ int swz(int r) { return ((2 * (r & 7)) ^ ((r >> 2) & 3)) & 7; }
__device__ __forceinline__ int slot_of(int r, int c) { return kRowChunks * r + (c ^ swz(r)); }

// This wave's share of the DMA for tile T (tokens [32T, 32T + 32)) of one
// sequence.  LDS slot q = 64 i + lane of instruction i receives cache chunk
// (r, c) with slot_of(r, c) = q.  Tokens outside [kbeg, kend) read as zero.
__device__ __forceinline__ void dma_tile(lds_char_t *buf, const uint16_t *kv, int page, int T,
                                         int kbeg, int kend, int wave, int lane)
{
    const __amdgpu_buffer_rsrc_t rsrc =
        make_rsrc(reinterpret_cast<const char *>(kv) + (int64_t)page * kPageBytes, kPageBytes);
    const int row0 = (T & 1) * kTileKeys;   // tile's first row inside its page
    // recompute the per-lane offsets each tile rather than keep 9 of them live
    asm volatile("" : "+v"(lane));
#pragma unroll
    for (int u = 0; u < kDmaPerWave; ++u) {
        const int i = wave * kDmaPerWave + u;
        const int q = 64 * i + lane;
        const int r = q / kRowChunks;
        const int c = (q - kRowChunks * r) ^ swz(r);
        const int key = T * kTileKeys + r;
        const int voff =
            (key >= kbeg && key < kend) ? (row0 + r) * kRowBytes + 16 * c : 0x40000000;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (void __attribute__((address_space(3))) *)(buf + 1024 * i), 16, voff, 0, 0, 0);
    }
}

// S^T[32 keys][32 rows] = K Q^T over the 576 dims of one 32-token tile: 36
// v_mfma_f32_32x32x16_bf16 with A = K rows from LDS (ds_read_b128, four in
// flight) and B = Q^T from registers.  The chain is written out here so that
// its accumulator lives in VGPRs while the value accumulators occupy all 256
// AGPRs.  Hazards the compiler cannot see inside the block are covered in
// it: each MFMA waits for its own K fragment (LDS returns in order), chained
// MFMAs accumulate into exactly the same registers (forwarded back to back),
// and 24 wait states after the last one cover the longest XDL-write ->
// VALU-access requirement (12 on gfx950) before the caller reads S.
#define MLA_QF(i) "v"(qf[i])
__device__ __forceinline__ void qk_tile(f32x16_t &s, const int kb[4], const bf16x8_t qf[kKSteps])
{
    bf16x8_t k0, k1, k2, k3;
    asm volatile(
        "ds_read_b128 %1, %5\n"
        "ds_read_b128 %2, %6\n"
        "ds_read_b128 %3, %7\n"
        "ds_read_b128 %4, %8\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %1, %9, 0\n"
        "ds_read_b128 %1, %5 offset:128\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %2, %10, %0\n"
        "ds_read_b128 %2, %6 offset:128\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %3, %11, %0\n"
        "ds_read_b128 %3, %7 offset:128\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %4, %12, %0\n"
        "ds_read_b128 %4, %8 offset:128\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %1, %13, %0\n"
        "ds_read_b128 %1, %5 offset:256\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %2, %14, %0\n"
        "ds_read_b128 %2, %6 offset:256\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %3, %15, %0\n"
        "ds_read_b128 %3, %7 offset:256\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %4, %16, %0\n"
        "ds_read_b128 %4, %8 offset:256\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %1, %17, %0\n"
        "ds_read_b128 %1, %5 offset:384\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %2, %18, %0\n"
        "ds_read_b128 %2, %6 offset:384\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %3, %19, %0\n"
        "ds_read_b128 %3, %7 offset:384\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %4, %20, %0\n"
        "ds_read_b128 %4, %8 offset:384\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %1, %21, %0\n"
        "ds_read_b128 %1, %5 offset:512\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %2, %22, %0\n"
        "ds_read_b128 %2, %6 offset:512\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %3, %23, %0\n"
        "ds_read_b128 %3, %7 offset:512\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %4, %24, %0\n"
        "ds_read_b128 %4, %8 offset:512\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %1, %25, %0\n"
        "ds_read_b128 %1, %5 offset:640\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %2, %26, %0\n"
        "ds_read_b128 %2, %6 offset:640\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %3, %27, %0\n"
        "ds_read_b128 %3, %7 offset:640\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %4, %28, %0\n"
        "ds_read_b128 %4, %8 offset:640\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %1, %29, %0\n"
        "ds_read_b128 %1, %5 offset:768\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %2, %30, %0\n"
        "ds_read_b128 %2, %6 offset:768\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %3, %31, %0\n"
        "ds_read_b128 %3, %7 offset:768\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %4, %32, %0\n"
        "ds_read_b128 %4, %8 offset:768\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %1, %33, %0\n"
        "ds_read_b128 %1, %5 offset:896\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %2, %34, %0\n"
        "ds_read_b128 %2, %6 offset:896\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %3, %35, %0\n"
        "ds_read_b128 %3, %7 offset:896\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %4, %36, %0\n"
        "ds_read_b128 %4, %8 offset:896\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %1, %37, %0\n"
        "ds_read_b128 %1, %5 offset:1024\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %2, %38, %0\n"
        "ds_read_b128 %2, %6 offset:1024\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %3, %39, %0\n"
        "ds_read_b128 %3, %7 offset:1024\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %4, %40, %0\n"
        "ds_read_b128 %4, %8 offset:1024\n"
        "s_waitcnt lgkmcnt(3)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %1, %41, %0\n"
        "s_waitcnt lgkmcnt(2)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %2, %42, %0\n"
        "s_waitcnt lgkmcnt(1)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %3, %43, %0\n"
        "s_waitcnt lgkmcnt(0)\n"
        "v_mfma_f32_32x32x16_bf16 %0, %4, %44, %0\n"
        "s_nop 7\n"
        "s_nop 7\n"
        "s_nop 7\n"
        : "=&v"(s), "=&v"(k0), "=&v"(k1), "=&v"(k2), "=&v"(k3)
        : "v"(kb[0]), "v"(kb[1]), "v"(kb[2]), "v"(kb[3]),
          MLA_QF(0), MLA_QF(1), MLA_QF(2), MLA_QF(3), MLA_QF(4), MLA_QF(5), MLA_QF(6),
          MLA_QF(7), MLA_QF(8), MLA_QF(9), MLA_QF(10), MLA_QF(11), MLA_QF(12), MLA_QF(13),
          MLA_QF(14), MLA_QF(15), MLA_QF(16), MLA_QF(17), MLA_QF(18), MLA_QF(19), MLA_QF(20),
          MLA_QF(21), MLA_QF(22), MLA_QF(23), MLA_QF(24), MLA_QF(25), MLA_QF(26), MLA_QF(27),
          MLA_QF(28), MLA_QF(29), MLA_QF(30), MLA_QF(31), MLA_QF(32), MLA_QF(33), MLA_QF(34),
          MLA_QF(35)
        : "memory");
}
#undef MLA_QF

struct WideRow {
    float m;    // exponent origin (log2 units), -inf before the first visible key
    float l;    // this lane's share of sum 2^(s - m) (gives the lse)
    float lr;   // the same over the bf16-rounded weights (normalizes the output)
};

__global__ __launch_bounds__(kWThreads, 1) void decode_wide_kernel(
    DecodeParams p, const int32_t *__restrict__ bt, const int32_t *__restrict__ seqlens,
    const int32_t *__restrict__ meta)
{
    __shared__ __attribute__((aligned(1024))) char tiles[kStages * kTileBytes];
    // redo requests, by tile parity: a flag written while tile t is processed
    // is read only after the barrier that opens tile t + 1, and written again
    // no earlier than tile t + 2 (after the next barrier), so every wave reads
    // the same value
    __shared__ int redo[2];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n32 = lane & 31;        // query row of this lane inside the wave's block
    const int g = lane >> 5;          // half: keys 4g.. of each 8-key group
    const int part = blockIdx.x;
    const int rt = blockIdx.y;
    const int R = p.s_q * p.h_q;

    const int32_t *rec = meta + part * kPartInts;
    const int s0 = rec[0];
    if (s0 < 0) return;
    const int t0 = rec[1], s1 = rec[2], t1 = rec[3], slot0 = rec[4];
    const int32_t *split_off = meta + p.num_parts * kPartInts;
    lds_char_t *lds = (lds_char_t *)tiles;
    const int lds_addr = (int)(uintptr_t)lds;
    if (threadIdx.x == 0) redo[0] = redo[1] = 0;

    // K^T fragment (A operand) of k-step kk: row n32, chunk 2kk + g, i.e.
    // slot 72 n32 + 8 (kk / 4) + ((2 (kk % 4) + g) ^ swz(n32))
    const int ksw = swz(n32);
    int kbase[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) kbase[j] = 16 * (kRowChunks * n32 + ((2 * j + g) ^ ksw));

    // V^T fragment addresses: lane 16G + 4e + c (G: g' = G >> 1, h = G & 1)
    // points at key 16 kk + 4 g' + e (+8), dims 32d + 16h + 4c .. +3, which is
    // chunk 4d + 2h + c/2 = 8 (d / 2) + (4 (d % 2) + 2h + c/2), half c % 2
    int vbase[2][2][2];   // [kk][second read][d parity]
    {
        const int trG = lane >> 4;
        const int tg = trG >> 1, th = trG & 1;
        const int te = (lane >> 2) & 3, tc = lane & 3;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int rd = 0; rd < 2; ++rd) {
                const int key = 16 * kk + 4 * tg + te + 8 * rd;
#pragma unroll
                for (int par = 0; par < 2; ++par)
                    vbase[kk][rd][par] =
                        16 * (kRowChunks * key + ((4 * par + 2 * th + (tc >> 1)) ^ swz(key))) +
                        8 * (tc & 1);
            }
    }

    for (int seq = s0; seq <= s1; ++seq) {
        const int n = seqlens[seq];
        const int ks = seq == s0 ? t0 : 0;
        const int ke = seq == s1 ? t1 : n;
        if (ks >= ke) continue;
        const int nsplit = split_off[seq + 1] - split_off[seq];
        const int slot = seq == s0 ? slot0 : split_off[seq];
        const int32_t *bt_row = bt + (int64_t)seq * p.bt_stride;
        const int T0 = ks / kTileKeys;
        const int ntiles = (ke + kTileKeys - 1) / kTileKeys - T0;

        const int row = rt * kWRows + 32 * wave + n32;
        int limit = ke;
        if (p.causal) limit = min(ke, n - p.s_q + 1 + row / p.h_q);

        bf16x8_t qf[kKSteps];
        float m_hint = -INFINITY;     // origin floor after a redo
        WideRow st;
        f32x16_t o[kDBlocks];
        for (int attempt = 0;; ++attempt) {
            // start the first tiles' DMA (and, once per segment, the Q^T loads)
#pragma unroll
            for (int sg = 0; sg < kStages - 1; ++sg)
                if (sg < ntiles)
                    dma_tile(lds + sg * kTileBytes, p.kv, bt_row[(T0 + sg) >> 1], T0 + sg, ks,
                             ke, wave, lane);
            if (attempt == 0) {
                const uint16_t *qrow = p.q + ((int64_t)seq * R + row) * kDqk + 8 * g;
#pragma unroll
                for (int kk = 0; kk < kKSteps; ++kk)
                    qf[kk] = *reinterpret_cast<const bf16x8_t *>(qrow + 16 * kk);
            }
            st = WideRow{m_hint, 0.f, 0.f};
            // fragment addresses in the stage of tile 0, advanced per tile
            int kb[4], vb[2][2][2];
#pragma unroll
            for (int j = 0; j < 4; ++j) kb[j] = lds_addr + kbase[j];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                vb[j >> 2][(j >> 1) & 1][j & 1] = lds_addr + vbase[j >> 2][(j >> 1) & 1][j & 1];
#pragma unroll
            for (int d = 0; d < kDBlocks; ++d) o[d] = f32x16_t{};

            for (int t = 0; t < ntiles; ++t) {
                const int T = T0 + t;
                // wait for this wave's part of tile t (tile t + 1 may still be
                // in flight); the barrier makes the tile visible and guarantees
                // every wave is done with tile t - 1, whose buffer the DMA for
                // tile t + 2 reuses
                if (t + 1 < ntiles)
                    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kDmaPerWave) : "memory");
                else
                    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                __syncthreads();
                if (t > 0 && redo[(t - 1) & 1]) break;   // uniform: a redo was asked for
                if (t + kStages - 1 < ntiles)
                    dma_tile(lds + ((t + kStages - 1) % kStages) * kTileBytes, p.kv,
                             bt_row[(T + kStages - 1) >> 1], T + kStages - 1, ks, ke, wave, lane);
                // ---- S^T[32 keys][32 rows] = K Q^T ----
                f32x16_t s;
                qk_tile(s, kb, qf);

                // ---- mask, exponent origin, weights (lane: row n32, keys
                //      8(r/4) + 4g + r%4 of the tile) ----
                float tmax = -INFINITY;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = T * kTileKeys + 8 * (r >> 2) + 4 * g + (r & 3);
                    s[r] = (key >= ks && key < limit) ? s[r] * p.scale_log2 : -INFINITY;
                    tmax = fmaxf(tmax, s[r]);
                }
                tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
                if (st.m == -INFINITY) st.m = tmax;   // first visible key: O, l still 0
                if (tmax > st.m + kWOriginSlack) {    // origin too low: redo the segment
                    m_hint = tmax;
                    redo[t & 1] = 1;
                }
                const float m_use = st.m == -INFINITY ? 0.f : st.m;
                uint32_t pw[8];
#pragma unroll
                for (int r = 0; r < 16; r += 2) {
                    const float e0 = fast_exp2(s[r] - m_use), e1 = fast_exp2(s[r + 1] - m_use);
                    st.l += e0 + e1;
                    pw[r >> 1] = pack_bf16x2(e0, e1);
                    st.lr += bf16_lo(pw[r >> 1]) + bf16_hi(pw[r >> 1]);
                }
                // P^T operand of k-step kk: this lane's weights 8kk .. 8kk+7
                const bf16x8_t pf0 =
                    __builtin_bit_cast(bf16x8_t, u32x4_t{pw[0], pw[1], pw[2], pw[3]});
                const bf16x8_t pf1 =
                    __builtin_bit_cast(bf16x8_t, u32x4_t{pw[4], pw[5], pw[6], pw[7]});

                // ---- O^T[512 dims][32 rows] += V^T P^T ----
                __builtin_amdgcn_sched_barrier(0);
                // step j = 2 d + kk; fragments read kPvAhead steps ahead
                i16x4_t vlo[kPvAhead], vhi[kPvAhead];
#pragma unroll
                for (int j = 0; j < kPvAhead; ++j) {
                    const int d = j >> 1, kk = j & 1, off = 128 * (d >> 1);
                    vlo[j] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (i16x4_t __attribute__((address_space(3))) *)(uintptr_t)(vb[kk][0][d & 1] + off));
                    vhi[j] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (i16x4_t __attribute__((address_space(3))) *)(uintptr_t)(vb[kk][1][d & 1] + off));
                }
#pragma unroll
                for (int j = 0; j < 2 * kDBlocks; ++j) {
                    const int d = j >> 1, kk = j & 1;
                    const i16x4_t lo = vlo[j % kPvAhead], hi = vhi[j % kPvAhead];
                    const i16x8_t a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                    o[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        __builtin_bit_cast(bf16x8_t, a), kk ? pf1 : pf0, o[d], 0, 0, 0);
                    const int nj = j + kPvAhead;
                    if (nj < 2 * kDBlocks) {
                        const int nd = nj >> 1, nkk = nj & 1, off = 128 * (nd >> 1);
                        vlo[j % kPvAhead] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (i16x4_t __attribute__((address_space(3))) *)(uintptr_t)(vb[nkk][0][nd & 1] + off));
                        vhi[j % kPvAhead] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (i16x4_t __attribute__((address_space(3))) *)(uintptr_t)(vb[nkk][1][nd & 1] + off));
                    }
                }
#pragma unroll
                for (int j = 0; j < 2 * kPvAhead; ++j) __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);
#pragma unroll
                for (int j = 0; j < 2 * kDBlocks; ++j) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
                    if (j + kPvAhead < 2 * kDBlocks) __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
                }
                // next tile's stage
                const int step = (t % kStages == kStages - 1) ? -(kStages - 1) * kTileBytes : kTileBytes;
#pragma unroll
                for (int j = 0; j < 4; ++j) kb[j] += step;
#pragma unroll
                for (int j = 0; j < 8; ++j) vb[j >> 2][(j >> 1) & 1][j & 1] += step;
            }
            // drain the DMA pipeline; every wave sees the same redo flag
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            const int again = redo[0] | redo[1];
            __syncthreads();
            if (!again) break;
            if (threadIdx.x == 0) redo[0] = redo[1] = 0;
            m_hint = fmaxf(m_hint, __shfl_xor(m_hint, 32));
            m_hint = fmaxf(m_hint, st.m);
        }

        // ---- epilogue: this wave's 32 rows, no cross-wave merge ----
        st.l += __shfl_xor(st.l, 32);
        st.lr += __shfl_xor(st.lr, 32);
        const float inv = st.lr > 0.f ? 1.f / st.lr : 0.f;
        const float lse_v = st.l > 0.f ? (st.m + fast_log2(st.l)) * kLn2 : -INFINITY;
        if (nsplit == 1) {
            uint16_t *dst = p.out + ((int64_t)seq * R + row) * kDv + 4 * g;
#pragma unroll
            for (int d = 0; d < kDBlocks; ++d)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    u32x2_t v;
                    v[0] = pack_bf16x2(o[d][4 * q4] * inv, o[d][4 * q4 + 1] * inv);
                    v[1] = pack_bf16x2(o[d][4 * q4 + 2] * inv, o[d][4 * q4 + 3] * inv);
                    *reinterpret_cast<u32x2_t *>(dst + 32 * d + 8 * q4) = v;
                }
            if (g == 0) p.lse[(int64_t)seq * R + row] = lse_v;
        } else {
            float *dst = p.o_part + ((int64_t)slot * R + row) * kDv + 4 * g;
#pragma unroll
            for (int d = 0; d < kDBlocks; ++d)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4)
                    *reinterpret_cast<f32x4_t *>(dst + 32 * d + 8 * q4) =
                        f32x4_t{o[d][4 * q4] * inv, o[d][4 * q4 + 1] * inv,
                                o[d][4 * q4 + 2] * inv, o[d][4 * q4 + 3] * inv};
            if (g == 0) p.lse_part[(int64_t)slot * R + row] = lse_v;
        }
    }
}

hipError_t launch_decode_wide(const DecodeParams &p, int num_parts, int row_tiles,
                              hipStream_t stream)
{
    hipLaunchKernelGGL(decode_wide_kernel, dim3(num_parts, row_tiles), dim3(kWThreads), 0,
                       stream, p, p.block_table, p.seqlens, p.meta);
    return hipGetLastError();
}

}  // namespace mla
