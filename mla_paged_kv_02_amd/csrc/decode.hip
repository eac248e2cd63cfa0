// decode.hip -- paged MLA decode for one 16-row tile of a sequence's queries.
//
// Operation: softmax(scale * Q K^T) V per query row over a paged latent cache
// (FlashMLA, "DeepSeek publica FlashMLA como codigo abierto", release bullets:
// BF16, 64-token pages, variable lengths).  K is the whole 576-wide latent
// row, V its first 512 dims, so every cache byte is fetched once per tile.
//
// Mapping onto gfx950 (one workgroup = 4 waves = one CU's worth of registers):
//  * A workgroup owns one scheduler part (a contiguous run of 16-token chunks,
//    possibly spanning sequences) and one 16-row tile of queries.
//  * The four waves take the part's chunks round-robin and run fully
//    independent online softmaxes: no barrier inside the key loop.
//  * Chunk rows are loaded straight from HBM into registers in the MFMA
//    operand layout, double-buffered so one chunk is in flight while the
//    previous one is computed.  Keys outside the part read as zero through a
//    buffer descriptor (no divergent branch around the loads).
//  * S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (18 k-steps over 576 dims); the
//    result layout (4 keys x 1 row per lane) is exactly the P^T operand of
//    the value product, so probabilities never leave registers.
//  * The value part of the chunk is written to the wave's own LDS slot and
//    read back transposed with ds_read_b64_tr_b16, giving the V^T operand of
//    v_mfma_f32_16x16x16_bf16 (32 output tiles of 16 dims).
//  * Softmax statistics are fp32 in the log2 domain; the running max is
//    only moved (and O rescaled) when a new score exceeds it by more than
//    2^8, so most chunks skip the rescale.
//  * At the end of a sequence segment the four wave states are merged in
//    LDS; the result is either the final output (bf16 out + lse) or an fp32
//    partial for the split-KV merge.
#include "mla_device.h"
#include "kernels.h"
#include "stamps.h"

namespace mla {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kQkSteps = kDqk / 32;   // 18
constexpr int kVSteps = kDv / 32;     // 16 of the 18 steps hold value dims
constexpr int kDTiles = kDv / 16;     // 32
constexpr int kVStride = kDv + 16;    // bf16 per staged value row (1056 B)
constexpr int kOStride = kDv + 16;    // fp32 per merge row
constexpr int kStageBytes = kWaves * 16 * kVStride * 2;   // 67584
constexpr int kMergeBytes = kWaves * 16 * kOStride * 4;   // 135168
// the waves' value stages are used inside the key loop, the merge rows after
// it, in the same bytes
static_assert(kStageBytes <= kMergeBytes, "value stages lie inside the merge area");
constexpr int kQStride = kDqk + 8;    // bf16 per query row in LDS (1168 B: 16 rows hit distinct banks)
constexpr int kStatBytes = kWaves * 16 * 4 * 4;   // m, l, l_rounded, pad
constexpr int kQOffset = kMergeBytes + kStatBytes;
constexpr int kLdsBytes = kQOffset + 16 * kQStride * 2;   // 154880
constexpr float kRescaleSlack = 8.0f;  // log2 units

#if MLA_STAMPS
// Instrumented build only: the record buffer of stamps.h, or null.
__device__ uint64_t *g_stamps_r16;
hipError_t set_stamps_r16(uint64_t *buf)
{
    return hipMemcpyToSymbol(HIP_SYMBOL(g_stamps_r16), &buf, sizeof(buf));
}
#endif


typedef u32x4_t ChunkRegs[kQkSteps];

// Issue the loads of one 16-token chunk: lane (key r16, group g) receives
// dims [32t + 8g, 32t + 8g + 8) of key 16c + r16 for t < 18.  Keys at or
// past `key_end` read as zero.
__device__ __forceinline__ void load_chunk(ChunkRegs &k, const DecodeParams &p,
                                           const int32_t *__restrict__ bt, int seq, int c,
                                           int key_end, int r16, int g)
{
    // columns past the table's width repeat its last one; entries outside
    // the cache are clamped into it (negative ones too, as unsigned)
    const int64_t col = min((int64_t)(c >> 2), p.bt_stride - 1);
    const uint32_t page = min((uint32_t)bt[(int64_t)seq * p.bt_stride + col], p.page_max);
    const char *base = reinterpret_cast<const char *>(p.kv) + (int64_t)page * kPageBytes;
    const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(base, kPageBytes);
    const int key = c * kChunk + r16;
    const int voff = key < key_end ? ((c & 3) * kChunk + r16) * kRowBytes + g * 16 : 0x40000000;
#pragma unroll
    for (int t = 0; t < kQkSteps; ++t)
        k[t] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, voff + t * 64, 0, 0);
}

struct RowState {
    float m;        // running max (log2 units) used as the exponent origin
    float l;        // this lane's share of sum_j 2^(s_j - m), fp32 (gives the lse)
    float lr;       // the same sum over the weights as fed to the value
                    // product, both bf16 terms (normalizes the output)
};

__device__ __forceinline__ void process_chunk(const ChunkRegs &k, const lds_short_t *qs,
                                              f32x4_t (&o)[kDTiles], RowState &st, int c,
                                              int limit, float scale_log2, lds_short_t *stage,
                                              int r16, int g)
{
    // S^T[key 4g+i][row r16] for the chunk's 16 keys; the query fragment
    // (B operand: row r16, dims 32t + 8g ..) comes from the tile in LDS
    f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < kQkSteps; ++t) {
        const bf16x8_t qf = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8_t *>(
            qs + r16 * kQStride + 32 * t + 8 * g);
        s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, k[t]), qf, s,
                                                    0, 0, 0);
    }

    // value rows of the chunk -> this wave's LDS slot, row-major
#pragma unroll
    for (int t = 0; t < kVSteps; ++t)
        *reinterpret_cast<__attribute__((address_space(3))) u32x4_t *>(
            stage + r16 * kVStride + 32 * t + 8 * g) = k[t];

    float sv[4];
    float tmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int key = c * kChunk + 4 * g + i;
        sv[i] = key < limit ? s[i] * scale_log2 : -INFINITY;
        tmax = fmaxf(tmax, sv[i]);
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));

    // move the exponent origin only when a score outgrows it by the slack
    const bool grow = tmax > st.m + kRescaleSlack;
    if (__builtin_amdgcn_ballot_w64(grow)) {
        const float m_new = grow ? tmax : st.m;
        const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp2(st.m - m_new);
        st.l *= alpha;
        st.lr *= alpha;
#pragma unroll
        for (int d = 0; d < kDTiles; ++d) o[d] *= alpha;
        st.m = m_new;
    }
    const float m_use = (st.m == -INFINITY) ? 0.f : st.m;
    const float e0 = fast_exp2(sv[0] - m_use), e1 = fast_exp2(sv[1] - m_use);
    const float e2 = fast_exp2(sv[2] - m_use), e3 = fast_exp2(sv[3] - m_use);
    st.l += (e0 + e1) + (e2 + e3);
    // Each weight goes to the value product as two bf16 terms: its rounding
    // and the rounding residual (exact in fp32), so the product sees it to
    // ~2^-16 relative instead of 2^-8 (bf16 keeps 8 significant bits).
    // With one term, rows dominated by a few keys with far-apart values
    // carry an error of up to 2^-8 times that spread, on top of the
    // output's own bf16 rounding.
    const uint32_t p01 = pack_bf16x2(e0, e1);
    const uint32_t p23 = pack_bf16x2(e2, e3);
    const uint32_t q01 = pack_bf16x2(e0 - bf16_lo(p01), e1 - bf16_hi(p01));
    const uint32_t q23 = pack_bf16x2(e2 - bf16_lo(p23), e3 - bf16_hi(p23));
    // normalizing by the sum of the weights as fed keeps the output an exact
    // convex combination of value rows
    st.lr += ((bf16_lo(p01) + bf16_hi(p01)) + (bf16_lo(p23) + bf16_hi(p23))) +
             ((bf16_lo(q01) + bf16_hi(q01)) + (bf16_lo(q23) + bf16_hi(q23)));
    const i16x4_t pf = __builtin_bit_cast(i16x4_t, u32x2_t{p01, p23});
    const i16x4_t pl = __builtin_bit_cast(i16x4_t, u32x2_t{q01, q23});

    // O^T[16d + 4g + i][row r16] += V^T[16 dims][16 keys] . P^T[16 keys][16 rows]
    // transposed read: lane 16g + 4e + c points at value row 4g + e, dims
    // 16d + 4c .. +3; lane 16g + j receives rows 4g..4g+3 of dim 16d + j.
    const lds_short_t *vt = stage + (4 * g + (r16 >> 2)) * kVStride + 4 * (r16 & 3);
#pragma unroll
    for (int d = 0; d < kDTiles; ++d) {
        const i16x4_t vf = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (i16x4_t __attribute__((address_space(3))) *)(vt + 16 * d));
        o[d] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vf, pf, o[d], 0, 0, 0);
        o[d] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vf, pl, o[d], 0, 0, 0);
    }
}

// The int tables are separate restrict arguments: with no aliasing store the
// compiler can read them through the scalar cache (wave-uniform indices).
__global__ __launch_bounds__(kThreads, 1) void decode_r16_kernel(
    DecodeParams p, const int32_t *__restrict__ bt, const int32_t *__restrict__ seqlens,
    const int32_t *__restrict__ meta)
{
    __shared__ __attribute__((aligned(16))) char smem[kLdsBytes];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const int r16 = lane & 15;
    const int g = lane >> 4;
    const int part = blockIdx.x;
    const int rt = blockIdx.y;
    const int R = p.s_q * p.h_q;

    MLA_STAMP_BEGIN();
    const int32_t *rec = meta + part * kPartInts;
    const int s0 = rec[0];
    if (s0 < 0) {
        MLA_STAMP_END(g_stamps_r16);
        return;
    }
    const int t0 = rec[1], s1 = rec[2], t1 = rec[3], slot0 = rec[4];
    const int32_t *split_off = meta + p.num_parts * kPartInts;

    lds_short_t *stage = (lds_short_t *)smem + wave * 16 * kVStride;
    float *mo = reinterpret_cast<float *>(smem);
    float *ml = reinterpret_cast<float *>(smem + kMergeBytes);
    lds_short_t *qs = (lds_short_t *)(smem + kQOffset);

    for (int seq = s0; seq <= s1; ++seq) {
        const int n = min(seqlens[seq], kMaxSeqLen);
        const int ks = seq == s0 ? t0 : 0;
        const int ke = seq == s1 ? t1 : n;
        if (ks >= ke) continue;   // empty sequence inside the part (uniform)
        MLA_STAMP_SEGMENT();
        const int nsplit = split_off[seq + 1] - split_off[seq];
        const int slot = seq == s0 ? slot0 : split_off[seq];

        const int c_begin = ks / kChunk;
        const int c_end = (ke + kChunk - 1) / kChunk;
        const int mine = c_end - c_begin - wave;
        const int nc = mine > 0 ? (mine + kWaves - 1) / kWaves : 0;
        int c = c_begin + wave;

        // the tile's 16 query rows -> LDS (16 B per thread and pass).  The
        // wave's first chunk loads go out between the query loads and their
        // LDS stores, so the two memory round trips overlap; they are issued
        // even when the wave has no chunk (then all outside the buffer range)
        // so that the wait before the stores counts the same loads on every path.
        const uint16_t *qtile = p.q + ((int64_t)seq * R + rt * 16) * kDqk;
        constexpr int kQPieces = 16 * (kDqk / 8);
        constexpr int kQPer = (kQPieces + kThreads - 1) / kThreads;
        u32x4_t qv[kQPer];
#pragma unroll
        for (int j = 0; j < kQPer; ++j) {
            const int i = threadIdx.x + j * kThreads;
            const int qr = i / (kDqk / 8), qc = 8 * (i % (kDqk / 8));
            qv[j] = i < kQPieces ? *reinterpret_cast<const u32x4_t *>(qtile + qr * kDqk + qc)
                                 : u32x4_t{0u, 0u, 0u, 0u};
        }
        ChunkRegs ka, kb;
        load_chunk(ka, p, bt, seq, nc > 0 ? c : c_begin, nc > 0 ? ke : 0, r16, g);
#pragma unroll
        for (int j = 0; j < kQPer; ++j) {
            const int i = threadIdx.x + j * kThreads;
            const int qr = i / (kDqk / 8), qc = 8 * (i % (kDqk / 8));
            if (i < kQPieces)
                *reinterpret_cast<__attribute__((address_space(3))) u32x4_t *>(qs + qr * kQStride +
                                                                               qc) = qv[j];
        }
        __syncthreads();
        const int row = rt * 16 + r16;

        // keys visible to this lane's row
        int limit = ke;
        if (p.causal) limit = min(ke, n - p.s_q + 1 + row / p.h_q);

        RowState st = {-INFINITY, 0.f, 0.f};
        f32x4_t o[kDTiles];
#pragma unroll
        for (int d = 0; d < kDTiles; ++d) o[d] = f32x4_t{0.f, 0.f, 0.f, 0.f};

        MLA_STAMP_PHASE(0);
        if (nc > 0) {
            for (int it = 0;; it += 2) {
                const int cn = c + kWaves;
                // always issue the next loads; past the wave's last chunk they
                // fall outside the buffer range (zeros, no memory traffic)
                load_chunk(kb, p, bt, seq, it + 1 < nc ? cn : c, it + 1 < nc ? ke : 0, r16, g);
                __builtin_amdgcn_sched_barrier(0);   // keep the loads ahead of the compute
                process_chunk(ka, qs, o, st, c, limit, p.scale_log2, stage, r16, g);
                if (it + 1 >= nc) break;
                load_chunk(ka, p, bt, seq, it + 2 < nc ? cn + kWaves : cn, it + 2 < nc ? ke : 0,
                           r16, g);
                __builtin_amdgcn_sched_barrier(0);
                process_chunk(kb, qs, o, st, cn, limit, p.scale_log2, stage, r16, g);
                if (it + 2 >= nc) break;
                c = cn + kWaves;
            }
        }

        MLA_STAMP_PHASE(1);
        // ---- merge the four wave states --------------------------------
        st.l += __shfl_xor(st.l, 16);
        st.l += __shfl_xor(st.l, 32);
        st.lr += __shfl_xor(st.lr, 16);
        st.lr += __shfl_xor(st.lr, 32);
        __syncthreads();   // staging slots are reused by the merge buffer
#pragma unroll
        for (int d = 0; d < kDTiles; ++d)
            *reinterpret_cast<f32x4_t *>(mo + (wave * 16 + r16) * kOStride + 16 * d + 4 * g) = o[d];
        if (g == 0) {
            ml[(wave * 16 + r16) * 4 + 0] = st.m;
            ml[(wave * 16 + r16) * 4 + 1] = st.l;
            ml[(wave * 16 + r16) * 4 + 2] = st.lr;
        }
        __syncthreads();

        // wave w finishes dims [128w, 128w + 128) of all 16 rows: lane (row
        // nr, c) the 8-dim runs 128w + 32j + 8c, j < 4, so the four lanes of a
        // row store 64 (bf16) or 128 (fp32) contiguous bytes per instruction
        const int nr = lane >> 2;
        const int d0 = 128 * wave + 8 * (lane & 3);
        float mw[kWaves];
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            mw[w] = ml[(w * 16 + nr) * 4];
            M = fmaxf(M, mw[w]);
        }
        const float m_use = M == -INFINITY ? 0.f : M;
        float L = 0.f, Lr = 0.f;
        float acc[32];
#pragma unroll
        for (int e = 0; e < 32; ++e) acc[e] = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float a = fast_exp2(mw[w] - m_use);
            L += a * ml[(w * 16 + nr) * 4 + 1];
            Lr += a * ml[(w * 16 + nr) * 4 + 2];
            const float *src = mo + (w * 16 + nr) * kOStride + d0;
#pragma unroll
            for (int e = 0; e < 32; e += 4) {
                // acc[e..e+3] = dims d0 + 32 (e / 8) + e % 8 ..
                const f32x4_t v = *reinterpret_cast<const f32x4_t *>(src + 32 * (e >> 3) + (e & 7));
                acc[e] += a * v[0];
                acc[e + 1] += a * v[1];
                acc[e + 2] += a * v[2];
                acc[e + 3] += a * v[3];
            }
        }
        const float inv = Lr > 0.f ? 1.f / Lr : 0.f;
        const float lse_v = L > 0.f ? (M + fast_log2(L)) * kLn2 : -INFINITY;
        const int orow = rt * 16 + nr;
        if (nsplit == 1) {
            uint16_t *dst = p.out + ((int64_t)seq * R + orow) * kDv + d0;
#pragma unroll
            for (int e = 0; e < 32; e += 8) {
                u32x4_t v;
                v[0] = pack_bf16x2(acc[e] * inv, acc[e + 1] * inv);
                v[1] = pack_bf16x2(acc[e + 2] * inv, acc[e + 3] * inv);
                v[2] = pack_bf16x2(acc[e + 4] * inv, acc[e + 5] * inv);
                v[3] = pack_bf16x2(acc[e + 6] * inv, acc[e + 7] * inv);
                *reinterpret_cast<u32x4_t *>(dst + 32 * (e >> 3)) = v;
            }
            if (wave == 0 && (lane & 3) == 0) p.lse[(int64_t)seq * R + orow] = lse_v;
        } else {
            float *dst = p.o_part + ((int64_t)slot * R + orow) * kDv + d0;
#pragma unroll
            for (int e = 0; e < 32; e += 4)
                *reinterpret_cast<f32x4_t *>(dst + 32 * (e >> 3) + (e & 7)) =
                    f32x4_t{acc[e] * inv, acc[e + 1] * inv, acc[e + 2] * inv, acc[e + 3] * inv};
            if (wave == 0 && (lane & 3) == 0) p.lse_part[(int64_t)slot * R + orow] = lse_v;
        }
        __syncthreads();   // before the next segment reuses LDS
        MLA_STAMP_PHASE(2);
    }
    MLA_STAMP_END(g_stamps_r16);
}

hipError_t launch_decode_r16(const DecodeParams &p, int num_parts, int row_tiles,
                             hipStream_t stream)
{
    hipLaunchKernelGGL(decode_r16_kernel, dim3(num_parts, row_tiles), dim3(kThreads), 0, stream,
                       p, p.block_table, p.seqlens, p.meta);
    return hipGetLastError();
}

}  // namespace mla
