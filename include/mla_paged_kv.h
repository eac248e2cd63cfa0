/*
 * mla_paged_kv.h -- C ABI of libmla_paged_kv.so: multi-head latent attention
 * (MLA) decode over a paged latent KV cache on AMD MI355X (gfx950).
 *
 * The operation is the MLA decode kernel released as FlashMLA ("DeepSeek
 * publica FlashMLA como codigo abierto", release bullets): BF16, a paged KV
 * cache with 64-token blocks, variable-length sequences, forward only.  The
 * query up-projection and value down-projection are applied as sequential
 * batched matmuls rather than materialized absorbed weights ("[Attention] MLA
 * get rid of materialization", PR description).
 *
 * Conventions shared by every call
 *   - bf16 tensors are passed as their raw 16-bit patterns (uint16_t).
 *   - Pointers marked [device] must be device memory of the current HIP
 *     device; [host] pointers are ordinary host memory.  The caller owns all
 *     buffers; the library keeps no pointer after a call returns and
 *     allocates no device memory.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call that
 *     launches work only enqueues it on that stream and returns without
 *     synchronizing; results are ready once the stream reaches that point.
 *   - Every call returns an mla_status.  Arguments are validated on the host
 *     before anything is launched; on an error nothing is enqueued and
 *     mla_last_error() holds a one-line reason (per calling thread).  No
 *     call aborts or throws.
 *   - The contents of device buffers (sequence lengths, block-table entries)
 *     are trusted: every length must satisfy 0 <= n_b <= bt_stride * 64 and
 *     every block-table entry a sequence uses must lie in [0, num_pages).
 *     Entries past ceil(n_b / 64) are never read.
 *
 * Geometry (fixed by the model; other values return MLA_ERR_UNSUPPORTED)
 *   d_qk = 576: each cached token is one latent row of 512 compressed dims
 *               followed by 64 rope dims; keys are the whole row.
 *   d_v  = 512: values are the first 512 dims of the same row.
 *   page = 64 tokens; kv_cache is [num_pages][64][576] bf16, a page is
 *          73,728 contiguous bytes.
 *   Rows of a sequence: R = s_q * h_q, ordered (query i, head h) -> i*h_q+h.
 *   h_q must be 16, 32, 64 or 128; 1 <= s_q <= 16.
 */
#ifndef MLA_PAGED_KV_H
#define MLA_PAGED_KV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mla_status {
    MLA_OK = 0,
    MLA_ERR_INVALID_ARG = 1, /* null pointer, negative size, bad stride   */
    MLA_ERR_UNSUPPORTED = 2, /* shape outside the supported geometry      */
    MLA_ERR_WORKSPACE = 3,   /* workspace pointer null or too small       */
    MLA_ERR_HIP = 4          /* a HIP runtime call or launch failed       */
} mla_status;

/* Static name of a status code (never NULL). */
const char *mla_status_str(int status);

/* Reason for the last non-OK status returned on this thread ("" if none). */
const char *mla_last_error(void);

/* Number of compute units of HIP device `device` -> *cus [host]. */
int mla_device_cus(int device, int *cus);

/* Scheduler parts for a shape: how many key ranges the sequences are cut
 * into so that one workgroup per part and row tile fills the device once.
 * A row tile is 128 query rows when s_q * h_q >= 48 (the MFMA-dense
 * kernel; the last tile is partly empty unless s_q * h_q is a multiple of
 * 128), 32 rows when s_q * h_q = 32, else 16 rows.  Pure host arithmetic. */
int mla_default_num_parts(int num_cus, int batch, int s_q, int h_q);

/* int32 count of the metadata buffer for (batch, num_parts):
 *   8 * num_parts      part records {seq_begin, tok_begin, seq_end, tok_end,
 *                      slot_begin, 0, 0, 0}: the part covers tokens
 *                      [tok_begin, ...) of sequence seq_begin, every token of
 *                      the sequences strictly between, and [0, tok_end) of
 *                      seq_end (or [tok_begin, tok_end) when they are equal);
 *                      seq_begin = -1 marks an empty part.  slot_begin is the
 *                      partial-result slot of its first sequence.
 *   batch + 1          split_offsets: sequence b owns partial slots
 *                      [split_offsets[b], split_offsets[b+1]); a sequence
 *                      with exactly one slot is written in place.
 *   1                  total chunks (16-token units) over the batch.
 *   batch + 1          extra merge workgroups before each sequence: a
 *                      sequence with k > 32 slots gets 4 S - 1, S = 2 for
 *                      k < 64, 4 for k < 128, 8 for k < 256, else 16 (the
 *                      dim slices each of its rows is merged in); an
 *                      exclusive prefix, the last entry is the total. */
size_t mla_metadata_ints(int batch, int num_parts);

/* Bytes of decode workspace: fp32 partial outputs and log-sum-exps for up
 * to batch + num_parts splits of R rows:
 *   (batch + num_parts) * s_q * h_q * (512 + 1) * 4. */
size_t mla_workspace_bytes(int batch, int s_q, int h_q, int num_parts);

/*
 * Variable-length split scheduling (the FlashMLA release bullets name
 * serving batches of sequences of differing lengths as its target).  Reads
 * the sequence lengths on the device (no host synchronization) and cuts the
 * sequences, in batch order, into `num_parts` contiguous ranges of near-equal
 * cost, where a sequence costs its 16-token chunks plus a lead of C chunks
 * for starting it: with TC cost units in all and U = min(num_parts, TC),
 * part p < U takes the chunks whose units fall in [floor(p*TC/U),
 * floor((p+1)*TC/U)), chunk i of sequence b sitting at unit (units of the
 * sequences before b) + C + i.  A part whose range holds lead units only is
 * empty.  With R = s_q * h_q, let S = 16 when R is 16 or 32 and S = 24
 * from 48 rows on: S prices one segment (a part's run of one sequence) in
 * chunks.  For 16 or 32 rows C = S; for more, C is 0 or S, whichever gives
 * the smaller largest part when every part costs its chunks plus S per
 * segment (ties: S).  Writes the metadata
 * described above.  Compute once per decode step; it stays valid for every
 * layer while the lengths do not change.
 *   seqlens  [device] int32 [batch]; a negative length counts as 0 and one
 *            above 2^21 tokens as 2^21 (mla_decode applies the same cap)
 *   metadata [device] int32 [mla_metadata_ints(batch, num_parts)] (output),
 *            16-byte aligned (part records are written 16 bytes at a time)
 *   1 <= batch <= 8192, 1 <= num_parts <= 65536.
 */
int mla_get_metadata(const int32_t *seqlens, int batch, int s_q, int h_q, int num_parts,
                     int32_t *metadata, void *stream);

/*
 * Paged MLA decode: the MLA decoding kernel of "DeepSeek publica FlashMLA
 * como codigo abierto" (release bullets: BF16, paged KV cache with 64-token
 * blocks, variable-length sequences).  For every sequence b, query i and
 * head h, with
 * n = seqlens[b] and L = n (causal = 0) or L = n - s_q + 1 + i (causal = 1:
 * query i sits at absolute position n - s_q + i):
 *   s_j = scale * <q[b,i,h,:], kv_row(b, j)>         for j < L
 *   out[b,i,h,:] = sum_j softmax(s)_j * kv_row(b, j)[0:512]
 *   lse[b,i,h]   = ln sum_j exp(s_j)                   (natural log)
 * where kv_row(b, j) = kv_cache[block_table[b*bt_stride + j/64]][j%64][:].
 * A row with L <= 0 gets out = 0 and lse = -inf.  Softmax runs in fp32 on
 * bf16 MFMA products; out is rounded to bf16 (nearest even).  `scale` is the
 * softmax temperature and must be positive and finite (MLA_ERR_INVALID_ARG
 * otherwise): the 128-row kernel masks keys and takes row maxima on the
 * unscaled products, which is only order-preserving for scale > 0.
 * The caller keeps n <= 64*bt_stride and the entries a sequence uses in
 * [0, num_pages).  The kernels do not report a breach (the values live on
 * the device) but keep every read inside the buffers: n is capped at 2^21
 * tokens, j/64 at bt_stride - 1 (keys past the table's width reuse its last
 * column) and an entry outside [0, num_pages) reads page num_pages - 1.
 * With the environment variable MLA_DEBUG_CHECKS set (to anything but 0)
 * the call first copies seqlens and block_table to host memory on `stream`,
 * synchronizes it, and returns MLA_ERR_INVALID_ARG, launching nothing, if a
 * length exceeds 64*bt_stride or 2^21 or a used entry is out of range (so
 * the call is not capturable into a graph in that mode).
 *
 *   q           [device] bf16 [batch][s_q][h_q][576]
 *   kv_cache    [device] bf16 [num_pages][64][576]
 *   block_table [device] int32 [batch][bt_stride]
 *   seqlens     [device] int32 [batch]
 *   metadata    [device] from mla_get_metadata with the same batch, s_q, h_q,
 *               num_parts and lengths; read only, so one buffer can serve
 *               any number of calls, also concurrent ones.
 *   workspace   [device] >= mla_workspace_bytes(batch, s_q, h_q, num_parts)
 *   out         [device] bf16 [batch][s_q][h_q][512]
 *   lse         [device] fp32 [batch][s_q][h_q]
 * Sequences cut into several parts are merged by the combine kernel on the
 * same stream before the call's work completes; each row of a sequence cut
 * into more than 32 parts is merged by several workgroups, one per slice of
 * its 512 output dims.
 */
int mla_decode(const uint16_t *q, const uint16_t *kv_cache, int64_t num_pages,
               const int32_t *block_table, int64_t bt_stride, const int32_t *seqlens,
               int batch, int s_q, int h_q, int d_qk, int d_v, int page_size,
               float scale, int causal, const int32_t *metadata, int num_parts,
               void *workspace, size_t workspace_bytes, uint16_t *out, float *lse,
               void *stream);

/*
 * The same decode for callers that cannot allocate device memory -- code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation: identical arguments and results to mla_decode without the
 * workspace, whose partial results go instead to a scratch array the
 * library owns, MLA_NOALLOC_SCRATCH_BYTES (160 MiB) on each device it runs
 * on, held from the first call on that device until the process ends.
 * Returns MLA_ERR_WORKSPACE, launching nothing, when
 * mla_workspace_bytes(batch, s_q, h_q, num_parts) exceeds it (use mla_decode
 * there).  The call allocates nothing, copies nothing to the host and never
 * synchronizes (MLA_DEBUG_CHECKS does not apply to it).  Every call on one
 * device shares that device's array and leaves its contents behind; calls
 * that overlap in time on one device (other streams, other threads) race.
 */
#define MLA_NOALLOC_SCRATCH_BYTES ((size_t)160 << 20)
int mla_decode_noalloc(const uint16_t *q, const uint16_t *kv_cache, int64_t num_pages,
                       const int32_t *block_table, int64_t bt_stride, const int32_t *seqlens,
                       int batch, int s_q, int h_q, int d_qk, int d_v, int page_size, float scale,
                       int causal, const int32_t *metadata, int num_parts, uint16_t *out, float *lse,
                       void *stream);

/*
 * Split-KV merge of the decode's partial results, the step that lets the
 * variable-length schedule of "DeepSeek publica FlashMLA como codigo
 * abierto" (release bullets) cut one sequence's keys over several
 * workgroups; the merge formula is the log-sum-exp combination of
 * softmax partials.  Sequence b's partial results are slots
 * [split_offsets[b], split_offsets[b+1]) of o_part / lse_part; each slot
 * holds a normalized partial output and its natural-log lse over a disjoint
 * key range (lse = -inf marks an empty range).  With M = max_s lse_s:
 *   lse = M + ln sum_s exp(lse_s - M),  out = sum_s exp(lse_s - lse) * o_s.
 * A sequence with no slot, or whose slots are all empty, gets out = 0 and
 * lse = -inf.
 *   o_part        [device] fp32 [total_slots][s_q*h_q][512]
 *   lse_part      [device] fp32 [total_slots][s_q*h_q]
 *   split_offsets [device] int32 [batch + 1], nondecreasing, from 0
 *   out           [device] bf16 [batch][s_q][h_q][512]
 *   lse           [device] fp32 [batch][s_q][h_q]
 */
int mla_combine(const float *o_part, const float *lse_part, const int32_t *split_offsets,
                int batch, int s_q, int h_q, int d_v, uint16_t *out, float *lse, void *stream);

/*
 * Per-head batched matmul for the non-materialized absorption ("[Attention]
 * MLA get rid of materialization", PR description):
 *   y[b, h, n] = sum_k x[b, h, k] * w[h, k, n]      (fp32 accumulate, bf16 out)
 * Used as q_lat = q_nope . W_UK (K = 128, N = 512, writing into the first 512
 * columns of the decode query) and as y = o_lat . W_UV (K = 512, N = 128).
 *   x [device] bf16, element (b, h, k) at x[b*x_stride_b + h*x_stride_h + k]
 *   w [device] bf16 [heads][K][N], contiguous
 *   y [device] bf16, element (b, h, n) at y[b*y_stride_b + h*y_stride_h + n]
 * K must be a positive multiple of 32 and N of 64; strides are in elements
 * and must keep every row 16-byte aligned (multiples of 8).  One workgroup
 * per head and 64 x 64 output tile: heads rounded up to 8, times
 * N/64 * ceil(batch/64) tiles, must stay below 2^24 (MLA_ERR_UNSUPPORTED
 * otherwise).  No device allocation; enqueued on `stream`.
 */
int mla_absorb_bmm(const uint16_t *x, int64_t x_stride_b, int64_t x_stride_h,
                   const uint16_t *w, int heads, int K, int N,
                   uint16_t *y, int64_t y_stride_b, int64_t y_stride_h, int batch,
                   void *stream);

/*
 * The same bmm with fp8 weights decompressed to bf16 inside the kernel (the
 * absorption PR stores the weights in fp8 and decompresses them to 16-bit
 * floats for the bmm, there being no fp8 bmm).  The format and the scale
 * granularity are not on the pages; this library reads them as OCP FP8 E4M3
 * codes (sign, 4-bit exponent with bias 7, 3-bit mantissa, subnormals,
 * S.1111.111 = NaN) with one fp32 scale per 128 x 128 block of each head's
 * K x N matrix:
 *   W[h, k, n] = bf16( e4m3(w[h, k, n]) * w_scale[h, k / 128, n / 128] )
 * (the exact product rounded once to nearest even), then y = x . W as in
 * mla_absorb_bmm (fp32 accumulate, bf16 out).
 *   w       [device] uint8 [heads][K][N] E4M3 codes, 16-byte aligned
 *   w_scale [device] fp32 [heads][ceil(K / 128)][ceil(N / 128)]
 * Other arguments, limits and errors as for mla_absorb_bmm.  Half the
 * weight bytes of the bf16 path.  No device allocation; enqueued on
 * `stream`.
 */
int mla_absorb_bmm_fp8w(const uint16_t *x, int64_t x_stride_b, int64_t x_stride_h,
                        const uint8_t *w, const float *w_scale, int heads, int K, int N,
                        uint16_t *y, int64_t y_stride_b, int64_t y_stride_h, int batch,
                        void *stream);

/*
 * Measurement probes: the rates this device reaches on the resources the
 * decode is bound by, so that achieved throughput can be quoted as a
 * fraction of what is attainable as well as of the published peaks.
 *
 * mla_probe_read: streams `bytes` of `buf` once (16-byte loads, 16 KB
 * contiguous per workgroup pass, `workgroups` workgroups of 256 threads
 * striding over the buffer) and writes nothing unless the XOR
 * of everything read hits one fixed 64-bit pattern (then sink[0]).
 *   buf  [device] 16-byte aligned, bytes a positive multiple of 16
 *   sink [device] uint32 [1]
 * mla_probe_mfma: `workgroups` workgroups of four waves; every wave issues
 * iters x 8 v_mfma_f32_32x32x16_bf16 (32768 flops each) on eight
 * independent accumulators, i.e. workgroups * 4 * iters * 8 * 32768 flops,
 * and writes one float per wave.
 *   sink [device] float [workgroups * 4]
 * mla_probe_lds: `workgroups` workgroups (one per CU: each holds 96 KB of
 * LDS) of `waves` waves; every wave issues iters x depth ds_read_b128 (1 KB
 * each, `depth` in flight at a time, bank-conflict free) and writes its
 * loop's shader clock cycles and 100 MHz real-time ticks: LDS bytes read per
 * clock per CU = waves * iters * depth * 1024 / (the slowest wave's cycles).
 *   waves in [1, 16]; depth 1, 2, 4, 8 or 16;
 *   ticks [device] uint32 [workgroups * waves][2]
 *   (cycles, ticks); sink [device] uint32 [1], written only on a fixed
 *   improbable XOR of what was read.
 * All are enqueued on `stream`; no device allocation.
 */
int mla_probe_read(const void *buf, int64_t bytes, int workgroups, uint32_t *sink, void *stream);
int mla_probe_mfma(int iters, int workgroups, float *sink, void *stream);
int mla_probe_lds(int waves, int depth, int iters, int workgroups, uint32_t *ticks,
                  uint32_t *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_PAGED_KV_H */
