// abi.cpp -- the extern "C" entry points of libmla_paged_kv.so.
//
// Every entry point validates its arguments on the host before touching the
// HIP runtime, so argument errors are reported without a device.  Work is
// only enqueued on the caller's stream; nothing here synchronizes, allocates
// device memory or keeps a pointer past the call.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "../../include/mla_paged_kv.h"
#include "kernels.h"

namespace {

thread_local char g_last_error[256] = "";

int fail(int status, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return status;
}

int ok()
{
    g_last_error[0] = '\0';
    return MLA_OK;
}

int hip_status(hipError_t e, const char *what)
{
    if (e != hipSuccess)
        return fail(MLA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool supported_heads(int h_q) { return h_q == 16 || h_q == 32 || h_q == 64 || h_q == 128; }

constexpr int kMaxSq = 16;

int check_rows(int batch, int s_q, int h_q)
{
    if (batch < 1) return fail(MLA_ERR_INVALID_ARG, "batch must be >= 1 (got %d)", batch);
    if (s_q < 1 || s_q > kMaxSq)
        return fail(MLA_ERR_UNSUPPORTED, "s_q must be in [1, %d] (got %d)", kMaxSq, s_q);
    if (!supported_heads(h_q))
        return fail(MLA_ERR_UNSUPPORTED, "h_q must be 16, 32, 64 or 128 (got %d)", h_q);
    return MLA_OK;
}

// MLA_DEBUG_CHECKS set to a value other than 0: before launching, copy the
// lengths and the block table to host memory (on the caller's stream, which
// this synchronizes) and reject a length above 64 * bt_stride or 2^21 and a
// used entry outside [0, num_pages).  Without it the kernels clamp such
// values instead (every read stays inside the buffers, no error).
bool debug_checks()
{
    const char *v = std::getenv("MLA_DEBUG_CHECKS");
    return v != nullptr && v[0] != '\0' && !(v[0] == '0' && v[1] == '\0');
}

int check_tables(const int32_t *seqlens, const int32_t *block_table, int64_t bt_stride,
                 int batch, int64_t num_pages, hipStream_t st)
{
    std::vector<int32_t> n((size_t)batch);
    std::vector<int32_t> bt((size_t)batch * (size_t)bt_stride);
    hipError_t e = hipMemcpyAsync(n.data(), seqlens, n.size() * 4, hipMemcpyDeviceToHost, st);
    if (e == hipSuccess)
        e = hipMemcpyAsync(bt.data(), block_table, bt.size() * 4, hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) return hip_status(e, "debug check copy");
    for (int b = 0; b < batch; ++b) {
        if ((int64_t)n[b] > 64 * bt_stride || n[b] > mla::kMaxSeqLen)
            return fail(MLA_ERR_INVALID_ARG,
                        "seqlens[%d] = %d exceeds 64 * bt_stride = %lld or 2^21", b, n[b],
                        (long long)(64 * bt_stride));
        for (int64_t t = 0; t < ((int64_t)n[b] + 63) / 64; ++t) {
            const int32_t page = bt[(size_t)b * (size_t)bt_stride + (size_t)t];
            if (page < 0 || page >= num_pages)
                return fail(MLA_ERR_INVALID_ARG,
                            "block_table[%d][%lld] = %d is outside [0, %lld)", b, (long long)t,
                            page, (long long)num_pages);
        }
    }
    return MLA_OK;
}

// The per-head bmm behind both absorb entry points: bf16 weights w, or E4M3
// weights w8 with their block scales.
int absorb(const uint16_t *x, int64_t x_stride_b, int64_t x_stride_h, const uint16_t *w,
           const uint8_t *w8, const float *wscale, int heads, int K, int N, uint16_t *y,
           int64_t y_stride_b, int64_t y_stride_h, int batch, void *stream)
{
    if (!x || !y) return fail(MLA_ERR_INVALID_ARG, "x and y must be non-null");
    if (batch < 1 || heads < 1) return fail(MLA_ERR_INVALID_ARG, "batch and heads must be >= 1");
    if (K < 32 || K % 32 != 0 || N < 64 || N % 64 != 0)
        return fail(MLA_ERR_UNSUPPORTED, "K must be a multiple of 32 and N of 64 (got %d, %d)", K,
                    N);
    if (heads > 65535) return fail(MLA_ERR_UNSUPPORTED, "heads must be <= 65535");
    if ((int64_t)((heads + 7) / 8 * 8) * (N / 64) * ((batch + 63) / 64) >= (int64_t)1 << 24)
        return fail(MLA_ERR_UNSUPPORTED, "too many (head, tile) workgroups: %d heads, N %d, batch %d",
                    heads, N, batch);
    if (x_stride_b % 8 || x_stride_h % 8 || y_stride_b % 8 || y_stride_h % 8 ||
        x_stride_b < 0 || x_stride_h < 0 || y_stride_b < 0 || y_stride_h < 0)
        return fail(MLA_ERR_INVALID_ARG, "strides must be non-negative multiples of 8 elements");
    if (!aligned(x, 16) || !aligned(y, 16))
        return fail(MLA_ERR_INVALID_ARG, "x and y must be 16-byte aligned");
    mla::AbsorbParams p;
    p.x = x;
    p.x_sb = x_stride_b;
    p.x_sh = x_stride_h;
    p.w = w;
    p.w8 = w8;
    p.wscale = wscale;
    p.K = K;
    p.N = N;
    p.y = y;
    p.y_sb = y_stride_b;
    p.y_sh = y_stride_h;
    p.batch = batch;
    p.heads = heads;
    return hip_status(mla::launch_absorb(p, heads, static_cast<hipStream_t>(stream)),
                      "absorb kernel launch");
}

}  // namespace

namespace mla {



int set_error(int status, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return status;
}

int decode_call(const uint16_t *q, const uint16_t *kv_cache, int64_t num_pages,
                const int32_t *block_table, int64_t bt_stride, const int32_t *seqlens, int batch,
                int s_q, int h_q, int d_qk, int d_v, int page_size, float scale, int causal,
                const int32_t *metadata, int num_parts, const WorkspaceSource &ws, uint16_t *out,
                float *lse, void *stream)
{
    if (!q || !kv_cache || !block_table || !seqlens || !metadata || !out || !lse)
        return fail(MLA_ERR_INVALID_ARG, "q, kv_cache, block_table, seqlens, metadata, out and "
                                         "lse must be non-null");
    if (int st = check_rows(batch, s_q, h_q)) return st;
    if (batch > mla::kMetaMaxBatch)
        return fail(MLA_ERR_UNSUPPORTED, "batch must be <= %d (got %d)", mla::kMetaMaxBatch, batch);
    if (d_qk != 576 || d_v != 512)
        return fail(MLA_ERR_UNSUPPORTED, "d_qk must be 576 and d_v 512 (got %d, %d)", d_qk, d_v);
    if (page_size != 64)
        return fail(MLA_ERR_UNSUPPORTED, "page_size must be 64 (got %d)", page_size);
    if (num_pages < 1) return fail(MLA_ERR_INVALID_ARG, "num_pages must be >= 1");
    if (bt_stride < 1) return fail(MLA_ERR_INVALID_ARG, "bt_stride must be >= 1");
    if (causal != 0 && causal != 1) return fail(MLA_ERR_INVALID_ARG, "causal must be 0 or 1");
    if (!std::isfinite(scale) || !(scale > 0.f))
        return fail(MLA_ERR_INVALID_ARG, "scale must be positive and finite (got %g)", (double)scale);
    if (num_parts < 1 || num_parts > mla::kMaxParts)
        return fail(MLA_ERR_INVALID_ARG, "num_parts must be in [1, %d] (got %d)", mla::kMaxParts,
                    num_parts);
    if (!aligned(q, 16) || !aligned(kv_cache, 16) || !aligned(out, 16) || !aligned(lse, 4) ||
        !aligned(block_table, 4) || !aligned(seqlens, 4) || !aligned(metadata, 4))
        return fail(MLA_ERR_INVALID_ARG, "q, kv_cache and out must be 16-byte aligned");
    const size_t need = mla_workspace_bytes(batch, s_q, h_q, num_parts);
    void *workspace = ws.ptr;
    if (ws.resolve == nullptr) {
        if (workspace == nullptr || ws.bytes < need || !aligned(workspace, 16))
            return fail(MLA_ERR_WORKSPACE, "workspace needs %zu bytes (16-byte aligned), got %zu",
                        need, workspace == nullptr ? (size_t)0 : ws.bytes);
    } else {
        if (need > ws.bytes)
            return fail(MLA_ERR_WORKSPACE,
                        "this shape needs %zu bytes of workspace, more than the %zu of the "
                        "library's own scratch buffer; use mla_decode with a workspace",
                        need, ws.bytes);
        if (int st = ws.resolve(&workspace)) return st;
    }

    hipStream_t st = static_cast<hipStream_t>(stream);
    if (ws.debug_checks && debug_checks())
        if (int bad = check_tables(seqlens, block_table, bt_stride, batch, num_pages, st))
            return bad;

    const int rows = s_q * h_q;
    const size_t slots = (size_t)batch + (size_t)num_parts;
    float *o_part = static_cast<float *>(workspace);
    float *lse_part = o_part + slots * (size_t)rows * 512;

    mla::DecodeParams p;
    p.q = q;
    p.kv = kv_cache;
    p.block_table = block_table;
    p.bt_stride = bt_stride;
    p.page_max = (uint32_t)std::min<int64_t>(num_pages - 1, INT32_MAX);
    p.seqlens = seqlens;
    p.meta = metadata;
    p.num_parts = num_parts;
    p.s_q = s_q;
    p.h_q = h_q;
    p.causal = causal;
    p.scale_log2 = scale * 1.4426950408889634f;
    p.o_part = o_part;
    p.lse_part = lse_part;
    p.out = out;
    p.lse = lse;
    // 128-row tiles (the last one possibly partly empty) from 48 rows on,
    // one shared-row 32-row tile at 32 rows, else 16-row tiles
    const int row_tiles = mla::decode_row_tiles(rows);
    const hipError_t e =
        mla::use_wide(rows)     ? mla::launch_decode_wide(p, num_parts, row_tiles, st)
        : mla::use_wide32(rows) ? mla::launch_decode_wide32(p, num_parts, row_tiles, st)
                                : mla::launch_decode_r16(p, num_parts, row_tiles, st);
    if (e != hipSuccess) return hip_status(e, "decode kernel launch");

    // heavily split sequences get the schedule's extra merge workgroups
    const mla::MetaLayout L{batch, num_parts};
    mla::CombineParams c;
    c.o_part = o_part;
    c.lse_part = lse_part;
    c.split_off = metadata + L.split_off();
    c.extra_off = metadata + L.extra_off();
    c.rows = rows;
    c.skip_single = 1;
    c.out = out;
    c.lse = lse;
    return hip_status(mla::launch_combine(c, batch, (int)L.extra_max(), st),
                      "combine kernel launch");
}

}  // namespace mla

extern "C" {

const char *mla_status_str(int status)
{
    switch (status) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_INVALID_ARG: return "MLA_ERR_INVALID_ARG";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED";
    case MLA_ERR_WORKSPACE: return "MLA_ERR_WORKSPACE";
    case MLA_ERR_HIP: return "MLA_ERR_HIP";
    default: return "MLA_ERR_UNKNOWN";
    }
}

const char *mla_last_error(void) { return g_last_error; }

int mla_device_cus(int device, int *cus)
{
    if (cus == nullptr) return fail(MLA_ERR_INVALID_ARG, "cus is null");
    int v = 0;
    hipError_t e = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, device);
    if (e != hipSuccess) return hip_status(e, "hipDeviceGetAttribute");
    *cus = v;
    return ok();
}

int mla_default_num_parts(int num_cus, int batch, int s_q, int h_q)
{
    (void)batch;
    if (num_cus < 1) num_cus = 1;
    const int rows = (s_q > 0 && h_q > 0) ? s_q * h_q : 16;
    const int row_tiles = mla::decode_row_tiles(rows);
    int parts = num_cus / row_tiles;
    if (parts < 1) parts = 1;
    if (parts > mla::kMaxParts) parts = mla::kMaxParts;
    return parts;
}

size_t mla_metadata_ints(int batch, int num_parts)
{
    if (batch < 0 || num_parts < 0) return 0;
    return (size_t)mla::MetaLayout{batch, num_parts}.ints();
}

size_t mla_workspace_bytes(int batch, int s_q, int h_q, int num_parts)
{
    if (batch < 0 || s_q < 0 || h_q < 0 || num_parts < 0) return 0;
    return ((size_t)batch + (size_t)num_parts) * (size_t)s_q * (size_t)h_q * (512 + 1) * 4;
}

int mla_get_metadata(const int32_t *seqlens, int batch, int s_q, int h_q, int num_parts,
                     int32_t *metadata, void *stream)
{
    if (seqlens == nullptr || metadata == nullptr)
        return fail(MLA_ERR_INVALID_ARG, "seqlens and metadata must be non-null");
    if (!aligned(seqlens, 4) || !aligned(metadata, 16))
        return fail(MLA_ERR_INVALID_ARG, "metadata must be 16-byte aligned, seqlens 4-byte");
    if (int st = check_rows(batch, s_q, h_q)) return st;
    if (batch > mla::kMetaMaxBatch)
        return fail(MLA_ERR_UNSUPPORTED, "batch must be <= %d (got %d)", mla::kMetaMaxBatch, batch);
    if (num_parts < 1 || num_parts > mla::kMaxParts)
        return fail(MLA_ERR_INVALID_ARG, "num_parts must be in [1, %d] (got %d)", mla::kMaxParts,
                    num_parts);
    const int rows = s_q * h_q;
    return hip_status(mla::launch_metadata(seqlens, batch, num_parts, mla::segment_cost(rows),
                                           mla::use_wide(rows), metadata,
                                           static_cast<hipStream_t>(stream)),
                      "metadata kernel launch");
}

int mla_decode(const uint16_t *q, const uint16_t *kv_cache, int64_t num_pages,
               const int32_t *block_table, int64_t bt_stride, const int32_t *seqlens,
               int batch, int s_q, int h_q, int d_qk, int d_v, int page_size,
               float scale, int causal, const int32_t *metadata, int num_parts,
               void *workspace, size_t workspace_bytes, uint16_t *out, float *lse,
               void *stream)
{
    mla::WorkspaceSource ws;
    ws.ptr = workspace;
    ws.bytes = workspace_bytes;
    return mla::decode_call(q, kv_cache, num_pages, block_table, bt_stride, seqlens, batch, s_q,
                            h_q, d_qk, d_v, page_size, scale, causal, metadata, num_parts, ws,
                            out, lse, stream);
}

int mla_combine(const float *o_part, const float *lse_part, const int32_t *split_offsets,
                int batch, int s_q, int h_q, int d_v, uint16_t *out, float *lse, void *stream)
{
    if (!o_part || !lse_part || !split_offsets || !out || !lse)
        return fail(MLA_ERR_INVALID_ARG, "all pointers must be non-null");
    if (int st = check_rows(batch, s_q, h_q)) return st;
    if (d_v != 512) return fail(MLA_ERR_UNSUPPORTED, "d_v must be 512 (got %d)", d_v);
    if (!aligned(o_part, 16) || !aligned(out, 16))
        return fail(MLA_ERR_INVALID_ARG, "o_part and out must be 16-byte aligned");
    mla::CombineParams c;
    c.o_part = o_part;
    c.lse_part = lse_part;
    c.split_off = split_offsets;
    c.extra_off = nullptr;   // no schedule: four waves per row of a heavy sequence
    c.rows = s_q * h_q;
    c.skip_single = 0;
    c.out = out;
    c.lse = lse;
    return hip_status(mla::launch_combine(c, batch, 0, static_cast<hipStream_t>(stream)),
                      "combine kernel launch");
}

int mla_absorb_bmm(const uint16_t *x, int64_t x_stride_b, int64_t x_stride_h,
                   const uint16_t *w, int heads, int K, int N,
                   uint16_t *y, int64_t y_stride_b, int64_t y_stride_h, int batch,
                   void *stream)
{
    if (!w) return fail(MLA_ERR_INVALID_ARG, "w must be non-null");
    if (!aligned(w, 16)) return fail(MLA_ERR_INVALID_ARG, "w must be 16-byte aligned");
    return absorb(x, x_stride_b, x_stride_h, w, nullptr, nullptr, heads, K, N, y, y_stride_b,
                  y_stride_h, batch, stream);
}

int mla_absorb_bmm_fp8w(const uint16_t *x, int64_t x_stride_b, int64_t x_stride_h,
                        const uint8_t *w, const float *w_scale, int heads, int K, int N,
                        uint16_t *y, int64_t y_stride_b, int64_t y_stride_h, int batch,
                        void *stream)
{
    if (!w || !w_scale) return fail(MLA_ERR_INVALID_ARG, "w and w_scale must be non-null");
    if (!aligned(w, 16) || !aligned(w_scale, 4))
        return fail(MLA_ERR_INVALID_ARG, "w must be 16-byte aligned and w_scale 4-byte");
    return absorb(x, x_stride_b, x_stride_h, nullptr, w, w_scale, heads, K, N, y, y_stride_b,
                  y_stride_h, batch, stream);
}

int mla_probe_read(const void *buf, int64_t bytes, int workgroups, uint32_t *sink, void *stream)
{
    if (!buf || !sink) return fail(MLA_ERR_INVALID_ARG, "buf and sink must be non-null");
    if (bytes < 16 || bytes % 16 != 0 || !aligned(buf, 16))
        return fail(MLA_ERR_INVALID_ARG, "buf must be 16-byte aligned and bytes a positive "
                                         "multiple of 16");
    if (workgroups < 1 || workgroups > (1 << 20))
        return fail(MLA_ERR_INVALID_ARG, "workgroups must be in [1, 2^20]");
    return hip_status(mla::launch_probe_read(buf, bytes, workgroups, sink,
                                             static_cast<hipStream_t>(stream)),
                      "read probe launch");
}

int mla_probe_mfma(int iters, int workgroups, float *sink, void *stream)
{
    if (!sink) return fail(MLA_ERR_INVALID_ARG, "sink must be non-null");
    if (iters < 1 || workgroups < 1 || workgroups > (1 << 20))
        return fail(MLA_ERR_INVALID_ARG, "iters must be >= 1 and workgroups in [1, 2^20]");
    return hip_status(mla::launch_probe_mfma(iters, workgroups, sink,
                                             static_cast<hipStream_t>(stream)),
                      "mfma probe launch");
}

#if MLA_STAMPS
// instrumented build only (not part of the public header): the buffer the
// decode kernels write each workgroup's timing record to (layout in
// stamps.h), or null
int mla_stamps_set(uint64_t *buf)
{
    if (hipError_t e = mla::set_stamps_r16(buf)) return hip_status(e, "stamps (16-row kernel)");
    return hip_status(mla::set_stamps_wide(buf), "stamps (128-row kernel)");
}
#endif

int mla_probe_lds(int waves, int depth, int iters, int workgroups, uint32_t *ticks,
                  uint32_t *sink, void *stream)
{
    if (!ticks || !sink) return fail(MLA_ERR_INVALID_ARG, "ticks and sink must be non-null");
    if (waves < 1 || waves > 16 || iters < 1 || workgroups < 1 || workgroups > (1 << 20))
        return fail(MLA_ERR_INVALID_ARG,
                    "waves must be in [1, 16], iters >= 1 and workgroups in [1, 2^20]");
    if (depth != 1 && depth != 2 && depth != 4 && depth != 8 && depth != 16)
        return fail(MLA_ERR_INVALID_ARG, "depth must be 1, 2, 4, 8 or 16 (got %d)", depth);
    return hip_status(mla::launch_probe_lds(waves, depth, iters, workgroups, ticks, sink,
                                            static_cast<hipStream_t>(stream)),
                      "lds probe launch");
}

}  // extern "C"
