// noalloc.hip -- mla_decode_noalloc: the paged MLA decode with its split-KV
// partial results in a scratch array that the library owns, for callers that
// cannot allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid allocation).
//
// The array is a file-scope __device__ variable, so every device the library
// runs on holds one copy of it from the first call on that device until the
// process ends.  In host code its name is only a stand-in for the symbol:
// the device address of each device's copy comes from hipGetSymbolAddress,
// called once per device with that device current, and only that address is
// handed to the kernels.  The decode writes every partial it reads in the
// same call, so nothing in the array has to start at zero and no clearing is
// needed.  All calls on one
// device share its array: calls that overlap in time on one device race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/mla_paged_kv.h"
#include "kernels.h"

namespace {

constexpr size_t kScratchBytes = MLA_NOALLOC_SCRATCH_BYTES;   // per device
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void *g_scratch[kMaxDevices];   // device address of each device's copy (null: not yet)

int resolve_scratch(void **out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return mla::set_error(MLA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return mla::set_error(MLA_ERR_UNSUPPORTED, "device %d beyond the %d the scratch table holds",
                              dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_scratch[dev] == nullptr) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || ptr == nullptr)
            return mla::set_error(MLA_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                                  hipGetErrorString(e));
        g_scratch[dev] = ptr;
    }
    *out = g_scratch[dev];
    return MLA_OK;
}

}  // namespace

extern "C" {

int mla_decode_noalloc(const uint16_t *q, const uint16_t *kv_cache, int64_t num_pages,
                       const int32_t *block_table, int64_t bt_stride, const int32_t *seqlens,
                       int batch, int s_q, int h_q, int d_qk, int d_v, int page_size, float scale,
                       int causal, const int32_t *metadata, int num_parts, uint16_t *out, float *lse,
                       void *stream)
{
    mla::WorkspaceSource ws;
    ws.bytes = kScratchBytes;
    ws.resolve = resolve_scratch;
    ws.debug_checks = false;   // no host copies or synchronization on this path
    return mla::decode_call(q, kv_cache, num_pages, block_table, bt_stride, seqlens, batch, s_q,
                            h_q, d_qk, d_v, page_size, scale, causal, metadata, num_parts, ws, out,
                            lse, stream);
}

}  // extern "C"
