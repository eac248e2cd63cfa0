// stamps.h -- per-workgroup timing of the decode kernels, compiled only into
// the instrumented library (MLA_STAMPS=1, built by `build.py --stamps`); in
// the default build every macro below is empty.
//
// Each decode workgroup keeps, in registers, the time it spends in three
// phases of each sequence segment it runs -- set-up (query tile and first
// cache loads), the key loop, and the merge of the wave states with the
// result stores -- and at its end thread 0 writes one record of
// kStampWords 64-bit words to the buffer set by mla_stamps_set:
//   [0] start, [1] end (s_memrealtime, 100 MHz ticks),
//   [2] set-up, [3] key loop, [4] merge and stores (ticks summed over the
//   workgroup's segments, as seen by wave 0), [5] segments, [6], [7] zero.
// Records are indexed by the workgroup's dispatch number (x fastest).  Time
// between segments (an empty sequence skipped) belongs to no phase.
#pragma once
#include <cstdint>

namespace mla {
constexpr int kStampWords = 8;
}

#if MLA_STAMPS
#define MLA_CLOCK() __builtin_amdgcn_s_memrealtime()
// The state lives in LDS, kept by thread 0, so no register is held across
// the kernel for it (the 128-row kernel has none to spare): the start, the
// last mark (low 32 bits: unsigned differences are exact below 2^32 ticks,
// 42 s), the three phase sums, the segment count and the record's index
// (taken at the start, so the end needs no register for the grid size).
#define MLA_STAMP_BEGIN()                                                                 \
    __shared__ uint32_t stp_s[8];                                                         \
    if (threadIdx.x == 0) {                                                               \
        const uint64_t stp_t = MLA_CLOCK();                                               \
        stp_s[0] = (uint32_t)stp_t;                                                       \
        stp_s[1] = (uint32_t)(stp_t >> 32);                                               \
        stp_s[2] = (uint32_t)stp_t;                                                       \
        stp_s[3] = stp_s[4] = stp_s[5] = stp_s[6] = 0;                                    \
        stp_s[7] = blockIdx.y * gridDim.x + blockIdx.x;                                   \
    }
#define MLA_STAMP_SEGMENT()                                                               \
    do {                                                                                  \
        if (threadIdx.x == 0) {                                                           \
            stp_s[2] = (uint32_t)MLA_CLOCK();                                             \
            ++stp_s[6];                                                                   \
        }                                                                                 \
    } while (0)
#define MLA_STAMP_PHASE(PH)                                                               \
    do {                                                                                  \
        if (threadIdx.x == 0) {                                                           \
            const uint32_t stp_t = (uint32_t)MLA_CLOCK();                                 \
            stp_s[3 + (PH)] += stp_t - stp_s[2];                                          \
            stp_s[2] = stp_t;                                                             \
        }                                                                                 \
    } while (0)
#define MLA_STAMP_END(BUF)                                                                \
    do {                                                                                  \
        if (threadIdx.x == 0 && (BUF) != nullptr) {                                       \
            uint64_t *stp_r = (BUF) + kStampWords * (int64_t)stp_s[7];                    \
            stp_r[0] = (uint64_t)stp_s[0] | ((uint64_t)stp_s[1] << 32);                   \
            stp_r[1] = MLA_CLOCK();                                                       \
            stp_r[2] = stp_s[3];                                                          \
            stp_r[3] = stp_s[4];                                                          \
            stp_r[4] = stp_s[5];                                                          \
            stp_r[5] = stp_s[6];                                                          \
            stp_r[6] = 0;                                                                 \
            stp_r[7] = 0;                                                                 \
        }                                                                                 \
    } while (0)
#else
#define MLA_STAMP_BEGIN() ((void)0)
#define MLA_STAMP_SEGMENT() ((void)0)
#define MLA_STAMP_PHASE(PH) ((void)0)
#define MLA_STAMP_END(BUF) ((void)0)
#endif
