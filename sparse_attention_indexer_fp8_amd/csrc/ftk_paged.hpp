// Keys in a paged cache (FlashTopK README, "Roadmap": a paged KV cache, where
// the released kernel needs one contiguous key array).  Logical key s of a call lives in page
// block_table[s / page_size] at slot s % page_size of a page pool
// [num_pages, page_size, 128] (its scale in a pool [num_pages, page_size]).
//
// k_gather_pages copies the call's keys (and scales) into one contiguous
// array in the workspace, after which the call runs as if its keys had been
// contiguous: one streaming pass, 2 x 128 B (FP8) or 2 x 256 B (BF16) per
// key, HBM-bound, a few microseconds at 128K keys against the scan's
// milliseconds.  A page id outside [0, num_pages) (a precondition violation)
// reads as zero keys with zero scale instead of touching memory.
#pragma once

#include "ftk_common.hpp"

namespace ftk {

constexpr int kGatherThreads = 256;
constexpr int kGatherUnroll = 4;  // 16-byte pieces per thread, all loads in flight together

template <int DT>
__global__ __launch_bounds__(kGatherThreads) void k_gather_pages(const uint8_t *pages, const float *spages,
                                                                 const int32_t *table, int page_size,
                                                                 int64_t num_pages, int64_t num_kv, uint8_t *kv,
                                                                 float *sig)
{
    constexpr int RB = RowBytes<DT>::value, PPK = RB / 16;  // 16-byte pieces per key
    const int64_t npieces = num_kv * PPK;
    const int64_t base = ((int64_t)blockIdx.x * kGatherThreads * kGatherUnroll) + threadIdx.x;
    v4i v[kGatherUnroll];
    int64_t src[kGatherUnroll];
#pragma unroll
    for (int u = 0; u < kGatherUnroll; ++u) {
        const int64_t c = base + (int64_t)u * kGatherThreads;
        src[u] = -1;
        v[u] = v4i{0, 0, 0, 0};
        if (c < npieces) {
            const int64_t s = c / PPK;
            const int64_t page = table[s / page_size];
            if (page >= 0 && page < num_pages) src[u] = page * page_size + s % page_size;
        }
    }
#pragma unroll
    for (int u = 0; u < kGatherUnroll; ++u) {
        const int64_t c = base + (int64_t)u * kGatherThreads;
        if (src[u] >= 0) v[u] = *reinterpret_cast<const v4i *>(pages + src[u] * RB + (c % PPK) * 16);
    }
#pragma unroll
    for (int u = 0; u < kGatherUnroll; ++u) {
        const int64_t c = base + (int64_t)u * kGatherThreads;
        if (c >= npieces) continue;
        *reinterpret_cast<v4i *>(kv + c * 16) = v[u];
        if (sig && c % PPK == 0) sig[c / PPK] = (src[u] >= 0 && spages) ? spages[src[u]] : 0.0f;
    }
}

}  // namespace ftk
