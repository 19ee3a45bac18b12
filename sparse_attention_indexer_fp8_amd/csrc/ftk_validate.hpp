// Device check of a call's preconditions (flashtopk_options.validate).
//
// The library does not check its data preconditions on the default path: the
// windows lie inside the keys (0 <= ks <= ke <= num_kv), the operands hold no
// NaN or infinity codes (E4M3 "fn" has no infinity; its NaN is S.1111.111;
// BF16 NaN and infinity have an all-ones exponent), weights are finite, key
// scales finite and non-negative, and page ids lie in the pool.  With the
// option set the call runs this kernel first and reports the violations as
// bit flags (flashtopk_info.invalid), and the call fails before any scoring
// kernel runs: no kernel reads out of bounds and no NaN reaches the scan.
#pragma once

#include "ftk_common.hpp"

namespace ftk {

enum InvalidFlag : unsigned {
    kBadWindow = 1u,   // a window outside [0, num_kv] or with ks > ke
    kBadQ = 2u,        // a NaN / infinity code in q
    kBadKv = 4u,       // a NaN / infinity code in the keys
    kBadWeight = 8u,   // a non-finite weight
    kBadScale = 16u,   // a negative or non-finite key scale
    kBadPage = 32u,    // a page id outside the pool
};

struct ValidateArgs {
    const uint8_t *q;
    int64_t q_pieces;          // 16-byte pieces of q
    const uint8_t *kv;         // contiguous keys, or null
    int64_t kv_pieces;
    const float *w;
    int64_t nw;
    const float *scales;       // or null
    int64_t nscales;
    const int32_t *ks;
    const int32_t *ke;
    int64_t num_q;
    int64_t num_kv;
    const int32_t *table;      // page ids, or null
    int64_t ntable;
    int64_t num_pages;
    int dtype;                 // kFP8 / kBF16
    unsigned *flags;           // zeroed before the launch
};

// Some byte of the word is an E4M3 NaN code (low 7 bits all ones).
__device__ __forceinline__ bool has_nan_e4m3(uint32_t x)
{
    const uint32_t v = (x & 0x7F7F7F7Fu) ^ 0x7F7F7F7Fu;  // a zero byte where the low 7 bits are ones
    return ((v - 0x01010101u) & ~v & 0x80808080u) != 0u;
}

// Some half of the word is a BF16 NaN or infinity (exponent all ones).
__device__ __forceinline__ bool has_naninf_bf16(uint32_t x)
{
    return (x & 0x7F80u) == 0x7F80u || (x & 0x7F800000u) == 0x7F800000u;
}

__device__ __forceinline__ bool bad_piece(const uint8_t *p, int64_t i, int dtype)
{
    const v4i v = reinterpret_cast<const v4i *>(p)[i];
    bool bad = false;
#pragma unroll
    for (int e = 0; e < 4; ++e)
        bad |= dtype == kFP8 ? has_nan_e4m3((uint32_t)v[e]) : has_naninf_bf16((uint32_t)v[e]);
    return bad;
}

__global__ __launch_bounds__(256) void k_validate(ValidateArgs a)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t i0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    unsigned f = 0u;
    for (int64_t i = i0; i < a.q_pieces; i += stride)
        if (bad_piece(a.q, i, a.dtype)) f |= kBadQ;
    for (int64_t i = i0; i < a.kv_pieces; i += stride)
        if (bad_piece(a.kv, i, a.dtype)) f |= kBadKv;
    for (int64_t i = i0; i < a.nw; i += stride)
        if (!__builtin_isfinite(a.w[i])) f |= kBadWeight;
    for (int64_t i = i0; i < a.nscales; i += stride) {
        const float s = a.scales[i];
        if (!__builtin_isfinite(s) || s < 0.0f) f |= kBadScale;
    }
    for (int64_t i = i0; i < a.num_q; i += stride) {
        const int64_t lo = a.ks[i], hi = a.ke[i];
        if (lo < 0 || hi > a.num_kv || lo > hi) f |= kBadWindow;
    }
    for (int64_t i = i0; i < a.ntable; i += stride) {
        const int64_t pg = a.table[i];
        if (pg < 0 || pg >= a.num_pages) f |= kBadPage;
    }
    // one atomic per wave
    unsigned m = 0u;
#pragma unroll
    for (int b = 0; b < 6; ++b)
        if (__ballot((f >> b) & 1u)) m |= 1u << b;
    if ((threadIdx.x & 63) == 0 && m) atomicOr(a.flags, m);
}

__global__ void k_zero_word(unsigned *p)
{
    if (threadIdx.x == 0 && blockIdx.x == 0) *p = 0u;
}

}  // namespace ftk
