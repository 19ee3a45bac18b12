// MFMA operand fragments of the scoring and bound kernels, and the per-key
// scale factor they apply.
//
// Both operands of an MFMA use the same assignment of the 128 dimensions to
// (lane group, byte) slots -- lane group g = lane / 16 holds dimensions
// [32g, 32g+32) -- so a contraction covers every dimension exactly once.
//   A (keys, M = 16 rows): lane (n, g) holds row n's slice, read from global.
//   B (queries, N = 16 columns): lane (n, g) holds column n's slice, read
//   from the q tile in LDS (slot layout: see stage_q_heads).
#pragma once

#include "ftk_common.hpp"

namespace ftk {

template <int DT> struct KFrag;
template <> struct KFrag<kFP8> { v8i a; };
template <> struct KFrag<kBF16> { v4i a[4]; };

// Where the key fragments of a 64-key step come from and where the step's
// scores land, per dtype.  A lane's fragment kt (kt < 4) holds the slice of
// key frag_key(kt) of the step that starts frag_byte(kt) bytes into the key
// row (32 bytes FP8, 64 bytes BF16); after the head sum the lane holds the
// score of key out_base + KSTR kt + i for output element (kt, i).
//   FP8, 16x16x128 MFMAs, four 16-key subtiles: lane (n, g) = (lane % 16,
//   lane / 16) loads key 16 kt + n, dimensions [32 g, 32 g + 32), and ends
//   with keys 4 g + 16 kt + i of query n.
//   BF16, 32x32x16 MFMAs, two 32-key subtiles: lane l loads key
//   32 (kt / 2) + l % 32, dimensions [64 (l / 32) + 32 (kt % 2), +32) (the
//   K steps 4 (kt % 2) .. +3 of its subtile); the MFMA leaves it keys
//   8 (r / 4) + 4 (l / 32) + r % 4 (r < 16) of both subtiles, and the head
//   halves' swap leaves lanes of half (l / 16) % 2 with subtile half's keys.
template <int DT> struct StepLayout;
template <> struct StepLayout<kFP8> {
    static constexpr int KSTR = 16;
    __device__ static __forceinline__ int frag_key(int kt, int lane) { return 16 * kt + (lane & 15); }
    __device__ static __forceinline__ int frag_byte(int, int lane) { return 32 * (lane >> 4); }
    __device__ static __forceinline__ int out_base(int lane) { return 4 * (lane >> 4); }
};
template <> struct StepLayout<kBF16> {
    static constexpr int KSTR = 8;
    __device__ static __forceinline__ int frag_key(int kt, int lane) { return 32 * (kt >> 1) + (lane & 31); }
    __device__ static __forceinline__ int frag_byte(int kt, int lane) { return 128 * (lane >> 5) + 64 * (kt & 1); }
    __device__ static __forceinline__ int out_base(int lane) { return 32 * ((lane >> 4) & 1) + 4 * (lane >> 5); }
};

// A key fragment from its slice (p: first byte).
__device__ __forceinline__ void load_kfrag_at(KFrag<kFP8> &f, const uint8_t *p)
{
    const v4i *src = reinterpret_cast<const v4i *>(p);
    const v4i lo = src[0], hi = src[1];
    f.a = (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

__device__ __forceinline__ void load_kfrag_at(KFrag<kBF16> &f, const uint8_t *p)
{
    const v4i *src = reinterpret_cast<const v4i *>(p);
#pragma unroll
    for (int m = 0; m < 4; ++m) f.a[m] = src[m];
}

// Raw buffer access: a resource (base, size in bytes) held in scalar
// registers, a per-lane 32-bit offset and a wave-uniform offset.  Word 3 of
// the resource selects 32-bit data for the gfx9-family buffer unit; reads at
// or past the size return zeros instead of touching memory.
constexpr int kBufWord3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, kBufWord3);
}

__device__ __forceinline__ v4i buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
{
    return __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
}

// Key fragment through a buffer resource: voff is the lane's byte offset of
// its slice within the key row block, soff the wave's (plus any offset that
// is the same for every lane, so the lane offset needs no vector add).
__device__ __forceinline__ void load_kfrag_buf(KFrag<kFP8> &f, __amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
{
    const v4i lo = buf_load16(r, voff, soff), hi = buf_load16(r, voff, soff + 16);
    f.a = (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

__device__ __forceinline__ void load_kfrag_buf(KFrag<kBF16> &f, __amdgpu_buffer_rsrc_t r, uint32_t voff,
                                               uint32_t soff)
{
#pragma unroll
    for (int m = 0; m < 4; ++m) f.a[m] = buf_load16(r, voff, soff + 16 * m);
}

template <int DT> struct BFrag;
template <> struct BFrag<kFP8> { v8i a; };
template <> struct BFrag<kBF16> { v4i a[4]; };

// A query fragment of the LDS q tile; qp points at the lane's slot of the head.
__device__ __forceinline__ void load_bfrag(BFrag<kFP8> &f, const uint8_t *qp)
{
    const v4i lo = *reinterpret_cast<const v4i *>(qp);
    const v4i hi = *reinterpret_cast<const v4i *>(qp + 1024);
    f.a = (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

__device__ __forceinline__ void load_bfrag(BFrag<kBF16> &f, const uint8_t *qp)
{
#pragma unroll
    for (int m = 0; m < 4; ++m) f.a[m] = *reinterpret_cast<const v4i *>(qp + m * 1024);
}

// Scale factor of key p as the scoring kernels apply it (sigh): sigma on the
// BF16 path, sigma / 2 on the FP8 path (its score is sigma/2 * (...)).
template <int DT>
__device__ __forceinline__ float sigh_of(const float *sigma, int p)
{
    const float sg = sigma ? sigma[p] : 1.0f;
    return DT == kFP8 ? sg * 0.5f : sg;
}

}  // namespace ftk
