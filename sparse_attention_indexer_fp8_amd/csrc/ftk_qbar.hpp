// Head-weighted query sum for the FP8 score path.
//
// With ReLU(x) = (x + |x|) / 2 the indexer score (FlashTopK README, "Quick
// start", indexer-score equation) splits into
//     sum_h w[t,h] ReLU(x_h) = ( sum_h w[t,h] |x_h|  +  qbar[t] . kv[s] ) / 2,
//     qbar[t] = sum_h w[t,h] q[t,h,:],
// an identity of real numbers.  The |x_h| half costs one fused multiply-add
// per (row, head, key) in the vector ALUs, half of max + multiply-add; the
// linear half is one more dot product per (row, key), done on the matrix
// cores.  The FP8 MFMA takes 8-bit operands only, so qbar (binary32) is
// scaled by a per-row power of two 2^e (largest component in [128, 256)) and
// written as the sum of three FP8 E4M3 parts, each the truncation of what the
// previous parts left over; the matrix cores then accumulate
// sum_p part_p . kv[s] and the kernel multiplies by 2^-e.  Three parts carry
// 12 significant bits of every component: exact whenever qbar's components
// have at most 12 (integer-valued operands with dyadic weights), and about
// 2^-12 relative to the row's largest component otherwise.  Rows with short
// windows (kPlainKeys) are scored without it.
#pragma once

#include "ftk_common.hpp"

namespace ftk {

constexpr int kQbarParts = 3;

// OCP E4M3 ("fn") code -> binary32, exact.  The 7 magnitude bits placed at
// bits 26..20 of a binary32 read as 2^(e - 127) (1 + m / 8), or as the
// subnormal (m / 8) 2^-126 when e = 0; times 2^120 both are the E4M3 value
// (binary32 subnormals are kept: the kernels run with f32 denormals on).
// Branch-free: three instructions.
__device__ __forceinline__ float e4m3_to_f32(uint32_t c)
{
    const float mag = __uint_as_float((c & 0x7Fu) << 20) * 0x1p120f;
    return __uint_as_float(__float_as_uint(mag) | ((c & 0x80u) << 24));
}

// binary32 with |v| <= 448 -> E4M3 code, truncating toward zero (selects,
// no branches).
__device__ __forceinline__ uint32_t f32_to_e4m3_trunc(float v)
{
    const uint32_t b = __float_as_uint(v), s = (b >> 24) & 0x80u;
    const int E = (int)((b >> 23) & 0xFFu) - 127;
    const uint32_t sub = (uint32_t)(fabsf(v) * 512.0f);                   // below 2^-6: trunc(|v| / 2^-9), 0 below 2^-9
    const uint32_t nrm = ((uint32_t)(E + 7) << 3) | ((b >> 20) & 7u);   // normal: top 3 mantissa bits
    return s | (E < -6 ? sub : nrm);
}

// Rows 4 blk .. 4 blk + 3, one wave per query row (a 256-thread
// workgroup); lane l owns dimensions 2l and 2l+1.  Writes parts[t][p][d]
// (E4M3 codes) and qscale[t] = 2^-e, and with q1 non-null
// q1[t] = sum_h |w[t,h]| ||q[t,h,:]||_1 (the score bound's rounding margin).
// Run by k_prep.
__device__ __forceinline__ void qbar_rows(const uint8_t *q, const float *w, int64_t num_q, uint8_t *parts,
                                          float *qscale, float *q1, int64_t blk)
{
    const int lane = threadIdx.x & 63;
    const int64_t t = blk * 4 + (threadIdx.x >> 6);
    if (t >= num_q) return;
    const uint8_t *qr = q + t * kHeads * kDim + 2 * lane;
    uint32_t c[kHeads];
    float wv[kHeads];
#pragma unroll
    for (int h = 0; h < kHeads; ++h) {  // every load in flight before the FMAs
        c[h] = *reinterpret_cast<const uint16_t *>(qr + h * kDim);
        wv[h] = w[t * kHeads + h];
    }
    float v0 = 0.0f, v1 = 0.0f, l1 = 0.0f;
#pragma unroll
    for (int h = 0; h < kHeads; ++h) {
        const float d0 = e4m3_to_f32(c[h] & 0xFFu), d1 = e4m3_to_f32(c[h] >> 8);
        v0 = __builtin_fmaf(wv[h], d0, v0);
        v1 = __builtin_fmaf(wv[h], d1, v1);
        l1 = __builtin_fmaf(fabsf(wv[h]), fabsf(d0) + fabsf(d1), l1);
    }
    if (q1) {
        for (int off = 32; off > 0; off >>= 1) l1 += __shfl_xor(l1, off);
        if (lane == 0) q1[t] = l1;
    }
    float m = fmaxf(fabsf(v0), fabsf(v1));
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    int k = 0;
    if (m > 0.0f) {
        int E;
        frexpf(m, &E);  // m = f * 2^E, f in [0.5, 1)
        k = 8 - E;      // m * 2^k in [128, 256)
    }
    float r0 = ldexpf(v0, k), r1 = ldexpf(v1, k);
    uint8_t *out = parts + t * kQbarParts * kDim + 2 * lane;
    for (int p = 0; p < kQbarParts; ++p) {
        const uint32_t c0 = f32_to_e4m3_trunc(r0), c1 = f32_to_e4m3_trunc(r1);
        r0 -= e4m3_to_f32(c0);  // exact: the part holds the leading bits of r0
        r1 -= e4m3_to_f32(c1);
        *reinterpret_cast<uint16_t *>(out + p * kDim) = (uint16_t)(c0 | (c1 << 8));
    }
    if (lane == 0) qscale[t] = ldexpf(1.0f, -k);
}

// The same parts for the 16 columns of a q tile staged in LDS (heads 0-31 in
// the tile's slot layout: byte d of head h of column n at
// ((2 h + (d / 16) % 2) * 64 + n + 16 (d / 32)) * 16 + d % 16), written to
// heads 32-34 of the tile, and each column's 2^-e to s_qsc[n].  s_w[h * 16 +
// n] holds the column's weights.  The sums, the scale and the truncations
// are those of qbar_rows, in the same order, so the parts have the same bits
// as the ones the preparation pass writes.  NT threads (the whole
// workgroup); one wave per column, lane l owning dimensions 2l and 2l + 1.
// Columns without a row (s_row[n] < 0) are skipped: their scores are never
// kept, whatever their parts hold.
template <int NT>
__device__ __forceinline__ void qbar_tile_lds(uint8_t *s_q, const float *s_w, float *s_qsc, const int *s_row)
{
    constexpr int NW = NT / 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int d = 2 * lane;
    const int off = ((d >> 4) & 1) * 64 * 16 + (d >> 5) * 16 * 16 + (d & 15);  // byte d's place within a head
    for (int n = wave; n < 16; n += NW) {
        if (s_row[n] < 0) continue;  // wave-uniform
        uint32_t c[kHeads];
#pragma unroll
        for (int h = 0; h < kHeads; ++h) c[h] = *reinterpret_cast<const uint16_t *>(s_q + h * 2 * 64 * 16 + n * 16 + off);
        float v0 = 0.0f, v1 = 0.0f;
#pragma unroll
        for (int h = 0; h < kHeads; ++h) {
            const float wv = s_w[h * 16 + n];
            v0 = __builtin_fmaf(wv, e4m3_to_f32(c[h] & 0xFFu), v0);
            v1 = __builtin_fmaf(wv, e4m3_to_f32(c[h] >> 8), v1);
        }
        float m = fmaxf(fabsf(v0), fabsf(v1));
        for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
        int k = 0;
        if (m > 0.0f) {
            int E;
            frexpf(m, &E);
            k = 8 - E;
        }
        float r0 = ldexpf(v0, k), r1 = ldexpf(v1, k);
        for (int p = 0; p < kQbarParts; ++p) {
            const uint32_t c0 = f32_to_e4m3_trunc(r0), c1 = f32_to_e4m3_trunc(r1);
            r0 -= e4m3_to_f32(c0);
            r1 -= e4m3_to_f32(c1);
            *reinterpret_cast<uint16_t *>(s_q + (kHeads + p) * 2 * 64 * 16 + n * 16 + off) = (uint16_t)(c0 | (c1 << 8));
        }
        if (lane == 0) s_qsc[n] = ldexpf(1.0f, -k);
    }
}

}  // namespace ftk
