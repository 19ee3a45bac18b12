// Score-bound key pruning and its per-call decision.
//
// FlashTopK README, "Highlights": per-key-block upper bounds on the score let
// whole blocks of keys be skipped when the bound is below the row's
// threshold, and the method decides per call whether that pays ("Performance":
// with untrained indexers the bound skips few keys and the kernel mostly
// scans; architecture diagram: "Adaptive planner", "SM90/SM100 pruning").  The
// pages give no bound formula; this file uses the box bound over a block's
// per-dimension key extremes.
//
// Bound.  A block b is the 64 keys [64 b, 64 b + 64) (one 64-key step of the
// scoring kernels).  With kmax[b,d] / kmin[b,d] the largest / smallest value
// of dimension d over the block's keys, q+ = max(q, 0) and q- = min(q, 0),
//     q[t,h,:] . k  <=  ub[t,h,b] = q+[t,h,:] . kmax[b,:] + q-[t,h,:] . kmin[b,:]
// for every key k of the block, and with sigma >= 0
//     I[t,s]  <=  U[t,b] = sigmax[b] * sum_{h : w[t,h] > 0} w[t,h] ReLU(ub[t,h,b]).
// kmax and kmin are elements of the key set, so they are exact FP8 / BF16
// codes, and so are q+ and q-: the ub terms are one more pair of 128-dim
// contractions per (row, head, block), run on the same MFMAs as the score
// (A = 16 blocks' extremes, B = 16 queries' q+ / q-).  That is 2 MFMAs per
// head per 16 x 16 (query, block) tile against 64 for scoring the same keys,
// about 3 % of the scan.
//
// Soundness against rounding.  The scan keeps a key when its binary32 score
// reaches the threshold; the score differs from the exact one by less than
// 2^-9 * sigmax[b] * kabs[b] * Q1[t], where kabs[b] is the largest |k| in the
// block and Q1[t] = sum_h |w[t,h]| * ||q[t,h,:]||_1 (the matrix cores' dot
// products, whose error on MI355X is below 2^-16 of sum_d |q_d k_d| for FP8
// operands and at binary32 rounding for BF16, the fp32 head sum, and on the
// FP8 identity path the 12-bit split of the head-weighted query sum, whose
// error is below 2^-11 of each component plus 2^-16 of the largest).  A block
// is skipped for a tile of 16 rows only when
//     U[t,b] + 2^-8 * sigmax[b] * kabs[b] * Q1[t]  <  tau[t]
// for every row of the tile whose window meets the block, so no skipped key
// could have passed the scan's test, and the candidate lists -- hence the
// results -- are bit-identical to the scan's.  A block holding a negative or
// non-finite scale is never skipped.
//
// Decision.  The bound costs about 3 % of the scan it can save, so it is
// only evaluated where it is likely to pay.  While the sample scores are
// computed (the q tile is in LDS then), each tile also evaluates the left
// side of the skip test for kPlanGroups groups of 16 blocks spread over its
// windows.  Once the thresholds are known, every scan work item reads its
// tile's sample and evaluates the bound for its own keys only when at least
// 1/8 of the sampled (row, key) pairs would be skipped -- an adaptive,
// per-tile decision taken on the device, so the call never waits for the
// host and needs no extra pass.  The forced prune path evaluates it always.
#pragma once

#include "ftk_common.hpp"
#include "ftk_frag.hpp"
#include "ftk_qbar.hpp"

namespace ftk {

constexpr int kBlockKeys = kStepKeys;   // keys per bound block
constexpr int kPlanGroups = 2;          // 16-block groups of each tile in the planner sample
// The auto path evaluates the planner sample only for tiles whose sampled
// rows' windows span at least this many keys: the sample costs the same for
// every tile, while what pruning can save grows with the window, and below
// about eight times the sample's 2048 keys a tile's scan is cheap anyway.
// Other tiles are scanned (their planner entries read as not prunable).
constexpr int kPlanMinKeys = 16384;

// ---------------------------------------------------------------------------
// Per-key pass: the scale factor of the scoring kernels (sigh, see sigh_of)
// for [0, num_kv + 64), and with `bounds` set the block extremes:
// kb[b][0][:] = per-dimension max, kb[b][1][:] = min (codes of the operand
// dtype), meta[b] = (sigmax, kabs) with sigmax NaN when the block holds a
// negative or non-finite scale.  One wave per 64 keys.  Block 0 also clears
// the call's statistics (nstats counters), which later kernels accumulate.
//
// Codes are compared as sign-magnitude integers: for finite E4M3 and BF16
// codes the magnitude bits order like the values, and +0 / -0 both map to 0.

template <int DT>
__device__ __forceinline__ int code_ord(uint32_t c)
{
    constexpr uint32_t S = DT == kFP8 ? 0x80u : 0x8000u;
    return (c & S) ? -(int)(c & (S - 1)) : (int)c;
}

template <int DT>
__device__ __forceinline__ uint32_t ord_code(int v)
{
    constexpr uint32_t S = DT == kFP8 ? 0x80u : 0x8000u;
    return v >= 0 ? (uint32_t)v : (S | (uint32_t)(-v));
}

template <int DT>
__device__ __forceinline__ void keyprep_blocks(const uint8_t *kv, const float *sigma, int num_kv, int nblocks,
                                               float *sigh, int bounds, uint8_t *kb, float2 *meta,
                                               unsigned long long *stats, int nstats, int blk)
{
    constexpr int RB = RowBytes<DT>::value;
    constexpr int EPL = DT == kFP8 ? 16 : 8;     // elements per 16-byte load
    constexpr int LPR = kDim / EPL;               // lanes per key row
    constexpr int KPL = 64 / LPR;                 // key rows per load instruction
    constexpr int NLD = kBlockKeys / KPL;         // loads per lane
    if (blk == 0 && (int)threadIdx.x < nstats) stats[threadIdx.x] = 0ull;
    const int lane = threadIdx.x & 63;
    const int b = blk * 4 + (threadIdx.x >> 6);
    const int p0 = b * kBlockKeys;
    if (p0 >= num_kv + 64) return;
    const int p = p0 + lane;
    float sg = 0.0f;
    if (p < num_kv + 64) {
        sg = p < num_kv ? (sigma ? sigma[p] : 1.0f) : 0.0f;
        sigh[p] = p < num_kv ? sigh_of<DT>(sigma, p) : 0.0f;
    }
    if (!bounds || b >= nblocks) return;

    const int p1 = min(p0 + kBlockKeys, num_kv);
    const int sub = lane % LPR, r0 = lane / LPR;  // lane's dims [EPL sub, ...), rows r0, r0 + KPL, ...
    v4i c[NLD];
#pragma unroll
    for (int u = 0; u < NLD; ++u) {  // every load in flight at once
        const int pp = min(p0 + r0 + u * KPL, p1 - 1);
        c[u] = *reinterpret_cast<const v4i *>(kv + (int64_t)pp * RB + sub * 16);
    }
    int mx[EPL], mn[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
        mx[e] = -0x10000;
        mn[e] = 0x10000;
    }
#pragma unroll
    for (int u = 0; u < NLD; ++u) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            const uint32_t word = (uint32_t)c[u][e / (EPL / 4)];
            const int sh = DT == kFP8 ? 8 * (e & 3) : 16 * (e & 1);
            const int v = code_ord<DT>((word >> sh) & (DT == kFP8 ? 0xFFu : 0xFFFFu));
            mx[e] = max(mx[e], v);
            mn[e] = min(mn[e], v);
        }
    }
    // Lanes with the same dims (same lane % LPR) combine.
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1)
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            mx[e] = max(mx[e], __shfl_xor(mx[e], off));
            mn[e] = min(mn[e], __shfl_xor(mn[e], off));
        }
    int am = 0;  // largest code magnitude
#pragma unroll
    for (int e = 0; e < EPL; ++e) am = max(am, max(mx[e], -mn[e]));
    if (lane < LPR) {
        v4i ox, on;
#pragma unroll
        for (int wd = 0; wd < 4; ++wd) {
            uint32_t x = 0, n = 0;
#pragma unroll
            for (int y = 0; y < EPL / 4; ++y) {
                const int e = wd * (EPL / 4) + y, sh = DT == kFP8 ? 8 * y : 16 * y;
                x |= ord_code<DT>(mx[e]) << sh;
                n |= ord_code<DT>(mn[e]) << sh;
            }
            ox[wd] = (int)x;
            on[wd] = (int)n;
        }
        uint8_t *dst = kb + (int64_t)b * 2 * RB + sub * 16;
        *reinterpret_cast<v4i *>(dst) = ox;
        *reinterpret_cast<v4i *>(dst + RB) = on;
    }
    for (int off = 32; off > 0; off >>= 1) am = max(am, __shfl_xor(am, off));
    // scales of the block's keys (lane u: key p0 + u)
    const bool bad = __any(p < p1 && (!(sg >= 0.0f) || !__builtin_isfinite(sg)));
    float smax = p < p1 ? sg : 0.0f;
    for (int off = 32; off > 0; off >>= 1) smax = fmaxf(smax, __shfl_xor(smax, off));
    if (lane == 0) {
        const float ka = DT == kFP8 ? e4m3_to_f32((uint32_t)am) : __uint_as_float((uint32_t)am << 16);
        meta[b] = make_float2(bad ? __builtin_nanf("") : smax, ka);
    }
}

// The call's two independent prologue passes in one launch: workgroups
// [0, key_blocks) run the per-key pass (4 blocks of 64 keys each), the rest
// the FP8 query sums (4 rows each, qbar_rows).  Both are short and
// latency-bound, so sharing a launch overlaps them and saves a kernel
// boundary.
struct PrepArgs {
    const uint8_t *kv;
    const float *sigma;
    int num_kv;
    int nblocks;
    float *sigh;
    int bounds;
    uint8_t *kb;
    float2 *meta;
    unsigned long long *stats;
    int nstats;
    int key_blocks;            // workgroups of the per-key pass
    const uint8_t *q;          // FP8 query sums (q null: none)
    const float *w;
    int64_t num_q;
    uint8_t *parts;
    float *qscale;
    float *q1;                 // Q1 per row (score-bound paths) or null
};

template <int DT>
__global__ __launch_bounds__(256) void k_prep(PrepArgs a)
{
    if ((int)blockIdx.x < a.key_blocks)
        keyprep_blocks<DT>(a.kv, a.sigma, a.num_kv, a.nblocks, a.sigh, a.bounds, a.kb, a.meta, a.stats, a.nstats,
                           (int)blockIdx.x);
    else if (DT == kFP8)
        qbar_rows(a.q, a.w, a.num_q, a.parts, a.qscale, a.q1, (int64_t)blockIdx.x - a.key_blocks);
}

// ---------------------------------------------------------------------------
// Bound of one 16-block group for a tile: lane (n, g) gets, for the blocks
// 16 c + 4 g + i (i < 4) and query n, u[i] = sum_h max(w[n,h], 0) ReLU(ub).
// qp is the lane's slot of head 0 in the LDS q tile (head stride HB bytes),
// s_w the tile's weights [h][16].  A-operand rows past the last block read
// the last block (their outputs are ignored by the caller).

// Splits a fragment of codes into its non-negative and non-positive parts
// (a negative code keeps its bits in qn and becomes +0 in qp).
__device__ __forceinline__ void split_sign(const BFrag<kFP8> &f, BFrag<kFP8> &qp, BFrag<kFP8> &qn)
{
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int neg = (int)((((uint32_t)f.a[i] >> 7) & 0x01010101u) * 0xFFu);
        qp.a[i] = f.a[i] & ~neg;
        qn.a[i] = f.a[i] & neg;
    }
}

__device__ __forceinline__ void split_sign(const BFrag<kBF16> &f, BFrag<kBF16> &qp, BFrag<kBF16> &qn)
{
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int neg = (int)((((uint32_t)f.a[m][i] >> 15) & 0x00010001u) * 0xFFFFu);
            qp.a[m][i] = f.a[m][i] & ~neg;
            qn.a[m][i] = f.a[m][i] & neg;
        }
}

// x = kmax . q+ + kmin . q-  (16 blocks x 16 queries)
__device__ __forceinline__ v4f mfma_ub(const KFrag<kFP8> &kx, const KFrag<kFP8> &kn, const BFrag<kFP8> &qp,
                                       const BFrag<kFP8> &qn)
{
    const v4f z = {0.0f, 0.0f, 0.0f, 0.0f};
    v4f x = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(kx.a, qp.a, z, 0, 0, 0, 0, 0, 0);
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(kn.a, qn.a, x, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ v4f mfma_ub(const KFrag<kBF16> &kx, const KFrag<kBF16> &kn, const BFrag<kBF16> &qp,
                                       const BFrag<kBF16> &qn)
{
    v4f x = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int m = 0; m < 4; ++m)
        x = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, kx.a[m]), __builtin_bit_cast(v8bf, qp.a[m]),
                                                    x, 0, 0, 0);
#pragma unroll
    for (int m = 0; m < 4; ++m)
        x = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, kn.a[m]), __builtin_bit_cast(v8bf, qn.a[m]),
                                                    x, 0, 0, 0);
    return x;
}

// UNR heads are unrolled (their LDS reads and MFMA chains overlap): many
// where registers are plentiful (the sample kernel), few in the scan.
template <int DT, int UNR = 2>
__device__ __forceinline__ v4f bound_group(const uint8_t *kb, int nblocks, int c, const uint8_t *qp, int HB,
                                           const float *s_w, int lane)
{
    const int n = lane & 15, g = lane >> 4;
    KFrag<DT> kx, kn;
    const int bb = min(c * 16 + n, nblocks - 1);  // A row n = block 16 c + n
    constexpr int RB = RowBytes<DT>::value;  // the 16x16 MFMA slices: lane group g holds [RB g / 4, RB (g + 1) / 4)
    load_kfrag_at(kx, kb + (int64_t)(2 * bb) * RB + (RB / 4) * g);
    load_kfrag_at(kn, kb + (int64_t)(2 * bb + 1) * RB + (RB / 4) * g);
    v4f u = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll UNR
    for (int h = 0; h < kHeads; ++h) {
        BFrag<DT> qf, qpos, qneg;
        load_bfrag(qf, qp + h * HB);
        split_sign(qf, qpos, qneg);
        const float wv = fmaxf(s_w[h * kTileQ + n], 0.0f);
        const v4f x = mfma_ub(kx, kn, qpos, qneg);
#pragma unroll
        for (int i = 0; i < 4; ++i) u[i] = __builtin_fmaf(wv, relu_bits(x[i]), u[i]);
    }
    return u;
}

// Left side of the skip test for (row, block): U sigmax + 2^-8 sigmax kabs Q1.
// NaN when the block holds a negative or non-finite scale (never skipped).
__device__ __forceinline__ float bound_value(float u, float2 meta, float q1)
{
    return __builtin_fmaf(0.00390625f * meta.y, q1 * meta.x, u * meta.x);
}

// Keys of the row window [rks, rke) inside block b.
__device__ __forceinline__ int block_overlap(int rks, int rke, int b)
{
    return max(0, min(rke, (b + 1) * kBlockKeys) - max(rks, b * kBlockKeys));
}

}  // namespace ftk
