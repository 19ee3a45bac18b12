// Fused indexer scoring on gfx950 MFMA.
//
// The score (FlashTopK README, "Quick start", indexer-score equation)
//     I[t,s] = sigma[s] * sum_{h<32} w[t,h] * ReLU(q[t,h,:] . kv[s,:])
// is a dense contraction over d = 128 followed by a per-head nonlinearity and
// a 32-term weighted sum.  One kernel body serves every caller so that the
// score of a (row, key) pair has the same bits on every path:
//   * sample mode  -- scores a strided lattice of each row's window and writes
//                     the sample scores (input of the per-row threshold);
//   * filter mode  -- scores the windows and keeps only keys whose score
//                     reaches the row's threshold (the hot loop);
//   * dense mode   -- scores whole windows of flagged rows into scratch for
//                     exact recovery.
//
// Mapping onto the matrix cores.  A work item is a tile of 16 query rows and
// a chunk of keys.  The tile's q (16 rows x 32 heads x 128) is staged once in
// LDS.  Each wave owns 64-key steps of the chunk; for each head h it issues
// one 16x16 MFMA per 16-key subtile with A = 16 keys (M rows, read straight
// from HBM/L2 into registers) and B = the 16 queries' head-h vectors (N
// columns, read from LDS).  The 16x16 fp32 output leaves each lane four keys
// of ONE query, so the nonlinearity, the w[t,h] weighting and the sum over
// heads all stay inside the lane.  The [T, S] score matrix never reaches HBM.
//
//   FP8 (v_mfma_f32_16x16x128_f8f6f4, one MFMA per 128-dim dot product): the
//   score is evaluated as sigma/2 * (sum_h w |x_h| + qbar . k) (see
//   ftk_qbar.hpp), one vector FMA per (row, head, key) plus three MFMAs per
//   (row, key) on the FP8 parts of qbar, staged in LDS as three extra heads.
//   FP8 MFMAs are fast enough that the vector ALUs would otherwise bound the
//   loop.  Rows with short windows (kPlainKeys) take the plain form instead;
//   a tile that holds one runs the step with a per-lane choice of form, at
//   one more vector op per (row, head, key).
//   BF16 (v_mfma_f32_16x16x32_bf16, four chained MFMAs per dot product): the
//   matrix cores are the bound, so the plain form sigma * sum_h w ReLU(x_h)
//   is kept (ReLU as an integer max on the bit pattern, then an FMA).
//
// Both operands of an MFMA use the same assignment of the 128 dimensions to
// (lane group, byte) slots -- lane group g holds dimensions [32g, 32g+32) --
// so the contraction covers every dimension exactly once.
#pragma once

#include "ftk_bound.hpp"
#include "ftk_common.hpp"
#include "ftk_frag.hpp"
#include "ftk_qbar.hpp"
#include "ftk_tau.hpp"

namespace ftk {

constexpr int kModeFilter = 0;
constexpr int kModeSample = 1;
constexpr int kModeDense = 2;


// q-tile "heads" in LDS: the 32 heads, plus the qbar parts on the FP8 path.
template <int DT> struct TileHeads { static constexpr int value = DT == kFP8 ? kHeads + kQbarParts : kHeads; };

// Per-dtype launch shape.
//   FP8: 16 waves per workgroup (4 per SIMD, up to 128 VGPRs each: the
//   linear half accumulates with the row scale applied inside the MFMA, so
//   its fold needs no extra registers) so that while one wave waits on LDS
//   or memory the others keep the matrix cores and vector ALUs busy; each
//   wave loads its next step's keys as soon as its last MFMA of a step has
//   issued.  The candidate rings then fill the rest of the 160 KiB of LDS.
//   BF16: the q tile takes 128 KiB of LDS and each wave's key fragments 64
//   VGPRs, so 8 waves (2 per SIMD) with the next step's keys prefetched.
// Candidate ring per (wave, query) in filter mode: survivors are staged in LDS
// and flushed to the row's candidate list with one atomic per query.  The
// stride between the 16 rings of a wave is odd in 8-byte entries (ring + 1),
// so the rings start on distinct LDS banks.
//   Sample mode (more bookkeeping registers) uses the 8-wave prefetching
//   shape for both dtypes; BF16 dense mode too.  FP8 dense mode takes the
//   scan's 16-wave shape (122 VGPRs, no candidate rings): 4 waves per SIMD
//   instead of 2 scored the 64-row decode call 10 % faster and the
//   recover-all path of the 4096 x 131072 chunk in 2.4 ms instead of 4.3.
//   The looping dense form (recovery, LOOP) runs 8 waves with one fragment
//   set.  For FP8 the loop's state pushes it 36 bytes per lane past 256
//   registers into scratch memory, and it still recovered every row of the
//   4096 x 131072 chunk in 4.2 ms against 5.6 ms with 4 waves of 512
//   registers; BF16 fits (a packed 65536-row sequence with 57344 rows
//   recovered: 12.5 against 14.2 ms).  The 16-wave form spills 172 bytes.
template <int DT, int MODE, bool LOOP = false> struct ScoreCfg {
    static constexpr bool wide = DT == kFP8 && (MODE == 0 || (MODE == 2 && !LOOP));  // 0: filter, 2: dense
    static constexpr int waves = wide ? 16 : 8;
    static constexpr int ring = DT == kFP8 ? 40 : 24;
    static constexpr bool prefetch = !wide && !LOOP && DT == kFP8;
};
template <int DT> struct RingEntries { static constexpr int value = ScoreCfg<DT, 0>::ring; };
template <int DT> struct RingStride { static constexpr int value = RingEntries<DT>::value + 1; };

struct ScoreArgs {
    const uint8_t *q;          // [num_q, 32, 128] codes
    const uint8_t *kv;         // [num_kv, 128] codes
    const float *sigma;        // [num_kv] or null
    const float *sigh;         // [num_kv + 64]: sigma (BF16) or sigma / 2 (FP8), zero padded
    const float *w;            // [num_q, 32]
    const int32_t *ks;         // [num_q]
    const int32_t *ke;         // [num_q]
    const uint8_t *qbar;       // [num_q, 3, 128] FP8 parts (FP8 path)
    const float *qscale;       // [num_q] 2^-e of the parts (FP8 path)
    int num_q;
    int num_kv;
    int ntiles;                // tiles along the grid's fast index
    int chunk;                 // keys per work item (filter and dense modes)
    int cap;                   // candidate capacity per row
    // filter mode
    const float *tau;          // [num_q] per-row threshold (-inf: take all)
    uint32_t *cnt;             // [num_q] candidate counters
    uint64_t *cand;            // [num_q, cap] candidate keys
    // sample mode
    uint32_t *samp;            // [num_q, sample_target] sample score codes
    int sample_target;
    int sample_min_stride;     // power of two, see sample_stride
    int sample_split;          // workgroups per tile in sample mode
    int tau_in_sample;         // sample mode, one workgroup per tile: it also sets the thresholds
    // dense mode: batch entry e (e < row_limit) is entry row_base + e of the
    // flagged-row list (present while below *nrows), or, with no list, row
    // row_base + e (present while below nrows_direct)
    const int32_t *rowlist;    // flagged rows, or null: every row
    const unsigned long long *nrows;  // device count of flagged rows
    int nrows_direct;          // rows of the call (no list)
    int row_base;              // first entry of this batch
    int row_limit;             // entries per batch
    float *scratch;            // [row_limit, scratch_stride] window scores (dense mode)
    int64_t scratch_stride;
    int32_t *wlen;             // dense mode, or null: window length of each row scored
    // dense mode without the per-call preparation pass: the FP8 query sums
    // come from the staged q tile, the per-key factor from sigma (or the
    // page pool's scales) as each step loads it
    int own_prep;
    // score-bound pruning (sample and filter modes)
    int prune;                 // 0: off; 1: per tile, from its planner sample; 2: always
    const uint8_t *kb;         // [nblocks, 2, 128] block extremes
    const float2 *meta;        // [nblocks] (sigmax, kabs)
    float *q1;                 // [num_q] sum_h |w| ||q_h||_1 (written by sample mode)
    int nblocks;
    float *vplan;              // [ntiles, kPlanGroups, 16 blocks, 16 rows] planner sample
    unsigned long long *plan;  // PlanCounter slots
    // sample mode: the threshold of each row is computed by the tile's
    // workgroup when it is the only one (sample_split 1)
    int topk;
    float rank_scale;
    float *tau_w;              // [rows] written threshold
    // 64-head indexers: row t's heads 0-31 and 32-63 are the tile columns 2t
    // and 2t + 1 (q [num_q / 2, 64, 128] read as [num_q, 32, 128], weights
    // likewise, num_q counting columns); the two columns' head sums are
    // added before the threshold, and only even columns emit results, for
    // row column / 2.
    int pair;
    // dense mode over a paged key cache: kv and sigma are the page pools
    const int32_t *table;      // [ceil(num_kv / page_size)] page ids, or null (contiguous keys)
    int page_size;
    int64_t num_pages;
};

// LDS layout of the q tile: for head h, the 64 lanes' fragments are stored as
// consecutive 16-byte slots, slot (h, sub, lane) at ((h*SUB + sub)*64 + lane)*16
// where lane = n + 16 g (query n, lane group g) and sub indexes the 16-byte
// pieces of the lane's 32 (FP8) or 64 (BF16) bytes.  Each ds_read_b128 of a
// head reads 1 KiB of consecutive LDS, free of bank conflicts.  On the FP8
// path heads 32..34 hold the qbar parts.
// NT threads (the whole workgroup) stage NH heads; each thread's global loads
// (at most 16, else batches of 8) are all issued before their LDS stores, so
// the latency of the tile's reads is paid once or twice, not once per piece.  The loads
// are unconditional (a column without a row reads row 0 and stores zeros,
// a piece past the tile re-reads the last piece and stores nothing): a load
// under a branch would be waited for inside that branch.
template <int DT, int NH, int NT>
__device__ __forceinline__ void stage_q_heads(uint8_t *s_q, const uint8_t *q, const uint8_t *qbar, const int *s_row)
{
    constexpr int RB = RowBytes<DT>::value;
    constexpr int CPR = RB / 16;    // 16-byte pieces per head row
    constexpr int SUB = CPR / 4;    // pieces per lane group
    constexpr int NCH = kTileQ * NH * CPR;
    constexpr int ITER = (NCH + NT - 1) / NT;
    constexpr int BATCH = ITER <= 16 ? ITER : 8;
#pragma unroll
    for (int base = 0; base < ITER; base += BATCH) {
        v4i v[BATCH];
        bool live[BATCH];
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
            const int id = min(threadIdx.x + (base + u) * NT, NCH - 1);
            const int n = id / (NH * CPR);
            const int h = (id / CPR) % NH;
            const int c = id % CPR;
            const int t = s_row[n];
            live[u] = t >= 0;
            const int64_t tt = max(t, 0);
            const uint8_t *src = (h < kHeads) ? q + (tt * kHeads + h) * RB
                                              : qbar + (tt * kQbarParts + (h - kHeads)) * RB;
            v[u] = *reinterpret_cast<const v4i *>(src + c * 16);
        }
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
            const int id = threadIdx.x + (base + u) * NT;
            if (base + u < ITER && id < NCH) {
                const int n = id / (NH * CPR);
                const int h = (id / CPR) % NH;
                const int c = id % CPR;
                const int sub = c % SUB, g = c / SUB;
                *reinterpret_cast<v4i *>(s_q + ((h * SUB + sub) * 64 + n + 16 * g) * 16) =
                    live[u] ? v[u] : (v4i){0, 0, 0, 0};
            }
        }
    }
}

template <int DT, int NT>
__device__ __forceinline__ void stage_q_tile(uint8_t *s_q, const ScoreArgs &a, const int *s_row)
{
    stage_q_heads<DT, TileHeads<DT>::value, NT>(s_q, a.q, a.qbar, s_row);
}

// ---------------------------------------------------------------------------
// One 64-key step of one wave: score kSub subtiles x 4 keys for the lane's
// query.  s_w holds the tile's weights, s_w[h * 16 + n] = w[row n, h].
//
// Software pipeline over heads: the MFMAs of a head are issued while the VALU
// epilogue of an earlier head runs, so the matrix cores and the vector ALUs
// work at the same time; result sets rotate so no copies are needed.  The
// head loop stays rolled so each group of heads is its own scheduling region:
// the compiler cannot hoist every head's operands (or sink every epilogue),
// which would need far more than 256 registers.

struct StepOut {
    float acc[kSub][4];   // FP8: qbar . k + sum_h w |x|;  BF16: sum_h w ReLU(x)
};

__device__ __forceinline__ void epi_abs(float (&acc)[kSub][4], const v4f (&x)[kSub], float w)
{
#pragma unroll
    for (int kt = 0; kt < kSub; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[kt][i] = __builtin_fmaf(w, __builtin_fabsf(x[kt][i]), acc[kt][i]);
}

__device__ __forceinline__ void epi_relu(float (&acc)[kSub][4], const v4f (&x)[kSub], float w)
{
#pragma unroll
    for (int kt = 0; kt < kSub; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[kt][i] = __builtin_fmaf(w, relu_bits(x[kt][i]), acc[kt][i]);
}

// q fragment of one head: qp points at the lane's slot of head 0 (s_q + lane
// * 16); head h adds h * 2 KiB.
__device__ __forceinline__ v8i load_qfrag_fp8(const uint8_t *qp)
{
    const v4i lo = *reinterpret_cast<const v4i *>(qp);
    const v4i hi = *reinterpret_cast<const v4i *>(qp + 1024);
    return (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

__device__ __forceinline__ void mfma_fp8_head(v4f (&x)[kSub], const KFrag<kFP8> (&kf)[kSub], const v8i &qf,
                                              const v4f (&c)[kSub])
{
#pragma unroll
    for (int kt = 0; kt < kSub; ++kt)
        x[kt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(kf[kt].a, qf, c[kt], 0, 0, 0, 0, 0, 0);
}

// The linear half: the qbar parts times the keys, scaled by the row's power
// of two through the B operand's E8M0 scale (A unscaled: code 127).
__device__ __forceinline__ void mfma_lin(v4f (&x)[kSub], const KFrag<kFP8> (&kf)[kSub], const v8i &qf,
                                         const v4f (&c)[kSub], int sb)
{
#pragma unroll
    for (int kt = 0; kt < kSub; ++kt)
        x[kt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(kf[kt].a, qf, c[kt], 0, 0, 0, 127, 0, sb);
}

__device__ __forceinline__ void epi_abs_lin(float (&acc)[kSub][4], const v4f (&x)[kSub], float w, const v4f (&lin)[kSub])
{
#pragma unroll
    for (int kt = 0; kt < kSub; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[kt][i] = __builtin_fmaf(w, __builtin_fabsf(x[kt][i]), lin[kt][i]);
}

// Tiles that hold a plain-form row (kPlainKeys): each lane scores its own
// row's form.  pl = 1 (plain) sums w 2 ReLU(x) from zero; pl = 0 (identity)
// sums w |x| from the linear half, the same bits as epi_abs / epi_abs_lin.
__device__ __forceinline__ void epi_mixed(float (&acc)[kSub][4], const v4f (&x)[kSub], float w, float pl)
{
#pragma unroll
    for (int kt = 0; kt < kSub; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[kt][i] = __builtin_fmaf(w, relu2_or_abs(pl, x[kt][i]), acc[kt][i]);
}

__device__ __forceinline__ void epi_mixed_lin(float (&acc)[kSub][4], const v4f (&x)[kSub], float w, float pl,
                                              const v4f (&lin)[kSub])
{
#pragma unroll
    for (int kt = 0; kt < kSub; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            acc[kt][i] = __builtin_fmaf(w, relu2_or_abs(pl, x[kt][i]), pl != 0.0f ? 0.0f : lin[kt][i]);
}

// One epilogue of the FP8 step, in the tile's variant.
template <bool MIXED>
__device__ __forceinline__ void epi_fp8(float (&acc)[kSub][4], const v4f (&x)[kSub], float w, float pl)
{
    if constexpr (MIXED) epi_mixed(acc, x, w, pl);
    else epi_abs(acc, x, w);
}

// MIXED: the tile holds a plain-form row; pl is the lane's row form (1
// plain, 0 identity).
template <bool MIXED, typename AfterMfma>
__device__ __forceinline__ void score_step(StepOut &o, const KFrag<kFP8> (&kf)[kSub], const uint8_t *s_q,
                                           const float *s_w, int lane, float qsc, float pl, AfterMfma after_mfma)
{
    constexpr int EV = MIXED ? 8 : 4;  // epilogue VALU ops per MFMA
    constexpr int HB = 2048;  // LDS bytes per head of the q tile
    const v4f z[kSub] = {};
    const uint8_t *qp = s_q + lane * 16;
    const float *wp = s_w + (lane & 15);
    // q fragments are double-buffered: the next head's fragment is read from
    // LDS while the MFMAs of the current one issue.
    // The linear half first: the qbar parts (heads 32..34) accumulate in the
    // MFMA with the row's power-of-two scale as the B operand's E8M0 block
    // scale (A unscaled: code 127), so lin = qscale * (qbar . k) exactly, and
    // it seeds acc in the first epilogue; the 16 lin registers are dead
    // after the second head.
    // While its MFMAs issue the wave runs at raised priority: the matrix
    // cores are the bound, so waves that feed them go before waves in their
    // survivor sink (which has no MFMA), and the sink fills the gaps.
    __builtin_amdgcn_s_setprio(1);
    const uint8_t *pp = s_q + lane * 16 + kHeads * HB;
    const int sb = (int)((__float_as_uint(qsc) >> 23) & 0xFFu);  // E8M0 code of qscale (a power of two)
    v4f lin[kSub];
    v8i qa = load_qfrag_fp8(pp), qb = load_qfrag_fp8(pp + HB);
    mfma_lin(lin, kf, qa, z, sb);           // part 0
    qa = load_qfrag_fp8(qp);
    mfma_lin(lin, kf, qb, lin, sb);         // part 1
    qb = load_qfrag_fp8(pp + 2 * HB);
    v4f xa[kSub], xb[kSub];
    mfma_fp8_head(xa, kf, qa, z);  // head 0
    qa = load_qfrag_fp8(qp + HB);
    mfma_lin(lin, kf, qb, lin, sb);         // part 2
    qb = load_qfrag_fp8(qp + 2 * HB);
    mfma_fp8_head(xb, kf, qa, z);  // head 1
    if constexpr (MIXED) epi_mixed_lin(o.acc, xa, wp[0], pl, lin);
    else epi_abs_lin(o.acc, xa, wp[0], lin);
    qa = load_qfrag_fp8(qp + 3 * HB);
    mfma_fp8_head(xa, kf, qb, z);  // head 2
    epi_fp8<MIXED>(o.acc, xb, wp[kTileQ], pl);
    qp += 2 * HB;
    wp += 2 * kTileQ;
    // Loop invariant: qa holds head h's fragment, xa head h-1's results.
#pragma unroll 2
    for (int h = 3; h < kHeads - 1; h += 2) {
        __builtin_amdgcn_sched_barrier(0);
        const float w0 = wp[0], w1 = wp[kTileQ];
        qb = load_qfrag_fp8(qp + 2 * HB);  // head h + 1
        mfma_fp8_head(xb, kf, qa, z);      // head h
        epi_fp8<MIXED>(o.acc, xa, w0, pl); // head h - 1
        qa = load_qfrag_fp8(qp + 3 * HB);  // head h + 2 (at most head 31)
        mfma_fp8_head(xa, kf, qb, z);      // head h + 1
        epi_fp8<MIXED>(o.acc, xb, w1, pl); // head h
        qp += 2 * HB;
        wp += 2 * kTileQ;
        // Issue order: one MFMA, then four epilogue FMAs, so each wave keeps
        // the matrix core fed while its vector work fills the gaps; the LDS
        // reads of the next fragments go out early.
        __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, EV, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, EV, 0);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    mfma_fp8_head(xb, kf, qa, z);  // head 31
    __builtin_amdgcn_s_setprio(0);
    after_mfma();  // the key fragments are free from here on
    epi_fp8<MIXED>(o.acc, xa, wp[0], pl);
    epi_fp8<MIXED>(o.acc, xb, wp[kTileQ], pl);
}

// BF16: v_mfma_f32_32x32x16_bf16, A = 32 keys x 16 dimensions (the lane's
// fragments), B = 16 dimensions x 32 columns from the q tile.  The 32
// columns are the tile's 16 queries for head hp (columns 0-15) and for head
// hp + 16 (columns 16-31), so one chain of 8 MFMAs (K = 128) scores 32 keys
// x 16 queries x 2 heads; the step's two 32-key subtiles interleave their
// chains.  A lane (column l % 32: query l % 16, head half (l / 16) % 2)
// sums ReLU of its half's 16 heads in order, weighted, for 16 keys of each
// subtile; then lanes l and l ^ 16 exchange one subtile's sums (one row
// swap), so that each lane adds the other head half to the subtile it keeps
// (half 0: subtile 0, half 1: subtile 1).  Every score is (heads 0-15) +
// (heads 16-31), each half summed in head order.

typedef float v16f __attribute__((ext_vector_type(16)));

// B fragment of K step s of a head: lane (column n = l % 32, k group
// kb = l / 32) takes dimensions [64 kb + 8 s, +8) of its column's head row,
// piece c = 8 kb + s of the q tile's slot layout (lane group c / 4, sub c % 4).
// qp points at the lane's slot of head 0 of its half: s_q + half * 16 * HB +
// (l % 16 + 32 kb) * 16.
__device__ __forceinline__ v4i bfrag_bf16(const uint8_t *qp, int s)
{
    return *reinterpret_cast<const v4i *>(qp + (s & 3) * 1024 + (s >> 2) * 256);
}

__device__ __forceinline__ void mfma_bf16_pair(v16f (&x)[2], const KFrag<kBF16> (&kf)[kSub], const uint8_t *qp)
{
    const v16f z = {};
    v4i qa = bfrag_bf16(qp, 0), qb;
#pragma unroll
    for (int st = 0; st < 8; st += 2) {
        qb = bfrag_bf16(qp, st + 1);
#pragma unroll
        for (int u = 0; u < 2; ++u)
            x[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, kf[2 * u + (st >> 2)].a[st & 3]),
                                                          __builtin_bit_cast(v8bf, qa), st ? x[u] : z, 0, 0, 0);
        if (st + 2 < 8) qa = bfrag_bf16(qp, st + 2);
#pragma unroll
        for (int u = 0; u < 2; ++u)
            x[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(v8bf, kf[2 * u + ((st + 1) >> 2)].a[(st + 1) & 3]), __builtin_bit_cast(v8bf, qb), x[u],
                0, 0, 0);
    }
}

__device__ __forceinline__ void epi_relu16(float (&acc)[2][16], const v16f (&x)[2], float w)
{
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[u][r] = __builtin_fmaf(w, relu_bits(x[u][r]), acc[u][r]);
}

// BF16 rows always take the plain form: MIXED and pl are unused.
template <bool MIXED, typename AfterMfma>
__device__ __forceinline__ void score_step(StepOut &o, const KFrag<kBF16> (&kf)[kSub], const uint8_t *s_q,
                                           const float *s_w, int lane, float /*qsc*/, float /*pl*/,
                                           AfterMfma after_mfma)
{
    constexpr int HB = 4096;  // LDS bytes per head of the q tile
    const int half = (lane >> 4) & 1;
    const uint8_t *qp = s_q + half * 16 * HB + ((lane & 15) + 32 * (lane >> 5)) * 16;
    const float *wp = s_w + half * 16 * kTileQ + (lane & 15);  // head hp + 16 half: wp[hp * kTileQ]
    float acc[2][16];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[u][r] = 0.0f;
    v16f xa[2], xb[2];
    __builtin_amdgcn_s_setprio(1);  // as on the FP8 path
    mfma_bf16_pair(xa, kf, qp);
#pragma unroll 1
    for (int hp = 1; hp < 15; hp += 2) {
        const float w0 = wp[0], w1 = wp[kTileQ];
        mfma_bf16_pair(xb, kf, qp + HB);
        epi_relu16(acc, xa, w0);
        mfma_bf16_pair(xa, kf, qp + 2 * HB);
        epi_relu16(acc, xb, w1);
        qp += 2 * HB;
        wp += 2 * kTileQ;
    }
    mfma_bf16_pair(xb, kf, qp + HB);
    __builtin_amdgcn_s_setprio(0);
    after_mfma();
    epi_relu16(acc, xa, wp[0]);
    epi_relu16(acc, xb, wp[kTileQ]);
    // Lane l keeps subtile (l / 16) % 2: the swap hands lane l ^ 16 the
    // subtile it keeps and brings back this lane's.
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(acc[0][r]), __float_as_uint(acc[1][r]), false,
                                                         false);
        o.acc[r >> 2][r & 3] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    }
}

// The score of output element (kt, i) from the step accumulators; sh is the
// key's scale factor as stored in sigh (sigma / 2 on the FP8 path, whose acc
// is qbar . k + sum_h w |x|).
template <int DT>
__device__ __forceinline__ float score_of(const StepOut &o, int kt, int i, float sh)
{
    return o.acc[kt][i] * sh;
}

// ---------------------------------------------------------------------------

// Wave-local LDS ordering: wait for this wave's LDS operations to finish
// before other lanes of the wave read what they wrote.
__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
}

// Moves a wave's staged candidates to the rows' candidate lists: one atomic
// per query reserves the slots, then the wave copies.  Slots past the
// capacity are dropped; the counter still counts them (overflow triage).
template <int RS>
__device__ __forceinline__ void ring_flush(const uint64_t *ring, uint32_t ring_cnt, int n, int g, int t,
                                           uint32_t *cnt, uint64_t *cand, int cap)
{
    wave_lds_sync();
    uint32_t base = 0;
    if (g == 0 && ring_cnt > 0 && t >= 0) base = atomicAdd(cnt + t, ring_cnt);
    base = __shfl(base, n);
    if (t >= 0) {
        for (uint32_t k = g; k < ring_cnt; k += 4) {
            const uint64_t v = ring[n * RS + k];
            if (base + k < (uint32_t)cap) cand[(int64_t)t * cap + base + k] = v;
        }
    }
    wave_lds_sync();
}

// ---------------------------------------------------------------------------

// Sample mode with one workgroup per tile (sample_split == 1) and the
// thresholds asked of it (tau_in_sample), after the workgroup's samples are
// written: it sets the threshold of each of the tile's rows from the row's
// samples, each wave taking its rows together (wave_tau_rows), and resets
// the row's candidate counter.  The samples were written by this
// workgroup's own waves, so workgroup-scope ordering is all it needs (an
// agent-scope fence would write back and invalidate the L2 and cost more
// than the thresholds).  hist: NW * kTauBuckets words of LDS that nothing
// else uses any more.  Called by every thread of the workgroup.
template <int NW, bool PAIR>
__device__ __forceinline__ void tile_tau(const ScoreArgs &a, int tile, uint32_t *hist, const int *s_row, const int *s_ks,
                                         const int *s_ke, const int *s_nl)
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __syncthreads();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    constexpr int R = PAIR ? kTileQ / 2 : kTileQ;  // rows per tile
    constexpr int K = (R + NW - 1) / NW;           // rows per wave, computed together
    const int64_t nrows = PAIR ? (int64_t)a.num_q >> 1 : (int64_t)a.num_q;
    const uint32_t *sp[K];
    int ns[K];
    uint32_t rk[K];
    int64_t tt[K];
    bool sampled[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
        // the row's window and lattice as the workgroup set them up (its
        // first column); unsampled rows take their whole window
        const int rr = wave + k * NW, col = PAIR ? 2 * rr : rr;
        const int64_t t = (int64_t)tile * R + rr;
        tt[k] = rr < R && t < nrows ? t : -1;
        sampled[k] = tt[k] >= 0 && s_row[col] >= 0;
        ns[k] = sampled[k] ? s_nl[col] : 1;
        rk[k] = sampled[k] ? tau_rank(a.topk, ns[k], (int64_t)s_ke[col] - s_ks[col], a.rank_scale) : 1u;
        sp[k] = a.samp + (sampled[k] ? tt[k] : 0) * a.sample_target;
    }
    float tv[K];
    wave_tau_rows<K>(sp, ns, rk, hist + wave * kTauBuckets, lane, tv);
#pragma unroll
    for (int k = 0; k < K; ++k)
        if (lane == 0 && tt[k] >= 0) {
            a.tau_w[tt[k]] = sampled[k] ? tv[k] : -__builtin_inff();
            a.cnt[tt[k]] = 0u;
        }
}

// PAIR: 64-head rows, two tile columns each (see ScoreArgs::pair).  LOOP
// (dense mode only): each workgroup loops over work items, for a grid
// smaller than the work (the recovery batches, whose row count only the
// device knows); without it a workgroup scores one item, which keeps the
// register allocation of the one-item body.
template <int DT, int MODE, bool PAIR, bool LOOP = false>
__global__ __launch_bounds__((64 * ScoreCfg<DT, MODE, LOOP>::waves)) void k_score(ScoreArgs a)
{
    static_assert(!LOOP || MODE == kModeDense, "only dense mode loops");
    using Cfg = ScoreCfg<DT, MODE, LOOP>;
    constexpr int kWaves = Cfg::waves;
    constexpr int RB = RowBytes<DT>::value;
    constexpr int TH = TileHeads<DT>::value;
    constexpr int RING = (MODE == kModeFilter) ? RingEntries<DT>::value : 1;
    constexpr int RS = (MODE == kModeFilter) ? RingStride<DT>::value : 1;
    // One LDS block carved by hand: weights (2 KiB) then the q tile, so the
    // weight and q-fragment reads of the head loop fit the 16-bit immediate
    // offset of ds_read; the candidate rings last.
    constexpr int QB = kTileQ * TH * RB;
    constexpr int WB = kHeads * kTileQ * 4;
    constexpr int RGB = (MODE == kModeFilter) ? kWaves * kTileQ * RS * 8 : 0;
    __shared__ __attribute__((aligned(16))) uint8_t smem[WB + QB + RGB];
    __shared__ int s_row[kTileQ], s_ks[kTileQ], s_ke[kTileQ], s_d[kTileQ];
    __shared__ int s_nl[MODE == kModeSample ? kTileQ : 1];  // sample mode: lattice size of each column
    // output row of each column (-1: none; with pair, odd columns), and its
    // scratch slot in dense mode
    __shared__ int s_out[PAIR ? kTileQ : 1], s_slot[PAIR ? kTileQ : 1];
    // Filter mode with pruning: offsets (from jlo) of the steps whose block
    // is not skipped, in order.
    constexpr int kMaxSteps = kMaxChunk / kStepKeys;
    __shared__ uint16_t s_steps[MODE == kModeFilter ? kMaxSteps : 1];
    __shared__ uint16_t s_skip[MODE == kModeFilter ? kMaxSteps / 16 + 1 : 1];  // per 16-block group
    __shared__ int s_wcnt[kWaves];
    __shared__ float s_tau[kTileQ], s_q1[kTileQ];
    __shared__ float s_qsc[MODE == kModeDense ? kTileQ : 1];  // dense mode without the preparation pass: 2^-e
    __shared__ float s_l1[MODE == kModeSample ? kTileQ * kHeads : 1];
    __shared__ unsigned long long s_pp[2];  // planner sample: pairs, prunable pairs
    __shared__ int s_next;                  // sample mode: next unclaimed step
    float *s_w = reinterpret_cast<float *>(smem);
    uint8_t *s_q = smem + WB;
    uint64_t *s_ring = reinterpret_cast<uint64_t *>(smem + WB + QB);

    // Dense mode loops over its work items (a grid smaller than the work, or
    // a batch whose row count is only known on the device): the tiles that
    // hold present entries times the key chunks.
    int ntiles = a.ntiles, nitems = 1;
    if constexpr (LOOP) {
        int64_t ent = a.rowlist ? (int64_t)*a.nrows - a.row_base : (int64_t)a.nrows_direct - a.row_base;
        ent = min(max(ent, (int64_t)0), (int64_t)a.row_limit);
        ntiles = (int)(((ent << (PAIR ? 1 : 0)) + kTileQ - 1) / kTileQ);
        nitems = ntiles * max(1, (a.num_kv + a.chunk - 1) / a.chunk);
    }
    for (int item = blockIdx.x; !LOOP || item < nitems; item += gridDim.x) {
    auto body = [&]() {
    // Work item: tile (fast index) x chunk; in sample mode the "chunk" is the
    // part of the tile's sample lattice (sample_split parts).  The filter
    // scan takes its items last tile and last chunk first: with causal or
    // packed windows the later rows of a document have the longer windows,
    // so the long items start early and short ones fill the end of the
    // grid (packed BF16 sequence: scan 4.16 -> 3.91 ms).
    const int witem = (MODE == kModeFilter) ? (int)gridDim.x - 1 - item : item;
    const int chunk = witem / ntiles;
    const int tile = witem - chunk * ntiles;
    // Sample mode: every workgroup, with or without work, ends here; with
    // one workgroup per tile it sets the tile's thresholds (the q tile's LDS
    // is free by then and holds the histograms).
    static_assert(MODE != kModeSample || QB >= kWaves * kTauBuckets * 4, "histograms fit the q tile");
    auto finish = [&]() {
        if constexpr (MODE == kModeSample)
            if (a.tau_in_sample) tile_tau<kWaves, PAIR>(a, tile, reinterpret_cast<uint32_t *>(s_q), s_row, s_ks, s_ke, s_nl);
    };

    if (threadIdx.x < kTileQ) {
        const int n = threadIdx.x;
        const int ps = PAIR ? 1 : 0;  // two columns per row
        int t = -1, slot = -1;  // t: the column's q row (row, or 2 row + half)
        if (MODE == kModeDense) {
            const int e = (tile * kTileQ + n) >> ps;
            if (e < a.row_limit) {
                if (a.rowlist) {
                    if ((unsigned long long)(a.row_base + e) < *a.nrows) {
                        t = (a.rowlist[a.row_base + e] << ps) + (n & ps);
                        slot = e;
                    }
                } else if (a.row_base + e < a.nrows_direct) {
                    t = ((a.row_base + e) << ps) + (n & ps);
                    slot = e;
                }
            }
        } else {
            const int64_t tt = (int64_t)tile * kTileQ + n;
            if (tt < a.num_q) t = (int)tt;
        }
        int lo = 0, hi = 0, d = 1;
        if (t >= 0) {
            lo = a.ks[t >> ps];
            hi = a.ke[t >> ps];
            if (hi < lo) hi = lo;
        }
        if (MODE == kModeSample) {
            if (t >= 0 && hi - lo > a.cap) {
                d = sample_stride(hi - lo, a.sample_target, a.sample_min_stride);
                const int dsh = __builtin_ctz((unsigned)d);
                s_nl[n] = (int)min(lattice_count(lo, hi, dsh, lattice_slot(tile, dsh)), (int64_t)a.sample_target);
            } else {
                t = -1;
                lo = hi = 0;
            }
        }
        if (MODE == kModeDense && !LOOP && a.wlen && t >= 0 && (n & ps) == 0 && chunk == 0) a.wlen[t >> ps] = hi - lo;
        s_row[n] = t;
        s_ks[n] = lo;
        s_ke[n] = hi;
        s_d[n] = d;
        if (PAIR) {
            s_out[n] = (t >= 0 && (n & 1) == 0) ? (t >> 1) : -1;
            s_slot[n] = (n & 1) == 0 ? slot : -1;
        }
        if (MODE == kModeFilter) s_tau[n] = t >= 0 ? a.tau[t >> ps] : __builtin_inff();
        // Q1 of the FP8 rows comes from the query-sum pass; BF16 sampling
        // computes it below.
        if ((MODE == kModeFilter || (MODE == kModeSample && DT == kFP8)) && a.prune)
            s_q1[n] = t >= 0 ? a.q1[t] : 0.0f;
        if (n < 2) s_pp[n] = 0ull;
        if (n == 0) s_next = 0;
    }
    __syncthreads();

    // Union (lo, hi) and intersection (ilo, ihi) of the tile's windows; the
    // lattice stride of the tile's samples.
    int lo = 0x7fffffff, hi = 0, ilo = 0, ihi = 0x7fffffff, dmin = 0x40000000;
#pragma unroll
    for (int n = 0; n < kTileQ; ++n) {
        if (s_row[n] >= 0 && s_ke[n] > s_ks[n]) {
            lo = min(lo, s_ks[n]);
            hi = max(hi, s_ke[n]);
            ilo = max(ilo, s_ks[n]);
            ihi = min(ihi, s_ke[n]);
            dmin = min(dmin, s_d[n]);
        }
    }
    // Workgroup-uniform: keep them (and what derives from them) in scalar registers.
    lo = __builtin_amdgcn_readfirstlane(lo);
    hi = __builtin_amdgcn_readfirstlane(hi);
    ilo = __builtin_amdgcn_readfirstlane(ilo);
    ihi = __builtin_amdgcn_readfirstlane(ihi);
    dmin = __builtin_amdgcn_readfirstlane(dmin);
    if (hi <= lo) {
        finish();
        return;
    }

    // Keys of this work item, in 64-key steps [jlo, jhi).  In sample mode the
    // steps index the tile's lattice (stride dmin): step j holds lattice
    // indices e_first + 64 j + [0, 64), e_first the multiple of 64 at or
    // below the index of the first lattice key at or after lo.
    int jlo, jhi, msh = 0, msl = 0;
    int64_t e_first = 0;
    if (MODE == kModeSample) {
        msh = __builtin_ctz((unsigned)dmin);  // power of two
        msl = lattice_slot(tile, msh);
        static_assert(kRunKeys >= 4 && kStepKeys % kRunKeys == 0, "a lane's 4 outputs share a run");
        e_first = lattice_prefix_sh(lo, msh, msl) & ~(int64_t)(kStepKeys - 1);
        const int nsteps = (int)((lattice_prefix_sh(hi, msh, msl) - e_first + kStepKeys - 1) / kStepKeys);
        // With few tiles the lattice is split over a.sample_split workgroups
        // (the chunk index is the part).
        const int per = (nsteps + a.sample_split - 1) / a.sample_split;
        jlo = chunk * per;
        jhi = min(nsteps, jlo + per);
        if (jhi <= jlo) {
            finish();
            return;
        }
    } else {
        const int64_t c0 = (int64_t)chunk * a.chunk;
        const int64_t klo = max((int64_t)lo, c0), khi = min((int64_t)hi, c0 + a.chunk);
        if (khi <= klo) return;
        jlo = (int)(klo / kStepKeys);
        jhi = (int)((khi + kStepKeys - 1) / kStepKeys);
    }

    // Without the preparation pass (dense mode only) the FP8 query sums are
    // computed here from the staged heads.
    const bool own_prep = MODE == kModeDense && !LOOP && a.own_prep;  // workgroup-uniform; recovery (LOOP) reads the prep pass
    // The weights load first so their latency overlaps the q tile's.
    constexpr int WR = (kHeads * kTileQ + 64 * kWaves - 1) / (64 * kWaves);
    float wv[WR];
#pragma unroll
    for (int u = 0; u < WR; ++u) {
        const int i = min((int)threadIdx.x + u * 64 * kWaves, kHeads * kTileQ - 1);
        const int rt = s_row[i & (kTileQ - 1)];
        wv[u] = a.w[(int64_t)max(rt, 0) * kHeads + i / kTileQ];
    }
    if (DT == kFP8 && own_prep) stage_q_heads<DT, kHeads, 64 * kWaves>(s_q, a.q, a.qbar, s_row);
    else stage_q_tile<DT, 64 * kWaves>(s_q, a, s_row);
#pragma unroll
    for (int u = 0; u < WR; ++u) {
        const int i = threadIdx.x + u * 64 * kWaves;
        if (i < kHeads * kTileQ) s_w[i] = s_row[i & (kTileQ - 1)] >= 0 ? wv[u] : 0.0f;
    }
    __syncthreads();
    if (DT == kFP8 && own_prep) {
        qbar_tile_lds<64 * kWaves>(s_q, s_w, s_qsc, s_row);
        __syncthreads();
    }

    int nstep = jhi - jlo;
    bool use_skip = false;  // workgroup-uniform
    // Auto path: does this tile evaluate the planner sample (sample mode)?
    const bool plan = MODE == kModeSample && a.prune == 1 && hi > lo && hi - lo >= kPlanMinKeys;
    if (MODE == kModeSample && DT == kBF16 && (a.prune == 2 || plan)) {
        // Q1[t] = sum_h |w[t,h]| ||q[t,h,:]||_1 of the sampled rows (the
        // bound's rounding margin), from the q tile in LDS: one (row, head)
        // per thread, then one thread per row.
        static_assert(MODE != kModeSample || 64 * kWaves == kTileQ * kHeads, "one (row, head) pair per thread");
        constexpr int SUB = RB / 64;
        const int rn = threadIdx.x & (kTileQ - 1), h = threadIdx.x >> 4;
        float l1 = 0.0f;
#pragma unroll
        for (int gg = 0; gg < 4; ++gg)
#pragma unroll
            for (int sub = 0; sub < SUB; ++sub) {
                const v4i v = *reinterpret_cast<const v4i *>(s_q + ((h * SUB + sub) * 64 + rn + 16 * gg) * 16);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t u = (uint32_t)v[e];
                    if (DT == kFP8) {
#pragma unroll
                        for (int y = 0; y < 4; ++y) l1 += e4m3_to_f32((u >> (8 * y)) & 0x7Fu);
                    } else {
                        l1 += __uint_as_float((u << 16) & 0x7FFF0000u) + __uint_as_float(u & 0x7FFF0000u);
                    }
                }
            }
        s_l1[rn * kHeads + h] = fabsf(s_w[h * kTileQ + rn]) * l1;
        __syncthreads();
        if (threadIdx.x < kTileQ) {
            float q1 = 0.0f;
            for (int hh = 0; hh < kHeads; ++hh) q1 += s_l1[threadIdx.x * kHeads + hh];
            s_q1[threadIdx.x] = q1;
            if (s_row[threadIdx.x] >= 0) a.q1[s_row[threadIdx.x]] = q1;
        }
        __syncthreads();
    }
    if (MODE == kModeSample && a.prune == 1 && !plan && threadIdx.x < 64 * kPlanGroups) {
        // a tile of short windows: its entries read as not prunable
        const int ln = threadIdx.x & 63, wv = threadIdx.x >> 6;
        const int n = ln & 15, g = ln >> 4;
#pragma unroll
        for (int i = 0; i < 4; ++i) a.vplan[(((int64_t)tile * kPlanGroups + wv) * 16 + 4 * g + i) * 16 + n] = __builtin_inff();
    }
    if (MODE == kModeSample && plan && threadIdx.x < 64 * kPlanGroups) {
        // Planner sample: the skip test's left side for kPlanGroups groups
        // spread over the union of ALL the tile's windows (take-all rows
        // included: they can never be skipped, value +inf).
        const int ln = threadIdx.x & 63, wv = threadIdx.x >> 6;
        const int n = ln & 15, g = ln >> 4;
        const int64_t tt = (int64_t)tile * kTileQ + n;
        int rlo = 0, rhi = 0;
        if (tt < a.num_q) {
            rlo = a.ks[tt];
            rhi = max(a.ke[tt], rlo);
        }
        int ulo = rhi > rlo ? rlo : 0x7fffffff, uhi = rhi > rlo ? rhi : 0;
        for (int off = 1; off < 16; off <<= 1) {
            ulo = min(ulo, __shfl_xor(ulo, off));
            uhi = max(uhi, __shfl_xor(uhi, off));
        }
        const int g0 = ulo / (16 * kBlockKeys), g1 = (uhi + 16 * kBlockKeys - 1) / (16 * kBlockKeys);
        const int gs = g0 + ((2 * wv + 1) * (g1 - g0)) / (2 * kPlanGroups);
        const v4f u = bound_group<DT, 8>(a.kb, a.nblocks, gs, s_q + ln * 16, 16 * RB, s_w, ln);
        const bool sampled = s_row[n] >= 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int b = gs * 16 + 4 * g + i;
            const int ov = (b < a.nblocks) ? block_overlap(rlo, rhi, b) : 0;
            const float v = ov == 0 ? -__builtin_inff()
                                    : (sampled ? bound_value(u[i], a.meta[min(b, a.nblocks - 1)], s_q1[n])
                                               : __builtin_inff());
            a.vplan[(((int64_t)tile * kPlanGroups + wv) * 16 + 4 * g + i) * 16 + n] = v;
        }
    }
    if (MODE == kModeFilter && a.prune) {
        bool any_sampled = false;
#pragma unroll
        for (int n = 0; n < kTileQ; ++n) any_sampled |= s_row[n] >= 0 && s_tau[n] > -__builtin_inff();
        if (a.prune == 2) {
            use_skip = true;
        } else if (any_sampled) {
            // Read the tile's planner sample: (group, block, row) per thread.
            const int id = threadIdx.x;
            if (id < kPlanGroups * 256) {
                const int k = id >> 8, blk = (id >> 4) & 15, rn = id & 15;
                const int g0 = lo / (16 * kBlockKeys), g1 = (hi + 16 * kBlockKeys - 1) / (16 * kBlockKeys);
                const int gs = g0 + ((2 * k + 1) * (g1 - g0)) / (2 * kPlanGroups);
                const int b = gs * 16 + blk;
                const int ov = (s_row[rn] >= 0 && b < a.nblocks) ? block_overlap(s_ks[rn], s_ke[rn], b) : 0;
                const float v = a.vplan[(((int64_t)tile * kPlanGroups + k) * 16 + blk) * 16 + rn];
                const bool ok = ov == 0 || v < s_tau[rn];
                const unsigned long long bal = __ballot(ok);
                const bool all = ((bal >> (threadIdx.x & 48)) & 0xFFFFull) == 0xFFFFull;
                int sov = ov;
                for (int off = 1; off < 16; off <<= 1) sov += __shfl_xor(sov, off);
                if (rn == 0 && sov > 0) {
                    atomicAdd(&s_pp[0], (unsigned long long)sov);
                    if (all) atomicAdd(&s_pp[1], (unsigned long long)sov);
                }
            }
            __syncthreads();
            use_skip = s_pp[1] > 0 && s_pp[1] * 8ull >= s_pp[0];
        }
    }
    if (MODE == kModeFilter && use_skip) {
        // The bound of this work item's blocks, one 16-block group per wave
        // at a time; s_skip[c - c0] bit e = block 16 c + e is skipped.
        const int ln = threadIdx.x & 63, wv = threadIdx.x >> 6;
        const int n = ln & 15, g = ln >> 4;
        const int c0 = jlo >> 4, c1 = (jhi + 15) >> 4;
        const int rt = s_row[n], rks = s_ks[n], rke = s_ke[n];
        const float rtau = s_tau[n], rq1 = s_q1[n];
        unsigned long long pr = 0;
        for (int c = c0 + wv; c < c1; c += kWaves) {
            const v4f u = bound_group<DT>(a.kb, a.nblocks, c, s_q + ln * 16, 16 * RB, s_w, ln);
            uint32_t bits = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int b = c * 16 + 4 * g + i;
                const int ov = (rt >= 0 && b >= jlo && b < jhi) ? block_overlap(rks, rke, b) : 0;
                const bool ok = ov == 0 || bound_value(u[i], a.meta[min(b, a.nblocks - 1)], rq1) < rtau;
                const unsigned long long bal = __ballot(ok);
#pragma unroll
                for (int gg = 0; gg < 4; ++gg)
                    if (((bal >> (16 * gg)) & 0xFFFFull) == 0xFFFFull) bits |= 1u << (4 * gg + i);
                if ((bits >> (4 * g + i)) & 1u) pr += (unsigned long long)ov;
            }
            if (ln == 0) s_skip[c - c0] = (uint16_t)bits;
        }
        for (int off = 32; off > 0; off >>= 1) pr += __shfl_xor(pr, off);
        if (ln == 0 && pr) atomicAdd(a.plan + kPlanPruned, pr);
        if (threadIdx.x == 0) atomicAdd(a.plan + kPlanItems, 1ull);
        __syncthreads();
        // Order-preserving compaction of the steps that are not skipped, one
        // step per thread and round.
        int total = 0;
        for (int r0 = 0; r0 < nstep; r0 += 64 * kWaves) {
            const int i = r0 + threadIdx.x;
            bool keep = false;
            if (i < nstep) {
                const int j = jlo + i;
                keep = !((s_skip[(j >> 4) - c0] >> (j & 15)) & 1u);
            }
            const unsigned long long bal = __ballot(keep);
            if (ln == 0) s_wcnt[wv] = __popcll(bal);
            __syncthreads();
            int base = total;
            for (int v = 0; v < kWaves; ++v) {
                base += v < wv ? s_wcnt[v] : 0;
                total += s_wcnt[v];
            }
            if (keep) s_steps[base + __popcll(bal & ((1ull << ln) - 1ull))] = (uint16_t)i;
            __syncthreads();  // s_wcnt is read before the next round writes it
        }
        nstep = __builtin_amdgcn_readfirstlane(total);
    }

    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 15, g = lane >> 4;
    const int t = s_row[n];
    const int to = PAIR ? s_out[n] : t;  // the row this lane's results belong to, or -1
    const int rks = s_ks[n], rke = s_ke[n];
    const int S = a.num_kv;
    const float qsc = (DT == kFP8 && t >= 0) ? (own_prep ? s_qsc[MODE == kModeDense ? n : 0] : a.qscale[t]) : 1.0f;
    // FP8 row forms: the lane's (1 plain, 0 identity) and whether the tile
    // holds any plain row (workgroup-uniform).  Sample scores only steer the
    // threshold, so sampling keeps the identity for every row.
    bool mixed = false;
    float pl = 0.0f;
    if constexpr (DT == kFP8 && MODE != kModeSample) {
#pragma unroll
        for (int c = 0; c < kTileQ; ++c) mixed |= s_row[c] >= 0 && plain_row(s_ks[c], s_ke[c]);
        mixed = __builtin_amdgcn_readfirstlane(mixed ? 1 : 0) != 0;
        pl = t >= 0 && plain_row(rks, rke) ? 1.0f : 0.0f;
    }

    float tau = __builtin_inff();
    if (MODE == kModeFilter && to >= 0) tau = a.tau[to];
    // Sample mode: the row's lattice (stride dn, a multiple of dmin) holds
    // the tile's runs whose step index is a multiple of dn; a key's slot in
    // the row's sample is its lattice rank within the window.
    const int dn = s_d[n];                       // power of two
    const int dsh = __builtin_ctz((unsigned)dn);
    const int rsl = MODE == kModeSample ? lattice_slot(tile, dsh) : 0;
    const int64_t rank0 = MODE == kModeSample ? lattice_prefix_sh(rks, dsh, rsl) : 0;
    uint64_t *ring = s_ring + (MODE == kModeFilter ? wave * kTileQ * RS : 0);
    uint32_t ring_cnt = 0;

    // Key fragments of step j: this lane loads key row 16 kt + n of the step.
    // Filter mode addresses keys and scale factors by 32-bit offsets from the
    // work item's first key (a workgroup-uniform base held in scalar
    // registers), which keeps the hot loop's vector registers free.
    // Keys past num_kv read as zeros (their scores are masked by the windows).
    const int kbase = jlo * kStepKeys;
    const int kspan = min(S - kbase, a.chunk + kStepKeys);
    const __amdgpu_buffer_rsrc_t kvr = make_rsrc(a.kv + (int64_t)kbase * RB, (uint32_t)kspan * RB);
    const __amdgpu_buffer_rsrc_t shr = make_rsrc(a.sigh + kbase, (uint32_t)(kspan + kStepKeys) * 4u);
    using LY = StepLayout<DT>;
    constexpr int KSTR = LY::KSTR;
    // the lane's slice of its fragment-0 key (fragment kt adds a constant)
    const uint32_t klane = (uint32_t)(LY::frag_key(0, lane) * RB + LY::frag_byte(0, lane));
    auto load_step = [&](KFrag<DT>(&f)[kSub], int j) {
#pragma unroll
        for (int kt = 0; kt < kSub; ++kt) {
            const int e = j * kStepKeys + LY::frag_key(kt, lane);
            if (MODE == kModeFilter) {
                const uint32_t soff = (uint32_t)(j * kStepKeys - kbase) * RB;
                const uint32_t kofs = (uint32_t)((LY::frag_key(kt, 0) - LY::frag_key(0, 0)) * RB +
                                                 (LY::frag_byte(kt, 0) - LY::frag_byte(0, 0)));  // compile-time
                load_kfrag_buf(f[kt], kvr, klane, soff + kofs);
            } else {
                int p = e;
                if (MODE == kModeSample)
                    p = (int)min(lattice_key(e_first + e, msh, msl), (int64_t)S - 1);
                p = min(p, S - 1);
                if (MODE == kModeDense && !LOOP && a.table) {
                    // paged keys: logical key p is row p % page_size of its
                    // page (a page id out of range reads the pool's first row;
                    // its scale factor is 0)
                    const int64_t pg = a.table[p / a.page_size];
                    const int64_t slot = (pg >= 0 && pg < a.num_pages) ? pg * a.page_size + p % a.page_size : 0;
                    load_kfrag_at(f[kt], a.kv + slot * RB + LY::frag_byte(kt, lane));
                } else {
                    load_kfrag_at(f[kt], a.kv + (int64_t)p * RB + LY::frag_byte(kt, lane));
                }
            }
        }
    };

    // Scores one step and hands its 16 outputs per lane to the mode's sink;
    // `next` runs as soon as the step's MFMAs no longer need the key
    // fragments (it issues the next step's key loads).
    // mx: std::true_type for the tile variant with plain-form rows (FP8).
    auto process = [&](KFrag<DT>(&kf)[kSub], int j, auto next, auto mx) {
        const int sb = j * kStepKeys + LY::out_base(lane);  // key of element (kt, i) is sb + KSTR kt + i
        // Scale factors of the step's outputs (4 consecutive keys per
        // subtile).  With the prefetching (2-wave) shape they load before the
        // MFMA work so their latency hides; with 4 waves per SIMD other waves
        // hide it and the registers stay free during the head loop.
        v4f shv[kSub];
        auto load_sh = [&]() {
            if (MODE == kModeFilter) {
                const uint32_t soff = (uint32_t)(j * kStepKeys - kbase) * 4u;
#pragma unroll
                for (int kt = 0; kt < kSub; ++kt)
                    shv[kt] = __builtin_bit_cast(v4f, buf_load16(shr, (uint32_t)(4 * LY::out_base(lane)), soff + 4u * KSTR * kt));
            } else if (MODE == kModeSample) {
                // A lane's 4 outputs of a subtile are one run of 4
                // consecutive keys: one aligned load of the padded factors
                // (runs past the keys read the padding; their scores are
                // never kept).
                const int64_t sal = ((int64_t)S + 3) & ~(int64_t)3;
#pragma unroll
                for (int kt = 0; kt < kSub; ++kt) {
                    const int64_t p0 = lattice_key(e_first + sb + KSTR * kt, msh, msl);
                    shv[kt] = *reinterpret_cast<const v4f *>(a.sigh + min(p0, sal));
                }
            } else if (own_prep) {
                // the factor the preparation pass would store: sigma / 2
                // (FP8) or sigma, 0 past the keys and for a page out of range
#pragma unroll
                for (int kt = 0; kt < kSub; ++kt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int p = sb + KSTR * kt + i;
                        float sg = 0.0f;
                        if (p < S) {
                            if (a.table) {
                                const int64_t pg = a.table[p / a.page_size];
                                const bool ok = pg >= 0 && pg < a.num_pages;
                                sg = !ok ? 0.0f : (a.sigma ? a.sigma[pg * a.page_size + p % a.page_size] : 1.0f);
                            } else {
                                sg = a.sigma ? a.sigma[p] : 1.0f;
                            }
                        }
                        shv[kt][i] = DT == kFP8 ? sg * 0.5f : sg;
                    }
            } else {
#pragma unroll
                for (int kt = 0; kt < kSub; ++kt) shv[kt] = *reinterpret_cast<const v4f *>(a.sigh + sb + KSTR * kt);
            }
        };
        // The factors load before the MFMA work where registers allow (their
        // latency hides behind it); otherwise right after the last MFMA and
        // before the next step's key loads (loads complete in order, so
        // waiting for them does not wait for the keys).  BF16 sampling keeps
        // its registers for the key fragments.
        constexpr bool early = Cfg::prefetch && !(DT == kBF16 && MODE == kModeSample);
        if (early) load_sh();
        StepOut o;
        auto after_mfma = [&]() {
            if (!early) load_sh();
            next();
        };
        score_step<decltype(mx)::value>(o, kf, s_q, s_w, lane, qsc, pl, after_mfma);
        if (PAIR) {
            // a row's two columns are neighbouring lanes: add their head sums
#pragma unroll
            for (int kt = 0; kt < kSub; ++kt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    o.acc[kt][i] += __int_as_float(__builtin_amdgcn_update_dpp(
                        0, __float_as_int(o.acc[kt][i]), 0xB1 /* quad_perm [1,0,3,2] */, 0xf, 0xf, false));
        }
        if (MODE == kModeFilter) {
            // Keep (row, key) when the key is in the row's window and its
            // score reaches the row's threshold (take-all rows: -inf).
            // Elements outside the window become NaN, which fails every test.
            float sc[kSub * 4];
#pragma unroll
            for (int kt = 0; kt < kSub; ++kt)
#pragma unroll
                for (int i = 0; i < 4; ++i) sc[kt * 4 + i] = score_of<DT>(o, kt, i, shv[kt][i]);
            const bool inside = j * kStepKeys >= ilo && (j + 1) * kStepKeys <= ihi;  // wave-uniform
            if (__builtin_expect(!inside, 0)) {
#pragma unroll
                for (int b = 0; b < kSub * 4; ++b) {
                    const int s = sb + KSTR * (b >> 2) + (b & 3);
                    if (s < rks || s >= rke) sc[b] = __builtin_nanf("");
                }
            }
            uint32_t m = 0;
#pragma unroll
            for (int b = 0; b < kSub * 4; ++b) m += (sc[b] >= tau) ? 1u : 0u;
            // Survivors of the 4 lanes that hold query n (lanes n + 16 g'):
            // total and this lane's offset, by two row swaps in the VALU (no
            // LDS round trip).  A swap returns the lane's own value in one
            // output and its partner's in the other, so their sum is the
            // pair's: p16 = counts of g and g ^ 1, tot = all four.
            const auto s16 = __builtin_amdgcn_permlane16_swap(m, m, false, false);
            const uint32_t p16 = s16[0] + s16[1];
            const auto s32 = __builtin_amdgcn_permlane32_swap(p16, p16, false, false);
            uint32_t tot = s32[0] + s32[1];
            const uint32_t pre = ((g & 2) ? tot - p16 : 0u) + ((g & 1) ? p16 - m : 0u);
            if (__builtin_expect(__any(ring_cnt + tot > (uint32_t)RING), 0)) {
                ring_flush<RS>(ring, ring_cnt, n, g, to, a.cnt, a.cand, a.cap);
                ring_cnt = 0;
            }
            bool direct = false;
            if (__builtin_expect(__any(tot > (uint32_t)RING), 0)) {
                // More than a ring holds: reserve slots in the row's list directly.
                uint32_t base = 0;
                direct = tot > (uint32_t)RING;
                if (direct && g == 0 && to >= 0) base = atomicAdd(a.cnt + to, tot);
                base = __shfl(base, n);
                uint32_t pos = base + pre;
                if (direct && to >= 0) {
#pragma unroll
                    for (int b = 0; b < kSub * 4; ++b) {
                        if (sc[b] >= tau) {
                            if (pos < (uint32_t)a.cap)
                                a.cand[(int64_t)to * a.cap + pos] = raw_cand(sc[b], sb + KSTR * (b >> 2) + (b & 3));
                            ++pos;
                        }
                    }
                }
            }
            if (__builtin_expect(!direct && __any(m != 0), 1)) {
                uint64_t *rp = ring + n * RS + ring_cnt + pre;
#pragma unroll
                for (int b = 0; b < kSub * 4; ++b) {
                    if (sc[b] >= tau) {
                        *rp = raw_cand(sc[b], sb + KSTR * (b >> 2) + (b & 3));
                        ++rp;
                    }
                }
            }
            ring_cnt += direct ? 0u : tot;
        } else if (MODE == kModeSample) {
            // The lane's 4 outputs of a subtile are one run of the tile's
            // lattice; when the run is on the row's lattice and inside its
            // window they take consecutive sample slots and go out as one
            // 16-byte store where aligned.
            uint32_t *srow = a.samp + (int64_t)(to < 0 ? 0 : to) * a.sample_target;
#pragma unroll
            for (int kt = 0; kt < kSub; ++kt) {
                const int64_t p0 = lattice_key(e_first + sb + KSTR * kt, msh, msl);
                const bool on_row = to >= 0 && ((p0 >> kRunShift) & (dn - 1)) == rsl;
                if (!on_row) continue;
                const int64_t idx0 = lattice_prefix_sh(p0, dsh, rsl) - rank0;
                if (p0 >= rks && p0 + 3 < rke && (idx0 & 3) == 0 && idx0 + 3 < a.sample_target) {
                    v4i v;
#pragma unroll
                    for (int i = 0; i < 4; ++i) v[i] = (int)ord_of(score_of<DT>(o, kt, i, shv[kt][i]));
                    *reinterpret_cast<v4i *>(srow + idx0) = v;
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int64_t p = p0 + i;
                        if (p < rks || p >= rke || idx0 + i >= a.sample_target) continue;
                        srow[idx0 + i] = ord_of(score_of<DT>(o, kt, i, shv[kt][i]));
                    }
                }
            }
        } else {
            const int slot = PAIR ? s_slot[n] : (t >= 0 ? tile * kTileQ + n : -1);
#pragma unroll
            for (int kt = 0; kt < kSub; ++kt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int s = sb + KSTR * kt + i;
                    if (slot < 0 || s < rks || s >= rke) continue;
                    a.scratch[(int64_t)slot * a.scratch_stride + (s - rks)] = score_of<DT>(o, kt, i, shv[kt][i]);
                }
        }
    };

    // Steps of this wave in filter and dense modes: the wave-th,
    // (wave + kWaves)-th, ... step of the work item (all of [jlo, jhi), or
    // the ones not skipped).
    auto step_of = [&](int i) { return use_skip ? jlo + __builtin_amdgcn_readfirstlane((int)s_steps[i]) : jlo + i; };
    auto nop = []() {};
    if (MODE == kModeSample) {
        // Sample mode claims steps from a workgroup counter, so the waves that
        // evaluated the planner sample first take fewer of them.  Each wave
        // claims a step when it issues its key loads, one step ahead.
        auto claim = [&]() {
            int v = 0;
            if (lane == 0) v = atomicAdd(&s_next, 1);
            return __builtin_amdgcn_readfirstlane(__shfl(v, 0));
        };
        if constexpr (DT == kFP8) {
            KFrag<DT> ka[kSub], kb[kSub];
            int i = claim();
            if (i < nstep) load_step(ka, step_of(i));
            while (i < nstep) {
                const int i2 = claim();
                if (i2 < nstep) load_step(kb, step_of(i2));
                process(ka, step_of(i), nop, std::false_type{});
                if (i2 >= nstep) break;
                const int i3 = claim();
                if (i3 < nstep) load_step(ka, step_of(i3));
                process(kb, step_of(i2), nop, std::false_type{});
                i = i3;
            }
        } else {
            // one fragment set (BF16's 32x32 step needs the registers): the
            // next claimed step's keys load as soon as this step's last MFMA
            // has issued
            KFrag<DT> kf[kSub];
            int i = claim();
            if (i < nstep) load_step(kf, step_of(i));
            while (i < nstep) {
                const int i2 = claim();
                process(
                    kf, step_of(i), [&]() {
                        if (i2 < nstep) load_step(kf, step_of(i2));
                    },
                    std::false_type{});
                i = i2;
            }
        }
    } else {
      // Filter and dense modes: one copy of the step loop per tile variant,
      // so each keeps its own register allocation.
      auto scan = [&](auto mx) {
        if constexpr (Cfg::prefetch) {
            // Two fragment sets alternate so the next step's keys load while
            // this step computes.
            KFrag<DT> ka[kSub], kb[kSub];
            int i = wave;
            if (i < nstep) load_step(ka, step_of(i));
            for (; i < nstep; i += 2 * kWaves) {
                if (i + kWaves < nstep) load_step(kb, step_of(i + kWaves));
                process(ka, step_of(i), nop, mx);
                if (i + kWaves >= nstep) break;
                if (i + 2 * kWaves < nstep) load_step(ka, step_of(i + 2 * kWaves));
                process(kb, step_of(i + kWaves), nop, mx);
            }
        } else {
            // One fragment set: the next step's keys load into it as soon as
            // this step's last MFMA is issued, so the sink hides their
            // latency.  The load is unconditional (the last step re-reads its
            // own keys) so the code after it has one path and the wait for
            // the scale factors never covers these loads.
            KFrag<DT> kf[kSub];
            int i = wave;
            if (i < nstep) load_step(kf, step_of(i));
            for (; i < nstep; i += kWaves) {
                const int in = min(i + kWaves, nstep - 1);
                process(kf, step_of(i), [&]() { load_step(kf, step_of(in)); }, mx);
            }
        }
      };
      if (DT == kFP8 && mixed) scan(std::true_type{});
      else scan(std::false_type{});
    }
    if (MODE == kModeFilter) {
        if (__any(ring_cnt > 0)) ring_flush<RS>(ring, ring_cnt, n, g, to, a.cnt, a.cand, a.cap);
    }
    finish();
    };  // body
    body();
    if (!LOOP) break;
    __syncthreads();  // the next item reuses the LDS
    }
}

}  // namespace ftk
