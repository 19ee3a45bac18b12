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
// of ONE query, so the ReLU, the w[t,h] weighting and the sum over heads all
// stay inside the lane: acc = fma(w[t,h], ReLU(x), acc) for h = 0..31 in
// order, then I = sigma[s] * acc.  The [T, S] score matrix never reaches HBM.
//   FP8:  v_mfma_f32_16x16x128_f8f6f4, one MFMA covers the full d = 128.
//   BF16: v_mfma_f32_16x16x32_bf16, four chained MFMAs cover d = 128.
// Both operands of an MFMA use the same assignment of the 128 dimensions to
// (lane group, byte) slots -- lane group g holds dimensions [32g, 32g+32) --
// so the contraction covers every dimension exactly once.
#pragma once

#include "ftk_common.hpp"

namespace ftk {

constexpr int kModeFilter = 0;
constexpr int kModeSample = 1;
constexpr int kModeDense = 2;

// Candidate ring per (wave, query) in filter mode: survivors are staged in LDS
// and flushed to the row's candidate list with one atomic per query.
template <int DT> struct RingEntries { static constexpr int value = DT == kFP8 ? 88 : 24; };

struct ScoreArgs {
    const uint8_t *q;          // [num_q, 32, 128] codes
    const uint8_t *kv;         // [num_kv, 128] codes
    const float *sigma;        // [num_kv] or null
    const float *w;            // [num_q, 32]
    const int32_t *ks;         // [num_q]
    const int32_t *ke;         // [num_q]
    int64_t num_q;
    int64_t num_kv;
    int ntiles;                // tiles along the grid's fast index
    int cap;                   // candidate capacity per row
    // filter mode
    const float *tau;          // [num_q] per-row threshold (-inf: take all)
    uint32_t *cnt;             // [num_q] candidate counters
    uint64_t *cand;            // [num_q, cap] candidate keys
    // sample mode
    uint32_t *samp;            // [num_q, sample_target] sample score codes
    int sample_target;
    // dense mode
    const int32_t *rowlist;    // flagged rows
    const int32_t *nrows;      // device count of flagged rows
    int row_base;              // first flagged entry of this batch
    int row_limit;             // entries per batch
    uint64_t *scratch;         // [row_limit, scratch_stride] keys
    int64_t scratch_stride;
};

// ---------------------------------------------------------------------------
// Operand fragments.

template <int DT> struct KFrag;
template <> struct KFrag<kFP8> { v8i a; };
template <> struct KFrag<kBF16> { v4i a[4]; };

// Key row p, lane group g: dimensions [32g, 32g+32).
__device__ __forceinline__ void load_kfrag(KFrag<kFP8> &f, const uint8_t *kv, int64_t p, int g)
{
    const v4i *src = reinterpret_cast<const v4i *>(kv + p * 128 + 32 * g);
    v4i lo = src[0];
    v4i hi = src[1];
    f.a = (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

__device__ __forceinline__ void load_kfrag(KFrag<kBF16> &f, const uint8_t *kv, int64_t p, int g)
{
    const v4i *src = reinterpret_cast<const v4i *>(kv + p * 256 + 64 * g);
#pragma unroll
    for (int m = 0; m < 4; ++m) f.a[m] = src[m];
}

// LDS layout of the q tile: for head h, the 64 lanes' fragments are stored as
// consecutive 16-byte slots, slot (h, sub, lane) at ((h*SUB + sub)*64 + lane)*16
// where lane = n + 16 g (query n, lane group g) and sub indexes the 16-byte
// pieces of the lane's 32 (FP8) or 64 (BF16) bytes.  Each ds_read_b128 of a
// head reads 1 KiB of consecutive LDS, free of bank conflicts.
template <int DT>
__device__ __forceinline__ void stage_q_tile(uint8_t *s_q, const uint8_t *q, const int *s_row)
{
    constexpr int RB = RowBytes<DT>::value;
    constexpr int CPR = RB / 16;    // 16-byte pieces per head row
    constexpr int SUB = CPR / 4;    // pieces per lane group
    constexpr int NCH = kTileQ * kHeads * CPR;
    for (int id = threadIdx.x; id < NCH; id += kThreads) {
        int n = id / (kHeads * CPR);
        int h = (id / CPR) % kHeads;
        int c = id % CPR;
        int t = s_row[n];
        v4i v = {0, 0, 0, 0};
        if (t >= 0) v = *reinterpret_cast<const v4i *>(q + ((int64_t)t * kHeads + h) * RB + c * 16);
        int sub = c % SUB, g = c / SUB;
        *reinterpret_cast<v4i *>(s_q + ((h * SUB + sub) * 64 + n + 16 * g) * 16) = v;
    }
}

// Scores of kSub subtiles x 4 keys for the lane's query, accumulated over all
// heads.  kf: the lane's key fragments; s_w: the tile's weights in LDS,
// s_w[h * 16 + n] = w[row n, h].
//
// Software pipeline over heads: the MFMAs of head h are issued while the VALU
// epilogue (ReLU, weight, sum) of head h-1 runs, so the matrix cores and the
// vector ALUs work at the same time; the q fragment and weight of head h+1 are
// read from LDS one head ahead.  The head loop is kept rolled so each head is
// its own scheduling region: the compiler cannot hoist every head's operands
// (or sink every epilogue), which would need far more than 256 registers.
__device__ __forceinline__ void head_epilogue(float (&acc)[kSub][4], const v4f (&x)[kSub], float w)
{
#pragma unroll
    for (int kt = 0; kt < kSub; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[kt][i] = __builtin_fmaf(w, relu_bits(x[kt][i]), acc[kt][i]);
}

// qp points at the lane's slot of head 0 (s_q + lane * 16); head h adds h * 2 KiB.
__device__ __forceinline__ void mfma_fp8_heads(v4f (&x)[kSub], const KFrag<kFP8> (&kf)[kSub], const uint8_t *qp)
{
    const v4f z = {0.0f, 0.0f, 0.0f, 0.0f};
    const v4i lo = *reinterpret_cast<const v4i *>(qp);
    const v4i hi = *reinterpret_cast<const v4i *>(qp + 1024);
    const v8i qf = (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
    for (int kt = 0; kt < kSub; ++kt)
        x[kt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(kf[kt].a, qf, z, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ void score_step(float (&acc)[kSub][4], const KFrag<kFP8> (&kf)[kSub],
                                           const uint8_t *s_q, const float *s_w, int lane)
{
    constexpr int HB = 2048;  // LDS bytes per head of the q tile
#pragma unroll
    for (int kt = 0; kt < kSub; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[kt][i] = 0.0f;
    const uint8_t *qp = s_q + lane * 16;
    const float *wp = s_w + (lane & 15);
    // Two result sets alternate so no copies are needed between heads.
    v4f xa[kSub], xb[kSub];
    mfma_fp8_heads(xa, kf, qp);
#pragma unroll 1
    for (int h = 1; h < kHeads - 1; h += 2) {
        const float w0 = wp[0], w1 = wp[kTileQ];
        mfma_fp8_heads(xb, kf, qp + HB);
        head_epilogue(acc, xa, w0);
        mfma_fp8_heads(xa, kf, qp + 2 * HB);
        head_epilogue(acc, xb, w1);
        qp += 2 * HB;
        wp += 2 * kTileQ;
    }
    mfma_fp8_heads(xb, kf, qp + HB);
    head_epilogue(acc, xa, wp[0]);
    head_epilogue(acc, xb, wp[kTileQ]);
}

__device__ __forceinline__ v4f mfma_bf16_d128(const KFrag<kBF16> &k, const v4i (&qf)[4])
{
    v4f x = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int m = 0; m < 4; ++m)
        x = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, k.a[m]), __builtin_bit_cast(v8bf, qf[m]),
                                                    x, 0, 0, 0);
    return x;
}

// qp points at the lane's slot of head 0 (s_q + lane * 16); head h adds h * 4 KiB.
__device__ __forceinline__ void mfma_bf16_heads(v4f (&x)[kSub], const KFrag<kBF16> (&kf)[kSub], const uint8_t *qp)
{
    v4i qf[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) qf[m] = *reinterpret_cast<const v4i *>(qp + m * 1024);
#pragma unroll
    for (int kt = 0; kt < kSub; ++kt) x[kt] = mfma_bf16_d128(kf[kt], qf);
}

__device__ __forceinline__ void score_step(float (&acc)[kSub][4], const KFrag<kBF16> (&kf)[kSub],
                                           const uint8_t *s_q, const float *s_w, int lane)
{
    constexpr int HB = 4096;
#pragma unroll
    for (int kt = 0; kt < kSub; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[kt][i] = 0.0f;
    const uint8_t *qp = s_q + lane * 16;
    const float *wp = s_w + (lane & 15);
    v4f xa[kSub], xb[kSub];
    mfma_bf16_heads(xa, kf, qp);
#pragma unroll 1
    for (int h = 1; h < kHeads - 1; h += 2) {
        const float w0 = wp[0], w1 = wp[kTileQ];
        mfma_bf16_heads(xb, kf, qp + HB);
        head_epilogue(acc, xa, w0);
        mfma_bf16_heads(xa, kf, qp + 2 * HB);
        head_epilogue(acc, xb, w1);
        qp += 2 * HB;
        wp += 2 * kTileQ;
    }
    mfma_bf16_heads(xb, kf, qp + HB);
    head_epilogue(acc, xa, wp[0]);
    head_epilogue(acc, xb, wp[kTileQ]);
}

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
template <int RING>
__device__ __forceinline__ void ring_flush(const uint64_t *ring, uint32_t ring_cnt, int n, int g, int t,
                                           uint32_t *cnt, uint64_t *cand, int cap)
{
    wave_lds_sync();
    uint32_t base = 0;
    if (g == 0 && ring_cnt > 0 && t >= 0) base = atomicAdd(cnt + t, ring_cnt);
    base = __shfl(base, n);
    if (t >= 0) {
        for (uint32_t k = g; k < ring_cnt; k += 4) {
            uint64_t v = ring[n * RING + k];
            if (base + k < (uint32_t)cap) cand[(int64_t)t * cap + base + k] = v;
        }
    }
    wave_lds_sync();
}

// ---------------------------------------------------------------------------

template <int DT, int MODE>
__global__ __launch_bounds__(kThreads) void k_score(ScoreArgs a)
{
    constexpr int RB = RowBytes<DT>::value;
    constexpr int RING = (MODE == kModeFilter) ? RingEntries<DT>::value : 1;
    // One LDS block carved by hand so the q tile sits at offset 0 and every
    // q-fragment read fits the 16-bit immediate offset of ds_read.
    constexpr int QB = kTileQ * kHeads * RB;
    constexpr int WB = kHeads * kTileQ * 4;
    constexpr int RGB = (MODE == kModeFilter) ? kWaves * kTileQ * RING * 8 : 0;
    __shared__ __attribute__((aligned(16))) uint8_t smem[QB + WB + RGB];
    __shared__ int s_row[kTileQ], s_ks[kTileQ], s_ke[kTileQ], s_d[kTileQ];
    uint8_t *s_q = smem;
    float *s_w = reinterpret_cast<float *>(smem + QB);
    uint64_t *s_ring = reinterpret_cast<uint64_t *>(smem + QB + WB);

    int tile, chunk;
    if (MODE == kModeSample) {
        tile = blockIdx.x;
        chunk = 0;
    } else {
        chunk = blockIdx.x / a.ntiles;
        tile = blockIdx.x - chunk * a.ntiles;
    }

    if (threadIdx.x < kTileQ) {
        int n = threadIdx.x, t = -1;
        if (MODE == kModeDense) {
            int e = tile * kTileQ + n;
            if (e < a.row_limit && a.row_base + e < *a.nrows) t = a.rowlist[a.row_base + e];
        } else {
            int64_t tt = (int64_t)tile * kTileQ + n;
            if (tt < a.num_q) t = (int)tt;
        }
        int lo = 0, hi = 0, d = 1;
        if (t >= 0) {
            lo = a.ks[t];
            hi = a.ke[t];
            if (hi < lo) hi = lo;
        }
        if (MODE == kModeSample) {
            if (t >= 0 && hi - lo > a.cap) {
                d = sample_stride(hi - lo, a.sample_target);
            } else {
                t = -1;
                lo = hi = 0;
            }
        }
        s_row[n] = t;
        s_ks[n] = lo;
        s_ke[n] = hi;
        s_d[n] = d;
    }
    __syncthreads();

    // Union of the tile's windows; the lattice stride of the tile's samples.
    int lo = 0x7fffffff, hi = 0, dmin = 0x40000000;
#pragma unroll
    for (int n = 0; n < kTileQ; ++n) {
        if (s_row[n] >= 0 && s_ke[n] > s_ks[n]) {
            lo = min(lo, s_ks[n]);
            hi = max(hi, s_ke[n]);
            dmin = min(dmin, s_d[n]);
        }
    }
    if (hi <= lo) return;

    // Keys of this work item, in 64-key steps [jlo, jhi).  In sample mode the
    // steps index the lattice first_b + e * dmin, e < nlat.
    int64_t jlo, jhi, first_b = 0, nlat = 0;
    if (MODE == kModeSample) {
        first_b = ((int64_t)lo + dmin - 1) / dmin * dmin;
        nlat = lattice_count(lo, hi, dmin);
        jlo = 0;
        jhi = (nlat + kStepKeys - 1) / kStepKeys;
    } else {
        int64_t c0 = (int64_t)chunk * kChunkKeys;
        int64_t klo = max((int64_t)lo, c0), khi = min((int64_t)hi, c0 + kChunkKeys);
        if (khi <= klo) return;
        jlo = klo / kStepKeys;
        jhi = (khi + kStepKeys - 1) / kStepKeys;
    }

    stage_q_tile<DT>(s_q, a.q, s_row);
    for (int i = threadIdx.x; i < kHeads * kTileQ; i += kThreads) {
        const int rn = i & (kTileQ - 1), h = i / kTileQ;
        const int rt = s_row[rn];
        s_w[i] = rt >= 0 ? a.w[(int64_t)rt * kHeads + h] : 0.0f;
    }
    __syncthreads();

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n = lane & 15, g = lane >> 4;
    const int t = s_row[n];
    const int rks = s_ks[n], rke = s_ke[n];

    float tau = __builtin_inff();
    if (MODE == kModeFilter && t >= 0) tau = a.tau[t];
    int dn = s_d[n];
    int64_t first_n = ((int64_t)rks + dn - 1) / dn * dn;
    uint64_t *ring = s_ring + (MODE == kModeFilter ? wave * kTileQ * RING : 0);
    uint32_t ring_cnt = 0;
    const int64_t S = a.num_kv;

    // Key fragments of step j: this lane loads key row 16 kt + n of the step.
    auto load_step = [&](KFrag<DT>(&f)[kSub], int64_t j) {
#pragma unroll
        for (int kt = 0; kt < kSub; ++kt) {
            int64_t e = j * kStepKeys + 16 * kt + n;
            int64_t p = (MODE == kModeSample) ? first_b + e * dmin : e;
            p = min(p, S - 1);
            load_kfrag(f[kt], a.kv, p, g);
        }
    };
    KFrag<DT> kf[kSub];
    if (jlo + wave < jhi) load_step(kf, jlo + wave);
    for (int64_t j = jlo + wave; j < jhi; j += kWaves) {
        KFrag<DT> kn[kSub];
        if (j + kWaves < jhi) load_step(kn, j + kWaves);  // prefetch the wave's next step
        float acc[kSub][4];
        score_step(acc, kf, s_q, s_w, lane);

        // Output element (kt, i) of this lane: key row 16 kt + 4 g + i, query n.
        if (MODE == kModeFilter) {
            // Keep (row, key) when the key is in the row's window and its
            // score reaches the row's threshold (take-all rows: -inf).
            uint32_t mask = 0;
            float sc[kSub * 4];
#pragma unroll
            for (int kt = 0; kt < kSub; ++kt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    int64_t s = j * kStepKeys + 16 * kt + 4 * g + i;
                    float sg = a.sigma ? a.sigma[min(s, S - 1)] : 1.0f;
                    float I = sg * acc[kt][i];
                    sc[kt * 4 + i] = I;
                    bool ok = (s >= rks) && (s < rke) && (I >= tau);
                    mask |= (uint32_t)ok << (kt * 4 + i);
                }
            const int64_t sbase = j * kStepKeys + 4 * g;
            // Survivors of the 4 lanes that hold query n: total and this lane's offset.
            uint32_t m = __builtin_popcount(mask);
            uint32_t c0 = __shfl(m, n), c1 = __shfl(m, n + 16), c2 = __shfl(m, n + 32), c3 = __shfl(m, n + 48);
            uint32_t tot = c0 + c1 + c2 + c3;
            uint32_t pre = (g > 0 ? c0 : 0) + (g > 1 ? c1 : 0) + (g > 2 ? c2 : 0);
            if (__any(ring_cnt + tot > (uint32_t)RING)) {
                ring_flush<RING>(ring, ring_cnt, n, g, t, a.cnt, a.cand, a.cap);
                ring_cnt = 0;
            }
            if (__any(tot > (uint32_t)RING)) {
                // More than a ring holds: reserve slots in the row's list directly.
                uint32_t base = 0;
                bool direct = tot > (uint32_t)RING;
                if (direct && g == 0 && t >= 0) base = atomicAdd(a.cnt + t, tot);
                base = __shfl(base, n);
                uint32_t pos = base + pre;
                if (direct && t >= 0) {
#pragma unroll
                    for (int b = 0; b < kSub * 4; ++b) {
                        if (mask & (1u << b)) {
                            int64_t s = sbase + 16 * (b >> 2) + (b & 3);
                            if (pos < (uint32_t)a.cap) a.cand[(int64_t)t * a.cap + pos] = sel_key(sc[b], (int32_t)s);
                            ++pos;
                        }
                    }
                    mask = 0;
                    tot = 0;
                }
            }
            uint32_t pos = ring_cnt + pre;
#pragma unroll
            for (int b = 0; b < kSub * 4; ++b) {
                if (mask & (1u << b)) {
                    int64_t s = sbase + 16 * (b >> 2) + (b & 3);
                    ring[n * RING + pos] = sel_key(sc[b], (int32_t)s);
                    ++pos;
                }
            }
            ring_cnt += tot;
        } else if (MODE == kModeSample) {
#pragma unroll
            for (int kt = 0; kt < kSub; ++kt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    int64_t e = j * kStepKeys + 16 * kt + 4 * g + i;
                    if (t < 0 || e >= nlat) continue;
                    int64_t p = first_b + e * dmin;
                    if (p < rks || p >= rke || (p & (dn - 1)) != 0) continue;
                    float sg = a.sigma ? a.sigma[p] : 1.0f;
                    float I = sg * acc[kt][i];
                    int64_t idx = (p - first_n) / dn;
                    a.samp[(int64_t)t * a.sample_target + idx] = ord_of(I);
                }
        } else {
            const int slot = tile * kTileQ + n;
#pragma unroll
            for (int kt = 0; kt < kSub; ++kt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    int64_t s = j * kStepKeys + 16 * kt + 4 * g + i;
                    if (t < 0 || s < rks || s >= rke) continue;
                    float sg = a.sigma ? a.sigma[s] : 1.0f;
                    float I = sg * acc[kt][i];
                    a.scratch[(int64_t)slot * a.scratch_stride + (s - rks)] = sel_key(I, (int32_t)s);
                }
        }
#pragma unroll
        for (int kt = 0; kt < kSub; ++kt) kf[kt] = kn[kt];
    }
    if (MODE == kModeFilter) {
        if (__any(ring_cnt > 0)) ring_flush<RING>(ring, ring_cnt, n, g, t, a.cnt, a.cand, a.cap);
    }
}

}  // namespace ftk
