// Indexer scoring for calls with at most kFewRows query rows (decode, a few
// speculative tokens): the same three modes as k_score (sample, filter,
// dense), with the 32 heads on the MFMA's M dimension instead of 16 query
// rows.
//
// The score (FlashTopK README, "Quick start", indexer-score equation)
//     I[t,s] = sigma[s] * sum_{h<32} w[t,h] * ReLU(q[t,h,:] . kv[s,:])
// With one to four rows, a 16-row query tile would leave most MFMA columns
// empty and give each workgroup little work for its q-tile staging.  Here an
// MFMA takes A = 16 heads of one row (M) and B = 16 keys (N): two MFMAs give
// all 32 heads' dot products of 16 keys, each lane holding 4 heads x 1 key.
// ReLU and the w weighting happen in the lane, the head sum is finished by
// two cross-lane additions (lanes n, n+16, n+32, n+48 share key n), and sigma
// scales the sum.  The work is bound by reading the keys once (128 B per key
// FP8, 256 B BF16); the matrix cores and vector ALUs have room to spare.
//
// Keys may sit in a paged cache (a.table non-null: logical key p is row
// p % page_size of page table[p / page_size]); each lane then reads its key
// from its page, so such calls need no gathered copy of the keys.
//
// Every mode of a call with at most kFewRows rows uses this arithmetic, so a
// row's scores have the same bits on every path of such a call (the sums run
// in another order than k_score's, so a row's last bits may differ between a
// call with few rows and one with many).
#pragma once

#include "ftk_common.hpp"
#include "ftk_frag.hpp"
#include "ftk_score.hpp"
#include "ftk_tau.hpp"

namespace ftk {

constexpr int kFewRows = 4;
constexpr int kFewWaves = 4;
constexpr int kFewThreads = 64 * kFewWaves;

// 16-key groups per wave step (key fragments of a step stay in registers).
template <int DT> struct FewGroups { static constexpr int value = DT == kFP8 ? 4 : 2; };
// Keys per workgroup in filter and dense modes: a multiple of every wave's
// step, kFewWaves * 16 * groups.
constexpr int kFewChunk = 256;
// Sample mode: lattice entries per workgroup.
constexpr int kFewSamplePart = 256;

// Scores of 16 keys (the lanes' B fragment) for one row whose A fragments
// (heads 0-15, 16-31) are a0, a1; w4 holds the lane's 8 weights (heads
// 4g + i and 16 + 4g + i, g = lane / 16).  Returns the head sum of key
// lane % 16 in every lane.
__device__ __forceinline__ float few_sum(const KFrag<kFP8> &kf, const KFrag<kFP8> &a0, const KFrag<kFP8> &a1,
                                         const float (&w8)[8])
{
    const v4f z = {0.0f, 0.0f, 0.0f, 0.0f};
    const v4f x0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a0.a, kf.a, z, 0, 0, 0, 0, 0, 0);
    const v4f x1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a1.a, kf.a, z, 0, 0, 0, 0, 0, 0);
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) s = __builtin_fmaf(w8[i], relu_bits(x0[i]), s);
#pragma unroll
    for (int i = 0; i < 4; ++i) s = __builtin_fmaf(w8[4 + i], relu_bits(x1[i]), s);
    s += __shfl_xor(s, 16);
    s += __shfl_xor(s, 32);
    return s;
}

__device__ __forceinline__ float few_sum(const KFrag<kBF16> &kf, const KFrag<kBF16> &a0, const KFrag<kBF16> &a1,
                                         const float (&w8)[8])
{
    v4f x0 = {0.0f, 0.0f, 0.0f, 0.0f}, x1 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        x0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a0.a[m]), __builtin_bit_cast(v8bf, kf.a[m]),
                                                     x0, 0, 0, 0);
        x1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a1.a[m]), __builtin_bit_cast(v8bf, kf.a[m]),
                                                     x1, 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) s = __builtin_fmaf(w8[i], relu_bits(x0[i]), s);
#pragma unroll
    for (int i = 0; i < 4; ++i) s = __builtin_fmaf(w8[4 + i], relu_bits(x1[i]), s);
    s += __shfl_xor(s, 16);
    s += __shfl_xor(s, 32);
    return s;
}

// Resource over keys [p0, p1) (at most kFewChunk of them, so every lane
// offset is small); reads past them return zeros.
template <int DT>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t few_key_rsrc(const uint8_t *kv, int64_t p0, int64_t p1)
{
    constexpr int RB = RowBytes<DT>::value;
    return make_rsrc(kv + p0 * RB, (uint32_t)(max(p1 - p0, (int64_t)0) * RB));
}

template <int DT, int MODE>
__global__ __launch_bounds__(kFewThreads) void k_score_few(ScoreArgs a)
{
    constexpr int RB = RowBytes<DT>::value, G = FewGroups<DT>::value;
    // A fragments of every row in LDS: [row][half][lane] slices of RB / 4 bytes.
    __shared__ __attribute__((aligned(16))) uint8_t s_a[kFewRows * 2 * 64 * (RB / 4)];
    __shared__ float s_w[kFewRows * kHeads];
    __shared__ uint64_t s_out[MODE == kModeFilter ? kFewRows * kFewChunk : 1];
    __shared__ uint32_t s_n[kFewRows], s_base[kFewRows];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, n = lane & 15;

    // Rows of this workgroup and the keys it scores.
    int r0 = 0, r1 = 0;         // rows [r0, r1) (indices into the call's rows)
    int64_t klo = 0, khi = 0;   // filter / dense: key range; sample: lattice entries
    int t_dense = -1, e_dense = 0;
    int64_t first = 0, d = 1;   // sample lattice
    int64_t nlat = 0;
    if (MODE == kModeSample) {
        // Workgroup 0 clears the call's statistics; a row that takes its
        // whole window gets threshold -inf; a sampled row's threshold comes
        // from its last workgroup (below).
        if (blockIdx.x == 0 && tid < a.nstats) a.stats[tid] = 0ull;
        const int parts = (a.sample_target + kFewSamplePart - 1) / kFewSamplePart;
        const int t = blockIdx.x / parts, part = blockIdx.x - t * parts;
        if (t >= a.num_q) return;
        const int64_t lo = a.ks[t], hi = max((int64_t)a.ke[t], lo);
        if (hi - lo <= a.cap) {
            if (part == 0 && tid == 0) {
                a.tau_w[t] = -__builtin_inff();
                a.cnt[t] = 0u;
            }
            return;
        }
        d = sample_stride(hi - lo, a.sample_target, a.sample_min_stride);
        first = (lo + d - 1) / d * d;
        nlat = lattice_count(lo, hi, (int)d);
        klo = (int64_t)part * kFewSamplePart;
        khi = max(klo, min(nlat, klo + kFewSamplePart));  // may be empty: the workgroup still counts
        r0 = t;
        r1 = t + 1;
    } else if (MODE == kModeDense) {
        const int nch = (int)((a.num_kv + kFewChunk - 1) / kFewChunk);
        e_dense = blockIdx.x / max(nch, 1);
        const int ch = blockIdx.x - e_dense * max(nch, 1);
        if (e_dense >= a.row_limit || (unsigned long long)(a.row_base + e_dense) >= *a.nrows) return;
        t_dense = a.rowlist[a.row_base + e_dense];
        const int64_t lo = a.ks[t_dense], hi = max((int64_t)a.ke[t_dense], lo);
        klo = max(lo, (int64_t)ch * kFewChunk);
        khi = min(hi, (int64_t)ch * kFewChunk + kFewChunk);
        if (khi <= klo) return;
        r0 = t_dense;
        r1 = t_dense + 1;
    } else {
        klo = (int64_t)blockIdx.x * kFewChunk;
        khi = min((int64_t)a.num_kv, klo + kFewChunk);
        r0 = 0;
        r1 = a.num_q;
        if (khi <= klo) return;
    }
    const int nr = r1 - r0;

    // Stage the rows' A fragments and weights.
    for (int i = tid; i < nr * 2 * 64; i += kFewThreads) {
        const int rr = i >> 7, half = (i >> 6) & 1, ln = i & 63;
        const uint8_t *src = a.q + ((int64_t)(r0 + rr) * kHeads + half * 16 + (ln & 15)) * RB + (ln >> 4) * (RB / 4);
        uint8_t *dst = s_a + ((rr * 2 + half) * 64 + ln) * (RB / 4);
#pragma unroll
        for (int c = 0; c < RB / 64; ++c)
            reinterpret_cast<v4i *>(dst)[c] = reinterpret_cast<const v4i *>(src)[c];
    }
    for (int i = tid; i < nr * kHeads; i += kFewThreads) s_w[i] = a.w[(int64_t)r0 * kHeads + i];
    if (MODE == kModeFilter && tid < kFewRows) s_n[tid] = 0u;
    __syncthreads();

    auto load_a = [&](KFrag<DT> &f, int rr, int half) {
        const uint8_t *p = s_a + ((rr * 2 + half) * 64 + lane) * (RB / 4);
        if constexpr (DT == kFP8) {
            const v4i lo = reinterpret_cast<const v4i *>(p)[0], hi = reinterpret_cast<const v4i *>(p)[1];
            f.a = (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        } else {
#pragma unroll
            for (int m = 0; m < 4; ++m) f.a[m] = reinterpret_cast<const v4i *>(p)[m];
        }
    };
    auto weights = [&](float (&w8)[8], int rr) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            w8[i] = s_w[rr * kHeads + 4 * g + i];
            w8[4 + i] = s_w[rr * kHeads + 16 + 4 * g + i];
        }
    };

    // Wave steps: G groups of 16 keys (lattice entries in sample mode).
    constexpr int STEP = 16 * G;
    const int64_t nsteps = (khi - klo + STEP - 1) / STEP;
    // filter / dense: keys [klo, khi) through a buffer resource (keys past it
    // read as zeros and are dropped); sample: lattice keys by plain loads,
    // entries past the lattice reread its first key.
    const __amdgpu_buffer_rsrc_t rs = few_key_rsrc<DT>(a.kv, klo, min(khi, (int64_t)a.num_kv));
    for (int64_t st = wave; st < nsteps; st += kFewWaves) {
        const int64_t e0 = klo + st * STEP;  // first key (or lattice entry) of the step
        KFrag<DT> kf[G];
        float sig[G];
#pragma unroll
        for (int gi = 0; gi < G; ++gi) {
            const int64_t e = e0 + 16 * gi + n;
            const bool in = e < khi;
            const int64_t p = MODE == kModeSample ? first + (in ? e : 0) * d : e;
            if (a.table) {
                // paged keys: the lane reads its key's row from its page
                // (a page id out of range reads the pool's first row with
                // scale 0); p is in range here, so the table read is too
                const int64_t pq = in ? p : (MODE == kModeSample ? first : klo);
                const int64_t pg = a.table[pq / a.page_size];
                const bool ok = pg >= 0 && pg < a.num_pages;
                const int64_t slot = ok ? pg * a.page_size + pq % a.page_size : 0;
                load_kfrag(kf[gi], a.kv + slot * RB, 0, g);
                sig[gi] = !ok ? 0.0f : (a.sigma ? a.sigma[slot] : 1.0f);
            } else {
                if (MODE == kModeSample)
                    load_kfrag(kf[gi], a.kv, (int)p, g);
                else
                    load_kfrag_buf(kf[gi], rs, in ? (uint32_t)((e - klo) * RB + g * (RB / 4)) : 0xFFFFFFF0u, 0u);
                sig[gi] = (in && a.sigma) ? a.sigma[p] : 1.0f;
            }
        }
        for (int rr = 0; rr < nr; ++rr) {
            const int t = r0 + rr;
            KFrag<DT> a0, a1;
            load_a(a0, rr, 0);
            load_a(a1, rr, 1);
            float w8[8];
            weights(w8, rr);
            const int64_t lo = a.ks[t], hi = max((int64_t)a.ke[t], lo);
            const float tau = MODE == kModeFilter ? a.tau[t] : 0.0f;
#pragma unroll
            for (int gi = 0; gi < G; ++gi) {
                const float sc = few_sum(kf[gi], a0, a1, w8) * sig[gi];
                const int64_t e = e0 + 16 * gi + n;
                if (MODE == kModeSample) {
                    if (g == 0 && e < khi) a.samp[(int64_t)t * a.sample_target + e] = ord_of(sc);
                } else if (MODE == kModeDense) {
                    if (g == 0 && e < khi)
                        a.scratch[(int64_t)e_dense * a.scratch_stride + (e - lo)] = sc;
                } else {
                    const bool keep = g == 0 && e < khi && e >= lo && e < hi && sc >= tau;
                    const uint64_t bal = __ballot(keep);
                    if (bal) {
                        uint32_t base = 0;
                        if (lane == 0) base = atomicAdd(&s_n[rr], (uint32_t)__builtin_popcountll(bal));
                        base = __shfl(base, 0);
                        if (keep)
                            s_out[rr * kFewChunk + base + __builtin_popcountll(bal & ((1ull << lane) - 1ull))] =
                                raw_cand(sc, (int32_t)e);
                    }
                }
            }
        }
    }
    if (MODE == kModeSample) {
        // The row's last workgroup to finish (a self-resetting counter)
        // computes its threshold from all of its samples.
        __shared__ uint32_t s_hist[kTauBuckets];
        __shared__ uint32_t s_red[3 * kFewWaves + 1];
        __shared__ int s_last;
        const int t = r0;
        const int parts = (a.sample_target + kFewSamplePart - 1) / kFewSamplePart;
        __threadfence();
        __syncthreads();
        if (tid == 0) s_last = atomicInc(&a.ticket[t], (unsigned)(parts - 1)) == (unsigned)(parts - 1);
        __syncthreads();
        if (!s_last) return;
        __threadfence();
        const int64_t lo = a.ks[t], hi = max((int64_t)a.ke[t], lo);
        const float tv = block_tau<kFewThreads>(a.samp + (int64_t)t * a.sample_target, (int)nlat,
                                                tau_rank(a.topk, nlat, hi - lo, a.rank_scale), s_hist, s_red);
        if (tid == 0) {
            a.tau_w[t] = tv;
            a.cnt[t] = 0u;
        }
    }
    if (MODE == kModeFilter) {
        // One global atomic per row reserves the workgroup's survivors.
        __syncthreads();
        if (tid < nr && s_n[tid]) s_base[tid] = atomicAdd(&a.cnt[r0 + tid], s_n[tid]);
        __syncthreads();
        for (int rr = 0; rr < nr; ++rr) {
            const uint32_t cnt = s_n[rr], base = s_base[rr];
            for (uint32_t i = tid; i < cnt; i += kFewThreads)
                if (base + i < (uint32_t)a.cap) a.cand[(int64_t)(r0 + rr) * a.cap + base + i] = s_out[rr * kFewChunk + i];
        }
    }
}

}  // namespace ftk
