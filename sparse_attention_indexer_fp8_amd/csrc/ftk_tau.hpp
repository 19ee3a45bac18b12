// Per-row threshold from the row's strided sample (FlashTopK README,
// "Highlights": the threshold comes from a strided sample of the row's own
// window).
//
// The threshold is the r-th largest sample score, r = ceil(2 * topk * n / L)
// for n samples of an L-key window, so about 2 topk keys of the window are
// expected to reach it.  The sample is bucketed linearly in score
// (kTauBuckets buckets between its minimum and maximum, highest first); the
// bucket that holds the r-th largest sample is found from the histogram, and
// when it holds at most 64 samples (the usual case) the r-th largest is
// picked from them exactly.  A denser bucket gives the threshold one bucket
// below its lower edge instead: at least r samples reach it, whatever the
// rounding of the bucket arithmetic.  When every lane holds a sample and
// r <= 64, the smallest of the 64 lanes' largest samples is a floor: at
// least 64 samples reach it, so the r-th largest does too, and only the
// samples at or above it are bucketed (between it and the maximum), which
// leaves most samples out of the histogram and spreads the top of the row
// over all buckets.  No threshold changes results -- triage catches any row
// it misjudges -- only the candidate count.
#pragma once

#include "ftk_common.hpp"

namespace ftk {

constexpr int kTauBuckets = 2048;
constexpr int kTauExactMax = 64;  // largest bucket searched for the exact r-th sample

// The r-th largest of the wave's samples, given the bucket b that holds it:
// v holds the lane's PER samples (NaN: absent), `above` the samples of the
// buckets before b and cb those of b (cb <= kTauExactMax), with the same
// bucket arithmetic (lo, vmax, scale) as the histogram.  buf: kTauExactMax words
// of LDS private to the wave.  Every lane returns the value.
template <int PER>
__device__ __forceinline__ float tau_exact_in_bucket(const float (&v)[PER], float lo, float vmax, float scale,
                                                     int b, uint32_t above, uint32_t cb, uint32_t r, uint32_t *buf,
                                                     int lane)
{
    auto in_b = [&](float x) {
        if (!(x >= lo)) return false;  // below the bucketed range (or NaN: absent)
        const float y = (vmax - x) * scale;
        const int bb = y < (float)(kTauBuckets - 1) ? (int)(uint32_t)y : kTauBuckets - 1;
        return bb == b;
    };
    // the bucket's samples, compacted into buf
    uint32_t mine = 0;
#pragma unroll
    for (int q = 0; q < PER; ++q) mine += in_b(v[q]) ? 1u : 0u;
    uint32_t pos = wave_incl_add(mine) - mine;
#pragma unroll
    for (int q = 0; q < PER; ++q)
        if (in_b(v[q])) buf[pos++] = __float_as_uint(v[q]);
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
    // lane j < cb: the rank of its sample among the bucket's (larger values
    // first, equal ones by position); the one of rank r - above - 1 wins.
    // Lane i's sample reaches the others through readlane (no LDS round
    // trip per comparison).
    const uint32_t want = r - above - 1;
    const bool mine_ok = (uint32_t)lane < cb;
    const uint32_t eb = mine_ok ? buf[lane] : 0u;
    const float e = __uint_as_float(eb);
    uint32_t rank = 0;
    for (uint32_t i = 0; i < cb; ++i) {
        const float f = __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)eb, (int)i));
        rank += (f > e || (f == e && i < (uint32_t)lane)) ? 1u : 0u;
    }
    if (!mine_ok) rank = 0xFFFFFFFFu;
    const uint64_t hit = __ballot(rank == want);
    const float t = __shfl(e, hit ? __builtin_ctzll(hit) : 0);
    __builtin_amdgcn_wave_barrier();  // every lane has read buf before the caller reuses the LDS
    return t;
}

// Rank of the threshold in a sample of n keys of an L-key window.
__device__ __forceinline__ uint32_t tau_rank(int topk, int64_t n, int64_t len, float rank_scale)
{
    const double want = ceil(2.0 * (double)topk * (double)n / (double)len * (double)rank_scale);
    return (uint32_t)min(max(want, 1.0), (double)n);
}

// One wave computes the threshold of one row from its n >= 1 sample codes
// (ord_of of the scores); hist is kTauBuckets words of LDS private to the
// wave.  Every lane returns the threshold.  Samples are read 2048 at a time
// (32 per lane, all loads in flight together); a row of at most 2048 samples
// is read once and kept in registers for both passes.
__device__ __forceinline__ float wave_tau(const uint32_t *samp, int n, uint32_t r, uint32_t *hist, int lane)
{
    constexpr int PER = kTauBuckets / 64;
    constexpr int PERL = 32;             // samples per lane per chunk
    constexpr int CHUNK = 64 * PERL;
    float v[PERL];
    // Loads are unconditional (index clamped, n >= 1) so all of a chunk's
    // loads are in flight before the first wait.
    auto load_chunk = [&](int base) {
        uint32_t u[PERL];
#pragma unroll
        for (int q = 0; q < PERL; ++q) u[q] = samp[min(base + lane + 64 * q, n - 1)];
#pragma unroll
        for (int q = 0; q < PERL; ++q) v[q] = base + lane + 64 * q < n ? float_of_ord(u[q]) : __builtin_nanf("");
    };
    float vmin = __builtin_inff(), vmax = -__builtin_inff();
    for (int base = 0; base < n; base += CHUNK) {
        load_chunk(base);
#pragma unroll
        for (int q = 0; q < PERL; ++q) {  // fminf / fmaxf ignore the NaN fill
            vmin = fminf(vmin, v[q]);
            vmax = fmaxf(vmax, v[q]);
        }
    }
    // wave extremes through DPP on the order codes (lanes with no sample hold +-inf)
    const float lmin = float_of_ord(~wave_max(~ord_of(vmax)));  // smallest lane maximum
    vmax = float_of_ord(wave_max(ord_of(vmax)));
    vmin = float_of_ord(~wave_max(~ord_of(vmin)));
    const float lo = (n >= 64 && r <= 64u) ? lmin : vmin;  // floor of the bucketed range
    const float scale = (float)kTauBuckets / (vmax - lo);
    if (!(vmax > lo) || !__builtin_isfinite(scale)) return lo;  // samples at the floor equal: admit them all
#pragma unroll
    for (int q = 0; q < PER; ++q) hist[lane + 64 * q] = 0u;
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the zeros land before any lane adds
    __builtin_amdgcn_wave_barrier();
    for (int base = 0; base < n; base += CHUNK) {
        if (n > CHUNK) load_chunk(base);  // a single chunk is still in registers
#pragma unroll
        for (int q = 0; q < PERL; ++q) {
            if (v[q] >= lo) {  // NaN fill fails
                const float x = (vmax - v[q]) * scale;
                atomicAdd(&hist[x < (float)(kTauBuckets - 1) ? (uint32_t)x : (uint32_t)(kTauBuckets - 1)], 1u);
            }
        }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
    // Lane l owns buckets [PER l, PER l + PER); exclusive prefix over lanes.
    // The counts are read twice from LDS rather than held in registers (more
    // waves fit per SIMD).
    uint32_t run = 0;
#pragma unroll
    for (int q = 0; q < PER; ++q) run += hist[lane * PER + q];
    uint32_t base = wave_incl_add(run) - run;
    int b = -1;
    uint32_t above = 0, cb = 0;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
        const uint32_t cq = hist[lane * PER + q];
        if (base < r && r <= base + cq) {
            b = lane * PER + q;
            above = base;
            cb = cq;
        }
        base += cq;
    }
    const uint64_t hit = __ballot(b >= 0);
    const int src = hit ? __builtin_ctzll(hit) : 0;
    b = __shfl(b, src);
    above = __shfl(above, src);
    cb = __shfl(cb, src);
    if (n <= CHUNK && cb <= (uint32_t)kTauExactMax) {
        __builtin_amdgcn_wave_barrier();  // every lane has read its counts before hist is reused
        return tau_exact_in_bucket<PERL>(v, lo, vmax, scale, b, above, cb, r, hist, lane);
    }
    return vmax - (float)(b + 2) / scale;
}

// wave_tau for K rows, each of n[k] <= 2048 samples: the same buckets and
// rule, with the K rows' sample loads and range reductions interleaved so
// their latencies overlap; the histogram passes then take the rows in turn.
// hist: kTauBuckets words of LDS private to the wave, 16-byte aligned.  Every lane gets the
// K thresholds.
template <int K>
__device__ __forceinline__ void wave_tau_rows(const uint32_t *const (&samp)[K], const int (&n)[K],
                                              const uint32_t (&r)[K], uint32_t *hist, int lane, float (&tv)[K])
{
    constexpr int PER = kTauBuckets / 64;  // buckets per lane, and samples per lane
    float v[K][PER];
    {
        uint32_t u[K][PER];
#pragma unroll
        for (int k = 0; k < K; ++k)
#pragma unroll
            for (int q = 0; q < PER; ++q) u[k][q] = samp[k][min(lane + 64 * q, n[k] - 1)];
#pragma unroll
        for (int k = 0; k < K; ++k)
#pragma unroll
            for (int q = 0; q < PER; ++q) v[k][q] = lane + 64 * q < n[k] ? float_of_ord(u[k][q]) : __builtin_nanf("");
    }
    float vmin[K], vmax[K], lo[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
        vmin[k] = __builtin_inff();
        vmax[k] = -__builtin_inff();
#pragma unroll
        for (int q = 0; q < PER; ++q) {  // fminf / fmaxf ignore the NaN fill
            vmin[k] = fminf(vmin[k], v[k][q]);
            vmax[k] = fmaxf(vmax[k], v[k][q]);
        }
    }
#pragma unroll
    for (int k = 0; k < K; ++k) {  // wave extremes through DPP on the order codes (lanes with no sample hold +-inf)
        const float lmin = float_of_ord(~wave_max(~ord_of(vmax[k])));  // smallest lane maximum
        vmax[k] = float_of_ord(wave_max(ord_of(vmax[k])));
        vmin[k] = float_of_ord(~wave_max(~ord_of(vmin[k])));
        lo[k] = (n[k] >= 64 && r[k] <= 64u) ? lmin : vmin[k];  // floor of the bucketed range
    }
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const float scale = (float)kTauBuckets / (vmax[k] - lo[k]);
        if (!(vmax[k] > lo[k]) || !__builtin_isfinite(scale)) {  // samples at the floor equal: admit them all
            tv[k] = lo[k];
            continue;
        }
#pragma unroll
        for (int q = 0; q < PER / 4; ++q) reinterpret_cast<v4i *>(hist)[lane + 64 * q] = (v4i){0, 0, 0, 0};
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the zeros land before any lane adds
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            if (v[k][q] >= lo[k]) {  // NaN fill fails
                const float x = (vmax[k] - v[k][q]) * scale;
                atomicAdd(&hist[x < (float)(kTauBuckets - 1) ? (uint32_t)x : (uint32_t)(kTauBuckets - 1)], 1u);
            }
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);
        __builtin_amdgcn_wave_barrier();
        // Lane l owns buckets [PER l, PER l + PER); exclusive prefix over lanes.
        uint32_t c[PER], run = 0;
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            c[q] = hist[lane * PER + q];
            run += c[q];
        }
        uint32_t base = wave_incl_add(run) - run;
        int b = -1;
        uint32_t above = 0, cb = 0;
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            if (base < r[k] && r[k] <= base + c[q]) {
                b = lane * PER + q;
                above = base;
                cb = c[q];
            }
            base += c[q];
        }
        const uint64_t hit = __ballot(b >= 0);
        const int src = hit ? __builtin_ctzll(hit) : 0;
        b = __shfl(b, src);
        above = __shfl(above, src);
        cb = __shfl(cb, src);
        __builtin_amdgcn_wave_barrier();  // every lane has read the counts before hist is reused
        if (cb <= (uint32_t)kTauExactMax) tv[k] = tau_exact_in_bucket<PER>(v[k], lo[k], vmax[k], scale, b, above, cb, r[k], hist, lane);
        else tv[k] = vmax[k] - (float)(b + 2) / scale;
        __builtin_amdgcn_wave_barrier();
    }
}

struct TauArgs {
    const int32_t *ks;
    const int32_t *ke;
    int64_t num_q;
    int topk;
    int cap;
    const uint32_t *samp;      // [num_q, sample_target] sample score codes
    int sample_target;
    int sample_min_stride;
    int pair;                  // 64-head rows: two tile columns per row
    float rank_scale;          // multiplies the rank of the threshold
    float *tau;                // [num_q]
    uint32_t *cnt;             // [num_q] candidate counters, reset here
};

// One wave per row: resets the row's candidate counter and sets its
// threshold (-inf for rows that take their whole window).  Used when the
// sample scores of a tile come from several workgroups, or when the tiles
// take more than one round of sample workgroups (otherwise the sample
// kernel sets the thresholds itself).
constexpr int kTauWaves = 4;

__global__ __launch_bounds__(64 * kTauWaves) __attribute__((amdgpu_waves_per_eu(5))) void k_tau(TauArgs a)
{
    __shared__ uint32_t s_hist[kTauWaves][kTauBuckets];
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t t = (int64_t)blockIdx.x * kTauWaves + wave;  // wave-uniform: scalar registers
    if (t >= a.num_q) return;
    const int64_t lo = a.ks[t], hi = a.ke[t];
    const int64_t len = hi > lo ? hi - lo : 0;
    if (lane == 0) a.cnt[t] = 0;
    float tv = -__builtin_inff();
    if (len > a.cap) {
        const int d = sample_stride(len, a.sample_target, a.sample_min_stride);
        const int dsh = __builtin_ctz((unsigned)d);
        const int64_t tile = (t << a.pair) / 16;  // the sample kernel's tile of the row's first column
        const int ns = (int)min(lattice_count(lo, hi, dsh, lattice_slot(tile, dsh)), (int64_t)a.sample_target);
        tv = wave_tau(a.samp + t * a.sample_target, ns, tau_rank(a.topk, ns, len, a.rank_scale), s_hist[wave], lane);
    }
    if (lane == 0) a.tau[t] = tv;
}

}  // namespace ftk
