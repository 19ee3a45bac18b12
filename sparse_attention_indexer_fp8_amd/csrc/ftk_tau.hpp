// Per-row threshold from the row's strided sample (FlashTopK README,
// "Highlights": the threshold comes from a strided sample of the row's own
// window).
//
// The threshold needs no exact rank -- only the candidate count it admits
// matters, and triage catches any row it misjudges -- so the sample is
// bucketed linearly in score (kTauBuckets buckets between the sample's
// minimum and maximum, highest first) and the threshold is one bucket below
// the lower edge of the bucket that holds the r-th largest sample: at least r
// samples reach it, whatever the rounding of the bucket arithmetic.  With
// r = ceil(2 * topk * n / L) for n samples of an L-key window, about 2 topk
// keys of the window are expected to reach it.
#pragma once

#include "ftk_common.hpp"

namespace ftk {

constexpr int kTauBuckets = 2048;

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
    for (int off = 32; off > 0; off >>= 1) {
        vmin = fminf(vmin, __shfl_xor(vmin, off));
        vmax = fmaxf(vmax, __shfl_xor(vmax, off));
    }
    const float scale = (float)kTauBuckets / (vmax - vmin);
    if (!(vmax > vmin) || !__builtin_isfinite(scale)) return vmin;  // all samples equal: admit them all
#pragma unroll
    for (int q = 0; q < PER; ++q) hist[lane + 64 * q] = 0u;
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the zeros land before any lane adds
    __builtin_amdgcn_wave_barrier();
    for (int base = 0; base < n; base += CHUNK) {
        if (n > CHUNK) load_chunk(base);  // a single chunk is still in registers
#pragma unroll
        for (int q = 0; q < PERL; ++q) {
            if (base + lane + 64 * q < n) {
                const float x = (vmax - v[q]) * scale;
                atomicAdd(&hist[x < (float)(kTauBuckets - 1) ? (uint32_t)x : (uint32_t)(kTauBuckets - 1)], 1u);
            }
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
    uint32_t x = run;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = __shfl_up(x, off);
        if (lane >= off) x += y;
    }
    uint32_t base = x - run;
    int b = -1;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
        if (base < r && r <= base + c[q]) b = lane * PER + q;
        base += c[q];
    }
    const uint64_t hit = __ballot(b >= 0);
    b = __shfl(b, hit ? __builtin_ctzll(hit) : 0);
    return vmax - (float)(b + 2) / scale;
}

// wave_tau for K rows, each of n[k] <= 2048 samples: the same buckets and
// rule, with the K rows' sample loads and range reductions interleaved so
// their latencies overlap; the histogram passes then take the rows in turn.
// hist: kTauBuckets words of LDS private to the wave.  Every lane gets the
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
    float vmin[K], vmax[K];
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
        vmax[k] = float_of_ord(wave_max(ord_of(vmax[k])));
        vmin[k] = float_of_ord(~wave_max(~ord_of(vmin[k])));
    }
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const float scale = (float)kTauBuckets / (vmax[k] - vmin[k]);
        if (!(vmax[k] > vmin[k]) || !__builtin_isfinite(scale)) {  // all samples equal: admit them all
            tv[k] = vmin[k];
            continue;
        }
#pragma unroll
        for (int q = 0; q < PER; ++q) hist[lane + 64 * q] = 0u;
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the zeros land before any lane adds
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            if (lane + 64 * q < n[k]) {
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
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            if (base < r[k] && r[k] <= base + c[q]) b = lane * PER + q;
            base += c[q];
        }
        const uint64_t hit = __ballot(b >= 0);
        b = __shfl(b, hit ? __builtin_ctzll(hit) : 0);
        tv[k] = vmax[k] - (float)(b + 2) / scale;
        __builtin_amdgcn_wave_barrier();  // every lane has read the counts before the next row clears them
    }
}

// The same threshold computed by a whole workgroup of NT threads from n <=
// kTauBuckets sample codes (at most kTauBuckets / NT per thread): the same
// buckets and rule as wave_tau.  hist is kTauBuckets words of LDS, red 3 *
// (NT / 64) + 1 words; every thread returns the threshold.
template <int NT>
__device__ float block_tau(const uint32_t *samp, int n, uint32_t r, uint32_t *hist, uint32_t *red)
{
    constexpr int NW = NT / 64, PER = kTauBuckets / NT;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    uint32_t c[PER];
    uint32_t hic = 0, nloc = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) c[j] = samp[min(tid + NT * j, max(n, 1) - 1)];  // all loads in flight
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int i = tid + NT * j;
        if (i >= n) c[j] = 0u;
        if (i < n) {
            hic = max(hic, c[j]);
            nloc = max(nloc, ~c[j]);
        }
    }
    hic = wave_max(hic);
    nloc = wave_max(nloc);
    if (lane == 0) {
        red[wave] = hic;
        red[NW + wave] = nloc;
    }
    for (int i = tid; i < kTauBuckets; i += NT) hist[i] = 0u;
    __syncthreads();
    for (int w = 0; w < NW; ++w) {
        hic = max(hic, red[w]);
        nloc = max(nloc, red[NW + w]);
    }
    const float vmin = float_of_ord(~nloc), vmax = float_of_ord(hic);
    const float scale = (float)kTauBuckets / (vmax - vmin);
    if (!(vmax > vmin) || !__builtin_isfinite(scale)) return vmin;  // all samples equal: admit them all
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        if (tid + NT * j < n) {
            const float x = (vmax - float_of_ord(c[j])) * scale;
            atomicAdd(&hist[x < (float)(kTauBuckets - 1) ? (uint32_t)x : (uint32_t)(kTauBuckets - 1)], 1u);
        }
    }
    __syncthreads();
    // Thread t owns buckets [PER t, PER t + PER); exclusive prefix over threads.
    uint32_t run = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        c[j] = hist[tid * PER + j];
        run += c[j];
    }
    const uint32_t x = wave_incl_add(run);
    if (lane == 63) red[2 * NW + wave] = x;
    if (tid == 0) red[3 * NW] = 0u;
    __syncthreads();
    uint32_t base = x - run;
    for (int w = 0; w < wave; ++w) base += red[2 * NW + w];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        if (base < r && r <= base + c[j]) red[3 * NW] = tid * PER + j;
        base += c[j];
    }
    __syncthreads();
    const uint32_t b = red[3 * NW];
    return vmax - (float)(b + 2) / scale;
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
    float rank_scale;          // multiplies the rank of the threshold
    float *tau;                // [num_q]
    uint32_t *cnt;             // [num_q] candidate counters, reset here
};

// One wave per row: resets the row's candidate counter and sets its
// threshold (-inf for rows that take their whole window).  Used when the
// sample scores of a tile come from several workgroups (with one, the
// sample kernel sets the thresholds itself).
constexpr int kTauWaves = 4;

__global__ __launch_bounds__(64 * kTauWaves) void k_tau(TauArgs a)
{
    __shared__ uint32_t s_hist[kTauWaves][kTauBuckets];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t t = (int64_t)blockIdx.x * kTauWaves + wave;
    if (t >= a.num_q) return;
    const int64_t lo = a.ks[t], hi = a.ke[t];
    const int64_t len = hi > lo ? hi - lo : 0;
    if (lane == 0) a.cnt[t] = 0;
    float tv = -__builtin_inff();
    if (len > a.cap) {
        const int d = sample_stride(len, a.sample_target, a.sample_min_stride);
        const int ns = (int)lattice_count(lo, hi, d);
        tv = wave_tau(a.samp + t * a.sample_target, ns, tau_rank(a.topk, ns, len, a.rank_scale), s_hist[wave], lane);
    }
    if (lane == 0) a.tau[t] = tv;
}

}  // namespace ftk
