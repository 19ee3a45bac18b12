// Per-row threshold, triage and exact selection kernels.
//
// Threshold ("gate"): FlashTopK README, "Highlights": each row's threshold
// comes from a strided sample of its own window.  The sample is the lattice of
// multiples of a power-of-two stride d inside [ks, ke) (at most
// `sample_target` keys); the threshold is the r-th largest sample score with
// r = ceil(alpha * topk * n_sample / L), alpha = 2, so about alpha * topk keys
// of the window are expected to reach it.
//
// Exactness ("What you can do": exact; rows the sampled threshold misses are
// rescored on the GPU): a row whose candidate count is below min(topk, L)
// (the threshold was too high) or above the candidate capacity (too low) is
// flagged by triage and rescored densely; every other row's candidates
// contain its whole top-k, because every key outside them scores below the
// threshold.
//
// Selection: the k-th largest 64-bit key (score code, complemented index) is
// found by an MSB-first radix select with 8-bit digits; keys at or above it --
// exactly k, since keys are distinct -- are gathered into LDS and sorted
// descending by a bitonic network.  Descending key order is score descending
// with the smaller index first on ties ("What you can do": deterministic).
#pragma once

#include "ftk_common.hpp"

namespace ftk {

constexpr int kSelThreads = 512;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kMaxTopk = 4096;

// ---------------------------------------------------------------------------
// Block-wide radix select.  `each(f)` calls f(key) for every element this
// thread owns.  Returns the smallest key T such that exactly k elements are
// >= T (the k-th largest key, or a lower bound with the same count).  All
// threads of the block must call it; k must satisfy 1 <= k <= n.

struct RadixLds {
    uint32_t hist[kSelWaves][256];
    uint32_t tot[256];
    uint32_t suf[257];
    uint32_t digit;
};

template <typename KeyT, int NDIGITS, typename Each>
__device__ KeyT radix_select_kth(RadixLds &L, Each each, uint32_t k)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    constexpr int BITS = 8 * sizeof(KeyT);
    KeyT prefix = 0;
    uint32_t remaining = k;
    for (int p = 0; p < NDIGITS; ++p) {
        const int shift = BITS - 8 * (p + 1);
        for (int i = tid; i < kSelWaves * 256; i += blockDim.x) (&L.hist[0][0])[i] = 0;
        __syncthreads();
        each([&](KeyT e, bool valid) {
            const bool match = valid && ((p == 0) || (((e ^ prefix) >> (shift + 8)) == 0));
            const uint32_t dig = (uint32_t)(e >> shift) & 255u;
            // Lanes that share the first active lane's digit add once: the
            // keys of a row crowd into few digits, and same-address LDS
            // atomics would serialise.
            const uint64_t act = __ballot(match);
            if (act) {
                const int leader = __builtin_ctzll(act);
                const uint32_t ld = __shfl(dig, leader);
                const bool same = match && dig == ld;
                const uint64_t sm = __ballot(same);
                if (lane == leader) atomicAdd(&L.hist[wave][ld], (uint32_t)__builtin_popcountll(sm));
                if (match && !same) atomicAdd(&L.hist[wave][dig], 1u);
            }
        });
        __syncthreads();
        if (tid < 256) {
            uint32_t s = 0;
#pragma unroll
            for (int w = 0; w < kSelWaves; ++w) s += L.hist[w][tid];
            L.tot[tid] = s;
        }
        __syncthreads();
        if (wave == 0) {
            // Suffix sums over bins, highest digit first: lane handles 4 bins.
            uint32_t v0 = L.tot[255 - 4 * lane], v1 = L.tot[254 - 4 * lane];
            uint32_t v2 = L.tot[253 - 4 * lane], v3 = L.tot[252 - 4 * lane];
            uint32_t c0 = v0, c1 = c0 + v1, c2 = c1 + v2, c3 = c2 + v3;
            uint32_t x = c3;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                uint32_t y = __shfl_up(x, off);
                if (lane >= off) x += y;
            }
            uint32_t ex = x - c3;
            L.suf[255 - 4 * lane] = ex + c0;
            L.suf[254 - 4 * lane] = ex + c1;
            L.suf[253 - 4 * lane] = ex + c2;
            L.suf[252 - 4 * lane] = ex + c3;
            if (lane == 0) L.suf[256] = 0;
        }
        __syncthreads();
        if (tid < 256 && L.suf[tid] >= remaining && L.suf[tid + 1] < remaining) L.digit = tid;
        __syncthreads();
        const uint32_t d = L.digit;
        const uint32_t above = L.suf[d + 1];
        const uint32_t inbin = L.tot[d];
        __syncthreads();
        remaining -= above;
        prefix |= (KeyT)d << shift;
        if (inbin == remaining) break;  // the whole bin is selected
    }
    return prefix;
}

// Elements of a row, as a visitor over the calling thread's share: either
// held in registers (NREG > 0: at most NREG per thread, all loads in flight
// at once) or streamed from memory on every visit (NREG == 0).
template <int NREG>
struct RowElems {
    static constexpr bool REG = NREG > 0;
    static constexpr int kRegPer = REG ? NREG : 1;
    const uint64_t *src;
    int64_t n;
    uint64_t r[kRegPer];

    __device__ __forceinline__ void load(const uint64_t *p, int64_t cnt)
    {
        src = p;
        n = cnt;
        if (REG) {
#pragma unroll
            for (int q = 0; q < kRegPer; ++q) {
                const int64_t i = threadIdx.x + (int64_t)q * blockDim.x;
                r[q] = i < n ? p[i] : 0ull;
            }
        }
    }
    // f(raw, valid): visits this thread's elements; REG visits every slot so
    // wave-wide operations inside f see all lanes.
    template <typename F>
    __device__ __forceinline__ void each(F f) const
    {
        if (REG) {
#pragma unroll
            for (int q = 0; q < kRegPer; ++q) {
                const int64_t i = threadIdx.x + (int64_t)q * blockDim.x;
                if (__any(i < n)) f(r[q], i < n);
            }
        } else {
            const int64_t rounds = (n + blockDim.x - 1) / blockDim.x;
            for (int64_t q = 0; q < rounds; ++q) {
                const int64_t i = threadIdx.x + q * blockDim.x;
                f(i < n ? src[i] : 0ull, i < n);
            }
        }
    }
};

// ---------------------------------------------------------------------------
// Per-row threshold from the row's strided sample.

struct TauArgs {
    const int32_t *ks;
    const int32_t *ke;
    int topk;
    int cap;
    const uint32_t *samp;
    int sample_target;
    float rank_scale;
    int recover_all;
    float *tau;
    uint32_t *cnt;
};

// The threshold needs no exact rank -- only the candidate count it admits
// matters, and triage catches any row it misjudges -- so the sample is
// bucketed linearly in score (kTauBuckets buckets between the sample's
// minimum and maximum, highest first) and the threshold is the lower edge of
// the bucket that holds the r-th largest sample.  At least r samples reach it.
constexpr int kTauThreads = 256;
constexpr int kTauBuckets = 2048;

__global__ __launch_bounds__(kTauThreads) void k_tau(TauArgs a)
{
    __shared__ uint32_t s_b[kTauBuckets];
    __shared__ float s_red[2 * (kTauThreads / 64)];
    __shared__ uint32_t s_tot[kTauThreads / 64];
    __shared__ float s_tau;
    const int t = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    constexpr int NW = kTauThreads / 64, PER = kTauBuckets / kTauThreads;
    const int64_t lo = a.ks[t], hi = a.ke[t];
    const int64_t len = hi > lo ? hi - lo : 0;
    if (tid == 0) a.cnt[t] = 0;
    if (a.recover_all || len <= a.cap) {
        if (tid == 0) a.tau[t] = a.recover_all ? __builtin_inff() : -__builtin_inff();
        return;
    }
    const int d = sample_stride(len, a.sample_target);
    const int ns = (int)lattice_count(lo, hi, d);
    const double want = ceil(2.0 * (double)a.topk * (double)ns / (double)len * (double)a.rank_scale);
    const uint32_t r = (uint32_t)min(max(want, 1.0), (double)ns);
    const uint32_t *row = a.samp + (int64_t)t * a.sample_target;
    // Visits this thread's samples in register chunks of 8 (loads in flight
    // together); one chunk covers the default sample size.
    constexpr int CH = 8;
    auto each = [&](auto f) {
        for (int base = 0; base < ns; base += CH * kTauThreads) {
            float v[CH];
#pragma unroll
            for (int q = 0; q < CH; ++q) {
                const int i = base + tid + q * kTauThreads;
                v[q] = i < ns ? float_of_ord(row[i]) : __builtin_nanf("");
            }
#pragma unroll
            for (int q = 0; q < CH; ++q)
                if (base + tid + q * kTauThreads < ns) f(v[q]);
        }
    };
    float vmin = __builtin_inff(), vmax = -__builtin_inff();
    each([&](float f) {
        vmin = fminf(vmin, f);
        vmax = fmaxf(vmax, f);
    });
    for (int off = 32; off > 0; off >>= 1) {
        vmin = fminf(vmin, __shfl_xor(vmin, off));
        vmax = fmaxf(vmax, __shfl_xor(vmax, off));
    }
    if (lane == 0) {
        s_red[wave] = vmin;
        s_red[NW + wave] = vmax;
    }
    for (int i = tid; i < kTauBuckets; i += kTauThreads) s_b[i] = 0;
    __syncthreads();
    vmin = s_red[0];
    vmax = s_red[NW];
    for (int w = 1; w < NW; ++w) {
        vmin = fminf(vmin, s_red[w]);
        vmax = fmaxf(vmax, s_red[NW + w]);
    }
    const float scale = (float)kTauBuckets / (vmax - vmin);
    if (!(vmax > vmin) || !__builtin_isfinite(scale)) {
        if (tid == 0) a.tau[t] = vmin;  // all samples equal: admit them all
        return;
    }
    each([&](float f) {
        const float x = (vmax - f) * scale;
        atomicAdd(&s_b[x < (float)(kTauBuckets - 1) ? (uint32_t)x : (uint32_t)(kTauBuckets - 1)], 1u);
    });
    __syncthreads();
    uint32_t c[PER], run = 0;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
        c[q] = s_b[tid * PER + q];
        run += c[q];
    }
    uint32_t x = run;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = __shfl_up(x, off);
        if (lane >= off) x += y;
    }
    if (lane == 63) s_tot[wave] = x;
    __syncthreads();
    uint32_t base = x - run;
    for (int w = 0; w < wave; ++w) base += s_tot[w];
#pragma unroll
    for (int q = 0; q < PER; ++q) {
        if (base < r && r <= base + c[q]) {
            // One bucket below the lower edge of bucket b, so rounding cannot
            // leave a sample of buckets 0..b under the threshold.
            const int b = tid * PER + q;
            s_tau = vmax - (float)(b + 2) / scale;
        }
        base += c[q];
    }
    __syncthreads();
    if (tid == 0) a.tau[t] = s_tau;
}

// ---------------------------------------------------------------------------
// Triage: one block classifies every row, lists the flagged rows in row
// order and gathers the statistics.

enum Stat {
    kStRows = 0, kStEmpty, kStTakeAll, kStSampled, kStUnder, kStOver, kStFlagged, kStMaxCand,
    kStWindow, kStPruned, kStPruneOn, kStCount
};

struct TriageArgs {
    const int32_t *ks;
    const int32_t *ke;
    int64_t num_q;
    int topk;
    int cap;
    const uint32_t *cnt;
    int recover_all;
    int32_t *rowflag;
    int32_t *rowlist;
    int32_t *nflagged;
    unsigned long long *stats;
    const unsigned long long *plan;  // pruning counters, or null (pruning off)
};

__global__ __launch_bounds__(1024) void k_triage(TriageArgs a)
{
    __shared__ unsigned long long s_st[kStCount];
    __shared__ uint32_t s_wave[16];
    __shared__ uint32_t s_base;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (tid < kStCount) s_st[tid] = 0;
    if (tid == 0) s_base = 0;
    __syncthreads();
    // Per-thread tallies, reduced per wave at the end (no per-row atomics).
    uint32_t n_empty = 0, n_take = 0, n_samp = 0, n_under = 0, n_over = 0, maxc = 0;
    unsigned long long win = 0;
    for (int64_t b0 = 0; b0 < a.num_q; b0 += 1024) {
        const int64_t t = b0 + tid;
        bool flag = false;
        if (t < a.num_q) {
            const int64_t lo = a.ks[t], hi = a.ke[t];
            const int64_t len = hi > lo ? hi - lo : 0;
            const uint32_t c = a.cnt[t];
            if (len == 0) {
                ++n_empty;
            } else if (a.recover_all) {
                flag = true;
            } else {
                const int64_t need = min((int64_t)a.topk, len);
                const bool under = (int64_t)c < need;
                const bool over = (int64_t)c > a.cap;
                flag = under || over;
                if (len <= a.cap) {
                    ++n_take;
                } else {
                    ++n_samp;
                    maxc = max(maxc, c);
                }
                n_under += under;
                n_over += over;
            }
            win += (unsigned long long)len;
            a.rowflag[t] = flag ? 1 : 0;
        }
        // Order-preserving compaction of the flagged rows.
        const uint64_t bal = __ballot(flag);
        const uint32_t below = __builtin_popcountll(bal & ((1ull << lane) - 1ull));
        if (lane == 0) s_wave[wave] = __builtin_popcountll(bal);
        __syncthreads();
        uint32_t off = s_base;
        for (int w = 0; w < wave; ++w) off += s_wave[w];
        if (flag) a.rowlist[off + below] = (int32_t)t;
        __syncthreads();
        if (tid == 0) {
            uint32_t sum = 0;
            for (int w = 0; w < 16; ++w) sum += s_wave[w];
            s_base += sum;
        }
        __syncthreads();
    }
    for (int off = 32; off > 0; off >>= 1) {
        n_empty += __shfl_xor(n_empty, off);
        n_take += __shfl_xor(n_take, off);
        n_samp += __shfl_xor(n_samp, off);
        n_under += __shfl_xor(n_under, off);
        n_over += __shfl_xor(n_over, off);
        maxc = max(maxc, (uint32_t)__shfl_xor(maxc, off));
        win += __shfl_xor(win, off);
    }
    if (lane == 0) {
        atomicAdd(&s_st[kStEmpty], (unsigned long long)n_empty);
        atomicAdd(&s_st[kStTakeAll], (unsigned long long)n_take);
        atomicAdd(&s_st[kStSampled], (unsigned long long)n_samp);
        atomicAdd(&s_st[kStUnder], (unsigned long long)n_under);
        atomicAdd(&s_st[kStOver], (unsigned long long)n_over);
        atomicMax(&s_st[kStMaxCand], (unsigned long long)maxc);
        atomicAdd(&s_st[kStWindow], win);
    }
    __syncthreads();
    if (tid == 0) {
        *a.nflagged = (int32_t)s_base;
        s_st[kStRows] = (unsigned long long)a.num_q;
        s_st[kStFlagged] = s_base;
        s_st[kStPruneOn] = (a.plan && a.plan[kPlanItems] > 0) ? 1ull : 0ull;
        s_st[kStPruned] = a.plan ? a.plan[kPlanPruned] : 0ull;
    }
    __syncthreads();
    if (tid < kStCount) a.stats[tid] = s_st[tid];
}

// ---------------------------------------------------------------------------
// Exact selection of one row per block.

struct SelectArgs {
    const int32_t *ks;
    const int32_t *ke;
    int topk;
    int cap;
    // candidate rows
    const uint32_t *cnt;
    const int32_t *rowflag;
    const uint64_t *cand;
    // dense (recovered) rows
    const int32_t *rowlist;
    const int32_t *nrows;
    int row_base;
    int row_limit;
    const uint64_t *scratch;
    int64_t scratch_stride;
    int32_t *out_idx;
    float *out_val;
};

// Bucketed selection.  The row's candidates are spread over kBuckets
// buckets linear in score between their minimum and maximum, highest scores
// in bucket 0.  The bucket function is monotone (a larger score never lands
// in a later bucket, equal scores share a bucket), so after one histogram and
// one prefix sum the bucket holding the k-th key is known, every key of an
// earlier bucket is selected, and a counting-sort scatter followed by a sort
// of each (small) bucket by full key yields the top k in order.  Rows whose
// buckets are too crowded (massive ties) use the radix select + bitonic sort.
constexpr int kBuckets = 4096;
constexpr int kSegMax = 48;
constexpr int kBinsPerThread = kBuckets / kSelThreads;

struct SelectLds {
    union {
        RadixLds radix;
        uint32_t bucket[kBuckets];
    };
    uint64_t sel[kMaxTopk + kSegMax];
    float redf[2 * kSelWaves];
    uint32_t redu[kSelWaves];
    uint32_t misc[4];
};

__device__ __forceinline__ float raw_score(uint64_t r) { return __uint_as_float((uint32_t)r); }

// NREG == 0: dense (recovered) rows streamed from scratch; otherwise the
// row's candidates (count <= NREG * kSelThreads) are held in registers.
template <int NREG>
__global__ __launch_bounds__(kSelThreads) void k_select(SelectArgs a)
{
    constexpr bool DENSE = NREG == 0;
    __shared__ SelectLds S;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int t;
    const uint64_t *src;
    int64_t n;
    if (DENSE) {
        const int e = blockIdx.x;
        if (e >= a.row_limit || a.row_base + e >= *a.nrows) return;
        t = a.rowlist[a.row_base + e];
        src = a.scratch + (int64_t)e * a.scratch_stride;
        const int64_t lo = a.ks[t], hi = a.ke[t];
        n = hi > lo ? hi - lo : 0;
    } else {
        t = blockIdx.x;
        if (a.rowflag[t]) return;
        src = a.cand + (int64_t)t * a.cap;
        n = min((int64_t)a.cnt[t], (int64_t)a.cap);  // a.cap <= NREG * kSelThreads
    }
    const uint32_t k = (uint32_t)min((int64_t)a.topk, n);
    int32_t *oi = a.out_idx + (int64_t)t * a.topk;
    float *ov = a.out_val ? a.out_val + (int64_t)t * a.topk : nullptr;
    RowElems<NREG> el;
    el.load(src, n);

    bool fast = false;
    float mx = 0.0f, scale = 0.0f;
    uint32_t kb = 0;
    if (k > 0) {
        // Score range of the candidates.
        float lo = __builtin_inff(), hi = -__builtin_inff();
        el.each([&](uint64_t r, bool v) {
            if (v) {
                const float f = raw_score(r);
                lo = fminf(lo, f);
                hi = fmaxf(hi, f);
            }
        });
        for (int off = 32; off > 0; off >>= 1) {
            lo = fminf(lo, __shfl_xor(lo, off));
            hi = fmaxf(hi, __shfl_xor(hi, off));
        }
        if (lane == 0) {
            S.redf[wave] = lo;
            S.redf[kSelWaves + wave] = hi;
        }
        for (int i = tid; i < kBuckets; i += blockDim.x) S.bucket[i] = 0;
        __syncthreads();
        lo = S.redf[0];
        hi = S.redf[kSelWaves];
        for (int w = 1; w < kSelWaves; ++w) {
            lo = fminf(lo, S.redf[w]);
            hi = fmaxf(hi, S.redf[kSelWaves + w]);
        }
        mx = hi;
        scale = (float)kBuckets / (hi - lo);
        fast = hi > lo && __builtin_isfinite(scale) && __builtin_isfinite(hi - lo);
    }
    auto bucket_of = [&](float f) -> uint32_t {
        const float x = (mx - f) * scale;
        return x < (float)(kBuckets - 1) ? (uint32_t)x : (uint32_t)(kBuckets - 1);
    };
    if (fast) {
        el.each([&](uint64_t r, bool v) {
            if (v) atomicAdd(&S.bucket[bucket_of(raw_score(r))], 1u);
        });
        __syncthreads();
        // Exclusive prefix over buckets; each thread owns kBinsPerThread
        // consecutive buckets and keeps their counts.
        uint32_t cntv[kBinsPerThread], run = 0;
#pragma unroll
        for (int q = 0; q < kBinsPerThread; ++q) {
            cntv[q] = S.bucket[tid * kBinsPerThread + q];
            run += cntv[q];
        }
        uint32_t x = run;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const uint32_t y = __shfl_up(x, off);
            if (lane >= off) x += y;
        }
        if (lane == 63) S.redu[wave] = x;
        __syncthreads();
        uint32_t base = x - run;
        for (int w = 0; w < wave; ++w) base += S.redu[w];
#pragma unroll
        for (int q = 0; q < kBinsPerThread; ++q) {
            const uint32_t b = tid * kBinsPerThread + q;
            S.bucket[b] = base;
            if (base <= k - 1 && k - 1 < base + cntv[q]) S.misc[0] = b;  // bucket of the k-th key
            base += cntv[q];
        }
        __syncthreads();
        kb = S.misc[0];
        uint32_t seg = 0;
#pragma unroll
        for (int q = 0; q < kBinsPerThread; ++q)
            if ((uint32_t)(tid * kBinsPerThread + q) <= kb) seg = max(seg, cntv[q]);
        for (int off = 32; off > 0; off >>= 1) seg = max(seg, (uint32_t)__shfl_xor(seg, off));
        if (lane == 0) S.redu[wave] = seg;
        __syncthreads();
        for (int w = 0; w < kSelWaves; ++w) seg = max(seg, S.redu[w]);
        fast = seg <= (uint32_t)kSegMax;
        if (fast) {
            el.each([&](uint64_t r, bool v) {
                if (v) {
                    const uint32_t b = bucket_of(raw_score(r));
                    if (b <= kb) S.sel[atomicAdd(&S.bucket[b], 1u)] = key_of_raw(r);
                }
            });
            __syncthreads();
            // Bucket b now spans [bucket[b-1], bucket[b]); sort it descending.
            for (uint32_t b = tid; b <= kb; b += blockDim.x) {
                const uint32_t s0 = b ? S.bucket[b - 1] : 0u, s1 = S.bucket[b];
                for (uint32_t i = s0 + 1; i < s1; ++i) {
                    const uint64_t v = S.sel[i];
                    uint32_t j = i;
                    while (j > s0 && S.sel[j - 1] < v) {
                        S.sel[j] = S.sel[j - 1];
                        --j;
                    }
                    S.sel[j] = v;
                }
            }
            __syncthreads();
        } else {
            __syncthreads();  // everyone has read the buckets before the radix scratch reuses them
        }
    }
    if (k > 0 && !fast) {
        uint64_t thr = 0;
        if ((int64_t)k < n)
            thr = radix_select_kth<uint64_t, 8>(
                S.radix, [&](auto f) { el.each([&](uint64_t r, bool v) { f(key_of_raw(r), v); }); }, k);
        if (tid == 0) S.misc[1] = 0;
        __syncthreads();
        el.each([&](uint64_t r, bool v) {
            const uint64_t e = key_of_raw(r);
            if (v && e >= thr) {
                const uint32_t pos = atomicAdd(&S.misc[1], 1u);
                if (pos < (uint32_t)kMaxTopk) S.sel[pos] = e;
            }
        });
        uint32_t P = 1;
        while (P < k) P <<= 1;
        __syncthreads();
        for (uint32_t i = k + tid; i < P; i += blockDim.x) S.sel[i] = 0;  // below every real key
        __syncthreads();
        for (uint32_t size = 2; size <= P; size <<= 1) {
            for (uint32_t stride = size >> 1; stride > 0; stride >>= 1) {
                for (uint32_t i = tid; i < P / 2; i += blockDim.x) {
                    const uint32_t l0 = 2 * i - (i & (stride - 1));
                    const uint32_t l1 = l0 + stride;
                    const bool desc = (l0 & size) == 0;
                    const uint64_t x = S.sel[l0], y = S.sel[l1];
                    if (desc ? (x < y) : (x > y)) {
                        S.sel[l0] = y;
                        S.sel[l1] = x;
                    }
                }
                __syncthreads();
            }
        }
    }
    for (int j = tid; j < a.topk; j += blockDim.x) {
        int32_t idx = -1;
        float v = -__builtin_inff();
        if ((uint32_t)j < k) {
            const uint64_t e = S.sel[j];
            idx = key_index(e);
            v = key_score(e);
        }
        oi[j] = idx;
        if (ov) ov[j] = v;
    }
}

}  // namespace ftk
