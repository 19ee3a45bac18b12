// Triage and exact selection kernels.
//
// Exactness (FlashTopK README, "What you can do": exact; rows the sampled
// threshold misses are rescored on the GPU): a row whose candidate count is
// below min(topk, L) (the threshold was too high) or above the candidate
// capacity (too low) is flagged by triage and rescored densely; every other
// row's candidates contain its whole top-k, because every key outside them
// scores below the threshold.
//
// Selection: the k-th largest 64-bit key (score code, complemented index) is
// located by bucketing the candidates by score (or, for massive ties, by an
// MSB-first radix select with 8-bit digits); keys at or above it -- exactly
// k, since keys are distinct -- are put in descending order.  Descending key
// order is score descending with the smaller index first on ties ("What you
// can do": deterministic).
#pragma once

#include "ftk_common.hpp"

namespace ftk {

constexpr int kSelThreads = 512;   // threads of the selection workgroups for large rows
constexpr int kMaxTopk = 4096;

// ---------------------------------------------------------------------------
// Block-wide radix select over NW waves.  `each(f)` calls f(key) for every
// element this thread owns.  Returns the smallest key T such that exactly k
// elements are >= T (the k-th largest key, or a lower bound with the same
// count).  All threads of the block must call it; k must satisfy 1 <= k <= n.

template <int NW>
struct RadixLds {
    uint32_t hist[NW][256];
    uint32_t tot[256];
    uint32_t suf[257];
    uint32_t digit;
};

template <typename KeyT, int NDIGITS, int NW, typename Each>
__device__ KeyT radix_select_kth(RadixLds<NW> &L, Each each, uint32_t k)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    constexpr int BITS = 8 * sizeof(KeyT);
    KeyT prefix = 0;
    uint32_t remaining = k;
    for (int p = 0; p < NDIGITS; ++p) {
        const int shift = BITS - 8 * (p + 1);
        for (int i = tid; i < NW * 256; i += 64 * NW) (&L.hist[0][0])[i] = 0;
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
        for (int b = tid; b < 256; b += 64 * NW) {
            uint32_t s = 0;
#pragma unroll
            for (int w = 0; w < NW; ++w) s += L.hist[w][b];
            L.tot[b] = s;
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
        for (int b = tid; b < 256; b += 64 * NW)
            if (L.suf[b] >= remaining && L.suf[b + 1] < remaining) L.digit = b;
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
    // f(q, raw, valid) for the register slots q (REG only; q is a
    // compile-time index after unrolling), every lane of the wave together.
    template <typename F>
    __device__ __forceinline__ void each_slot(F f) const
    {
#pragma unroll
        for (int q = 0; q < kRegPer; ++q) {
            const int64_t i = threadIdx.x + (int64_t)q * blockDim.x;
            if (__any(i < n)) f(q, r[q], i < n);
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
// Call statistics kept on the device (zeroed by the preparation pass at the
// start of every fused call): kStPruned / kStPruneOn are the scan's
// PlanCounter slots; kStFlagged is the length of the flagged-row list.  The
// row classes of flashtopk_info are counted on the host from each row's
// window length and candidate count when the record is read.

enum Stat { kStFlagged = 0, kStPruned, kStPruneOn, kStCount };
static_assert(kStPruneOn == kStPruned + kPlanItems, "the scan's counters live in the statistics");

// Triage of one row (the pages' "recovery triage"): a row with a non-empty
// window is rescored densely when its candidate count is below
// min(topk, L) (its threshold was too high) or above the capacity (too low:
// the list lost candidates).
__device__ __host__ __forceinline__ bool row_flagged(int64_t len, uint32_t c, int topk, int cap)
{
    if (len <= 0) return false;
    return (int64_t)c < (len < (int64_t)topk ? len : (int64_t)topk) || (int64_t)c > cap;
}

// ---------------------------------------------------------------------------
// Exact selection of one row per block.

// Output options (DeepSelect README, "Usage": sorted_index, indices_type).
enum OutFlag { kOutIndexOrder = 1, kOutInt64 = 2 };

struct SelectArgs {
    const int32_t *ks;
    const int32_t *ke;
    int topk;
    int cap;
    // candidate rows
    const uint32_t *cnt;
    const uint64_t *cand;
    // outputs
    void *out_idx;       // int32 or int64 (kOutInt64)
    float *out_val;
    int out_flags;       // OutFlag
    // triage: each row's workgroup records the row's window length and
    // appends a flagged row to the recovery list
    int32_t *wlen;                 // [rows]
    int32_t *rowlist;              // flagged rows, in no particular order
    unsigned long long *nflagged;  // length of the list
};

// Bucketed selection.  The row's candidates are spread over NBKT buckets
// linear in score between their minimum and maximum, highest scores in
// bucket 0.  The bucket function is monotone (a larger score never lands in
// a later bucket, equal scores share a bucket), so after one histogram and
// one prefix sum the bucket holding the k-th key is known, every key of an
// earlier bucket is selected, and a counting-sort scatter puts each bucket's
// keys in its slot range.  Each key then finds its place inside its bucket
// by counting the larger keys there (independent LDS reads, one key per
// thread, no serial insertion) and moves to it.  Rows with a bucket of more
// than kSegMax keys up to the k-th (massive ties) use the radix select +
// bitonic sort.
constexpr int kSegMax = 256;

template <int NT, int NBKT, int MAXK>
struct SelectLds {
    static constexpr int NW = NT / 64;
    union {
        RadixLds<NW> radix;
        uint32_t bucket[NBKT];
    };
    uint64_t sel[MAXK + kSegMax];
    uint32_t redu2[2 * NW];
    uint32_t redu[NW];
    uint32_t misc[4];
};

__device__ __forceinline__ float raw_score(uint64_t r) { return __uint_as_float((uint32_t)r); }

// Launch shapes of the selection kernel: NREG candidates per thread in
// registers, NT threads, NBKT buckets,
// rows of at most MAXK outputs.  Small candidate lists get small workgroups
// with small LDS, so more rows are in flight per compute unit.
// MINW is the launch bound's minimum waves per SIMD (0: none), which caps
// the registers so that many rows fit per compute unit.
template <int NREG, int NT, int NBKT, int MAXK, int MINW = 0> struct SelShape {
    static constexpr int nreg = NREG, nt = NT, nbkt = NBKT, maxk = MAXK, minw = MINW;
};
using SelSmall = SelShape<8, 256, 2048, 2048>;     // cap <= 2048
using SelSmallK = SelShape<8, 256, 2048, 512>;     // cap <= 2048, topk <= 512: 8 rows per compute unit
using SelMid = SelShape<8, 512, 4096, kMaxTopk>;   // cap <= 4096
using SelLarge = SelShape<8, 1024, 4096, kMaxTopk, 8>;  // cap <= 8192
using SelLargeK = SelShape<16, 512, 4096, 2048, 6>;     // cap <= 8192, topk <= 2048: 3 rows per compute unit, no spills
using SelHuge = SelShape<16, 1024, 8192, kMaxTopk, 8>;  // cap <= 16384: 2 rows per compute unit beat 1 without spills; 8192 buckets thin the dense ones

template <int NT, int NBKT, int MAXK, typename E>
__device__ void select_core(SelectLds<NT, NBKT, MAXK> &S, const E &el, int64_t n, uint32_t k, int topk,
                            void *oi, float *ov, int flags, int32_t ibase = 0);

// Row r's slots of an output index array of int32 or int64 entries.
__device__ __forceinline__ void *out_row(void *base, int64_t r, int topk, int flags)
{
    return (char *)base + r * topk * ((flags & kOutInt64) ? 8 : 4);
}

// Candidate mode: rows that triage flags (same predicate) are left to dense
// recovery; every other row's candidates hold its whole top k.
template <typename SH>
__global__ __launch_bounds__(SH::nt, SH::minw > 0 ? SH::minw : 1) void k_select(SelectArgs a)
{
    constexpr int NREG = SH::nreg, NT = SH::nt, NBKT = SH::nbkt, MAXK = SH::maxk;
    __shared__ SelectLds<NT, NBKT, MAXK> S;
    const int t = blockIdx.x;
    const int64_t lo = a.ks[t], hi = a.ke[t];
    const int64_t len = hi > lo ? hi - lo : 0;
    const uint32_t c = a.cnt[t];
    const bool flagged = row_flagged(len, c, a.topk, a.cap);
    if (threadIdx.x == 0) {
        a.wlen[t] = (int32_t)len;
        if (flagged) a.rowlist[atomicAdd(a.nflagged, 1ull)] = t;
    }
    if (flagged) return;  // block-uniform
    const uint64_t *src = a.cand + (int64_t)t * a.cap;
    const int64_t n = len > 0 ? min((int64_t)c, (int64_t)a.cap) : 0;  // a.cap <= NREG * NT
    const uint32_t k = (uint32_t)min((int64_t)a.topk, n);
    void *oi = out_row(a.out_idx, t, a.topk, a.out_flags);
    float *ov = a.out_val ? a.out_val + (int64_t)t * a.topk : nullptr;
    RowElems<NREG> el;
    el.load(src, n);
    select_core<NT, NBKT, MAXK>(S, el, n, k, a.topk, oi, ov, a.out_flags);
}

// Exact top k of one row's elements (raw candidates, see raw_cand) held by
// the visitor `el`, written to oi / ov (ov may be null) in key order -- or,
// with kOutIndexOrder, the same k keys by ascending index -- and padded to
// topk; indices (the elements' own plus ibase) as int32, or int64 with
// kOutInt64.  All threads of the block call it; S is the block's LDS.
// Element visitors with registers (E::REG) rank keys inside their buckets in
// parallel; streamed visitors sort each bucket serially and so only take the
// bucketed path for buckets of at most 48 keys.
template <int NT, int NBKT, int MAXK, typename E>
__device__ void select_core(SelectLds<NT, NBKT, MAXK> &S, const E &el, int64_t n, uint32_t k, int topk,
                            void *oi, float *ov, int flags, int32_t ibase)
{
    constexpr int NW = NT / 64, BPT = NBKT / NT;
    constexpr bool DENSE = !E::REG;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    bool fast = false;
    float mx = 0.0f, scale = 0.0f;
    uint32_t kb = 0;
    if (k > 0) {
        // Score range of the candidates, as order codes (maxima of the code
        // and of its complement).
        uint32_t hic = 0, nloc = 0;
        el.each([&](uint64_t r, bool v) {
            if (v) {
                const uint32_t c = ord_of(raw_score(r));
                hic = max(hic, c);
                nloc = max(nloc, ~c);
            }
        });
        hic = wave_max(hic);
        nloc = wave_max(nloc);
        if (lane == 0) {
            S.redu2[wave] = hic;
            S.redu2[NW + wave] = nloc;
        }
        for (int i = tid; i < NBKT; i += NT) S.bucket[i] = 0;
        __syncthreads();
        for (int w = 0; w < NW; ++w) {
            hic = max(hic, S.redu2[w]);
            nloc = max(nloc, S.redu2[NW + w]);
        }
        const float lo = float_of_ord(~nloc), hi = float_of_ord(hic);
        mx = hi;
        scale = (float)NBKT / (hi - lo);
        fast = hi > lo && __builtin_isfinite(scale) && __builtin_isfinite(hi - lo);
    }
    auto bucket_of = [&](float f) -> uint32_t {
        const float x = (mx - f) * scale;
        return x < (float)(NBKT - 1) ? (uint32_t)x : (uint32_t)(NBKT - 1);
    };
    if (fast) {
        el.each([&](uint64_t r, bool v) {
            if (v) atomicAdd(&S.bucket[bucket_of(raw_score(r))], 1u);
        });
        __syncthreads();
        // Exclusive prefix over buckets; each thread owns BPT consecutive
        // buckets and keeps their counts.
        uint32_t cntv[BPT], run = 0;
#pragma unroll
        for (int q = 0; q < BPT; ++q) {
            cntv[q] = S.bucket[tid * BPT + q];
            run += cntv[q];
        }
        const uint32_t x = wave_incl_add(run);
        if (lane == 63) S.redu[wave] = x;
        __syncthreads();
        uint32_t base = x - run;
        for (int w = 0; w < wave; ++w) base += S.redu[w];
#pragma unroll
        for (int q = 0; q < BPT; ++q) {
            const uint32_t b = tid * BPT + q;
            S.bucket[b] = base;
            if (base <= k - 1 && k - 1 < base + cntv[q]) S.misc[0] = b;  // bucket of the k-th key
            base += cntv[q];
        }
        __syncthreads();
        kb = S.misc[0];
        uint32_t seg = 0;
#pragma unroll
        for (int q = 0; q < BPT; ++q)
            if ((uint32_t)(tid * BPT + q) <= kb) seg = max(seg, cntv[q]);
        seg = wave_max(seg);
        if (lane == 0) S.redu[wave] = seg;
        __syncthreads();
        for (int w = 0; w < NW; ++w) seg = max(seg, S.redu[w]);
        fast = seg <= (DENSE ? 48u : (uint32_t)kSegMax);  // streamed rows sort buckets serially
        if (fast) {
            el.each([&](uint64_t r, bool v) {
                if (v) {
                    const uint32_t b = bucket_of(raw_score(r));
                    if (b <= kb) S.sel[atomicAdd(&S.bucket[b], 1u)] = key_of_raw(r);
                }
            });
            __syncthreads();
            // Bucket b now spans [bucket[b-1], bucket[b]).
            if constexpr (!DENSE) {
                // Place of each gathered key: the bucket start plus the
                // number of larger keys in the bucket (keys are distinct),
                // computed for all keys before any key moves.  The keys are
                // visited by their position in S.sel (bucket kb ends at
                // S.bucket[kb]), so the candidate registers are dead here.
                constexpr int PE = (MAXK + kSegMax + NT - 1) / NT;  // gathered keys per thread
                const uint32_t tot = S.bucket[kb];
                uint32_t place[PE];
                uint64_t key[PE];
#pragma unroll
                for (int m = 0; m < PE; ++m) {
                    const uint32_t jj = tid + m * NT;
                    place[m] = 0xFFFFFFFFu;
                    key[m] = 0;
                    if (jj < tot) {
                        const uint64_t e = S.sel[jj];
                        const uint32_t b = bucket_of(key_score(e));
                        const uint32_t s0 = b ? S.bucket[b - 1] : 0u, s1 = S.bucket[b];
                        // four independent LDS reads per step: buckets of
                        // tied scores (BF16 inputs) hold dozens of keys
                        uint32_t rank = 0, j = s0;
                        for (; j + 4 <= s1; j += 4) {
                            const uint64_t k0 = S.sel[j], k1 = S.sel[j + 1], k2 = S.sel[j + 2], k3 = S.sel[j + 3];
                            rank += (k0 > e ? 1u : 0u) + (k1 > e ? 1u : 0u) + (k2 > e ? 1u : 0u) + (k3 > e ? 1u : 0u);
                        }
                        for (; j < s1; ++j) rank += S.sel[j] > e ? 1u : 0u;
                        place[m] = s0 + rank;
                        key[m] = e;
                    }
                }
                __syncthreads();
#pragma unroll
                for (int m = 0; m < PE; ++m)
                    if (place[m] != 0xFFFFFFFFu) S.sel[place[m]] = key[m];
            } else {
                // Streamed rows (recovery): insertion sort of each bucket.
                for (uint32_t b = tid; b <= kb; b += NT) {
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
            }
            __syncthreads();
        } else {
            __syncthreads();  // everyone has read the buckets before the radix scratch reuses them
        }
    }
    if (k > 0 && !fast) {
        uint64_t thr = 0;
        if ((int64_t)k < n)
            thr = radix_select_kth<uint64_t, 8, NW>(
                S.radix, [&](auto f) { el.each([&](uint64_t r, bool v) { f(key_of_raw(r), v); }); }, k);
        if (tid == 0) S.misc[1] = 0;
        __syncthreads();
        el.each([&](uint64_t r, bool v) {
            const uint64_t e = key_of_raw(r);
            if (v && e >= thr) {
                const uint32_t pos = atomicAdd(&S.misc[1], 1u);
                if (pos < (uint32_t)MAXK) S.sel[pos] = e;
            }
        });
        uint32_t P = 1;
        while (P < k) P <<= 1;
        __syncthreads();
        for (uint32_t i = k + tid; i < P; i += NT) S.sel[i] = 0;  // below every real key
        __syncthreads();
        for (uint32_t size = 2; size <= P; size <<= 1) {
            for (uint32_t stride = size >> 1; stride > 0; stride >>= 1) {
                for (uint32_t i = tid; i < P / 2; i += NT) {
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
    if ((flags & kOutIndexOrder) && k > 1) {
        // S.sel[0, k) holds the selected keys; a bitonic sort on the low
        // word (the index's complement) descending orders them by index.
        // Padding with low word 0 sorts last.
        uint32_t P = 1;
        while (P < k) P <<= 1;
        __syncthreads();
        for (uint32_t i = k + tid; i < P; i += NT) S.sel[i] = 0;
        __syncthreads();
        for (uint32_t size = 2; size <= P; size <<= 1) {
            for (uint32_t stride = size >> 1; stride > 0; stride >>= 1) {
                for (uint32_t i = tid; i < P / 2; i += NT) {
                    const uint32_t l0 = 2 * i - (i & (stride - 1));
                    const uint32_t l1 = l0 + stride;
                    const bool desc = (l0 & size) == 0;
                    const uint64_t x = S.sel[l0], y = S.sel[l1];
                    const uint32_t xl = (uint32_t)x, yl = (uint32_t)y;
                    if (desc ? (xl < yl) : (xl > yl)) {
                        S.sel[l0] = y;
                        S.sel[l1] = x;
                    }
                }
                __syncthreads();
            }
        }
    }
    for (int j = tid; j < topk; j += NT) {
        int32_t idx = -1;
        float v = -__builtin_inff();
        if ((uint32_t)j < k) {
            const uint64_t e = S.sel[j];
            idx = key_index(e) + ibase;
            v = key_score(e);
        }
        if (flags & kOutInt64) ((int64_t *)oi)[j] = idx;
        else ((int32_t *)oi)[j] = idx;
        if (ov) ov[j] = v;
    }
}

}  // namespace ftk
