// Exact top-k over materialized score rows (DeepSelect README, "Usage" and
// "Variable-length rows": each row keeps its topk largest values among its
// first end[r] entries; shorter rows are padded).  Same order and padding as
// the indexer selection: value descending, smaller position first on ties
// (+0 and -0 equal), then index -1 / value -inf.
//
// One workgroup per row, one pass over the row in the common case:
//   1. a sample of the row (64 runs of 128 contiguous bytes spread over it)
//      sets a threshold tau that about three times topk entries of the row
//      reach (the same sampled-threshold idea as the indexer's filter);
//   2. one streaming pass gathers every entry >= tau into LDS and counts
//      them exactly;
//   3. when topk <= count <= capacity, the gathered set holds the whole top
//      k -- every entry tied with the k-th value included -- and the
//      candidate selection finishes the row exactly.
// Otherwise (a sample that misjudged the row, values crowding at the top)
// the row is redone by a two-pass digit histogram: pass 1 counts the top 12
// bits of each value's order code (4096 digits, an eighth of a binade each),
// pass 2 gathers every entry of the k-th value's digit or above, and the
// selection runs on that set, or, if even that does not fit, on the
// streamed row (radix select).
#pragma once

#include "ftk_common.hpp"
#include "ftk_frag.hpp"
#include "ftk_select.hpp"

namespace ftk {

// Launch shapes: NT threads, REGS gathered entries per thread (the LDS
// capacity is NT * REGS), and the selection's buckets and largest topk.
// Small rows outputs fit four workgroups per compute unit, so one
// workgroup's latency-bound phases (sample, selection) overlap the others'
// streaming.
template <int NT_, int REGS_, int NBKT_, int MAXK_> struct RowsShape {
    static constexpr int nt = NT_, regs = REGS_, cap = NT_ * REGS_, nbkt = NBKT_, maxk = MAXK_;
};
using RowsSmall = RowsShape<512, 8, 2048, 1024>;        // topk <= 1024, capacity 4096
using RowsLarge = RowsShape<1024, 8, 4096, kMaxTopk>;   // topk <= 4096, capacity 8192
constexpr int kRowsDigitShift = 20;                       // 12-bit digits
constexpr int kRowsBuckets = 1 << (32 - kRowsDigitShift);  // 4096
constexpr int kRowsTauBuckets = 2048;
constexpr int kRowsSampleRuns = 64;                       // 128-byte runs sampled per row
// 16-byte loads per thread and group; with the next group in flight while
// one is scanned, 64 bytes per thread are outstanding.
constexpr int kRowsUnroll = 2;

struct RowsArgs {
    const void *x;          // [rows, stride] float32 or BF16
    int64_t rows, cols, stride;
    const int32_t *ends;    // [rows] or null
    int topk;
    void *out_idx;          // [rows, topk] int32, or int64 (kOutInt64)
    float *out_val;         // [rows, topk] or null
    int32_t *nan_flag;      // set to 1 when a row holds a NaN; or null
    int out_flags;          // OutFlag
    // Window rows (dense scores of the fused call), when ks is set: input
    // row r is call row rowmap[row_base + r], present while row_base + r is
    // below *nrows (dense recovery of flagged rows), or, with no rowmap, call
    // row row_base + r, present while below rows_total (every row scored
    // densely); its outputs go to that call row, its length is the row's
    // window ke - ks (at most cols) and its indices are offset by the window
    // start ks.
    const int32_t *rowmap;
    const unsigned long long *nrows;
    int64_t row_base;
    const int32_t *ks;
    const int32_t *ke;
    int64_t rows_total;
};

// Output row, length and index offset of input row r (present = false: a
// mapped row past the list, nothing to do).
struct RowPlace {
    int64_t out, n;
    int32_t base;
    bool present;
};

__device__ __forceinline__ RowPlace row_place(const RowsArgs &a, int64_t r)
{
    if (a.ks) {
        int64_t t = a.row_base + r;
        if (a.rowmap) {
            if ((unsigned long long)t >= *a.nrows) return {0, 0, 0, false};
            t = a.rowmap[t];
        } else if (t >= a.rows_total) {
            return {0, 0, 0, false};
        }
        const int64_t lo = a.ks[t], hi = max((int64_t)a.ke[t], lo);
        return {t, min(hi - lo, a.cols), (int32_t)lo, true};
    }
    return {r, a.ends ? min(max((int64_t)a.ends[r], (int64_t)0), a.cols) : a.cols, 0, true};
}

template <typename T> __device__ __forceinline__ float entry_value(T v);
template <> __device__ __forceinline__ float entry_value<float>(float v) { return v; }
template <> __device__ __forceinline__ float entry_value<uint16_t>(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }

template <typename SH>
struct RowsLds {
    // The histograms, the gathered entries and the selection's state are
    // live one after another.
    union {
        uint32_t hist[kRowsBuckets];
        uint64_t cand[SH::cap];
        SelectLds<SH::nt, SH::nbkt, SH::maxk> sel;
    };
    uint32_t redu2[2 * (SH::nt / 64)];
    uint32_t redu[SH::nt / 64];
    uint32_t misc[4];
};

// Block-wide exclusive prefix over BPT counts per thread, taken in thread
// order; returns this thread's start.  Ends with the block synchronised.
template <int NT, int BPT>
__device__ __forceinline__ uint32_t block_prefix(const uint32_t (&c)[BPT], uint32_t *redu)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t run = 0;
#pragma unroll
    for (int q = 0; q < BPT; ++q) run += c[q];
    const uint32_t x = wave_incl_add(run);
    if (lane == 63) redu[wave] = x;
    __syncthreads();
    uint32_t base = x - run;
    for (int w = 0; w < wave; ++w) base += redu[w];
    __syncthreads();
    return base;
}

// Buffer resource over `entries` entries from p, rounded up to whole 16-byte
// chunks (the aligned chunk holding a valid entry is always readable) and
// clamped to the 32-bit size field; nothing if entries <= 0.  Loads past it
// read zeros, so every load is unconditional and no branch makes the
// compiler wait for it early.
template <typename T>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const T *p, int64_t entries)
{
    const uint64_t bytes = entries > 0 ? ((uint64_t)entries * sizeof(T) + 15) & ~(uint64_t)15 : 0;
    return make_rsrc(p, (bytes >> 32) ? 0xFFFFFFF0u : (uint32_t)bytes);
}

// One group of U 16-byte chunks per thread: chunk u of thread t covers
// entries g0 + (u NT + t) V ... + V - 1.  Chunks past the row read as zeros.
template <typename T, int NT, int U>
__device__ __forceinline__ void load_group(v4i (&raw)[U], const T *row, int64_t n, int64_t g0)
{
    const __amdgpu_buffer_rsrc_t rs = row_rsrc(row + g0, n - g0);
    const uint32_t voff = threadIdx.x * 16u;  // one lane offset; the chunk's goes in the scalar offset
#pragma unroll
    for (int u = 0; u < U; ++u) raw[u] = buf_load16(rs, voff, (uint32_t)(u * NT * 16));
}

// Threshold from the row's sample: linear buckets between the finite
// sample extremes, largest first; tau is one bucket below the lower edge of
// the bucket holding the r-th largest sample, so at least r samples reach
// it whatever the rounding.  r = ceil(target * samples / n).
// The count of entries reaching the r-th largest of ns samples of n entries
// is about r n / ns, with a relative spread of about 1 / sqrt(r) for
// independent values; the target t keeps topk four spreads below it
// (t - 4 sqrt(t n / ns) >= topk), but at most three times topk and no more
// than halfway from topk to the LDS capacity: rows far from independent
// values that miss both bounds (fewer than topk, more than the capacity)
// take the slower exact path.
__device__ __forceinline__ uint32_t rows_target(uint32_t k, uint32_t cap, uint32_t ns, int64_t n)
{
    const float m = ns > 0 ? (float)n / (float)ns : 1.0f;
    const float s = 2.0f * sqrtf(m) + sqrtf(4.0f * m + (float)k);
    const uint32_t t = (uint32_t)fminf(s * s + 1.0f, 4.0e9f);
    return min(min(max(t, k + 1u), 3u * k), k + (cap - k) / 2u);
}

// The sample: 64 runs of 128 bytes, run j starting at line floor(j lines / 64)
// of the row; chunk t (0 ... 511) is 16-byte chunk t % 8 of run t / 8.
// Returns the chunk's first entry, or -1 past the row.
template <typename T>
__device__ __forceinline__ int64_t sample_base(int64_t n, int t)
{
    constexpr int V = 16 / sizeof(T), CPR = 128 / 16;  // chunks per run
    const int run = t / CPR, sub = t % CPR;
    const int64_t nlines = (n * (int64_t)sizeof(T) + 127) / 128;
    const int64_t base = ((int64_t)run * nlines / kRowsSampleRuns * CPR + sub) * V;
    return run < kRowsSampleRuns && base < n ? base : -1;
}

template <typename T>
__device__ __forceinline__ v4i sample_load(const T *row, int64_t n, int t)
{
    const int64_t base = sample_base<T>(n, t);
    // (a row past 4 GiB wraps the offset to another in-row chunk: the sample
    // only steers speed)
    return buf_load16(row_rsrc(row, n), base >= 0 ? (uint32_t)(base * (int64_t)sizeof(T)) : 0xFFFFFFF0u, 0u);
}

template <typename T, typename SH>
__device__ float rows_sample_tau(RowsLds<SH> &L, const v4i &raw, int64_t n, uint32_t k)
{
    constexpr int NT = SH::nt, V = 16 / sizeof(T), NW = NT / 64;
    constexpr int BPT = kRowsTauBuckets / NT;
    static_assert(kRowsSampleRuns * 8 <= NT, "one sampled chunk per thread");
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    float v[V];
    bool ok[V];
    {
        const int64_t base = sample_base<T>(n, tid);
        const T *e = reinterpret_cast<const T *>(&raw);
#pragma unroll
        for (int j = 0; j < V; ++j) {
            v[j] = entry_value<T>(e[j]);
            ok[j] = base >= 0 && base + j < n;
        }
    }
    // finite sample extremes as order codes (maxima of the code and of its
    // complement), and the sample count
    uint32_t hic = 0, nloc = 0, ns = 0;
#pragma unroll
    for (int j = 0; j < V; ++j) {
        ns += ok[j] ? 1u : 0u;
        if (ok[j] && __builtin_isfinite(v[j])) {
            const uint32_t c = ord_of(v[j]);
            hic = max(hic, c);
            nloc = max(nloc, ~c);
        }
    }
    hic = wave_max(hic);
    nloc = wave_max(nloc);
    ns = wave_sum(ns);
    if (lane == 0) {
        L.redu2[wave] = hic;
        L.redu2[NW + wave] = nloc;
        L.redu[wave] = ns;
    }
    for (int i = tid; i < kRowsTauBuckets; i += NT) L.hist[i] = 0u;
    __syncthreads();
    ns = 0;
    for (int w = 0; w < NW; ++w) {
        hic = max(hic, L.redu2[w]);
        nloc = max(nloc, L.redu2[NW + w]);
        ns += L.redu[w];
    }
    const bool any = hic != 0u;  // a finite sample has a nonzero code
    const float lo = float_of_ord(~nloc), hi = float_of_ord(hic);
    const float scale = (float)kRowsTauBuckets / (hi - lo);
    const bool spread = any && hi > lo && __builtin_isfinite(scale) && scale > 0.0f;
    __syncthreads();  // the reductions are read before the prefix reuses redu
    if (!spread) return any && !(hi > lo) ? lo : -__builtin_inff();  // degenerate sample: let the count decide
    const uint32_t target = rows_target(k, SH::cap, ns, n);
    const uint32_t r = (uint32_t)min(max(ceil((double)target * (double)ns / (double)n), 1.0), (double)ns);
#pragma unroll
    for (int j = 0; j < V; ++j) {
        if (ok[j]) {
            const float x = (hi - v[j]) * scale;  // +inf -> -inf, -inf and NaN -> last bucket
            const uint32_t b = v[j] == __builtin_inff() ? 0u
                               : (x < (float)(kRowsTauBuckets - 1) ? (uint32_t)fmaxf(x, 0.0f) : (uint32_t)(kRowsTauBuckets - 1));
            atomicAdd(&L.hist[b], 1u);
        }
    }
    __syncthreads();
    uint32_t c[BPT];
#pragma unroll
    for (int q = 0; q < BPT; ++q) c[q] = L.hist[tid * BPT + q];
    uint32_t base = block_prefix<NT, BPT>(c, L.redu);
#pragma unroll
    for (int q = 0; q < BPT; ++q) {
        if (base < r && r <= base + c[q]) L.misc[0] = tid * BPT + q;
        base += c[q];
    }
    __syncthreads();
    const uint32_t b = L.misc[0];
    __syncthreads();
    return hi - (float)(b + 2) / scale;
}

// Appends the entries >= tau of one loaded group (row positions g0 ...) to
// L.cand, the first SH::cap of the row.  Each thread marks its keepers in a
// bit mask (entry e of the group at bit U V - 1 - e), reserves their slots
// with one LDS atomic and stores them in order; keepers are rare, so the
// store loop walks the mask's set bits and picks each keeper's word out of
// the group with a select chain.  TAIL: the group may pass the row's end.
template <typename T, typename SH, int U, bool TAIL>
__device__ __forceinline__ void scan_group(RowsLds<SH> &L, const v4i (&raw)[U], int64_t g0, int64_t n, float tau,
                                           bool &nan, int64_t ibase)
{
    constexpr int NT = SH::nt, V = 16 / sizeof(T), PER = sizeof(uint32_t) / sizeof(T);  // entries per word
    constexpr int E = U * V;
    static_assert(E <= 32, "one mask bit per entry");
    const int tid = threadIdx.x;
    const uint32_t rem = TAIL ? (uint32_t)min(n - g0, (int64_t)NT * E) : 0u;
    uint32_t mask = 0;
    bool bad = false;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const T *e = reinterpret_cast<const T *>(&raw[u]);
#pragma unroll
        for (int j = 0; j < V; ++j) {
            const float f = entry_value<T>(e[j]);
            const bool valid = !TAIL || (uint32_t)((u * NT + tid) * V + j) < rem;
            bad |= valid && f != f;
            mask = (mask << 1) | ((valid && f >= tau) ? 1u : 0u);
        }
    }
    nan |= bad;
    if (mask == 0) return;
    uint32_t pos = atomicAdd(&L.misc[3], (uint32_t)__builtin_popcount(mask));
    do {
        const int b = E - 1 - (31 - __builtin_clz(mask));  // the lowest-numbered keeper left
        mask &= ~(1u << (E - 1 - b));
        const int q = b / PER;  // word of the group
        uint32_t w = (uint32_t)raw[0][0];
#pragma unroll
        for (int x = 1; x < U * 4; ++x)
            if (q == x) w = (uint32_t)raw[x / 4][x % 4];
        float f;
        if (PER == 2) f = __uint_as_float((b & 1) ? (w & 0xFFFF0000u) : (w << 16));
        else f = __uint_as_float(w);
        const uint32_t li = (uint32_t)(((b / V) * NT + tid) * V + (b % V));
        if (pos < (uint32_t)SH::cap) L.cand[pos] = raw_cand(f, (int32_t)(ibase + g0 + li));
        ++pos;
    } while (mask);
}

template <typename T, typename SH, int U>
__device__ __forceinline__ void scan_any(RowsLds<SH> &L, const v4i (&raw)[U], int64_t g0, int64_t n, float tau,
                                         bool &nan, int64_t ibase)
{
    if (n - g0 >= (int64_t)(SH::nt * U * (16 / sizeof(T)))) scan_group<T, SH, U, false>(L, raw, g0, n, tau, nan, ibase);
    else scan_group<T, SH, U, true>(L, raw, g0, n, tau, nan, ibase);
}

// Gathers every valid entry >= tau (as raw candidates, their positions
// offset by ibase) into L.cand, the first SH::cap of them, and returns how
// many there are.  `a` holds the row's first group, already loaded.  Two
// register sets alternate, so one group is in flight while the other is
// scanned.
template <typename T, typename SH, int U>
__device__ uint32_t rows_gather(RowsLds<SH> &L, v4i (&a)[U], const T *row, int64_t n, float tau, bool &nan,
                                int64_t ibase = 0)
{
    constexpr int64_t G = (int64_t)SH::nt * U * (16 / sizeof(T));
    if (threadIdx.x == 0) L.misc[3] = 0u;
    __syncthreads();
    v4i b[U];
    for (int64_t g0 = 0; g0 < n; g0 += 2 * G) {
        load_group<T, SH::nt, U>(b, row, n, g0 + G);
        __builtin_amdgcn_sched_barrier(0);  // the loads go out before the scan
        scan_any<T, SH, U>(L, a, g0, n, tau, nan, ibase);
        if (g0 + G >= n) break;  // block-uniform
        load_group<T, SH::nt, U>(a, row, n, g0 + 2 * G);
        __builtin_amdgcn_sched_barrier(0);
        scan_any<T, SH, U>(L, b, g0 + G, n, tau, nan, ibase);
    }
    __syncthreads();
    const uint32_t cnt = L.misc[3];
    __syncthreads();
    return cnt;
}

// Visits a row's first n entries as (value, position, valid), every thread
// of the block the same number of times, with the loads of the next group in
// flight while a group is visited (as in rows_gather).
template <typename T, int NT, typename F>
__device__ __forceinline__ void visit_row(const T *row, int64_t n, F f)
{
    constexpr int V = 16 / sizeof(T), U = kRowsUnroll;
    constexpr int64_t G = (int64_t)NT * U * V;
    auto visit = [&](const v4i (&raw)[U], int64_t g0) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t base = g0 + ((int64_t)u * NT + threadIdx.x) * V;
            const T *e = reinterpret_cast<const T *>(&raw[u]);
#pragma unroll
            for (int j = 0; j < V; ++j) f(entry_value<T>(e[j]), base + j, base + j < n);
        }
    };
    v4i a[U], b[U];
    load_group<T, NT, U>(a, row, n, 0);
    for (int64_t g0 = 0; g0 < n; g0 += 2 * G) {
        load_group<T, NT, U>(b, row, n, g0 + G);
        __builtin_amdgcn_sched_barrier(0);
        visit(a, g0);
        if (g0 + G >= n) break;  // block-uniform
        load_group<T, NT, U>(a, row, n, g0 + 2 * G);
        __builtin_amdgcn_sched_barrier(0);
        visit(b, g0 + G);
    }
}

// A row of materialized scores as an element visitor of the candidate
// selection (streamed: every visit reads the row again).
template <typename T>
struct RowStream {
    static constexpr bool REG = false;
    static constexpr int kRegPer = 1;
    const T *row;
    int64_t n;
    template <typename F>
    __device__ __forceinline__ void each(F f) const
    {
        const int64_t rounds = (n + blockDim.x - 1) / blockDim.x;
        for (int64_t q = 0; q < rounds; ++q) {
            const int64_t i = threadIdx.x + q * blockDim.x;
            f(i < n ? raw_cand(entry_value<T>(row[i]), (int32_t)i) : 0ull, i < n);
        }
    }
};

// Fallback: boundary digit of the k-th value by a full histogram, then the
// entries of that digit or above.  Returns how many were gathered into
// L.cand, or a count above SH::cap when they do not fit.
template <typename T, typename SH>
__device__ uint32_t rows_digit_gather(RowsLds<SH> &L, const T *row, int64_t n, uint32_t k, bool &nan)
{
    constexpr int NT = SH::nt, BPT = kRowsBuckets / NT;
    const int tid = threadIdx.x, lane = tid & 63;
    for (int i = tid; i < kRowsBuckets; i += NT) L.hist[i] = 0u;
    __syncthreads();
    visit_row<T, NT>(row, n, [&](float v, int64_t, bool valid) {
        nan |= valid && v != v;
        const uint32_t d = ord_of(v) >> kRowsDigitShift;
        // Lanes sharing the first active lane's digit add once (rows crowd
        // into few digits).
        const uint64_t act = __ballot(valid);
        if (act) {
            const int leader = __builtin_ctzll(act);
            const uint32_t ld = __shfl(d, leader);
            const bool same = valid && d == ld;
            const uint64_t sm = __ballot(same);
            if (lane == leader) atomicAdd(&L.hist[ld], (uint32_t)__builtin_popcountll(sm));
            if (valid && !same) atomicAdd(&L.hist[d], 1u);
        }
    });
    __syncthreads();
    // Thread t owns digits 4095 - BPT t ... 4096 - BPT (t + 1), highest first.
    uint32_t c[BPT];
#pragma unroll
    for (int q = 0; q < BPT; ++q) c[q] = L.hist[kRowsBuckets - 1 - (BPT * tid + q)];
    uint32_t above = block_prefix<NT, BPT>(c, L.redu);
#pragma unroll
    for (int q = 0; q < BPT; ++q) {
        if (above < k && k <= above + c[q]) {
            L.misc[0] = (uint32_t)(kRowsBuckets - 1 - (BPT * tid + q));
            L.misc[1] = above + c[q];
        }
        above += c[q];
    }
    if (tid == 0) L.misc[3] = 0u;
    __syncthreads();
    const uint32_t bd = L.misc[0];
    const uint32_t m = L.misc[1];
    if (m > (uint32_t)SH::cap) return m;
    visit_row<T, NT>(row, n, [&](float v, int64_t i, bool valid) {
        const bool keep = valid && (ord_of(v) >> kRowsDigitShift) >= bd;
        const uint64_t bal = __ballot(keep);
        if (bal) {
            uint32_t base = 0;
            if (lane == 0) base = atomicAdd(&L.misc[3], (uint32_t)__builtin_popcountll(bal));
            base = __shfl(base, 0);
            if (keep) L.cand[base + __builtin_popcountll(bal & ((1ull << lane) - 1ull))] = raw_cand(v, (int32_t)i);
        }
    });
    __syncthreads();
    return m;
}

// Thresholds of many rows ahead of the row kernel, one wave per row: the
// same sample and bucket rule as rows_sample_tau, computed by a wave with the
// whole sample in registers (8 chunks per lane) and a private LDS histogram.
// The threshold's bits go to the row's first output index slot.  Rows of at
// most SH::cap entries take every entry and need none.
constexpr int kRowsTauWaves = 4;

template <typename T, typename SH>
__global__ __launch_bounds__(64 * kRowsTauWaves) void k_rows_tau(RowsArgs a)
{
    constexpr int V = 16 / sizeof(T), C = kRowsSampleRuns * 8 / 64, PER = kRowsTauBuckets / 64;
    __shared__ uint32_t s_hist[kRowsTauWaves][kRowsTauBuckets];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t r = (int64_t)blockIdx.x * kRowsTauWaves + wave;
    if (r >= a.rows) return;  // wave-uniform; no block barrier follows
    const RowPlace pl = row_place(a, r);
    if (!pl.present) return;
    const int64_t n = pl.n;
    const uint32_t k = (uint32_t)min((int64_t)a.topk, n);
    if (n <= SH::cap || k == 0) return;
    const T *row = reinterpret_cast<const T *>(a.x) + r * a.stride;
    uint32_t *hist = s_hist[wave];
    v4i raw[C];
#pragma unroll
    for (int c = 0; c < C; ++c) raw[c] = sample_load(row, n, lane + 64 * c);
    uint32_t hic = 0, nloc = 0, ns = 0;
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const int64_t base = sample_base<T>(n, lane + 64 * c);
        const T *e = reinterpret_cast<const T *>(&raw[c]);
#pragma unroll
        for (int j = 0; j < V; ++j) {
            const float v = entry_value<T>(e[j]);
            const bool ok = base >= 0 && base + j < n;
            ns += ok ? 1u : 0u;
            if (ok && __builtin_isfinite(v)) {
                const uint32_t cd = ord_of(v);
                hic = max(hic, cd);
                nloc = max(nloc, ~cd);
            }
        }
    }
    hic = wave_max(hic);
    nloc = wave_max(nloc);
    ns = wave_sum(ns);
    const bool any = hic != 0u;
    const float lo = float_of_ord(~nloc), hi = float_of_ord(hic);
    const float scale = (float)kRowsTauBuckets / (hi - lo);
    float tau;
    if (!(any && hi > lo && __builtin_isfinite(scale) && scale > 0.0f)) {
        tau = any && !(hi > lo) ? lo : -__builtin_inff();
    } else {
        const uint32_t rk = (uint32_t)min(max(ceil((double)rows_target(k, SH::cap, ns, n) * (double)ns / (double)n), 1.0),
                                          (double)ns);
#pragma unroll
        for (int q = 0; q < PER; ++q) hist[lane + 64 * q] = 0u;
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the zeros land before any lane adds
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int c = 0; c < C; ++c) {
            const int64_t base = sample_base<T>(n, lane + 64 * c);
            const T *e = reinterpret_cast<const T *>(&raw[c]);
#pragma unroll
            for (int j = 0; j < V; ++j) {
                const float v = entry_value<T>(e[j]);
                if (base >= 0 && base + j < n) {
                    const float x = (hi - v) * scale;
                    const uint32_t b = v == __builtin_inff() ? 0u
                                       : (x < (float)(kRowsTauBuckets - 1) ? (uint32_t)fmaxf(x, 0.0f)
                                                                           : (uint32_t)(kRowsTauBuckets - 1));
                    atomicAdd(&hist[b], 1u);
                }
            }
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);
        __builtin_amdgcn_wave_barrier();
        // Lane l owns buckets [PER l, PER l + PER), largest scores first.
        uint32_t cnt[PER], run = 0;
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            cnt[q] = hist[lane * PER + q];
            run += cnt[q];
        }
        uint32_t basec = wave_incl_add(run) - run;
        int b = -1;
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            if (basec < rk && rk <= basec + cnt[q]) b = lane * PER + q;
            basec += cnt[q];
        }
        const uint64_t hit = __ballot(b >= 0);
        b = __shfl(b, hit ? __builtin_ctzll(hit) : 0);
        tau = hi - (float)(b + 2) / scale;
    }
    if (lane == 0) *(int32_t *)out_row(a.out_idx, pl.out, a.topk, a.out_flags) = __float_as_int(tau);
}

// One workgroup per row.  With PRE_TAU the row's threshold was computed by
// k_rows_tau and parked in the first 4 bytes of the row's output indices
// (the outputs are written last); otherwise the workgroup reads the sample itself, with
// its first group of the row already in flight.
// Rows present in the call: all of them, or for rows mapped through the
// flagged-row list, those below its device-side length.
__device__ __forceinline__ int64_t rows_present(const RowsArgs &a)
{
    if (a.ks && a.rowmap) return min(a.rows, max((int64_t)*a.nrows - a.row_base, (int64_t)0));
    return a.rows;
}

// One workgroup per row; with LOOP the workgroups loop over the rows
// (grid-stride), so a batch of flagged rows whose count only the device
// knows costs one launch of at most the resident workgroups (the one-row
// form keeps the register allocation of the plain body).
template <typename T, typename SH, bool PRE_TAU, bool LOOP = false>
__global__ __launch_bounds__(SH::nt) __attribute__((amdgpu_waves_per_eu(LOOP ? 4 : 8))) void k_topk_rows(RowsArgs a)
{
    constexpr int NT = SH::nt, U = kRowsUnroll;
    __shared__ RowsLds<SH> L;
    const int tid = threadIdx.x;
    const int64_t nrow = LOOP ? rows_present(a) : a.rows;
    for (int64_t r = blockIdx.x; r < nrow; r += gridDim.x) {
    auto body = [&]() {
    const RowPlace pl = row_place(a, r);
    if (!pl.present) return;  // block-uniform
    const T *row = reinterpret_cast<const T *>(a.x) + r * a.stride;
    const int64_t n = pl.n;
    const uint32_t k = (uint32_t)min((int64_t)a.topk, n);
    void *oi = out_row(a.out_idx, pl.out, a.topk, a.out_flags);
    float *ov = a.out_val ? a.out_val + pl.out * a.topk : nullptr;
    if (k == 0) {
        for (int j = tid; j < a.topk; j += NT) {
            if (a.out_flags & kOutInt64) ((int64_t *)oi)[j] = -1;
            else ((int32_t *)oi)[j] = -1;
            if (ov) ov[j] = -__builtin_inff();
        }
        return;
    }
    bool nan = false;
    float tau = -__builtin_inff();
    if (PRE_TAU && n > SH::cap) tau = __int_as_float(__builtin_amdgcn_readfirstlane(*(const int32_t *)oi));
    v4i first[U];
    load_group<T, NT, U>(first, row, n, 0);  // in flight while the sample is read
    if (!PRE_TAU && n > SH::cap) {
        const v4i smp = sample_load(row, n, tid);
        tau = rows_sample_tau<T, SH>(L, smp, n, k);
    }
    uint32_t m = rows_gather<T, SH, U>(L, first, row, n, tau, nan);
    if (m < k || m > (uint32_t)SH::cap) m = rows_digit_gather<T, SH>(L, row, n, k, nan);
    if (a.nan_flag && __any(nan) && (tid & 63) == 0) atomicOr(a.nan_flag, 1);
    if (m <= (uint32_t)SH::cap) {
        RowElems<SH::regs> el;
        el.load(L.cand, m);
        __syncthreads();  // the gathered entries are in registers; the LDS becomes the selection's
        select_core<NT, SH::nbkt, SH::maxk>(L.sel, el, m, k, a.topk, oi, ov, a.out_flags, pl.base);
    } else {
        RowStream<T> el{row, n};
        select_core<NT, SH::nbkt, SH::maxk>(L.sel, el, n, k, a.topk, oi, ov, a.out_flags, pl.base);
    }
    };  // body
    body();
    if (!LOOP) break;
    __syncthreads();  // the next row reuses the LDS
    }
}

// ---------------------------------------------------------------------------
// Rows split over several workgroups (few rows: each row's latency-bound
// stream is shared out), in two launches.  k_topk_rows_part: workgroup (row
// r, part p) computes the row's threshold from the whole row's sample (every
// part gets the same value), gathers the entries of its slice that reach it
// and appends them to the row's candidate list in global memory.
// k_topk_rows_merge: one workgroup per row selects from the list, or, when
// the parts together kept fewer than k or more than the capacity, redoes the
// row alone by the digit histogram; it then clears the row's state, so the
// state reads zero between calls.  The launch boundary orders the parts'
// writes before the merge's reads (no fence inside either kernel: a
// device-scope fence writes back and invalidates the L2, which is slow when
// hundreds of workgroups do it).
struct RowsSplit {
    uint32_t *cnt;     // [rows] candidates appended
    uint32_t *over;    // [rows] a part held more than it could keep
    uint64_t *cand;    // [rows, cap] the row's candidates
    int parts;         // workgroups per row
};

template <typename T, typename SH>
__global__ __launch_bounds__(SH::nt) __attribute__((amdgpu_waves_per_eu(8))) void k_topk_rows_part(RowsArgs a,
                                                                                                  RowsSplit sp)
{
    constexpr int NT = SH::nt, U = kRowsUnroll, V = 16 / sizeof(T), CAP = SH::cap;
    __shared__ RowsLds<SH> L;
    __shared__ uint32_t s_base;
    const int tid = threadIdx.x;
    const int64_t r = blockIdx.x / sp.parts;
    const int part = (int)(blockIdx.x - r * sp.parts);
    const RowPlace pl = row_place(a, r);
    if (!pl.present) return;  // block-uniform
    const T *row = reinterpret_cast<const T *>(a.x) + r * a.stride;
    const int64_t n = pl.n;
    const uint32_t k = (uint32_t)min((int64_t)a.topk, n);
    if (k == 0) return;
    // This part's slice: whole 16-byte chunks.
    const int64_t per = ((n + sp.parts - 1) / sp.parts + V - 1) / V * V;
    const int64_t s0 = min((int64_t)part * per, n), s1 = min(s0 + per, n);
    bool nan = false;
    float tau = -__builtin_inff();
    v4i first[U];
    load_group<T, NT, U>(first, row + s0, s1 - s0, 0);  // in flight while the sample is read
    if (n > CAP) {
        const v4i smp = sample_load(row, n, tid);
        tau = rows_sample_tau<T, SH>(L, smp, n, k);
    }
    const uint32_t m = rows_gather<T, SH, U>(L, first, row + s0, s1 - s0, tau, nan, s0);
    if (a.nan_flag && __any(nan) && (tid & 63) == 0) atomicOr(a.nan_flag, 1);
    if (tid == 0) {
        if (m > (uint32_t)CAP) {
            atomicOr(sp.over + r, 1u);
            s_base = (uint32_t)CAP;
        } else {
            s_base = m ? atomicAdd(sp.cnt + r, m) : 0u;
        }
    }
    __syncthreads();
    const uint32_t base = s_base;
    if (m <= (uint32_t)CAP)
        for (uint32_t i = tid; i < m; i += NT)
            if (base + i < (uint32_t)CAP) sp.cand[r * CAP + base + i] = L.cand[i];
}

// One workgroup per row and few rows: occupancy does not matter, so the
// merge keeps its registers (no spill to scratch).
template <typename T, typename SH>
__global__ __launch_bounds__(SH::nt) __attribute__((amdgpu_waves_per_eu(SH::nt / 256))) void k_topk_rows_merge(RowsArgs a,
                                                                                                   RowsSplit sp)
{
    constexpr int NT = SH::nt, CAP = SH::cap;
    __shared__ RowsLds<SH> L;
    const int tid = threadIdx.x;
    const int64_t r = blockIdx.x;
    const RowPlace pl = row_place(a, r);
    if (!pl.present) return;  // block-uniform
    const T *row = reinterpret_cast<const T *>(a.x) + r * a.stride;
    const int64_t n = pl.n;
    const uint32_t k = (uint32_t)min((int64_t)a.topk, n);
    void *oi = out_row(a.out_idx, pl.out, a.topk, a.out_flags);
    float *ov = a.out_val ? a.out_val + pl.out * a.topk : nullptr;
    const uint32_t tot = sp.cnt[r], over = sp.over[r];
    __syncthreads();  // every thread has read the state before it is cleared
    if (tid == 0) {
        sp.cnt[r] = 0u;
        sp.over[r] = 0u;
    }
    if (k == 0) {
        for (int j = tid; j < a.topk; j += NT) {
            if (a.out_flags & kOutInt64) ((int64_t *)oi)[j] = -1;
            else ((int32_t *)oi)[j] = -1;
            if (ov) ov[j] = -__builtin_inff();
        }
        return;
    }
    if (!over && tot >= k && tot <= (uint32_t)CAP) {
        RowElems<SH::regs> el;
        el.load(sp.cand + r * CAP, tot);
        select_core<NT, SH::nbkt, SH::maxk>(L.sel, el, tot, k, a.topk, oi, ov, a.out_flags, pl.base);
    } else {
        bool nan = false;  // the parts have reported NaN already
        const uint32_t m = rows_digit_gather<T, SH>(L, row, n, k, nan);
        if (m <= (uint32_t)CAP) {
            RowElems<SH::regs> el;
            el.load(L.cand, m);
            __syncthreads();
            select_core<NT, SH::nbkt, SH::maxk>(L.sel, el, m, k, a.topk, oi, ov, a.out_flags, pl.base);
        } else {
            RowStream<T> el{row, n};
            select_core<NT, SH::nbkt, SH::maxk>(L.sel, el, n, k, a.topk, oi, ov, a.out_flags, pl.base);
        }
    }
}

}  // namespace ftk
