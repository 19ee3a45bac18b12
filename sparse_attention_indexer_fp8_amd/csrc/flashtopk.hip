// C ABI of the fused indexer top-k library (declared in include/flashtopk.h).
//
// Two call sequences, both entirely on the caller's stream and neither
// waiting on the host:
//
// Fused path (FlashTopK README, "Highlights": a per-row threshold from a
// strided sample of the row's own window, candidates, exact selection; rows
// the threshold misjudges are rescored):
//   0. k_prep           per-key scale factors (+ block extremes for the bound)
//                       and (FP8) head-weighted query sums split into FP8
//                       parts, in one launch; clears the call's counters
//   1. k_score<sample>  strided-sample scores of every long row     (MFMA);
//                       with one workgroup per tile and at most one round
//                       of workgroups it also sets the tile's per-row
//                       thresholds from those samples
//   2. k_tau            the thresholds otherwise (several workgroups per
//                       tile, or more tiles than compute units)
//   3. k_score<filter>  fused score (+ bound) + threshold filter -> candidates (MFMA, hot)
//   4. k_select         triage (flagged rows go to a list on the device) and
//                       the exact top-k of every other row
//   5. recovery         k_score<dense> + k_topk_rows over the flagged rows, in
//                       batches whose scratch fits the budget; launched
//                       without knowing how many rows were flagged (batch
//                       rows past the list's device-side length exit)
//
// Dense path (calls of few rows, and the forced recover-all path): every
// row's window scores are materialised (k_score_dec for at most 4 rows,
// otherwise k_score<dense>; both compute their own query sums and scale
// factors) and the row top-k kernels select from them;
// with few rows each row is split over several workgroups.
//
// Both paths score a (row, key) pair with the same instruction sequence, so
// a row's results do not depend on the path or on the other rows of the
// call.  Outputs are complete when the stream reaches the end of the call's
// work.  The counts of flashtopk_info are computed on the host, from each
// row's window length and candidate count, when the record is read.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <vector>

#include "flashtopk.h"
#include "ftk_bound.hpp"
#include "ftk_dec.hpp"
#include "ftk_paged.hpp"
#include "ftk_probe.hpp"
#include "ftk_rows.hpp"
#include "ftk_score.hpp"
#include "ftk_select.hpp"
#include "ftk_tau.hpp"
#include "ftk_validate.hpp"

using namespace ftk;

namespace {

constexpr int kMaxCap = 16384;
constexpr int kDefaultSampleTarget = 2048;
constexpr int64_t kDefaultRecoverBudget = int64_t(2) << 30;
// The auto path scores every row densely when the call's (row, key) pairs
// are at most this many: materialising the scores then costs less than the
// fused path's fixed passes (preparation, sample, thresholds, selection).
constexpr int64_t kDensePairs = int64_t(8) << 20;
// Smallest key chunk of a dense-mode work item.
constexpr int kMinDenseChunk = 512;
// Split-row top-k: at most this many workgroups per row, each streaming at
// least kMinSplitEntries entries.
constexpr int kMaxSplit = 64;
constexpr int64_t kMinSplitEntries = 4096;

// Grow-only device buffer.  zero: it must read zero when handed to a call
// (recorded by the sizing pass of the allocation-free entry point).
struct DevBuf {
    void *ptr = nullptr;
    size_t bytes = 0;
    bool zero = false;
};

// Record of the last call on a stream; its counts are computed from the
// workspace's device arrays when flashtopk_get_last_info reads it.
enum CallKind { kCallNone = 0, kCallFailed, kCallFused, kCallDense };

struct Workspace {
    int device = -1;
    hipStream_t stream = nullptr;
    std::mutex mu;  // held while a call is enqueued or its record read
    DevBuf tau, cnt, rowlist, stats, wlen, cand, samp, scratch, qbar, qscale, sigh;
    DevBuf kb, kmeta, vplan, q1;                 // score-bound pruning
    DevBuf scnt, sover, scand;                   // split-row top-k (counters read zero between calls)
    DevBuf pkv, psig;                            // keys and scales gathered from a paged cache
    DevBuf vflag;                                // precondition flags (options.validate)
    unsigned *host_flag = nullptr;               // pinned: the precondition flags
    hipEvent_t ev[7] = {};                       // phase boundaries when profiling
    int last_kind = kCallNone;
    flashtopk_info last{};                       // status, sizes, timings of the last call
    int last_topk = 0;
    // The allocation-free entry point's workspace: first a sizing pass
    // (ensure records the sizes a call needs), then the buffers are carved
    // from a fixed array and ensure only checks them.
    bool sizing = false;
    bool fixed = false;
};

std::mutex g_mu;
std::vector<Workspace *> g_ws;

// Scratch of the allocation-free entry point.  In host code `scratch` only
// names the symbol: its device address comes from hipGetSymbolAddress, once
// per device (each device holds its own copy).
constexpr size_t kNoAllocBytes = (size_t)FLASHTOPK_NOALLOC_SCRATCH_BYTES;
constexpr int64_t kNoAllocRecoverBudget = int64_t(32) << 20;
constexpr int kNoAllocMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[kNoAllocBytes];

struct NoAllocDevice {
    std::mutex mu;       // held for the whole call: calls from several host threads take turns
    uint8_t *base = nullptr;  // the device address of `scratch`
    Workspace ws;        // buffers carved from it
};
NoAllocDevice g_na[kNoAllocMaxDevices];

int hip_status(hipError_t e)
{
    if (e == hipSuccess) return FLASHTOPK_OK;
    if (e == hipErrorOutOfMemory) return FLASHTOPK_ERR_OUT_OF_MEMORY;
    return FLASHTOPK_ERR_HIP;
}

// Ensures `b` holds at least `bytes`; on growth the stream is drained first so
// no pending kernel still uses the old buffer.
int ensure(Workspace &w, DevBuf &b, size_t bytes)
{
    if (w.sizing) {
        b.bytes = std::max(b.bytes, bytes);
        return FLASHTOPK_OK;
    }
    if (b.bytes >= bytes && b.ptr) return FLASHTOPK_OK;
    if (w.fixed) return FLASHTOPK_ERR_WORKSPACE_LIMIT;
    size_t want = std::max(bytes, b.bytes + b.bytes / 4);
    if (b.ptr) {
        hipError_t e = hipStreamSynchronize(w.stream);
        if (e != hipSuccess) return hip_status(e);
        (void)hipFree(b.ptr);
        b.ptr = nullptr;
        b.bytes = 0;
    }
    hipError_t e = hipMalloc(&b.ptr, std::max<size_t>(want, 256));
    if (e != hipSuccess) {
        (void)hipGetLastError();
        b.ptr = nullptr;
        return hip_status(e);
    }
    b.bytes = std::max<size_t>(want, 256);
    return FLASHTOPK_OK;
}

// ensure() for a buffer that must read zero when (re)allocated.
int ensure_zeroed(Workspace &w, DevBuf &b, size_t bytes)
{
    if (w.sizing) b.zero = true;
    if (w.sizing || w.fixed || (b.bytes >= bytes && b.ptr)) return ensure(w, b, bytes);
    int st = ensure(w, b, bytes);
    if (st) return st;
    return hip_status(hipMemset(b.ptr, 0, b.bytes));
}

Workspace *get_ws(hipStream_t stream, int *status)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        *status = hip_status(e);
        return nullptr;
    }
    std::lock_guard<std::mutex> lk(g_mu);
    for (Workspace *w : g_ws)
        if (w->device == dev && w->stream == stream) return w;
    Workspace *w = new Workspace();
    w->device = dev;
    w->stream = stream;
    e = hipHostMalloc((void **)&w->host_flag, sizeof(unsigned), hipHostMallocDefault);
    if (e != hipSuccess) {
        delete w;
        *status = hip_status(e);
        return nullptr;
    }
    g_ws.push_back(w);
    return w;
}

struct Plan {
    int validate = 0;     // options.validate
    unsigned invalid = 0; // the flags it found
    int64_t T, S;
    int dtype, topk, cap, sample_target, sample_min_stride, path;
    float rank_scale;
    int64_t recover_budget;
    int profile;
    int out_flags;
    int heads;  // 32, or 64 (each row's halves are a pair of tile columns)
    // keys in a paged cache, read in place (dense path)
    const int32_t *table = nullptr;
    int page_size = 0;
    int64_t num_pages = 0;
};

int resolve(Plan &p, const flashtopk_options *opt)
{
    p.path = opt ? opt->path : FLASHTOPK_PATH_AUTO;
    if (p.path < FLASHTOPK_PATH_AUTO || p.path > FLASHTOPK_PATH_FUSED) return FLASHTOPK_ERR_INVALID_ARGUMENT;
    int cap = (opt && opt->cand_capacity > 0) ? opt->cand_capacity : std::min(kMaxCap, 4 * p.topk);
    p.cap = std::min(kMaxCap, std::max(cap, p.topk));
    p.sample_target = (opt && opt->sample_target > 0) ? std::min(opt->sample_target, (int)kTauBuckets)
                                                       : kDefaultSampleTarget;
    // The threshold is the r-th largest sample score with r about 2 topk / d
    // for stride d; r >= 64 (relative spread of the admitted count about
    // 1/8) is enough, so the stride need not go below topk / 32.
    p.sample_min_stride = 1;
    while (p.sample_min_stride * 2 <= p.topk / 32) p.sample_min_stride *= 2;
    p.rank_scale = (opt && opt->sample_rank_scale > 0.0f) ? opt->sample_rank_scale : 1.0f;
    p.out_flags = opt ? opt->out_flags : 0;
    p.heads = (opt && opt->heads) ? opt->heads : FLASHTOPK_HEADS;
    if (p.heads != 32 && p.heads != 64) return FLASHTOPK_ERR_INVALID_ARGUMENT;
    if (p.out_flags & ~(FLASHTOPK_OUT_INDEX_ORDER | FLASHTOPK_OUT_INT64)) return FLASHTOPK_ERR_INVALID_ARGUMENT;
    p.recover_budget = (opt && opt->recover_budget_bytes > 0) ? opt->recover_budget_bytes : kDefaultRecoverBudget;
    p.profile = (opt && opt->profile) ? 1 : 0;
    p.validate = (opt && opt->validate) ? 1 : 0;
    return FLASHTOPK_OK;
}

// Compute units of the current device (queried once).
int num_cu()
{
    static int n_cu = 0;
    if (n_cu == 0) {
        int dev = 0;
        hipDeviceProp_t prop{};
        if (hipGetDevice(&dev) == hipSuccess && hipGetDeviceProperties(&prop, dev) == hipSuccess)
            n_cu = std::max(1, prop.multiProcessorCount);
        else
            n_cu = 256;
    }
    return n_cu;
}

// Keys per work item (a power of two in [min_chunk, kMaxChunk]), from a cost
// model: a work item takes a whole compute unit (its LDS), so items run in
// rounds of one per CU, and an item costs a fixed part (setting up and
// staging the q tile, flushing candidates: about one wave step) plus the wave
// steps of each of its `waves` waves.  The chunk of least cost wins, the
// larger one on a tie: large chunks amortise the fixed part, small ones fill
// the GPU when the call has few tiles.
int chunk_keys(int ntiles, int64_t S, int waves, int min_chunk = kMinChunk)
{
    const int64_t n_cu = num_cu();
    int best = kMaxChunk;
    int64_t best_cost = INT64_MAX;
    for (int chunk = kMaxChunk; chunk >= min_chunk; chunk >>= 1) {
        const int64_t items = (int64_t)ntiles * ((S + chunk - 1) / chunk);
        const int64_t rounds = (items + n_cu - 1) / n_cu;
        // in 1 / waves of a wave step (the fixed part is `waves` of them):
        // an item's steps count exactly, not rounded up to whole steps per
        // wave, so of two chunks that both give each wave at most one step
        // the smaller one, on twice the compute units, wins
        const int64_t cost = rounds * (waves + chunk / kStepKeys);
        if (cost < best_cost) {
            best_cost = cost;
            best = chunk;
        }
    }
    return best;
}

// Workgroups per tile for the sample scores: with few tiles (decode-sized
// calls) each tile's lattice is split so the pass still spreads over the GPU.
int sample_split(int ntiles)
{
    int split = 1;
    while (split < 16 && (int64_t)ntiles * split * 2 <= num_cu()) split <<= 1;
    return split;
}

// Workgroups per row of the row top-k: rows that leave most compute units
// idle are split so the GPU streams them with about two workgroups per CU.
int split_parts(int64_t rows, int64_t cols)
{
    int parts = 1;
    while (parts < kMaxSplit && rows * parts * 2 <= 2 * (int64_t)num_cu() &&
           cols / (parts * 2) >= kMinSplitEntries)
        parts <<= 1;
    return parts;
}

// kModeDenseLoop: dense mode with workgroups looping over the work items.
constexpr int kModeDenseLoop = 3;

template <int DT>
void launch_score(int mode, dim3 grid, hipStream_t st, const ScoreArgs &a)
{
    constexpr int WD = 64 * ScoreCfg<DT, kModeDense>::waves, WL = 64 * ScoreCfg<DT, kModeDense, true>::waves;
    if (a.pair) {
        if (mode == kModeFilter) k_score<DT, kModeFilter, true><<<grid, 64 * ScoreCfg<DT, kModeFilter>::waves, 0, st>>>(a);
        else if (mode == kModeSample) k_score<DT, kModeSample, true><<<grid, 64 * ScoreCfg<DT, kModeSample>::waves, 0, st>>>(a);
        else if (mode == kModeDense) k_score<DT, kModeDense, true><<<grid, WD, 0, st>>>(a);
        else k_score<DT, kModeDense, true, true><<<grid, WL, 0, st>>>(a);
    } else {
        if (mode == kModeFilter) k_score<DT, kModeFilter, false><<<grid, 64 * ScoreCfg<DT, kModeFilter>::waves, 0, st>>>(a);
        else if (mode == kModeSample) k_score<DT, kModeSample, false><<<grid, 64 * ScoreCfg<DT, kModeSample>::waves, 0, st>>>(a);
        else if (mode == kModeDense) k_score<DT, kModeDense, false><<<grid, WD, 0, st>>>(a);
        else k_score<DT, kModeDense, false, true><<<grid, WL, 0, st>>>(a);
    }
}

template <typename SH>
void launch_select(int64_t blocks, hipStream_t st, const SelectArgs &a)
{
    k_select<SH><<<dim3((unsigned)blocks), SH::nt, 0, st>>>(a);
}

void launch_score_dt(int dtype, int mode, dim3 grid, hipStream_t st, const ScoreArgs &a)
{
    if (dtype == FLASHTOPK_FP8_E4M3) launch_score<kFP8>(mode, grid, st, a);
    else launch_score<kBF16>(mode, grid, st, a);
}

// Phase boundary i of a profiled call (no-op otherwise).
void mark(Workspace &w, const Plan &p, int i, hipStream_t stream)
{
    if (!p.profile) return;
    if (!w.ev[i]) (void)hipEventCreate(&w.ev[i]);
    (void)hipEventRecord(w.ev[i], stream);
}

float phase_ms(Workspace &w, const Plan &p, int i, int j)
{
    float ms = 0.0f;
    if (p.profile && w.ev[i] && w.ev[j] && hipEventElapsedTime(&ms, w.ev[i], w.ev[j]) != hipSuccess) {
        (void)hipGetLastError();
        ms = 0.0f;
    }
    return ms;
}

// Row top-k launch.  Few rows are split over several workgroups each (split
// non-null, split->parts > 1); with more rows than resident workgroups and
// pre_tau, the thresholds are computed up front by k_rows_tau, so that no
// row workgroup waits on its sample.
template <typename T, typename SH>
void launch_rows(const RowsArgs &a, hipStream_t s, bool pre_tau, const RowsSplit *split)
{
    if (split && split->parts > 1) {
        hipLaunchKernelGGL((k_topk_rows_part<T, SH>), dim3((unsigned)(a.rows * split->parts)), dim3(SH::nt), 0, s, a,
                           *split);
        hipLaunchKernelGGL((k_topk_rows_merge<T, SH>), dim3((unsigned)a.rows), dim3(SH::nt), 0, s, a, *split);
        return;
    }
    static int per_cu = 0;
    if (per_cu == 0) {
        int b = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, k_topk_rows<T, SH, true>, SH::nt, 0) != hipSuccess ||
            b < 1)
            b = 1;
        per_cu = b;
    }
    const int64_t resident = (int64_t)per_cu * num_cu();
    if (a.rowmap) {
        // flagged rows, counted on the device: the rows loop over at most the
        // resident workgroups
        hipLaunchKernelGGL((k_topk_rows<T, SH, false, true>), dim3((unsigned)std::min(a.rows, resident)),
                           dim3(SH::nt), 0, s, a);
    } else if (pre_tau && a.rows > resident) {
        const dim3 tgrid((unsigned)((a.rows + kRowsTauWaves - 1) / kRowsTauWaves));
        hipLaunchKernelGGL((k_rows_tau<T, SH>), tgrid, dim3(64 * kRowsTauWaves), 0, s, a);
        hipLaunchKernelGGL((k_topk_rows<T, SH, true>), dim3((unsigned)a.rows), dim3(SH::nt), 0, s, a);
    } else {
        hipLaunchKernelGGL((k_topk_rows<T, SH, false>), dim3((unsigned)a.rows), dim3(SH::nt), 0, s, a);
    }
}

template <typename T>
void launch_rows_k(const RowsArgs &a, hipStream_t s, bool pre_tau, const RowsSplit *split)
{
    if (a.topk <= RowsSmall::maxk) launch_rows<T, RowsSmall>(a, s, pre_tau, split);
    else launch_rows<T, RowsLarge>(a, s, pre_tau, split);
}

// Split-row state for `rows` rows of `parts` workgroups each (nothing when
// parts is 1).
int ensure_split(Workspace &w, int64_t rows, int parts, RowsSplit &sp)
{
    sp = RowsSplit{};
    sp.parts = parts;
    if (parts <= 1) return FLASHTOPK_OK;
    int st;
    if ((st = ensure_zeroed(w, w.scnt, sizeof(uint32_t) * (size_t)rows))) return st;
    if ((st = ensure_zeroed(w, w.sover, sizeof(uint32_t) * (size_t)rows))) return st;
    if ((st = ensure(w, w.scand, sizeof(uint64_t) * (size_t)rows * RowsLarge::cap))) return st;
    sp.cnt = (uint32_t *)w.scnt.ptr;
    sp.over = (uint32_t *)w.sover.ptr;
    sp.cand = (uint64_t *)w.scand.ptr;
    return FLASHTOPK_OK;
}

// Scratch rows of float window scores, 16-byte aligned (the row kernels'
// loads), and the rows per recovery / dense batch that fit the budget (a
// multiple of the 16-column tile).
int64_t scratch_stride(int64_t S) { return (std::max<int64_t>(S, 1) + 3) / 4 * 4; }

int64_t batch_rows(const Plan &p)
{
    const int64_t stride = scratch_stride(p.S);
    int64_t rcap = std::max<int64_t>(kTileQ, p.recover_budget / (int64_t)(sizeof(float) * stride));
    rcap = std::min<int64_t>(rcap, (p.T + kTileQ - 1) / kTileQ * kTileQ);
    return (rcap + kTileQ - 1) / kTileQ * kTileQ;
}

void begin_record(Workspace &w, const Plan &p, int kind)
{
    flashtopk_info &info = w.last;
    std::memset(&info, 0, sizeof(info));
    info.status = FLASHTOPK_OK;
    info.rows = p.T;
    info.invalid = (int32_t)p.invalid;
    w.last_kind = kind;
    w.last_topk = p.topk;
}

// Workspace of a dense call.
int prepare_dense(Workspace &w, const Plan &p, RowsSplit &sp)
{
    int st = FLASHTOPK_OK;
    const int64_t rcap = batch_rows(p);
    const int64_t brows = std::min(rcap, p.T);
    if ((st = ensure(w, w.scratch, sizeof(float) * (size_t)rcap * scratch_stride(p.S)))) return st;
    if ((st = ensure(w, w.wlen, sizeof(int32_t) * (size_t)p.T))) return st;
    return ensure_split(w, brows, split_parts(brows, p.S), sp);
}

// Every row scored densely: window scores in scratch, then the row top-k.
int run_dense(Workspace &w, const void *q, const void *kv, const float *kv_scales, const float *weights,
              const int32_t *ks, const int32_t *ke, void *out_idx, float *out_val, hipStream_t stream, const Plan &p)
{
    int st = FLASHTOPK_OK;
    const int64_t T = p.T, S = p.S;
    const int ps = p.heads == 64 ? 1 : 0;
    const int64_t stride = scratch_stride(S);
    const int64_t rcap = batch_rows(p);
    RowsSplit sp;
    if ((st = prepare_dense(w, p, sp))) return st;

    mark(w, p, 0, stream);
    for (int64_t rb = 0; rb < T; rb += rcap) {
        const int64_t nb = std::min(rcap, T - rb);
        ScoreArgs sa{};
        sa.q = (const uint8_t *)q;
        sa.kv = (const uint8_t *)kv;
        sa.sigma = kv_scales;
        sa.w = weights;
        sa.ks = ks;
        sa.ke = ke;
        sa.num_q = (int)(T << ps);
        sa.num_kv = (int)S;
        sa.pair = ps;
        sa.table = p.table;
        sa.page_size = p.page_size;
        sa.num_pages = p.num_pages;
        sa.rowlist = nullptr;
        sa.nrows_direct = (int)T;
        sa.row_base = (int)rb;
        sa.row_limit = (int)nb;
        sa.scratch = (float *)w.scratch.ptr;
        sa.scratch_stride = stride;
        sa.wlen = (int32_t *)w.wlen.ptr;
        sa.own_prep = 1;
        sa.ntiles = (int)(((nb << ps) + kTileQ - 1) / kTileQ);
        sa.chunk = chunk_keys(sa.ntiles, S,
                              p.dtype == FLASHTOPK_FP8_E4M3 ? ScoreCfg<kFP8, kModeDense>::waves
                                                            : ScoreCfg<kBF16, kModeDense>::waves,
                              kMinDenseChunk);
        const int nch = (int)std::max<int64_t>(1, (S + sa.chunk - 1) / sa.chunk);
        if (nb <= kDecRows && !ps && !p.table) {
            // A few rows: their heads on the MFMA's N dimension (same bits).
            const unsigned grid = (unsigned)std::max<int64_t>(1, ((S + kStepKeys - 1) / kStepKeys + kDecWaves - 1) / kDecWaves);
            if (p.dtype == FLASHTOPK_FP8_E4M3) k_score_dec<kFP8><<<grid, 64 * kDecWaves, 0, stream>>>(sa);
            else k_score_dec<kBF16><<<grid, 64 * kDecWaves, 0, stream>>>(sa);
        } else {
            launch_score_dt(p.dtype, kModeDense, dim3((unsigned)(sa.ntiles * nch)), stream, sa);
        }

        RowsArgs ra{};
        ra.x = w.scratch.ptr;
        ra.rows = nb;
        ra.cols = S;
        ra.stride = stride;
        ra.topk = p.topk;
        ra.out_idx = out_idx;
        ra.out_val = out_val;
        ra.out_flags = p.out_flags;
        ra.ks = ks;
        ra.ke = ke;
        ra.row_base = rb;
        ra.rows_total = T;
        launch_rows_k<float>(ra, stream, true, &sp);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_status(e);
    mark(w, p, 1, stream);

    begin_record(w, p, kCallDense);
    w.last.path = FLASHTOPK_PATH_RECOVER;
    w.last.cand_capacity = 0;
    w.last.sample_target = 0;
    if (p.profile) {
        (void)hipEventSynchronize(w.ev[1]);
        w.last.ms_recover = phase_ms(w, p, 0, 1);
    }
    return FLASHTOPK_OK;
}

// Score-bound pruning: on the auto / fused path (each scan work item decides
// from its tile's planner sample) and the forced prune path; not for 64
// heads.
bool bounds_on(const Plan &p) { return p.heads == 32 && p.S > 0 && p.path != FLASHTOPK_PATH_SCAN; }

// Workspace of a fused call.
int prepare_fused(Workspace &w, const Plan &p)
{
    int st = FLASHTOPK_OK;
    const int64_t T = p.T, S = p.S;
    const bool fp8 = p.dtype == FLASHTOPK_FP8_E4M3;
    const int64_t TC = T << (p.heads == 64 ? 1 : 0);
    const int ntiles = (int)((TC + kTileQ - 1) / kTileQ);
    const int nblocks = (int)((S + kBlockKeys - 1) / kBlockKeys);
    if ((st = ensure(w, w.tau, sizeof(float) * T))) return st;
    if ((st = ensure(w, w.cnt, sizeof(uint32_t) * T))) return st;
    if ((st = ensure(w, w.rowlist, sizeof(int32_t) * T))) return st;
    if ((st = ensure(w, w.wlen, sizeof(int32_t) * T))) return st;
    if ((st = ensure(w, w.stats, sizeof(unsigned long long) * kStCount))) return st;
    if (fp8) {
        if ((st = ensure(w, w.qbar, (size_t)TC * kQbarParts * kDim))) return st;
        if ((st = ensure(w, w.qscale, sizeof(float) * TC))) return st;
    }
    if ((st = ensure(w, w.sigh, sizeof(float) * (size_t)(S + 64)))) return st;
    if ((st = ensure(w, w.cand, sizeof(uint64_t) * (size_t)T * p.cap))) return st;
    if ((st = ensure(w, w.samp, sizeof(uint32_t) * (size_t)T * p.sample_target))) return st;
    if (bounds_on(p)) {
        if ((st = ensure(w, w.kb, (size_t)nblocks * 2 * (fp8 ? 128 : 256)))) return st;
        if ((st = ensure(w, w.kmeta, sizeof(float2) * (size_t)nblocks))) return st;
        if ((st = ensure(w, w.vplan, sizeof(float) * (size_t)ntiles * kPlanGroups * 256))) return st;
        if ((st = ensure(w, w.q1, sizeof(float) * (size_t)T))) return st;
    }
    // Recovery batches: rows of scratch that fit the budget.
    return ensure(w, w.scratch, sizeof(float) * (size_t)batch_rows(p) * scratch_stride(S));
}

// The fused path: sampled thresholds, the filtering scan, selection, and
// dense recovery of the rows the threshold misjudged.
int run_fused(Workspace &w, const void *q, const void *kv, const float *kv_scales, const float *weights,
              const int32_t *ks, const int32_t *ke, void *out_idx, float *out_val, hipStream_t stream, const Plan &p)
{
    int st = FLASHTOPK_OK;
    const int64_t T = p.T, S = p.S;
    if ((st = prepare_fused(w, p))) return st;
    const bool fp8 = p.dtype == FLASHTOPK_FP8_E4M3;
    // 64 heads: row t's two 32-head halves are tile columns 2t and 2t + 1.
    const int ps = p.heads == 64 ? 1 : 0;
    const int64_t TC = T << ps;  // tile columns
    const int ntiles = (int)((TC + kTileQ - 1) / kTileQ);
    const bool bounds = bounds_on(p);
    const int nblocks = (int)((S + kBlockKeys - 1) / kBlockKeys);
    const int64_t stride = scratch_stride(S);
    const int64_t rcap = batch_rows(p);

    const int chunk = chunk_keys(ntiles, S, fp8 ? ScoreCfg<kFP8, kModeFilter>::waves : ScoreCfg<kBF16, kModeFilter>::waves);
    const int nchunks = (int)std::max<int64_t>(1, (S + chunk - 1) / chunk);

    ScoreArgs sa{};
    sa.q = (const uint8_t *)q;
    sa.kv = (const uint8_t *)kv;
    sa.sigma = kv_scales;
    sa.sigh = (const float *)w.sigh.ptr;
    sa.w = weights;
    sa.ks = ks;
    sa.ke = ke;
    sa.num_q = (int)TC;
    sa.num_kv = (int)S;
    sa.pair = ps;
    sa.qbar = (const uint8_t *)w.qbar.ptr;
    sa.qscale = (const float *)w.qscale.ptr;
    sa.ntiles = ntiles;
    sa.chunk = chunk;
    sa.cap = p.cap;
    sa.tau = (const float *)w.tau.ptr;
    sa.cnt = (uint32_t *)w.cnt.ptr;
    sa.cand = (uint64_t *)w.cand.ptr;
    sa.samp = (uint32_t *)w.samp.ptr;
    sa.sample_target = p.sample_target;
    sa.sample_min_stride = p.sample_min_stride;
    sa.sample_split = sample_split(ntiles);
    if (bounds) {
        sa.prune = p.path == FLASHTOPK_PATH_PRUNE ? 2 : 1;
        sa.kb = (const uint8_t *)w.kb.ptr;
        sa.meta = (const float2 *)w.kmeta.ptr;
        sa.q1 = (float *)w.q1.ptr;
        sa.nblocks = nblocks;
        sa.vplan = (float *)w.vplan.ptr;
        sa.plan = (unsigned long long *)w.stats.ptr + kStPruned;
    }

    // The sample kernel sets the thresholds itself when each row's samples
    // come from one workgroup per tile and the tiles fit one round of
    // workgroups (the thresholds then add to the one round's span only);
    // with more tiles, k_tau follows it, so that each round of sample
    // workgroups ends without the thresholds on its critical path.
    const bool fused_tau = sa.sample_split == 1 && (int64_t)ntiles * sa.sample_split <= num_cu();
    sa.tau_in_sample = fused_tau ? 1 : 0;
    sa.topk = p.topk;
    sa.rank_scale = p.rank_scale;
    sa.tau_w = (float *)w.tau.ptr;

    mark(w, p, 0, stream);
    {
        // Per-key scale factors (and block extremes for the bound), the
        // statistics cleared, and (FP8) the query sums, in one launch.
        PrepArgs pa{};
        pa.key_blocks = (int)((S + 64 + 4 * kBlockKeys - 1) / (4 * kBlockKeys));
        pa.kv = (const uint8_t *)kv;
        pa.sigma = kv_scales;
        pa.num_kv = (int)S;
        pa.nblocks = nblocks;
        pa.sigh = (float *)w.sigh.ptr;
        pa.bounds = bounds ? 1 : 0;
        pa.kb = bounds ? (uint8_t *)w.kb.ptr : nullptr;
        pa.meta = bounds ? (float2 *)w.kmeta.ptr : nullptr;
        pa.stats = (unsigned long long *)w.stats.ptr;
        pa.nstats = kStCount;
        int64_t qblocks = 0;
        if (fp8) {
            pa.q = (const uint8_t *)q;
            pa.w = weights;
            pa.num_q = TC;
            pa.parts = (uint8_t *)w.qbar.ptr;
            pa.qscale = (float *)w.qscale.ptr;
            pa.q1 = bounds ? (float *)w.q1.ptr : nullptr;
            qblocks = (TC + 3) / 4;
        }
        const unsigned nwg = (unsigned)(pa.key_blocks + qblocks);
        if (fp8) k_prep<kFP8><<<nwg, 256, 0, stream>>>(pa);
        else k_prep<kBF16><<<nwg, 256, 0, stream>>>(pa);
    }
    launch_score_dt(p.dtype, kModeSample, dim3((unsigned)(ntiles * sa.sample_split)), stream, sa);
    mark(w, p, 1, stream);

    if (!fused_tau) {
        TauArgs ta{};
        ta.ks = ks;
        ta.ke = ke;
        ta.num_q = T;
        ta.topk = p.topk;
        ta.cap = p.cap;
        ta.samp = (const uint32_t *)w.samp.ptr;
        ta.sample_target = p.sample_target;
        ta.sample_min_stride = p.sample_min_stride;
        ta.pair = p.heads == 64 ? 1 : 0;
        ta.rank_scale = p.rank_scale;
        ta.tau = (float *)w.tau.ptr;
        ta.cnt = (uint32_t *)w.cnt.ptr;
        k_tau<<<dim3((unsigned)((T + kTauWaves - 1) / kTauWaves)), 64 * kTauWaves, 0, stream>>>(ta);
    }
    mark(w, p, 2, stream);

    launch_score_dt(p.dtype, kModeFilter, dim3((unsigned)(ntiles * nchunks)), stream, sa);
    mark(w, p, 3, stream);

    SelectArgs se{};
    se.ks = ks;
    se.ke = ke;
    se.topk = p.topk;
    se.cap = p.cap;
    se.cnt = (const uint32_t *)w.cnt.ptr;
    se.cand = (const uint64_t *)w.cand.ptr;
    se.out_idx = out_idx;
    se.out_val = out_val;
    se.out_flags = p.out_flags;
    se.wlen = (int32_t *)w.wlen.ptr;
    se.rowlist = (int32_t *)w.rowlist.ptr;
    se.nflagged = (unsigned long long *)w.stats.ptr + kStFlagged;
    if (p.cap <= SelSmallK::nreg * SelSmallK::nt && p.topk <= SelSmallK::maxk) launch_select<SelSmallK>(T, stream, se);
    else if (p.cap <= SelSmall::nreg * SelSmall::nt && p.topk <= SelSmall::maxk) launch_select<SelSmall>(T, stream, se);
    else if (p.cap <= SelMid::nreg * SelMid::nt) launch_select<SelMid>(T, stream, se);
    else if (p.cap <= SelLargeK::nreg * SelLargeK::nt && p.topk <= SelLargeK::maxk) launch_select<SelLargeK>(T, stream, se);
    else if (p.cap <= SelLarge::nreg * SelLarge::nt) launch_select<SelLarge>(T, stream, se);
    else launch_select<SelHuge>(T, stream, se);
    mark(w, p, 4, stream);

    // Dense recovery of the flagged rows, batch by batch: batch b covers
    // entries [b rcap, (b + 1) rcap) of the list; entries past its
    // device-side length exit at once, so a call that flags nothing pays
    // two near-empty launches per batch.
    for (int64_t rb = 0; rb < T; rb += rcap) {
        sa.rowlist = (const int32_t *)w.rowlist.ptr;
        sa.nrows = (const unsigned long long *)w.stats.ptr + kStFlagged;
        sa.row_limit = (int)rcap;
        sa.row_base = (int)rb;
        sa.scratch = (float *)w.scratch.ptr;
        sa.scratch_stride = stride;
        sa.ntiles = (int)((rcap << ps) / kTileQ);
        sa.chunk = chunk_keys(sa.ntiles, S, ScoreCfg<kFP8, kModeDense, true>::waves);
        // the work items loop over one workgroup per compute unit: a batch
        // with nothing flagged costs one short launch
        const int64_t items = (int64_t)sa.ntiles * std::max<int64_t>(1, (S + sa.chunk - 1) / sa.chunk);
        launch_score_dt(p.dtype, kModeDenseLoop, dim3((unsigned)std::min<int64_t>(items, num_cu())), stream, sa);
        // Exact top k of each batch row's window scores: the row top-k
        // kernels in mapped-row mode (outputs to the flagged row, indices
        // offset by its window start; entries past the list exit).
        RowsArgs ra{};
        ra.x = w.scratch.ptr;
        ra.rows = rcap;
        ra.cols = S;
        ra.stride = stride;
        ra.topk = p.topk;
        ra.out_idx = out_idx;
        ra.out_val = out_val;
        ra.out_flags = p.out_flags;
        ra.rowmap = (const int32_t *)w.rowlist.ptr;
        ra.nrows = (const unsigned long long *)w.stats.ptr + kStFlagged;
        ra.row_base = rb;
        ra.ks = ks;
        ra.ke = ke;
        launch_rows_k<float>(ra, stream, false, nullptr);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_status(e);
    mark(w, p, 5, stream);

    begin_record(w, p, kCallFused);
    w.last.cand_capacity = p.cap;
    w.last.sample_target = p.sample_target;
    if (p.profile) {
        (void)hipEventSynchronize(w.ev[5]);
        w.last.ms_sample = phase_ms(w, p, 0, 1);
        w.last.ms_tau = phase_ms(w, p, 1, 2);
        w.last.ms_filter = phase_ms(w, p, 2, 3);
        w.last.ms_select = phase_ms(w, p, 3, 4);
        w.last.ms_recover = phase_ms(w, p, 4, 5);
    }
    return FLASHTOPK_OK;
}

// The auto path's choice between the fused and the dense sequence.
bool dense_path(const Plan &p)
{
    if (p.path == FLASHTOPK_PATH_RECOVER) return true;
    if (p.path != FLASHTOPK_PATH_AUTO) return false;
    return p.T * std::max<int64_t>(p.S, 1) <= kDensePairs;
}

int run(Workspace &w, const void *q, const void *kv, const float *kv_scales, const float *weights, const int32_t *ks,
        const int32_t *ke, void *out_idx, float *out_val, hipStream_t stream, const Plan &p)
{
    if (dense_path(p)) return run_dense(w, q, kv, kv_scales, weights, ks, ke, out_idx, out_val, stream, p);
    return run_fused(w, q, kv, kv_scales, weights, ks, ke, out_idx, out_val, stream, p);
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Run once by flashtopk_reserve on its stream: the first launch of a kernel
// of this library loads its code object, and a kernel that keeps values in
// private (scratch) memory makes the runtime size the stream's private-memory
// area for it.  This kernel holds kWarmWords words per lane there, more than
// any kernel of the library spills, so both happen here and not in a later
// call.
constexpr int kWarmWords = 96;
__global__ __launch_bounds__(64) void k_warm(float *out, int n)
{
    float buf[kWarmWords];
    for (int i = 0; i < kWarmWords; ++i) buf[(i * 7 + (int)threadIdx.x) % kWarmWords] = (float)(i + n);
    const float v = buf[(n + (int)threadIdx.x) % kWarmWords];
    if (out && n > 0) out[threadIdx.x] = v;
}

// Zero fill of n words (clears what the allocation-free entry point hands to
// a call as zero; a kernel, so the call can be captured in a graph).
__global__ __launch_bounds__(256) void k_fill_zero(uint32_t *p, int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0u;
}

// Lays the buffers a call needs (the sizing pass's sizes) out in the fixed
// array and clears the ones that must read zero.  Returns
// FLASHTOPK_ERR_WORKSPACE_LIMIT when they do not fit.
int carve(Workspace &w, uint8_t *base, hipStream_t s)
{
    DevBuf *bufs[] = {&w.tau,   &w.cnt,     &w.rowlist, &w.stats, &w.wlen, &w.cand,  &w.samp,
                      &w.scratch, &w.qbar,  &w.qscale,  &w.sigh,  &w.kb,   &w.kmeta, &w.vplan,
                      &w.q1,    &w.scnt,    &w.sover,   &w.scand};
    size_t off = 0;
    for (DevBuf *b : bufs) {
        if (!b->bytes) continue;
        const size_t len = (b->bytes + 255) / 256 * 256;
        if (len > kNoAllocBytes - off) return FLASHTOPK_ERR_WORKSPACE_LIMIT;
        b->ptr = base + off;
        off += len;
    }
    for (DevBuf *b : bufs)
        if (b->bytes && b->zero) {
            const int64_t n = (int64_t)(b->bytes + 3) / 4;
            k_fill_zero<<<(unsigned)std::min<int64_t>(1024, (n + 255) / 256), 256, 0, s>>>((uint32_t *)b->ptr, n);
        }
    return hip_status(hipGetLastError());
}

// options.validate: runs k_validate on the call's inputs, waits for its flags
// (p.invalid) and, when it found any, fails the call before a scoring kernel
// runs, recording it as the stream's last call.
int check_inputs(Workspace &w, hipStream_t s, Plan &p, ValidateArgs va)
{
    int st = FLASHTOPK_OK;
    if ((st = ensure(w, w.vflag, sizeof(unsigned)))) return st;
    va.flags = (unsigned *)w.vflag.ptr;
    va.dtype = p.dtype == FLASHTOPK_FP8_E4M3 ? kFP8 : kBF16;
    const int64_t n = std::max({va.q_pieces, va.kv_pieces, va.nw, va.nscales, va.num_q, va.ntable, (int64_t)1});
    const unsigned grid = (unsigned)std::min<int64_t>(2048, (n + 255) / 256);
    k_zero_word<<<1, 64, 0, s>>>(va.flags);
    k_validate<<<grid, 256, 0, s>>>(va);
    hipError_t e = hipMemcpyAsync(w.host_flag, va.flags, sizeof(unsigned), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_status(e);
    p.invalid = *w.host_flag;
    if (p.invalid) {
        begin_record(w, p, kCallFailed);
        w.last.status = FLASHTOPK_ERR_INVALID_ARGUMENT;
        return FLASHTOPK_ERR_INVALID_ARGUMENT;
    }
    return FLASHTOPK_OK;
}

// Counts of the record from the last call's device arrays (the stream has
// been synchronised).
int fill_counts(Workspace &w)
{
    flashtopk_info &info = w.last;
    const int64_t T = info.rows;
    std::vector<int32_t> len((size_t)T);
    hipError_t e = hipMemcpy(len.data(), w.wlen.ptr, sizeof(int32_t) * (size_t)T, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_status(e);
    info.rows_empty = info.rows_take_all = info.rows_sampled = info.rows_underflow = info.rows_overflow = 0;
    info.rows_recovered = info.max_candidates = info.window_keys = info.pruned_keys = info.candidates = 0;
    if (w.last_kind == kCallDense) {
        for (int64_t t = 0; t < T; ++t) {
            info.window_keys += len[t];
            if (len[t] == 0) ++info.rows_empty;
            else ++info.rows_recovered;
        }
        return FLASHTOPK_OK;
    }
    std::vector<uint32_t> cnt((size_t)T);
    unsigned long long stats[kStCount];
    e = hipMemcpy(cnt.data(), w.cnt.ptr, sizeof(uint32_t) * (size_t)T, hipMemcpyDeviceToHost);
    if (e == hipSuccess) e = hipMemcpy(stats, w.stats.ptr, sizeof(stats), hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_status(e);
    const int64_t cap = info.cand_capacity;
    for (int64_t t = 0; t < T; ++t) {
        const int64_t L = len[t];
        const uint32_t c = cnt[t];
        info.window_keys += L;
        if (L == 0) {
            ++info.rows_empty;
            continue;
        }
        if ((int64_t)c < std::min<int64_t>(w.last_topk, L)) ++info.rows_underflow;
        if ((int64_t)c > cap) ++info.rows_overflow;
        if (row_flagged(L, c, w.last_topk, (int)cap)) ++info.rows_recovered;
        if (L <= cap) {
            ++info.rows_take_all;
        } else {
            ++info.rows_sampled;
            info.max_candidates = std::max<int64_t>(info.max_candidates, c);
            info.candidates += c;
        }
    }
    info.pruned_keys = (int64_t)stats[kStPruned];
    info.path = stats[kStPruneOn] ? FLASHTOPK_PATH_PRUNE : FLASHTOPK_PATH_SCAN;
    // the device's own count of the list (the recovery launches read it)
    if ((int64_t)stats[kStFlagged] != info.rows_recovered) return FLASHTOPK_ERR_HIP;
    return FLASHTOPK_OK;
}

Workspace *find_ws(hipStream_t stream)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return nullptr;
    std::lock_guard<std::mutex> lk(g_mu);
    for (Workspace *w : g_ws)
        if (w->device == dev && w->stream == stream) return w;
    return nullptr;
}

}  // namespace

extern "C" {

int flashtopk_select_ex(const void *q, const void *kv, const float *kv_scales, const float *weights,
                        const int32_t *ks, const int32_t *ke, int64_t num_q, int64_t num_kv, int dtype,
                        int topk, void *out_idx, float *out_val, void *stream,
                        const flashtopk_options *opt)
{
    if (dtype != FLASHTOPK_FP8_E4M3 && dtype != FLASHTOPK_BF16) return FLASHTOPK_ERR_UNSUPPORTED;
    if (num_q < 0 || num_kv < 0 || num_kv >= (int64_t(1) << 31) || num_q >= (int64_t(1) << 30))
        return FLASHTOPK_ERR_INVALID_ARGUMENT;
    if (topk < 1 || topk > FLASHTOPK_MAX_TOPK) return FLASHTOPK_ERR_INVALID_ARGUMENT;
    if (num_q == 0) return FLASHTOPK_OK;
    if (!q || !weights || !ks || !ke || !out_idx || (!kv && num_kv > 0)) return FLASHTOPK_ERR_INVALID_ARGUMENT;
    if (!aligned16(q) || (kv && !aligned16(kv))) return FLASHTOPK_ERR_INVALID_ARGUMENT;
    Plan p{};
    p.T = num_q;
    p.S = num_kv;
    p.dtype = dtype;
    p.topk = topk;
    int st = resolve(p, opt);
    if (st) return st;
    const hipStream_t s = (hipStream_t)stream;
    Workspace *w = get_ws(s, &st);
    if (!w) return st;
    std::lock_guard<std::mutex> lk(w->mu);
    if (p.validate) {
        const int64_t rb = dtype == FLASHTOPK_FP8_E4M3 ? kDim : 2 * kDim;
        ValidateArgs va{};
        va.q = (const uint8_t *)q;
        va.q_pieces = num_q * p.heads * rb / 16;
        va.kv = (const uint8_t *)kv;
        va.kv_pieces = kv ? num_kv * rb / 16 : 0;
        va.w = weights;
        va.nw = num_q * p.heads;
        va.scales = kv_scales;
        va.nscales = kv_scales ? num_kv : 0;
        va.ks = ks;
        va.ke = ke;
        va.num_q = num_q;
        va.num_kv = num_kv;
        if ((st = check_inputs(*w, s, p, va))) return st;
    }
    return run(*w, q, kv, kv_scales, weights, ks, ke, out_idx, out_val, s, p);
}

int flashtopk_select_paged(const void *q, const void *kv_pages, const float *scale_pages, const int32_t *block_table,
                           int page_size, int64_t num_pages, const float *weights, const int32_t *ks,
                           const int32_t *ke, int64_t num_q, int64_t num_kv, int dtype, int topk, void *out_idx,
                           float *out_val, void *stream, const flashtopk_options *opt)
{
    if (dtype != FLASHTOPK_FP8_E4M3 && dtype != FLASHTOPK_BF16) return FLASHTOPK_ERR_UNSUPPORTED;
    if (num_q < 0 || num_kv < 0 || num_kv >= (int64_t(1) << 31) || num_q >= (int64_t(1) << 30))
        return FLASHTOPK_ERR_INVALID_ARGUMENT;
    if (page_size < 1 || num_pages < 0) return FLASHTOPK_ERR_INVALID_ARGUMENT;
    if (topk < 1 || topk > FLASHTOPK_MAX_TOPK) return FLASHTOPK_ERR_INVALID_ARGUMENT;
    if (num_q == 0) return FLASHTOPK_OK;
    if (!q || !weights || !ks || !ke || !out_idx) return FLASHTOPK_ERR_INVALID_ARGUMENT;
    if (num_kv > 0 && (!kv_pages || !block_table || num_pages == 0)) return FLASHTOPK_ERR_INVALID_ARGUMENT;
    if (!aligned16(q) || (kv_pages && !aligned16(kv_pages))) return FLASHTOPK_ERR_INVALID_ARGUMENT;
    Plan p{};
    p.T = num_q;
    p.S = num_kv;
    p.dtype = dtype;
    p.topk = topk;
    int st = resolve(p, opt);
    if (st) return st;
    const hipStream_t s = (hipStream_t)stream;
    Workspace *w = get_ws(s, &st);
    if (!w) return st;
    std::lock_guard<std::mutex> lk(w->mu);
    if (p.validate) {
        // the pool may hold unused pages: q, weights, windows and page ids only
        const int64_t rb = dtype == FLASHTOPK_FP8_E4M3 ? kDim : 2 * kDim;
        ValidateArgs va{};
        va.q = (const uint8_t *)q;
        va.q_pieces = num_q * p.heads * rb / 16;
        va.w = weights;
        va.nw = num_q * p.heads;
        va.ks = ks;
        va.ke = ke;
        va.num_q = num_q;
        va.num_kv = num_kv;
        va.table = num_kv > 0 ? block_table : nullptr;
        va.ntable = num_kv > 0 ? (num_kv + page_size - 1) / page_size : 0;
        va.num_pages = num_pages;
        if ((st = check_inputs(*w, s, p, va))) return st;
    }
    if (num_kv == 0) return run(*w, q, nullptr, nullptr, weights, ks, ke, out_idx, out_val, s, p);
    if (dense_path(p)) {
        // the dense kernel reads each key from its page
        p.table = block_table;
        p.page_size = page_size;
        p.num_pages = num_pages;
        return run_dense(*w, q, kv_pages, scale_pages, weights, ks, ke, out_idx, out_val, s, p);
    }
    const bool fp8 = dtype == FLASHTOPK_FP8_E4M3;
    const int RB = fp8 ? 128 : 256;
    if ((st = ensure(*w, w->pkv, (size_t)num_kv * RB))) return st;
    if (scale_pages && (st = ensure(*w, w->psig, sizeof(float) * (size_t)num_kv))) return st;
    const int64_t pieces = num_kv * (RB / 16);
    const dim3 grid((unsigned)((pieces + kGatherThreads * kGatherUnroll - 1) / (kGatherThreads * kGatherUnroll)));
    float *sig = scale_pages ? (float *)w->psig.ptr : nullptr;
    if (fp8)
        k_gather_pages<kFP8><<<grid, kGatherThreads, 0, s>>>((const uint8_t *)kv_pages, scale_pages, block_table,
                                                             page_size, num_pages, num_kv, (uint8_t *)w->pkv.ptr, sig);
    else
        k_gather_pages<kBF16><<<grid, kGatherThreads, 0, s>>>((const uint8_t *)kv_pages, scale_pages, block_table,
                                                              page_size, num_pages, num_kv, (uint8_t *)w->pkv.ptr, sig);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_status(e);
    return run_fused(*w, q, w->pkv.ptr, sig, weights, ks, ke, out_idx, out_val, s, p);
}

int flashtopk_select_noalloc(const void *q, const void *kv, const float *kv_scales, const float *weights,
                             const int32_t *ks, const int32_t *ke, int64_t num_q, int64_t num_kv, int dtype,
                             int topk, void *out_idx, float *out_val, void *stream)
{
    if (dtype != FLASHTOPK_FP8_E4M3 && dtype != FLASHTOPK_BF16) return FLASHTOPK_ERR_UNSUPPORTED;
    if (num_q < 0 || num_kv < 0 || num_kv >= (int64_t(1) << 31) || num_q >= (int64_t(1) << 30))
        return FLASHTOPK_ERR_INVALID_ARGUMENT;
    if (topk < 1 || topk > FLASHTOPK_MAX_TOPK) return FLASHTOPK_ERR_INVALID_ARGUMENT;
    if (num_q == 0) return FLASHTOPK_OK;
    if (!q || !weights || !ks || !ke || !out_idx || (!kv && num_kv > 0)) return FLASHTOPK_ERR_INVALID_ARGUMENT;
    if (!aligned16(q) || (kv && !aligned16(kv))) return FLASHTOPK_ERR_INVALID_ARGUMENT;
    Plan p{};
    p.T = num_q;
    p.S = num_kv;
    p.dtype = dtype;
    p.topk = topk;
    int st = resolve(p, nullptr);
    if (st) return st;
    p.recover_budget = kNoAllocRecoverBudget;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e);
    if (dev < 0 || dev >= kNoAllocMaxDevices) return FLASHTOPK_ERR_HIP;
    NoAllocDevice &na = g_na[dev];
    std::lock_guard<std::mutex> lk(na.mu);
    if (!na.base) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr) {
            (void)hipGetLastError();
            return FLASHTOPK_ERR_HIP;
        }
        na.base = (uint8_t *)ptr;
    }
    const hipStream_t s = (hipStream_t)stream;
    Workspace &w = na.ws;
    w.device = dev;
    w.stream = s;
    DevBuf *bufs[] = {&w.tau,   &w.cnt,     &w.rowlist, &w.stats, &w.wlen, &w.cand,  &w.samp,
                      &w.scratch, &w.qbar,  &w.qscale,  &w.sigh,  &w.kb,   &w.kmeta, &w.vplan,
                      &w.q1,    &w.scnt,    &w.sover,   &w.scand, &w.pkv,  &w.psig,  &w.vflag};
    for (DevBuf *b : bufs) *b = DevBuf{};
    // sizing pass, then the buffers in the fixed array, then the call
    const bool dense = dense_path(p);
    w.fixed = false;
    w.sizing = true;
    RowsSplit sp;
    st = dense ? prepare_dense(w, p, sp) : prepare_fused(w, p);
    w.sizing = false;
    if (st) return st;
    w.fixed = true;
    st = carve(w, na.base, s);
    if (st == FLASHTOPK_OK)
        st = dense ? run_dense(w, q, kv, kv_scales, weights, ks, ke, out_idx, out_val, s, p)
                   : run_fused(w, q, kv, kv_scales, weights, ks, ke, out_idx, out_val, s, p);
    w.fixed = false;
    return st;
}

int flashtopk_select(const void *q, const void *kv, const float *kv_scales, const float *weights,
                     const int32_t *ks, const int32_t *ke, int64_t num_q, int64_t num_kv, int dtype, int topk,
                     void *out_idx, float *out_val, void *stream)
{
    return flashtopk_select_ex(q, kv, kv_scales, weights, ks, ke, num_q, num_kv, dtype, topk, out_idx, out_val,
                               stream, nullptr);
}

int flashtopk_topk_rows(const void *x, int score_dtype, int64_t rows, int64_t cols, int64_t row_stride,
                        const int32_t *ends, int topk, void *out_idx, float *out_val, int32_t *nan_flag,
                        int out_flags, void *stream)
{
    if (score_dtype != FLASHTOPK_SCORES_F32 && score_dtype != FLASHTOPK_SCORES_BF16) return FLASHTOPK_ERR_UNSUPPORTED;
    if (rows < 0 || rows >= (int64_t(1) << 31) || cols < 0 || cols >= (int64_t(1) << 31))
        return FLASHTOPK_ERR_INVALID_ARGUMENT;
    if (topk < 1 || topk > FLASHTOPK_MAX_TOPK) return FLASHTOPK_ERR_INVALID_ARGUMENT;
    if (rows == 0) return FLASHTOPK_OK;
    const int64_t esize = score_dtype == FLASHTOPK_SCORES_F32 ? 4 : 2;
    if (!out_idx || (!x && cols > 0)) return FLASHTOPK_ERR_INVALID_ARGUMENT;
    if (rows > 1 && row_stride < cols) return FLASHTOPK_ERR_INVALID_ARGUMENT;
    if (x && !aligned16(x)) return FLASHTOPK_ERR_INVALID_ARGUMENT;
    if (rows > 1 && (row_stride * esize) % 16 != 0) return FLASHTOPK_ERR_INVALID_ARGUMENT;
    if (out_flags & ~(FLASHTOPK_OUT_INDEX_ORDER | FLASHTOPK_OUT_INT64)) return FLASHTOPK_ERR_INVALID_ARGUMENT;
    RowsArgs a{};
    a.x = x;
    a.rows = rows;
    a.cols = cols;
    a.stride = row_stride;
    a.ends = ends;
    a.topk = topk;
    a.out_idx = out_idx;
    a.out_val = out_val;
    a.nan_flag = nan_flag;
    a.out_flags = out_flags;
    const hipStream_t s = (hipStream_t)stream;
    // Few rows are split over several workgroups each, with per-row state in
    // the stream's workspace.
    const int parts = split_parts(rows, cols);
    RowsSplit sp{};
    std::unique_lock<std::mutex> lk;
    if (parts > 1) {
        int st = FLASHTOPK_OK;
        Workspace *w = get_ws(s, &st);
        if (!w) return st;
        lk = std::unique_lock<std::mutex>(w->mu);
        if ((st = ensure_split(*w, rows, parts, sp))) return st;
    }
    if (score_dtype == FLASHTOPK_SCORES_F32) launch_rows_k<float>(a, s, true, &sp);
    else launch_rows_k<uint16_t>(a, s, true, &sp);
    return hip_status(hipGetLastError());
}

int flashtopk_reserve(int64_t max_q, int64_t max_kv, int max_topk, int dtype, void *stream)
{
    if (dtype != FLASHTOPK_FP8_E4M3 && dtype != FLASHTOPK_BF16) return FLASHTOPK_ERR_UNSUPPORTED;
    if (max_q < 0 || max_kv < 0 || max_kv >= (int64_t(1) << 31) || max_q >= (int64_t(1) << 30) || max_topk < 1 ||
        max_topk > FLASHTOPK_MAX_TOPK)
        return FLASHTOPK_ERR_INVALID_ARGUMENT;
    int st = FLASHTOPK_OK;
    Workspace *w = get_ws((hipStream_t)stream, &st);
    if (!w) return st;
    std::lock_guard<std::mutex> lk(w->mu);
    // Everything a call of at most these sizes with default options (either
    // head count, either path) grows the workspace to.
    const int64_t T = std::max<int64_t>(max_q, 1), S = max_kv;
    const int64_t TC = 2 * T;  // 64 heads: two tile columns per row
    const int cap = std::min(kMaxCap, std::max(4 * max_topk, max_topk));
    Plan p{};
    p.T = T;
    p.S = S;
    p.recover_budget = kDefaultRecoverBudget;
    const int64_t stride = scratch_stride(S);
    const int64_t rcap = batch_rows(p);
    const int64_t nblocks = (S + kBlockKeys - 1) / kBlockKeys;
    const int64_t ntiles = (T + kTileQ - 1) / kTileQ;
    if ((st = ensure(*w, w->tau, sizeof(float) * T))) return st;
    if ((st = ensure(*w, w->cnt, sizeof(uint32_t) * T))) return st;
    if ((st = ensure(*w, w->rowlist, sizeof(int32_t) * T))) return st;
    if ((st = ensure(*w, w->wlen, sizeof(int32_t) * T))) return st;
    if ((st = ensure(*w, w->stats, sizeof(unsigned long long) * kStCount))) return st;
    if ((st = ensure(*w, w->cand, sizeof(uint64_t) * (size_t)T * cap))) return st;
    if ((st = ensure(*w, w->samp, sizeof(uint32_t) * (size_t)T * kDefaultSampleTarget))) return st;
    if ((st = ensure(*w, w->sigh, sizeof(float) * (size_t)(S + 64)))) return st;
    if ((st = ensure(*w, w->scratch, sizeof(float) * (size_t)rcap * stride))) return st;
    if (dtype == FLASHTOPK_FP8_E4M3) {
        if ((st = ensure(*w, w->qbar, (size_t)TC * kQbarParts * kDim))) return st;
        if ((st = ensure(*w, w->qscale, sizeof(float) * TC))) return st;
    }
    if ((st = ensure(*w, w->kb, (size_t)std::max<int64_t>(nblocks, 1) * 2 * (dtype == FLASHTOPK_FP8_E4M3 ? 128 : 256))))
        return st;
    if ((st = ensure(*w, w->kmeta, sizeof(float2) * (size_t)std::max<int64_t>(nblocks, 1)))) return st;
    if ((st = ensure(*w, w->vplan, sizeof(float) * (size_t)ntiles * kPlanGroups * 256))) return st;
    if ((st = ensure(*w, w->q1, sizeof(float) * (size_t)T))) return st;
    // split-row state (dense path and row top-k of at most one row per compute
    // unit): its size depends on the rows only
    RowsSplit sp;
    const int64_t srows = std::min<int64_t>(T, num_cu());
    if ((st = ensure_split(*w, srows, split_parts(1, S), sp))) return st;
    // the code object and the private-memory area, see k_warm
    k_warm<<<1, 64, 0, (hipStream_t)stream>>>(nullptr, 0);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
    return hip_status(e);
}

int flashtopk_get_last_info(void *stream, flashtopk_info *out)
{
    if (!out) return FLASHTOPK_ERR_INVALID_ARGUMENT;
    std::memset(out, 0, sizeof(*out));
    Workspace *w = find_ws((hipStream_t)stream);
    if (!w) return FLASHTOPK_ERR_INVALID_ARGUMENT;
    std::lock_guard<std::mutex> lk(w->mu);
    if (w->last_kind == kCallNone) return FLASHTOPK_ERR_INVALID_ARGUMENT;
    if (w->last_kind != kCallFailed) {
        hipError_t e = hipStreamSynchronize(w->stream);
        if (e != hipSuccess) return hip_status(e);
        int st = fill_counts(*w);
        if (st) return st;
    }
    *out = w->last;
    return FLASHTOPK_OK;
}

int flashtopk_get_last_recovered(void *stream, int32_t *rows, int64_t max_rows, int64_t *count)
{
    if (!count || max_rows < 0 || (max_rows > 0 && !rows)) return FLASHTOPK_ERR_INVALID_ARGUMENT;
    *count = 0;
    Workspace *w = find_ws((hipStream_t)stream);
    if (!w) return FLASHTOPK_ERR_INVALID_ARGUMENT;
    std::lock_guard<std::mutex> lk(w->mu);
    if (w->last_kind == kCallNone) return FLASHTOPK_ERR_INVALID_ARGUMENT;
    if (w->last_kind == kCallFailed) return FLASHTOPK_OK;
    hipError_t e = hipStreamSynchronize(w->stream);
    if (e != hipSuccess) return hip_status(e);
    const int64_t T = w->last.rows;
    if (w->last_kind == kCallDense) {
        std::vector<int32_t> len((size_t)T);
        e = hipMemcpy(len.data(), w->wlen.ptr, sizeof(int32_t) * (size_t)T, hipMemcpyDeviceToHost);
        if (e != hipSuccess) return hip_status(e);
        int64_t n = 0;
        for (int64_t t = 0; t < T; ++t)
            if (len[t] > 0) {
                if (n < max_rows) rows[n] = (int32_t)t;
                ++n;
            }
        *count = n;
        return FLASHTOPK_OK;
    }
    unsigned long long nf = 0;
    e = hipMemcpy(&nf, (unsigned long long *)w->stats.ptr + kStFlagged, sizeof(nf), hipMemcpyDeviceToHost);
    if (e == hipSuccess && nf > 0 && max_rows > 0)
        e = hipMemcpy(rows, w->rowlist.ptr, sizeof(int32_t) * (size_t)std::min<int64_t>((int64_t)nf, max_rows),
                      hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_status(e);
    *count = (int64_t)nf;
    return FLASHTOPK_OK;
}

void flashtopk_release(void)
{
    std::lock_guard<std::mutex> lk(g_mu);
    for (Workspace *w : g_ws) {
        {
            std::lock_guard<std::mutex> wl(w->mu);
            int prev = 0;
            (void)hipGetDevice(&prev);
            (void)hipSetDevice(w->device);
            (void)hipStreamSynchronize(w->stream);
            DevBuf *bufs[] = {&w->tau,   &w->cnt,   &w->rowlist, &w->stats,  &w->wlen, &w->cand,
                              &w->samp,  &w->scratch, &w->qbar,  &w->qscale, &w->sigh, &w->kb,
                              &w->kmeta, &w->vplan, &w->q1,      &w->scnt,   &w->sover, &w->scand, &w->pkv,   &w->psig,    &w->vflag};
            for (DevBuf *b : bufs)
                if (b->ptr) (void)hipFree(b->ptr);
            if (w->host_flag) (void)hipHostFree(w->host_flag);
            for (hipEvent_t &ev : w->ev)
                if (ev) (void)hipEventDestroy(ev);
            (void)hipSetDevice(prev);
        }
        delete w;
    }
    g_ws.clear();
}

const char *flashtopk_status_string(int status)
{
    switch (status) {
    case FLASHTOPK_OK: return "ok";
    case FLASHTOPK_ERR_INVALID_ARGUMENT: return "invalid argument";
    case FLASHTOPK_ERR_UNSUPPORTED: return "unsupported dtype";
    case FLASHTOPK_ERR_OUT_OF_MEMORY: return "out of device memory";
    case FLASHTOPK_ERR_HIP: return "HIP runtime error";
    case FLASHTOPK_ERR_WORKSPACE_LIMIT: return "call too large for the fixed scratch array";
    default: return "unknown status";
    }
}

int flashtopk_probe_mfma(int dtype, int iters, void *stream, double *tflops)
{
    if (!tflops || iters <= 0 || (dtype != FLASHTOPK_FP8_E4M3 && dtype != FLASHTOPK_BF16))
        return FLASHTOPK_ERR_INVALID_ARGUMENT;
    *tflops = 0.0;
    (void)hipGetLastError();  // a stale error of an earlier call is not this call's
    hipStream_t s = (hipStream_t)stream;
    const unsigned grid = (unsigned)(4 * num_cu());  // four workgroups of four waves per compute unit
    const float never = __builtin_nanf("");
    auto launch = [&](int n) {
        if (dtype == FLASHTOPK_FP8_E4M3) k_probe_mfma<kFP8><<<grid, kProbeThreads, 0, s>>>(n, never);
        else k_probe_mfma<kBF16><<<grid, kProbeThreads, 0, s>>>(n, never);
    };
    hipEvent_t e0 = nullptr, e1 = nullptr;
    hipError_t e = hipEventCreate(&e0);
    if (e == hipSuccess) e = hipEventCreate(&e1);
    if (e == hipSuccess) {
        launch(std::max(1, iters / 8));  // warm-up: code object loaded, clocks up
        e = hipGetLastError();
    }
    if (e == hipSuccess) e = hipEventRecord(e0, s);
    if (e == hipSuccess) {
        launch(iters);
        e = hipGetLastError();
    }
    if (e == hipSuccess) e = hipEventRecord(e1, s);
    if (e == hipSuccess) e = hipEventSynchronize(e1);
    float ms = 0.0f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
    if (e0) (void)hipEventDestroy(e0);
    if (e1) (void)hipEventDestroy(e1);
    if (e != hipSuccess) {
        std::fprintf(stderr, "flashtopk_probe_mfma: %s\n", hipGetErrorString(e));
        (void)hipGetLastError();
        return hip_status(e);
    }
    const double per_mfma = dtype == FLASHTOPK_FP8_E4M3 ? 2.0 * 16 * 16 * 128 : 2.0 * 32 * 32 * 16;
    const double flops = (double)grid * (kProbeThreads / 64) * (double)iters * kProbeChains * per_mfma;
    *tflops = ms > 0.0f ? flops / ((double)ms * 1e-3) / 1e12 : 0.0;
    return FLASHTOPK_OK;
}

int flashtopk_version(void) { return 200; }

}  // extern "C"
