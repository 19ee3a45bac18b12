// C ABI of the fused indexer top-k library (declared in include/flashtopk.h).
//
// Launch sequence of one call, all on the caller's stream:
//   0. k_prep           per-key scale factors (+ block extremes for the bound)
//                       and (FP8) head-weighted query sums split into FP8
//                       parts, in one launch
//   1. k_score<sample>  strided-sample scores of every long row     (MFMA);
//                       with one workgroup per tile it also sets the
//                       tile's per-row thresholds from those samples
//   2. k_tau            (several workgroups per tile) the thresholds
//   3. k_score<filter>  fused score (+ bound) + threshold filter -> candidates (MFMA, hot)
//   4. k_triage         flag rows whose candidates under/overflowed
//   5. k_select         exact top-k of every unflagged row
//   6. (flagged rows)   k_score<dense> + the row top-k kernels in batches
// The triage counts are copied to pinned host memory behind step 4; the host
// waits for that copy (an event, while step 5 runs on the GPU) to size step
// 6, then returns.  Outputs are complete when the stream reaches the end of
// the call's work.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <vector>

#include "flashtopk.h"
#include "ftk_bound.hpp"
#include "ftk_few.hpp"
#include "ftk_paged.hpp"
#include "ftk_rows.hpp"
#include "ftk_score.hpp"
#include "ftk_select.hpp"
#include "ftk_tau.hpp"
#include "ftk_validate.hpp"

using namespace ftk;

namespace {

constexpr int kMaxCap = 16384;
constexpr int kDefaultSampleTarget = 2048;
constexpr int64_t kDefaultRecoverBudget = int64_t(1) << 30;

// Grow-only device buffer.
struct DevBuf {
    void *ptr = nullptr;
    size_t bytes = 0;
};

struct Workspace {
    int device = -1;
    hipStream_t stream = nullptr;
    DevBuf tau, cnt, rowlist, stats, cand, samp, scratch, qbar, qscale, sigh;
    DevBuf kb, kmeta, vplan, q1;               // score-bound pruning
    DevBuf ticket;                             // few-row sample finish counters (kept zero between calls)
    DevBuf pkv, psig;                          // keys and scales gathered from a paged cache
    DevBuf vflag;                              // precondition flags (options.validate)
    unsigned long long *host_stats = nullptr;  // pinned: kStCount statistics, then the precondition flags
    hipEvent_t ev[7] = {};                     // phase boundaries when profiling
    hipEvent_t stats_ev = nullptr;             // triage counts have reached the host
    flashtopk_info last{};
    bool has_last = false;
    bool last_pending = false;   // counts of `last` not yet read from host_stats
    bool last_recover_all = false;
};

std::mutex g_mu;
std::vector<Workspace *> g_ws;

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
    if (b.bytes >= bytes && b.ptr) return FLASHTOPK_OK;
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
    if (b.bytes >= bytes && b.ptr) return FLASHTOPK_OK;
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
    e = hipHostMalloc((void **)&w->host_stats, sizeof(unsigned long long) * (kStCount + 1), hipHostMallocDefault);
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
    // keys in a paged cache, read in place (calls with at most kFewRows rows)
    const int32_t *table = nullptr;
    int page_size = 0;
    int64_t num_pages = 0;
};

int resolve(Plan &p, const flashtopk_options *opt)
{
    p.path = opt ? opt->path : FLASHTOPK_PATH_AUTO;
    if (p.path < FLASHTOPK_PATH_AUTO || p.path > FLASHTOPK_PATH_RECOVER) return FLASHTOPK_ERR_INVALID_ARGUMENT;
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

// Keys per work item (a power of two in [kMinChunk, kMaxChunk]), from a cost
// model: a work item takes a whole compute unit (its LDS), so items run in
// rounds of one per CU, and an item costs a fixed part (setting up and
// staging the q tile, flushing candidates: about one wave step) plus the wave
// steps of each of its `waves` waves.  The chunk of least cost wins, the
// larger one on a tie: large chunks amortise the fixed part, small ones fill
// the GPU when the call has few tiles.
int chunk_keys(int ntiles, int64_t S, int waves)
{
    const int64_t n_cu = num_cu();
    int best = kMaxChunk;
    int64_t best_cost = INT64_MAX;
    for (int chunk = kMaxChunk; chunk >= kMinChunk; chunk >>= 1) {
        const int64_t items = (int64_t)ntiles * ((S + chunk - 1) / chunk);
        const int64_t rounds = (items + n_cu - 1) / n_cu;
        const int64_t steps = (chunk / kStepKeys + waves - 1) / waves;
        const int64_t cost = rounds * (1 + steps);
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

template <int DT>
void launch_score(int mode, dim3 grid, hipStream_t st, const ScoreArgs &a)
{
    if (a.pair) {
        if (mode == kModeFilter) k_score<DT, kModeFilter, true><<<grid, 64 * ScoreCfg<DT, kModeFilter>::waves, 0, st>>>(a);
        else if (mode == kModeSample) k_score<DT, kModeSample, true><<<grid, 64 * ScoreCfg<DT, kModeSample>::waves, 0, st>>>(a);
        else k_score<DT, kModeDense, true><<<grid, 64 * ScoreCfg<DT, kModeDense>::waves, 0, st>>>(a);
    } else {
        if (mode == kModeFilter) k_score<DT, kModeFilter, false><<<grid, 64 * ScoreCfg<DT, kModeFilter>::waves, 0, st>>>(a);
        else if (mode == kModeSample) k_score<DT, kModeSample, false><<<grid, 64 * ScoreCfg<DT, kModeSample>::waves, 0, st>>>(a);
        else k_score<DT, kModeDense, false><<<grid, 64 * ScoreCfg<DT, kModeDense>::waves, 0, st>>>(a);
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

// Calls with at most kFewRows rows score with k_score_few in every mode.
template <int DT>
void launch_few(int mode, dim3 grid, hipStream_t st, const ScoreArgs &a)
{
    if (mode == kModeSample) k_score_few<DT, kModeSample><<<grid, kFewThreads, 0, st>>>(a);
    else if (mode == kModeFilter) k_score_few<DT, kModeFilter><<<grid, kFewThreads, 0, st>>>(a);
    else k_score_few<DT, kModeDense><<<grid, kFewThreads, 0, st>>>(a);
}

void launch_few_dt(int dtype, int mode, dim3 grid, hipStream_t st, const ScoreArgs &a)
{
    if (dtype == FLASHTOPK_FP8_E4M3) launch_few<kFP8>(mode, grid, st, a);
    else launch_few<kBF16>(mode, grid, st, a);
}

// Phase boundary i of a profiled call (no-op otherwise).
void mark(Workspace &w, const Plan &p, int i, hipStream_t stream)
{
    if (!p.profile) return;
    if (!w.ev[i]) (void)hipEventCreate(&w.ev[i]);
    (void)hipEventRecord(w.ev[i], stream);
}

float phase_ms(Workspace &w, const Plan &p, int i)
{
    float ms = 0.0f;
    if (p.profile && w.ev[i] && w.ev[i + 1] && hipEventElapsedTime(&ms, w.ev[i], w.ev[i + 1]) != hipSuccess) {
        (void)hipGetLastError();
        ms = 0.0f;
    }
    return ms;
}

// Copies the statistics of the workspace's last call (already in pinned host
// memory) into its record.
void fill_counts(Workspace &w)
{
    flashtopk_info &info = w.last;
    const unsigned long long *hs = w.host_stats;
    info.path = w.last_recover_all ? FLASHTOPK_PATH_RECOVER
                                   : (hs[kStPruneOn] ? FLASHTOPK_PATH_PRUNE : FLASHTOPK_PATH_SCAN);
    info.rows_empty = (int64_t)hs[kStEmpty];
    info.rows_take_all = (int64_t)hs[kStTakeAll];
    info.rows_sampled = (int64_t)hs[kStSampled];
    info.rows_underflow = (int64_t)hs[kStUnder];
    info.rows_overflow = (int64_t)hs[kStOver];
    info.rows_recovered = (int64_t)hs[kStFlagged];
    info.max_candidates = (int64_t)hs[kStMaxCand];
    info.window_keys = (int64_t)hs[kStWindow];
    info.pruned_keys = (int64_t)hs[kStPruned];
    w.last_pending = false;
}

template <typename T, typename SH>
void launch_rows(const RowsArgs &a, hipStream_t s);

int run(const void *q, const void *kv, const float *kv_scales, const float *weights, const int32_t *ks,
        const int32_t *ke, void *out_idx, float *out_val, hipStream_t stream, const Plan &p)
{
    int st = FLASHTOPK_OK;
    Workspace *w = get_ws(stream, &st);
    if (!w) return st;
    const int64_t T = p.T, S = p.S;
    if ((st = ensure(*w, w->tau, sizeof(float) * T))) return st;
    if ((st = ensure(*w, w->cnt, sizeof(uint32_t) * T))) return st;
    if ((st = ensure(*w, w->rowlist, sizeof(int32_t) * T))) return st;
    if ((st = ensure(*w, w->stats, sizeof(unsigned long long) * kStCount))) return st;
    const bool recover_all = p.path == FLASHTOPK_PATH_RECOVER;
    const bool fp8 = p.dtype == FLASHTOPK_FP8_E4M3;
    // 64 heads: row t's two 32-head halves are tile columns 2t and 2t + 1.
    const int ps = p.heads == 64 ? 1 : 0;
    const int64_t TC = T << ps;  // tile columns
    if (fp8) {
        if ((st = ensure(*w, w->qbar, (size_t)TC * kQbarParts * kDim))) return st;
        if ((st = ensure(*w, w->qscale, sizeof(float) * TC))) return st;
    }
    if ((st = ensure(*w, w->sigh, sizeof(float) * (size_t)(S + 64)))) return st;
    if (!recover_all) {
        if ((st = ensure(*w, w->cand, sizeof(uint64_t) * (size_t)T * p.cap))) return st;
        if ((st = ensure(*w, w->samp, sizeof(uint32_t) * (size_t)T * p.sample_target))) return st;
    }

    const int ntiles = (int)((TC + kTileQ - 1) / kTileQ);
    // A few rows (decode) score with k_score_few, which has no bound pruning.
    const bool few = !ps && T <= kFewRows;
    // Score-bound pruning: on the auto path (each scan work item decides from
    // its tile's planner sample) and the forced prune path; not for 64 heads.
    const bool bounds = !few && !ps && S > 0 && (p.path == FLASHTOPK_PATH_AUTO || p.path == FLASHTOPK_PATH_PRUNE);
    const int nblocks = (int)((S + kBlockKeys - 1) / kBlockKeys);
    if (bounds) {
        if ((st = ensure(*w, w->kb, (size_t)nblocks * 2 * (fp8 ? 128 : 256)))) return st;
        if ((st = ensure(*w, w->kmeta, sizeof(float2) * (size_t)nblocks))) return st;
        if ((st = ensure(*w, w->vplan, sizeof(float) * (size_t)ntiles * kPlanGroups * 256))) return st;
        if ((st = ensure(*w, w->q1, sizeof(float) * (size_t)T))) return st;
    }
    const int chunk = chunk_keys(ntiles, S, fp8 ? ScoreCfg<kFP8, kModeFilter>::waves : ScoreCfg<kBF16, kModeFilter>::waves);
    const int nchunks = (int)std::max<int64_t>(1, (S + chunk - 1) / chunk);

    ScoreArgs sa{};
    sa.q = (const uint8_t *)q;
    sa.kv = (const uint8_t *)kv;
    sa.sigma = kv_scales;
    sa.sigh = (const float *)w->sigh.ptr;
    sa.w = weights;
    sa.ks = ks;
    sa.ke = ke;
    sa.num_q = (int)TC;
    sa.num_kv = (int)S;
    sa.pair = ps;
    sa.qbar = (const uint8_t *)w->qbar.ptr;
    sa.qscale = (const float *)w->qscale.ptr;
    sa.ntiles = ntiles;
    sa.chunk = chunk;
    sa.cap = p.cap;
    sa.tau = (const float *)w->tau.ptr;
    sa.cnt = (uint32_t *)w->cnt.ptr;
    sa.cand = (uint64_t *)w->cand.ptr;
    sa.samp = (uint32_t *)w->samp.ptr;
    sa.sample_target = p.sample_target;
    sa.sample_min_stride = p.sample_min_stride;
    sa.sample_split = sample_split(ntiles);
    sa.table = p.table;
    sa.page_size = p.page_size;
    sa.num_pages = p.num_pages;
    if (bounds) {
        sa.prune = p.path == FLASHTOPK_PATH_PRUNE ? 2 : 1;
        sa.kb = (const uint8_t *)w->kb.ptr;
        sa.meta = (const float2 *)w->kmeta.ptr;
        sa.q1 = (float *)w->q1.ptr;
        sa.nblocks = nblocks;
        sa.vplan = (float *)w->vplan.ptr;
        sa.plan = (unsigned long long *)w->stats.ptr + kStPruned;
    }

    // The sample kernel sets the thresholds itself when each row's samples
    // come from one workgroup per tile, or (few rows) from the row's last
    // workgroup to finish, which also clears the statistics (no per-key
    // pass); otherwise k_tau follows it.
    const bool few_sample = few && !recover_all;
    const bool fused_tau = !few && !recover_all && sa.sample_split == 1;
    sa.topk = p.topk;
    sa.rank_scale = p.rank_scale;
    sa.tau_w = (float *)w->tau.ptr;
    if (few_sample) {
        if ((st = ensure_zeroed(*w, w->ticket, sizeof(uint32_t) * (size_t)T))) return st;
        sa.ticket = (uint32_t *)w->ticket.ptr;
        sa.stats = (unsigned long long *)w->stats.ptr;
        sa.nstats = kStCount;
    }

    mark(*w, p, 0, stream);
    {
        // Per-key scale factors (and block extremes for the bound); with few
        // rows only the statistics are cleared (k_score_few reads sigma), and
        // those calls' sample kernel does even that.  FP8 calls of more rows
        // also get their query sums from the same launch.
        PrepArgs pa{};
        const int64_t Sp = few ? 0 : S;
        pa.key_blocks = few_sample ? 0 : (int)((Sp + 64 + 4 * kBlockKeys - 1) / (4 * kBlockKeys));
        pa.kv = (const uint8_t *)kv;
        pa.sigma = kv_scales;
        pa.num_kv = (int)Sp;
        pa.nblocks = nblocks;
        pa.sigh = (float *)w->sigh.ptr;
        pa.bounds = bounds ? 1 : 0;
        pa.kb = bounds ? (uint8_t *)w->kb.ptr : nullptr;
        pa.meta = bounds ? (float2 *)w->kmeta.ptr : nullptr;
        pa.stats = (unsigned long long *)w->stats.ptr;
        pa.nstats = kStCount;
        int64_t qblocks = 0;
        if (fp8 && !few) {
            pa.q = (const uint8_t *)q;
            pa.w = weights;
            pa.num_q = TC;
            pa.parts = (uint8_t *)w->qbar.ptr;
            pa.qscale = (float *)w->qscale.ptr;
            pa.q1 = bounds ? (float *)w->q1.ptr : nullptr;
            qblocks = (TC + 3) / 4;
        }
        const unsigned nwg = (unsigned)(pa.key_blocks + qblocks);
        if (nwg > 0) {
            if (fp8) k_prep<kFP8><<<nwg, 256, 0, stream>>>(pa);
            else k_prep<kBF16><<<nwg, 256, 0, stream>>>(pa);
        }
    }
    if (!recover_all) {
        if (few)
            launch_few_dt(p.dtype, kModeSample,
                          dim3((unsigned)(T * ((p.sample_target + kFewSamplePart - 1) / kFewSamplePart))), stream, sa);
        else
            launch_score_dt(p.dtype, kModeSample, dim3((unsigned)(ntiles * sa.sample_split)), stream, sa);
    }
    mark(*w, p, 1, stream);

    if (!recover_all && !few_sample && !fused_tau) {
        TauArgs ta{};
        ta.ks = ks;
        ta.ke = ke;
        ta.num_q = T;
        ta.topk = p.topk;
        ta.cap = p.cap;
        ta.samp = (const uint32_t *)w->samp.ptr;
        ta.sample_target = p.sample_target;
        ta.sample_min_stride = p.sample_min_stride;
        ta.rank_scale = p.rank_scale;
        ta.tau = (float *)w->tau.ptr;
        ta.cnt = (uint32_t *)w->cnt.ptr;
        k_tau<<<dim3((unsigned)((T + kTauWaves - 1) / kTauWaves)), 64 * kTauWaves, 0, stream>>>(ta);
    }
    mark(*w, p, 2, stream);

    if (!recover_all) {
        if (few)
            launch_few_dt(p.dtype, kModeFilter, dim3((unsigned)std::max<int64_t>(1, (S + kFewChunk - 1) / kFewChunk)),
                          stream, sa);
        else
            launch_score_dt(p.dtype, kModeFilter, dim3((unsigned)(ntiles * nchunks)), stream, sa);
    }
    mark(*w, p, 3, stream);

    SelectArgs se{};
    se.ks = ks;
    se.ke = ke;
    se.topk = p.topk;
    se.cap = p.cap;
    se.recover_all = recover_all ? 1 : 0;
    se.cnt = (const uint32_t *)w->cnt.ptr;
    se.cand = (const uint64_t *)w->cand.ptr;
    se.out_idx = out_idx;
    se.out_val = out_val;
    se.out_flags = p.out_flags;
    auto select_rows = [&]() {
        if (p.cap <= SelSmallK::nreg * SelSmallK::nt && p.topk <= SelSmallK::maxk) launch_select<SelSmallK>(T, stream, se);
        else if (p.cap <= SelSmall::nreg * SelSmall::nt && p.topk <= SelSmall::maxk) launch_select<SelSmall>(T, stream, se);
        else if (p.cap <= SelMid::nreg * SelMid::nt) launch_select<SelMid>(T, stream, se);
        else if (p.cap <= SelLargeK::nreg * SelLargeK::nt && p.topk <= SelLargeK::maxk) launch_select<SelLargeK>(T, stream, se);
        else if (p.cap <= SelLarge::nreg * SelLarge::nt) launch_select<SelLarge>(T, stream, se);
        else launch_select<SelHuge>(T, stream, se);
    };
    hipError_t e = hipSuccess;
    if (!w->stats_ev && (e = hipEventCreateWithFlags(&w->stats_ev, hipEventDisableTiming)) != hipSuccess)
        return hip_status(e);
    auto copy_stats = [&]() -> hipError_t {
        hipError_t ce = hipMemcpyAsync(w->host_stats, w->stats.ptr, sizeof(unsigned long long) * kStCount,
                                       hipMemcpyDeviceToHost, stream);
        if (ce == hipSuccess) ce = hipEventRecord(w->stats_ev, stream);
        return ce;
    };
    // Dense rescoring of flagged entries [rb, rb + rcap) of the list.
    auto recover_batch = [&](int64_t rb, int64_t rcap, int64_t stride) {
        sa.rowlist = (const int32_t *)w->rowlist.ptr;
        sa.nrows = (const unsigned long long *)w->stats.ptr + kStFlagged;
        sa.row_limit = (int)rcap;
        sa.scratch = (float *)w->scratch.ptr;
        sa.scratch_stride = stride;
        sa.row_base = (int)rb;
        if (few) {
            launch_few_dt(p.dtype, kModeDense,
                          dim3((unsigned)(rcap * std::max<int64_t>(1, (S + kFewChunk - 1) / kFewChunk))), stream, sa);
        } else {
            sa.ntiles = (int)((rcap << ps) / kTileQ);
            sa.chunk = chunk_keys(sa.ntiles, S, ScoreCfg<kFP8, kModeDense>::waves);
            const int rchunks = (int)std::max<int64_t>(1, (S + sa.chunk - 1) / sa.chunk);
            launch_score_dt(p.dtype, kModeDense, dim3((unsigned)(sa.ntiles * rchunks)), stream, sa);
        }
        // Exact top k of each batch row's window scores: the row top-k
        // kernels in mapped-row mode (outputs to the flagged row, indices
        // offset by its window start; entries past the list exit).
        RowsArgs ra{};
        ra.x = w->scratch.ptr;
        ra.rows = rcap;
        ra.cols = S;
        ra.stride = stride;
        ra.topk = p.topk;
        ra.out_idx = out_idx;
        ra.out_val = out_val;
        ra.out_flags = p.out_flags;
        ra.rowmap = (const int32_t *)w->rowlist.ptr;
        ra.nrows = (const unsigned long long *)w->stats.ptr + kStFlagged;
        ra.row_base = rb;
        ra.ks = ks;
        ra.ke = ke;
        if (p.topk <= RowsSmall::maxk) launch_rows<float, RowsSmall>(ra, stream);
        else launch_rows<float, RowsLarge>(ra, stream);
    };
    // Scratch rows of float scores, 16-byte aligned (the row kernels' loads).
    const int64_t stride = (std::max<int64_t>(S, 1) + 3) / 4 * 4;

    // Few rows whose whole windows fit the recovery budget: the selection
    // does each row's triage, recovery of every row is launched up front
    // (rows that need none exit at once), and the call returns without
    // waiting for the GPU; the statistics are read when asked for.
    const bool speculative = few && !p.profile && (int64_t)sizeof(float) * T * stride <= p.recover_budget;
    int64_t R = 0;
    if (speculative) {
        if ((st = ensure(*w, w->scratch, sizeof(float) * (size_t)T * stride))) return st;
        se.triage = 1;
        se.rowlist_w = (int32_t *)w->rowlist.ptr;
        se.stats_w = (unsigned long long *)w->stats.ptr;
        select_rows();
        mark(*w, p, 4, stream);
        mark(*w, p, 5, stream);
        mark(*w, p, 6, stream);
        recover_batch(0, T, stride);
        if ((e = copy_stats()) != hipSuccess) return hip_status(e);
        if ((e = hipGetLastError()) != hipSuccess) return hip_status(e);
    } else {
        TriageArgs tr{};
        tr.ks = ks;
        tr.ke = ke;
        tr.num_q = T;
        tr.topk = p.topk;
        tr.cap = p.cap;
        tr.cnt = (const uint32_t *)w->cnt.ptr;
        tr.recover_all = recover_all ? 1 : 0;
        tr.rowlist = (int32_t *)w->rowlist.ptr;
        tr.stats = (unsigned long long *)w->stats.ptr;
        if (T <= kTriageFewRows)
            k_triage<1><<<dim3((unsigned)((T + kTriageThreads - 1) / kTriageThreads)), kTriageThreads, 0, stream>>>(tr);
        else
            k_triage<16><<<dim3((unsigned)((T + 16 * kTriageThreads - 1) / (16 * kTriageThreads))), kTriageThreads, 0,
                           stream>>>(tr);
        // The triage counts go to pinned host memory right away; the host
        // waits for them (not for the stream) while the select kernel runs,
        // so the GPU never idles on the host between calls.
        if ((e = copy_stats()) != hipSuccess) return hip_status(e);
        mark(*w, p, 4, stream);
        select_rows();
        mark(*w, p, 5, stream);

        e = hipGetLastError();
        if (e == hipSuccess) e = hipEventSynchronize(w->stats_ev);
        if (e != hipSuccess) return hip_status(e);

        R = (int64_t)w->host_stats[kStFlagged];
        mark(*w, p, 6, stream);  // recovery timed from here (0 when nothing is flagged)
        if (R > 0) {
            // Dense rescoring of flagged rows, in batches that fit the budget.
            int64_t rcap = std::max<int64_t>(kTileQ, p.recover_budget / (int64_t)(sizeof(float) * stride));
            rcap = std::min<int64_t>(rcap, (R + kTileQ - 1) / kTileQ * kTileQ);
            rcap = (rcap + kTileQ - 1) / kTileQ * kTileQ;
            if ((st = ensure(*w, w->scratch, sizeof(float) * (size_t)rcap * stride))) return st;
            for (int64_t rb = 0; rb < R; rb += rcap) recover_batch(rb, rcap, stride);
            e = hipGetLastError();
            if (e != hipSuccess) return hip_status(e);
        }
    }
    float ms_rec = 0.0f;
    if (p.profile) {
        hipEvent_t end = nullptr;
        (void)hipEventCreate(&end);
        (void)hipEventRecord(end, stream);
        (void)hipEventSynchronize(end);
        if (hipEventElapsedTime(&ms_rec, w->ev[6], end) != hipSuccess) {
            (void)hipGetLastError();
            ms_rec = 0.0f;
        }
        (void)hipEventDestroy(end);
    }

    // The call's record; its counts are filled in from the statistics once
    // they have reached the host (now, or on the first read of a
    // speculative call's record).
    flashtopk_info &info = w->last;
    std::memset(&info, 0, sizeof(info));
    info.status = FLASHTOPK_OK;
    info.rows = T;
    info.cand_capacity = p.cap;
    info.sample_target = p.sample_target;
    info.ms_sample = phase_ms(*w, p, 0);
    info.ms_tau = phase_ms(*w, p, 1);
    info.ms_filter = phase_ms(*w, p, 2);
    info.ms_triage = phase_ms(*w, p, 3);
    info.ms_select = phase_ms(*w, p, 4);
    info.ms_recover = R > 0 ? ms_rec : 0.0f;
    info.invalid = (int32_t)p.invalid;
    w->last_recover_all = recover_all;
    w->has_last = true;
    w->last_pending = true;
    if (!speculative) fill_counts(*w);
    return FLASHTOPK_OK;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Row top-k launch.  When the rows take more than one wave of resident
// workgroups, the thresholds are computed up front by k_rows_tau, so that no
// row workgroup waits on its sample.
template <typename T, typename SH>
void launch_rows(const RowsArgs &a, hipStream_t s)
{
    static int per_cu = 0;
    if (per_cu == 0) {
        int b = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, k_topk_rows<T, SH, true>, SH::nt, 0) != hipSuccess ||
            b < 1)
            b = 1;
        per_cu = b;
    }
    const dim3 grid((unsigned)a.rows);
    if (a.rows > (int64_t)per_cu * num_cu()) {
        const dim3 tgrid((unsigned)((a.rows + kRowsTauWaves - 1) / kRowsTauWaves));
        hipLaunchKernelGGL((k_rows_tau<T, SH>), tgrid, dim3(64 * kRowsTauWaves), 0, s, a);
        hipLaunchKernelGGL((k_topk_rows<T, SH, true>), grid, dim3(SH::nt), 0, s, a);
    } else {
        hipLaunchKernelGGL((k_topk_rows<T, SH, false>), grid, dim3(SH::nt), 0, s, a);
    }
}

// options.validate: runs k_validate on the call's inputs, waits for its flags
// (p.invalid) and, when it found any, fails the call before a scoring kernel
// runs, recording it as the stream's last call.
int check_inputs(hipStream_t s, Plan &p, ValidateArgs va)
{
    int st = FLASHTOPK_OK;
    Workspace *w = get_ws(s, &st);
    if (!w) return st;
    if ((st = ensure(*w, w->vflag, sizeof(unsigned)))) return st;
    va.flags = (unsigned *)w->vflag.ptr;
    va.dtype = p.dtype == FLASHTOPK_FP8_E4M3 ? kFP8 : kBF16;
    const int64_t n = std::max({va.q_pieces, va.kv_pieces, va.nw, va.nscales, va.num_q, va.ntable, (int64_t)1});
    const unsigned grid = (unsigned)std::min<int64_t>(2048, (n + 255) / 256);
    k_zero_word<<<1, 64, 0, s>>>(va.flags);
    k_validate<<<grid, 256, 0, s>>>(va);
    unsigned *hf = reinterpret_cast<unsigned *>(w->host_stats + kStCount);
    hipError_t e = hipMemcpyAsync(hf, va.flags, sizeof(unsigned), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_status(e);
    p.invalid = *hf;
    if (p.invalid) {
        flashtopk_info &info = w->last;
        std::memset(&info, 0, sizeof(info));
        info.status = FLASHTOPK_ERR_INVALID_ARGUMENT;
        info.rows = p.T;
        info.invalid = (int32_t)p.invalid;
        w->has_last = true;
        w->last_pending = false;
        return FLASHTOPK_ERR_INVALID_ARGUMENT;
    }
    return FLASHTOPK_OK;
}

}  // namespace

extern "C" {

int flashtopk_select_ex(const void *q, const void *kv, const float *kv_scales, const float *weights,
                        const int32_t *ks, const int32_t *ke, int64_t num_q, int64_t num_kv, int dtype,
                        int topk, void *out_idx, float *out_val, void *stream,
                        const flashtopk_options *opt)
{
    if (dtype != FLASHTOPK_FP8_E4M3 && dtype != FLASHTOPK_BF16) return FLASHTOPK_ERR_UNSUPPORTED;
    if (num_q < 0 || num_kv < 0 || num_kv >= (int64_t(1) << 31) || num_q >= (int64_t(1) << 31))
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
        if ((st = check_inputs((hipStream_t)stream, p, va))) return st;
    }
    return run(q, kv, kv_scales, weights, ks, ke, out_idx, out_val, (hipStream_t)stream, p);
}

int flashtopk_select_paged(const void *q, const void *kv_pages, const float *scale_pages, const int32_t *block_table,
                           int page_size, int64_t num_pages, const float *weights, const int32_t *ks,
                           const int32_t *ke, int64_t num_q, int64_t num_kv, int dtype, int topk, void *out_idx,
                           float *out_val, void *stream, const flashtopk_options *opt)
{
    if (dtype != FLASHTOPK_FP8_E4M3 && dtype != FLASHTOPK_BF16) return FLASHTOPK_ERR_UNSUPPORTED;
    if (num_q < 0 || num_kv < 0 || num_kv >= (int64_t(1) << 31) || num_q >= (int64_t(1) << 31))
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
        if ((st = check_inputs((hipStream_t)stream, p, va))) return st;
    }
    if (num_kv == 0) return run(q, nullptr, nullptr, weights, ks, ke, out_idx, out_val, (hipStream_t)stream, p);
    const hipStream_t s = (hipStream_t)stream;
    if (num_q <= kFewRows && p.heads == 32) {
        // few rows read their keys from the pages directly
        p.table = block_table;
        p.page_size = page_size;
        p.num_pages = num_pages;
        return run(q, kv_pages, scale_pages, weights, ks, ke, out_idx, out_val, s, p);
    }
    Workspace *w = get_ws(s, &st);
    if (!w) return st;
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
    return run(q, w->pkv.ptr, sig, weights, ks, ke, out_idx, out_val, s, p);
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
    RowsArgs a{x, rows, cols, row_stride, ends, topk, out_idx, out_val, nan_flag, out_flags};
    const hipStream_t s = (hipStream_t)stream;
    const bool small = topk <= RowsSmall::maxk;
    if (score_dtype == FLASHTOPK_SCORES_F32) {
        if (small) launch_rows<float, RowsSmall>(a, s);
        else launch_rows<float, RowsLarge>(a, s);
    } else {
        if (small) launch_rows<uint16_t, RowsSmall>(a, s);
        else launch_rows<uint16_t, RowsLarge>(a, s);
    }
    return hip_status(hipGetLastError());
}

int flashtopk_reserve(int64_t max_q, int64_t max_kv, int max_topk, int dtype, void *stream)
{
    if (dtype != FLASHTOPK_FP8_E4M3 && dtype != FLASHTOPK_BF16) return FLASHTOPK_ERR_UNSUPPORTED;
    if (max_q < 0 || max_kv < 0 || max_topk < 1 || max_topk > FLASHTOPK_MAX_TOPK)
        return FLASHTOPK_ERR_INVALID_ARGUMENT;
    int st = FLASHTOPK_OK;
    Workspace *w = get_ws((hipStream_t)stream, &st);
    if (!w) return st;
    const int64_t T = std::max<int64_t>(max_q, 1);
    const int cap = std::min(kMaxCap, std::max(4 * max_topk, max_topk));
    if ((st = ensure(*w, w->tau, sizeof(float) * T))) return st;
    if ((st = ensure(*w, w->cnt, sizeof(uint32_t) * T))) return st;
    if ((st = ensure(*w, w->rowlist, sizeof(int32_t) * T))) return st;
    if ((st = ensure(*w, w->stats, sizeof(unsigned long long) * kStCount))) return st;
    if ((st = ensure(*w, w->cand, sizeof(uint64_t) * (size_t)T * cap))) return st;
    if ((st = ensure(*w, w->samp, sizeof(uint32_t) * (size_t)T * kDefaultSampleTarget))) return st;
    if ((st = ensure(*w, w->sigh, sizeof(float) * (size_t)(max_kv + 64)))) return st;
    if ((st = ensure(*w, w->q1, sizeof(float) * (size_t)T))) return st;
    if ((st = ensure_zeroed(*w, w->ticket, sizeof(uint32_t) * T))) return st;
    if (dtype == FLASHTOPK_FP8_E4M3) {
        if ((st = ensure(*w, w->qbar, (size_t)T * kQbarParts * kDim))) return st;
        if ((st = ensure(*w, w->qscale, sizeof(float) * T))) return st;
    }
    if (max_kv > 0) {
        const int64_t nblocks = (max_kv + kBlockKeys - 1) / kBlockKeys;
        const int64_t ntiles = (T + kTileQ - 1) / kTileQ;
        if ((st = ensure(*w, w->kb, (size_t)nblocks * 2 * (dtype == FLASHTOPK_FP8_E4M3 ? 128 : 256)))) return st;
        if ((st = ensure(*w, w->kmeta, sizeof(float2) * (size_t)nblocks))) return st;
        if ((st = ensure(*w, w->vplan, sizeof(float) * (size_t)ntiles * kPlanGroups * 256))) return st;
    }
    return FLASHTOPK_OK;
}

int flashtopk_get_last_info(void *stream, flashtopk_info *out)
{
    if (!out) return FLASHTOPK_ERR_INVALID_ARGUMENT;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e);
    std::lock_guard<std::mutex> lk(g_mu);
    for (Workspace *w : g_ws) {
        if (w->device == dev && w->stream == (hipStream_t)stream && w->has_last) {
            if (w->last_pending) {
                e = hipEventSynchronize(w->stats_ev);
                if (e != hipSuccess) return hip_status(e);
                fill_counts(*w);
            }
            *out = w->last;
            return FLASHTOPK_OK;
        }
    }
    std::memset(out, 0, sizeof(*out));
    return FLASHTOPK_ERR_INVALID_ARGUMENT;
}

void flashtopk_release(void)
{
    std::lock_guard<std::mutex> lk(g_mu);
    for (Workspace *w : g_ws) {
        int prev = 0;
        (void)hipGetDevice(&prev);
        (void)hipSetDevice(w->device);
        (void)hipStreamSynchronize(w->stream);
        DevBuf *bufs[] = {&w->tau, &w->cnt, &w->rowlist, &w->stats,
                          &w->cand, &w->samp, &w->scratch, &w->qbar, &w->qscale, &w->sigh,
                          &w->kb, &w->kmeta, &w->vplan, &w->q1, &w->ticket, &w->pkv, &w->psig, &w->vflag};
        for (DevBuf *b : bufs)
            if (b->ptr) (void)hipFree(b->ptr);
        if (w->host_stats) (void)hipHostFree(w->host_stats);
        for (hipEvent_t &ev : w->ev)
            if (ev) (void)hipEventDestroy(ev);
        if (w->stats_ev) (void)hipEventDestroy(w->stats_ev);
        (void)hipSetDevice(prev);
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
    default: return "unknown status";
    }
}

int flashtopk_version(void) { return 100; }

}  // extern "C"
