// Shared device definitions of the gfx950 indexer top-k kernels: geometry,
// operand vector types and the 64-bit selection key.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ftk {

// Indexer geometry: 32 heads of 128 dimensions sharing one key per token
// (FlashTopK README, "Support": indexers of 32 heads x 128).
constexpr int kHeads = 32;
constexpr int kDim = 128;

// Work decomposition.  A tile is 16 query rows: the N = 16 columns of a
// 16x16 MFMA output.  A wave scores kSub 16-key subtiles per step (the M = 16
// rows), the waves of a workgroup share a tile, and a work item covers one
// chunk of keys (a power of two between kMinChunk and kMaxChunk, chosen per
// call so there are enough work items to fill the GPU).
constexpr int kTileQ = 16;
constexpr int kSub = 4;
constexpr int kStepKeys = 16 * kSub;      // 64 keys per wave step
constexpr int kMinChunk = 1024;
constexpr int kMaxChunk = 131072;

constexpr int kFP8 = 0;
constexpr int kBF16 = 1;

// FP8 rows whose window holds at most this many keys are scored in the plain
// form sigma * sum_h w ReLU(x_h); longer rows through the linear identity.
// The identity's error is absolute (set by the query sum's truncation), while
// the score tolerance scales with the row's largest score, and on a short
// window that can be as small as one key's score.  The form depends only on
// the row's own window, so every path and batch gives a row the same bits.
constexpr int kPlainKeys = 4096;

__device__ __forceinline__ bool plain_row(int ks, int ke)
{
    return ke > ks && ke - ks <= kPlainKeys;
}

// 2 ReLU(x) for p = 1 and |x| for p = 0, exactly (one FMA, |x| as a source
// modifier): x + |x| is 2x or +0, and |x| + (+-0) is |x|.
__device__ __forceinline__ float relu2_or_abs(float p, float x)
{
    return __builtin_fmaf(p, x, __builtin_fabsf(x));
}

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// Bytes of one key row (or one query head row) per dtype.
template <int DT> struct RowBytes { static constexpr int value = DT == kFP8 ? 128 : 256; };

// Order-preserving map of a binary32 score onto uint32: a larger score gives
// a larger code, and -0 folds into +0 so the two compare equal.
__device__ __forceinline__ uint32_t ord_of(float f)
{
    uint32_t b = __float_as_uint(f);
    if (b == 0x80000000u) b = 0u;
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ float float_of_ord(uint32_t u)
{
    return __uint_as_float((u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
}

// 64-bit selection key: score code in the high word, the complement of the
// key index in the low word.  Ordering keys descending gives score
// descending and, among equal scores, the smaller key index first: the
// tie rule of the FlashTopK README, "What you can do" (an equal score at
// the k-th place goes to the lower index).  Keys of distinct indices are
// distinct.
__device__ __forceinline__ uint64_t sel_key(float score, int32_t s)
{
    return ((uint64_t)ord_of(score) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)s);
}

// Raw candidate as the scoring kernels write it: the binary32 score bits in
// the low word, the key index in the high word.  The selection kernels turn
// it into the ordered key above when they load it.
__device__ __forceinline__ uint64_t raw_cand(float score, int32_t s)
{
    return ((uint64_t)(uint32_t)s << 32) | (uint64_t)__float_as_uint(score);
}

__device__ __forceinline__ uint64_t key_of_raw(uint64_t r)
{
    return sel_key(__uint_as_float((uint32_t)r), (int32_t)(r >> 32));
}

__device__ __forceinline__ int32_t key_index(uint64_t k)
{
    return (int32_t)(0xFFFFFFFFu - (uint32_t)k);
}

__device__ __forceinline__ float key_score(uint64_t k)
{
    return float_of_ord((uint32_t)(k >> 32));
}

// ReLU as an integer max on the bit pattern: non-negative floats have
// non-negative int32 patterns, negative floats negative ones.  Exact for every
// finite input (and -0 becomes +0); one VALU op with no NaN canonicalisation.
__device__ __forceinline__ float relu_bits(float x)
{
    return __int_as_float(max(__float_as_int(x), 0));
}

// The row's strided sample is a lattice of short runs: the keys p with
// p mod (kRunKeys d) < kRunKeys, for a power of two d.  Runs of 4 keys let a
// lane's four outputs of a subtile (four consecutive lattice keys) share one
// scale-factor load and one sample store, while a 2048-key sample still
// spans 512 places of the window (keys with block structure need many
// independent places; 64-key runs gave 32 and misjudged such rows).
constexpr int kRunKeys = 4;
constexpr int kRunShift = 2;

// Stride of the row's sample: the smallest power of two d >= min_stride
// with len <= target * d.  The window then holds at most target + 2
// kRunKeys lattice keys (two partial runs); the kernels keep the first
// `target` of them.  (min_stride keeps the sample no denser than the
// threshold needs.)
__device__ __host__ __forceinline__ int sample_stride(int64_t len, int target, int min_stride)
{
    int d = min_stride;
    while (len > (int64_t)target * d) d <<= 1;
    return d;
}

// Which run of each period a lattice uses: slot sl of stride d holds the
// keys p with (p / kRunKeys) mod d == sl.  The slot comes from a hash of the
// 16-row tile that scores the row's sample, taken mod d: rows of one tile
// then share their keys (a row of stride dn >= dmin uses slot h mod dn,
// whose runs lie on the tile's lattice, slot h mod dmin), while different
// tiles sample different keys, so no single choice of keys biases every
// row's threshold the same way.
__device__ __host__ __forceinline__ uint32_t lattice_hash(int64_t tile)
{
    uint32_t x = (uint32_t)tile * 0x9E3779B1u;
    x ^= x >> 15;
    x *= 0x85EBCA77u;
    x ^= x >> 13;
    return x;
}

// Lattice keys (stride 2^dsh, slot sl) in [0, x).
__device__ __host__ __forceinline__ int64_t lattice_prefix_sh(int64_t x, int dsh, int sl)
{
    const int64_t y = x - (int64_t)sl * kRunKeys;
    if (y <= 0) return 0;
    const int64_t r = y & (((int64_t)kRunKeys << dsh) - 1);
    return ((y >> (kRunShift + dsh)) << kRunShift) + (r < kRunKeys ? r : kRunKeys);
}

// Key of lattice index e (stride 2^dsh, slot sl; index 0 is the slot's first key).
__device__ __host__ __forceinline__ int64_t lattice_key(int64_t e, int dsh, int sl)
{
    return (int64_t)sl * kRunKeys + ((e >> kRunShift) << (kRunShift + dsh)) + (e & (kRunKeys - 1));
}

// Lattice keys (stride d = 2^dsh, slot sl) in [lo, hi).
__device__ __host__ __forceinline__ int64_t lattice_count(int64_t lo, int64_t hi, int dsh, int sl)
{
    if (hi <= lo) return 0;
    return lattice_prefix_sh(hi, dsh, sl) - lattice_prefix_sh(lo, dsh, sl);
}

// Slot of stride 2^dsh for the rows of tile `tile`.
__device__ __host__ __forceinline__ int lattice_slot(int64_t tile, int dsh)
{
    return (int)(lattice_hash(tile) & ((1u << dsh) - 1u));
}

// ---------------------------------------------------------------------------
// Wave-wide scans and reductions over the 64 lanes through DPP lane moves
// (every lane must be active).  Rows of 16 lanes scan with row shifts of 1,
// 2, 4, 8 (lanes shifted in from outside the row read 0); row 15's and row
// 31's last lanes are then broadcast into the rows above them.

template <int CTRL, int ROW_MASK = 0xf, bool ZERO_FILL = true>
__device__ __forceinline__ uint32_t dpp_move(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xf, ZERO_FILL);
}

template <typename Op>
__device__ __forceinline__ uint32_t wave_scan_dpp(uint32_t x, Op op)
{
    x = op(x, dpp_move<0x111>(x));        // row_shr:1
    x = op(x, dpp_move<0x112>(x));        // row_shr:2
    x = op(x, dpp_move<0x114>(x));        // row_shr:4
    x = op(x, dpp_move<0x118>(x));        // row_shr:8
    x = op(x, dpp_move<0x142, 0xa>(x));   // row_bcast:15 into rows 1 and 3
    x = op(x, dpp_move<0x143, 0xc>(x));   // row_bcast:31 into rows 2 and 3
    return x;
}

// Inclusive prefix sum: lane l gets x_0 + ... + x_l.
__device__ __forceinline__ uint32_t wave_incl_add(uint32_t x)
{
    return wave_scan_dpp(x, [](uint32_t a, uint32_t b) { return a + b; });
}

// Sum and maximum over the wave, returned to every lane.
__device__ __forceinline__ uint32_t wave_sum(uint32_t x)
{
    return (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_add(x), 63);
}

__device__ __forceinline__ uint32_t wave_max(uint32_t x)
{
    return (uint32_t)__builtin_amdgcn_readlane(
        (int)wave_scan_dpp(x, [](uint32_t a, uint32_t b) { return a > b ? a : b; }), 63);
}

// Counters of the score-bound pruning, kept in the call's statistics (zeroed
// by the per-key pass, added to by the scan): (row, key) pairs skipped, and
// work items that evaluated the bound.
enum PlanCounter { kPlanPruned = 0, kPlanItems, kPlanCount };

}  // namespace ftk
