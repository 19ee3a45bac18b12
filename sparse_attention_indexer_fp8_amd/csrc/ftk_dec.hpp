// Dense scoring for calls of a few rows (decode, a few speculative tokens).
//
// The tile kernel puts 16 query rows on the MFMA's N dimension; with one row
// 15 of its 16 columns are empty.  Here the N dimension holds the row's heads
// instead: an FP8 16x16x128 MFMA takes 16 keys x 16 heads (two per 16 keys
// for 32 heads), a BF16 32x32x16 chain takes 32 keys x 32 heads.  Every
// (key, head) dot product is the same instruction on the same operand
// slices as in the tile kernel (the MFMA computes each output element from
// its own A row and B column), and the FP8 linear half q̄ . k is the tile
// kernel's own chain (its B columns are the rows, as there).  The products
// then go through LDS so that one lane holds all 32 heads of one (row, key)
// pair and sums them in the tile kernel's order: FP8 w |x| fused
// multiply-adds seeded with the linear half, heads 0..31; BF16 w ReLU(x)
// for heads 0..15 and 16..31 from zero, then the two halves added.  So the
// scores are bit-identical to the tile kernel's, and a row's results do not
// depend on which kernel scored it.
//
// One wave scores one 64-key step for every row of the call; the grid
// covers the union of the rows' windows in steps.  Scores go to the
// workspace (row e of the batch at scratch + e * stride, by window position)
// for the row top-k kernels, as in the tile kernel's dense mode.
#pragma once

#include "ftk_qbar.hpp"
#include "ftk_score.hpp"

namespace ftk {

constexpr int kDecRows = 4;    // rows per call scored this way
constexpr int kDecWaves = 4;
constexpr int kDecLd = 33;     // LDS words per key row of the transpose (32 heads + 1: no bank conflicts)

template <int DT>
__global__ __launch_bounds__(64 * kDecWaves) void k_score_dec(ScoreArgs a)
{
    static_assert(kDecRows <= kDecWaves, "one wave per row computes the query sums");
    constexpr int RB = RowBytes<DT>::value;
    __shared__ float s_x[kDecWaves][kStepKeys * kDecLd];   // per wave: [64 keys][32 heads (+1)]
    __shared__ float s_lin[kDecWaves][kStepKeys];          // FP8: the linear half of the row being summed
    __shared__ __attribute__((aligned(16))) uint8_t s_parts[kDecRows * kQbarParts * kDim];
    __shared__ float s_qsc[kDecRows];
    __shared__ float s_w[kDecRows * kHeads];
    __shared__ int s_ks[kDecRows], s_ke[kDecRows];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t nb = min((int64_t)a.nrows_direct - a.row_base, (int64_t)a.row_limit);
    const int T = (int)max<int64_t>(0, min<int64_t>(nb, kDecRows));
    const uint8_t *q0 = a.q + (int64_t)a.row_base * kHeads * RB;
    const float *w0 = a.w + (int64_t)a.row_base * kHeads;

    if (threadIdx.x < kDecRows) {
        const int e = threadIdx.x;
        int lo = 0, hi = 0;
        if (e < T) {
            lo = a.ks[a.row_base + e];
            hi = max(a.ke[a.row_base + e], lo);
            if (blockIdx.x == 0 && a.wlen) a.wlen[a.row_base + e] = hi - lo;
        }
        s_ks[e] = lo;
        s_ke[e] = hi;
    }
    for (int i = threadIdx.x; i < kDecRows * kHeads; i += blockDim.x)
        s_w[i] = (i / kHeads) < T ? w0[i] : 0.0f;
    if constexpr (DT == kFP8) {
        // The rows' query-sum parts and scales, by the preparation pass's own
        // code (one wave per row), into LDS.
        qbar_rows(q0, w0, T, s_parts, s_qsc, nullptr, 0);
        // parts of absent rows read as zeros
        for (int i = threadIdx.x; i < kDecRows * kQbarParts * kDim; i += blockDim.x)
            if (i / (kQbarParts * kDim) >= T) s_parts[i] = 0;
        if (threadIdx.x < kDecRows && (int)threadIdx.x >= T) s_qsc[threadIdx.x] = 1.0f;
    }
    __syncthreads();
    int lo = 0x7fffffff, hi = 0;
    for (int e = 0; e < T; ++e)
        if (s_ke[e] > s_ks[e]) {
            lo = min(lo, s_ks[e]);
            hi = max(hi, s_ke[e]);
        }
    if (hi <= lo) return;
    const int S = a.num_kv;
    using LY = StepLayout<DT>;
    float *xs = s_x[wave];

    for (int j = (lo >> 6) + blockIdx.x * kDecWaves + wave; j * kStepKeys < hi; j += gridDim.x * kDecWaves) {
        const int k0 = j * kStepKeys;
        KFrag<DT> kf[kSub];
#pragma unroll
        for (int kt = 0; kt < kSub; ++kt)
            load_kfrag_at(kf[kt], a.kv + (int64_t)min(k0 + LY::frag_key(kt, lane), S - 1) * RB + LY::frag_byte(kt, lane));
        // the lane's key of the summing phase and its scale factor (sigma / 2
        // on FP8, sigma on BF16, as the preparation pass stores them)
        const int key = k0 + lane;
        float sh = 0.0f;
        if (key < S) {
            const float sg = a.sigma ? a.sigma[key] : 1.0f;
            sh = DT == kFP8 ? sg * 0.5f : sg;
        }

        if constexpr (DT == kFP8) {
            // The linear half for every row at once: the tile kernel's chain,
            // B columns = rows (lane column n holds row n's part).
            const int n = lane & 15, g = lane >> 4;
            v4f lin[kSub];
            {
                const v4f z[kSub] = {};
                const int sb = (int)((__float_as_uint(n < kDecRows ? s_qsc[n] : 1.0f) >> 23) & 0xFFu);
                auto part = [&](int p) -> v8i {
                    if (n >= kDecRows) return (v8i){0, 0, 0, 0, 0, 0, 0, 0};
                    const v4i *src = reinterpret_cast<const v4i *>(s_parts + (n * kQbarParts + p) * kDim + 32 * g);
                    const v4i lo4 = src[0], hi4 = src[1];
                    return (v8i){lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
                };
                const v8i p0 = part(0), p1 = part(1), p2 = part(2);
#pragma unroll
                for (int kt = 0; kt < kSub; ++kt) {
                    lin[kt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(kf[kt].a, p0, z[kt], 0, 0, 0, 127, 0, sb);
                    lin[kt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(kf[kt].a, p1, lin[kt], 0, 0, 0, 127, 0, sb);
                    lin[kt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(kf[kt].a, p2, lin[kt], 0, 0, 0, 127, 0, sb);
                }
            }
            for (int e = 0; e < T; ++e) {
                // heads 16 hf + n of row e, dimensions [32 g, +32)
                const v4f z = {};
                v4f x[2][kSub];
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    const v4i *src =
                        reinterpret_cast<const v4i *>(q0 + ((int64_t)e * kHeads + 16 * hf + n) * RB + 32 * g);
                    const v4i lo4 = src[0], hi4 = src[1];
                    const v8i qf = (v8i){lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
#pragma unroll
                    for (int kt = 0; kt < kSub; ++kt)
                        x[hf][kt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(kf[kt].a, qf, z, 0, 0, 0, 0, 0, 0);
                }
                // transpose through LDS: key 16 kt + 4 g + i, head 16 hf + n
#pragma unroll
                for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                    for (int kt = 0; kt < kSub; ++kt)
#pragma unroll
                        for (int i = 0; i < 4; ++i) xs[(16 * kt + 4 * g + i) * kDecLd + 16 * hf + n] = x[hf][kt][i];
                if (n == e) {
#pragma unroll
                    for (int kt = 0; kt < kSub; ++kt)
#pragma unroll
                        for (int i = 0; i < 4; ++i) s_lin[wave][16 * kt + 4 * g + i] = lin[kt][i];
                }
                __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
                __builtin_amdgcn_wave_barrier();
                const float *xr = xs + lane * kDecLd;
                const float *wr = s_w + e * kHeads;
                const int rks = s_ks[e], rke = s_ke[e];
                // the row's form, as in the tile kernel: plain rows sum
                // w 2 ReLU(x) from zero, identity rows w |x| from the linear half
                const bool plain = plain_row(rks, rke);
                const float pl = plain ? 1.0f : 0.0f;
                float acc = __builtin_fmaf(wr[0], relu2_or_abs(pl, xr[0]), plain ? 0.0f : s_lin[wave][lane]);
#pragma unroll
                for (int h = 1; h < kHeads; ++h) acc = __builtin_fmaf(wr[h], relu2_or_abs(pl, xr[h]), acc);
                if (key >= rks && key < rke)
                    a.scratch[(int64_t)e * a.scratch_stride + (key - rks)] = acc * sh;
                __builtin_amdgcn_wave_barrier();  // every lane has read before the next row overwrites
            }
        } else {
            // BF16: per 32-key subtile u, a chain of 8 32x32x16 MFMAs with B
            // column l % 32 = head l % 32 of the row (dimensions [64 kb + 8 s,
            // +8) at K step s, kb = l / 32), as the tile kernel's chains.
            const int hcol = lane & 31, kb = lane >> 5;
            for (int e = 0; e < T; ++e) {
                const uint8_t *qr = q0 + ((int64_t)e * kHeads + hcol) * RB + 128 * kb;
                typedef float v16f_ __attribute__((ext_vector_type(16)));
                v16f_ x[2];
                const v16f_ z = {};
#pragma unroll
                for (int st = 0; st < 8; ++st) {
                    const v4i qf = *reinterpret_cast<const v4i *>(qr + 16 * st);
#pragma unroll
                    for (int u = 0; u < 2; ++u)
                        x[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            __builtin_bit_cast(v8bf, kf[2 * u + (st >> 2)].a[st & 3]), __builtin_bit_cast(v8bf, qf),
                            st ? x[u] : z, 0, 0, 0);
                }
                // lane l, register r: key 8 (r / 4) + 4 (l / 32) + r % 4 of subtile u, head l % 32
#pragma unroll
                for (int u = 0; u < 2; ++u)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        xs[(32 * u + 8 * (r >> 2) + 4 * kb + (r & 3)) * kDecLd + hcol] = x[u][r];
                __builtin_amdgcn_s_waitcnt(0xc07f);
                __builtin_amdgcn_wave_barrier();
                const float *xr = xs + lane * kDecLd;
                const float *wr = s_w + e * kHeads;
                float h0 = 0.0f, h1 = 0.0f;
#pragma unroll
                for (int h = 0; h < 16; ++h) {
                    h0 = __builtin_fmaf(wr[h], relu_bits(xr[h]), h0);
                    h1 = __builtin_fmaf(wr[16 + h], relu_bits(xr[16 + h]), h1);
                }
                const int rks = s_ks[e], rke = s_ke[e];
                if (key >= rks && key < rke)
                    a.scratch[(int64_t)e * a.scratch_stride + (key - rks)] = (h0 + h1) * sh;
                __builtin_amdgcn_wave_barrier();
            }
        }
    }
}

}  // namespace ftk
