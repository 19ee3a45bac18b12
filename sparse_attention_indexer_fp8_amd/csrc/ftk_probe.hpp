// Matrix-core throughput probe: the attainable rate of the scan's MFMA
// instructions on this GPU under sustained load, the ceiling the scan's
// roofline fraction is read against (the published dense peaks assume the
// 2.4 GHz peak engine clock).
//
// Every wave issues `iters` rounds of kProbeChains independent accumulation
// chains of one MFMA each, on operands held in registers (fixed per-lane
// pseudo-random codes of both signs, finite): no memory traffic and no other
// vector work in the loop.  FP8: v_mfma_f32_16x16x128_f8f6f4 (E4M3 x E4M3,
// 65536 FLOPs); BF16: v_mfma_f32_32x32x16_bf16 (32768 FLOPs).  Four waves per
// SIMD, as in the FP8 scan.
#pragma once

#include "ftk_common.hpp"

namespace ftk {

constexpr int kProbeChains = 4;
constexpr int kProbeThreads = 256;  // four waves per workgroup, four workgroups per compute unit

typedef float v16f_probe __attribute__((ext_vector_type(16)));

// Written only if the accumulators sum to `never` (the host passes a NaN,
// which no sum equals), so the MFMAs are live but nothing is stored.
__device__ float g_probe_sink[64];

__device__ __forceinline__ uint32_t probe_next(uint32_t &h)
{
    h ^= h << 13;  // xorshift32
    h ^= h >> 17;
    h ^= h << 5;
    return h;
}

template <int DT>
__global__ __launch_bounds__(kProbeThreads) __attribute__((amdgpu_waves_per_eu(4))) void k_probe_mfma(int iters, float never)
{
    const int lane = threadIdx.x & 63;
    uint32_t h = (blockIdx.x * (uint32_t)kProbeThreads + threadIdx.x) * 2654435761u + 0x9E3779B9u;
    float s = 0.0f;
    if constexpr (DT == kFP8) {
        v8i a[kProbeChains], b[kProbeChains];
        v4f c[kProbeChains];
#pragma unroll
        for (int k = 0; k < kProbeChains; ++k) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                // low bit of every byte cleared: no E4M3 NaN code (0x7F, 0xFF)
                a[k][e] = (int)(probe_next(h) & 0xFEFEFEFEu);
                b[k][e] = (int)(probe_next(h) & 0xFEFEFEFEu);
            }
            c[k] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};
        }
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int k = 0; k < kProbeChains; ++k)
                c[k] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[k], b[k], c[k], 0, 0, 0, 0, 0, 0);
        }
#pragma unroll
        for (int k = 0; k < kProbeChains; ++k) s += c[k][0] + c[k][1] + c[k][2] + c[k][3];
    } else {
        v4i a[kProbeChains], b[kProbeChains];
        v16f_probe c[kProbeChains];
#pragma unroll
        for (int k = 0; k < kProbeChains; ++k) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                // BF16 pairs with exponents 120..135 (magnitudes 2^-7 .. 2^8)
                auto code = [&]() {
                    const uint32_t r = probe_next(h);
                    return ((r & 0x8000u) | ((120u + ((r >> 7) & 15u)) << 7) | (r & 0x7Fu)) & 0xFFFFu;
                };
                a[k][e] = (int)(code() | (code() << 16));
                b[k][e] = (int)(code() | (code() << 16));
            }
            c[k] = (v16f_probe){};
        }
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int k = 0; k < kProbeChains; ++k)
                c[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, a[k]),
                                                              __builtin_bit_cast(v8bf, b[k]), c[k], 0, 0, 0);
        }
#pragma unroll
        for (int k = 0; k < kProbeChains; ++k)
#pragma unroll
            for (int r = 0; r < 16; ++r) s += c[k][r];
    }
    if (s == never) g_probe_sink[lane] = s;
}

}  // namespace ftk
