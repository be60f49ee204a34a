// lgn_wide.hpp -- the forward for groups wider than one workgroup tile
// (C = N/G a multiple of 256, up to LayerNorm over all N when G = 1).
//
// Same method as lgn_fused.hpp (POPCORNBENCH "Kimi-K2.6 l2_p37": linear with
// its bias, Swish, external bias, GroupNorm with population variance and eps
// inside the square root, per-channel affine).  A group now spans several
// 256-channel tiles, so its statistics cross workgroups; the transcripts'
// two-stage plan for a reduction wider than a tile (per-block partials, then
// a light second pass) is used:
//   kernel 1: the fused kernel in its WIDE mode (lgn_fused.hpp): the GEMM
//             tile, bias, Swish and bias, then per (row, 64-channel wave span)
//             the partial (mean, M2) -- lane two-pass, then lane^32 with equal
//             counts -- into the workspace, and u written to `out`;
//   kernel 2: one wave per (pair of rows, group) merges each row's partials
//             of the group in a fixed order and normalises `out` in place.
#pragma once

#include "lgn_fused.hpp"

namespace lgn {

constexpr int kWideSpan = 64;    // channels per partial (the fused tile's wave span)

// The (mean, M2) of the group whose partials start at pp: lane t merges
// partials t, t+64, ... in order (equal counts of TILE), then an xor
// butterfly (lower lane first, so both lanes of a pair hold the same bits)
// gives every lane the group's result.
template <int TILE>
__device__ __forceinline__ void wide_group_moments(const float2 *__restrict__ pp,
                                                   int tiles_per_group, int lane, float &mean,
                                                   float &m2) {
    float cnt = 0.f;
    mean = 0.f;
    m2 = 0.f;
    for (int t = lane; t < tiles_per_group; t += 64) {
        const float2 q = pp[t];
        if (cnt == 0.f) {
            mean = q.x;
            m2 = q.y;
        } else {
            const float d = q.x - mean;
            const float f = (float)TILE / (cnt + (float)TILE);
            mean = mean + d * f;
            m2 = m2 + q.y + d * d * (cnt * f);
        }
        cnt += (float)TILE;
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const float om = __shfl_xor(mean, off), om2 = __shfl_xor(m2, off), on = __shfl_xor(cnt, off);
        const bool lower = (lane & off) == 0;
        const float am = lower ? mean : om, am2 = lower ? m2 : om2, an = lower ? cnt : on;
        const float bm = lower ? om : mean, bm2 = lower ? om2 : m2, bn = lower ? on : cnt;
        const float nt = an + bn;
        if (bn == 0.f) {
            mean = am;
            m2 = am2;
        } else if (an == 0.f) {
            mean = bm;
            m2 = bm2;
        } else {
            const float d = bm - am;
            const float f = bn / nt;
            mean = am + d * f;
            m2 = am2 + bm2 + d * d * (an * f);
        }
        cnt = nt;
    }
}

// Kernel 2: one one-wave workgroup per (pair of rows, group) of C =
// tiles_per_group * TILE channels (TILE = channels per partial).  The wave
// forms each row's (mean, M2) from its partials, then normalises both rows'
// float4s of `out` in place, two float4s per row per step, with one load of
// gamma and beta serving both rows.  Against one wave per (row, group) in
// four-wave workgroups this measured 0.2255 -> 0.1965 ms (G = 1) and
// 0.2102 -> 0.1879 ms (G = 8) at 16384 x 8192, bitwise the same output.
constexpr int kWideNormRows = 2;
constexpr int kWideNormUnroll = 2;

template <int TILE>
__global__ __launch_bounds__(64) void lgn_wide_norm_kernel(
    const float2 *__restrict__ part, const float *__restrict__ gamma,
    const float *__restrict__ beta, long long M, int G, int tiles_per_group, int tiles_n,
    float eps, float *out) {
    constexpr int R = kWideNormRows, U = kWideNormUnroll;
    const int lane = threadIdx.x;
    const long long r0 = (long long)R * (blockIdx.x / G);
    const int g = (int)(blockIdx.x % G);
    if (r0 >= M) return;
    const int C = tiles_per_group * TILE;
    float rstd[R], nmr[R];
    f32x4 *rows[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        // a missing last row (odd M) repeats row M-1 and stores nothing
        const long long row = r0 + r < M ? r0 + r : M - 1;
        float mean, m2;
        wide_group_moments<TILE>(part + (size_t)row * tiles_n + (size_t)g * tiles_per_group,
                                 tiles_per_group, lane, mean, m2);
        rstd[r] = __builtin_amdgcn_rsqf(m2 / (float)C + eps);
        nmr[r] = -mean * rstd[r];
        rows[r] = reinterpret_cast<f32x4 *>(out + (size_t)row * (size_t)tiles_n * TILE +
                                            (size_t)g * C);
    }
    const f32x4 *gm = reinterpret_cast<const f32x4 *>(gamma + (size_t)g * C);
    const f32x4 *bt = reinterpret_cast<const f32x4 *>(beta + (size_t)g * C);
    for (int f0 = lane; f0 < C / 4; f0 += 64 * U) {
        f32x4 u[U][R], ga[U], be[U];
#pragma unroll
        for (int i = 0; i < U; ++i) {
            const int f = f0 + 64 * i;
            if (f < C / 4) {
#pragma unroll
                for (int r = 0; r < R; ++r) u[i][r] = rows[r][f];
                ga[i] = gm[f];
                be[i] = bt[f];
            }
        }
#pragma unroll
        for (int i = 0; i < U; ++i) {
            const int f = f0 + 64 * i;
            if (f < C / 4) {
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    f32x4 y;
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        y[j] = __builtin_fmaf(__builtin_fmaf(u[i][r][j], rstd[r], nmr[r]),
                                              ga[i][j], be[i][j]);
                    if (r0 + r < M) rows[r][f] = y;
                }
            }
        }
    }
}

}  // namespace lgn
