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
//   kernel 2: one wave per (row, group) merges the group's partials in a
//             fixed order and normalises `out` in place.
#pragma once

#include "lgn_fused.hpp"

namespace lgn {

constexpr int kWideSpan = 64;    // channels per partial (the fused tile's wave span)

// Kernel 2: one wave per (row, group) of C = tiles_per_group * TILE channels
// (TILE = channels per partial).
// Lane t merges the group's partials t, t+64, ... in order (equal counts),
// then an xor butterfly (lower lane first, so both lanes of a pair hold the
// same bits) gives every lane the group's (mean, M2); then the lanes
// normalise the group's float4s of `out` in place.
template <int TILE>
__global__ __launch_bounds__(256) void lgn_wide_norm_kernel(
    const float2 *__restrict__ part, const float *__restrict__ gamma,
    const float *__restrict__ beta, long long pairs, int G, int tiles_per_group, int tiles_n,
    float eps, float *out) {
    const int lane = threadIdx.x & 63;
    const long long p = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (p >= pairs) return;   // whole wave leaves together
    const long long row = p / G;
    const int g = (int)(p % G);
    const float2 *pp = part + (size_t)row * (size_t)tiles_n + (size_t)g * tiles_per_group;
    float mean = 0.f, m2 = 0.f, cnt = 0.f;
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
    const int C = tiles_per_group * TILE;
    const float rstd = __builtin_amdgcn_rsqf(m2 / (float)C + eps);
    const float nmr = -mean * rstd;
    f32x4 *row_g = reinterpret_cast<f32x4 *>(out + (size_t)row * (size_t)tiles_n * TILE +
                                             (size_t)g * C);
    const f32x4 *gm = reinterpret_cast<const f32x4 *>(gamma + (size_t)g * C);
    const f32x4 *bt = reinterpret_cast<const f32x4 *>(beta + (size_t)g * C);
    for (int f = lane; f < C / 4; f += 64) {
        const f32x4 u = row_g[f], ga = gm[f], be = bt[f];
        f32x4 y;
#pragma unroll
        for (int j = 0; j < 4; ++j) y[j] = __builtin_fmaf(__builtin_fmaf(u[j], rstd, nmr), ga[j], be[j]);
        row_g[f] = y;
    }
}

}  // namespace lgn
