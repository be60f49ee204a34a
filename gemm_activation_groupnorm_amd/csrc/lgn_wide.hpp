// lgn_wide.hpp -- the forward for groups wider than one workgroup tile
// (C = N/G a multiple of 256, up to LayerNorm over all N when G = 1).
//
// Same method as lgn_fused.hpp (POPCORNBENCH "Kimi-K2.6 l2_p37": linear with
// its bias, Swish, external bias, GroupNorm with population variance and eps
// inside the square root, per-channel affine).  A group now spans several
// 256-channel tiles, so its statistics cross workgroups; the transcripts'
// two-stage plan for a reduction wider than a tile (per-block partials, then
// a light second pass) is used:
//   kernel 1: the fused kernel's GEMM tile, bias, Swish and bias, then per
//             (row, 256-channel tile) the partial (mean, M2) -- lane two-pass,
//             lane^32, then the tile's waves through LDS, all equal counts in
//             a fixed order -- into the workspace, and u written to `out`;
//   kernel 2: one wave per (row, group) merges the group's tile partials in
//             tile order and normalises `out` in place.
#pragma once

#include "lgn_fused.hpp"

namespace lgn {

constexpr int kWideTile = 256;   // channels per partial

template <class DT, class Cfg, int RING>
__global__ __launch_bounds__(Cfg::NT) __attribute__((amdgpu_waves_per_eu(Cfg::OCC)))
void lgn_wide_partial_kernel(
    const typename dt_traits<DT>::storage *__restrict__ x,
    const typename dt_traits<DT>::storage *__restrict__ W, const float *__restrict__ b_lin,
    const float *__restrict__ b_add, int M, int K, int N, float *__restrict__ out,
    float2 *__restrict__ part, int tiles_m, int tiles_n) {
    static_assert(Cfg::BC == kWideTile, "one partial per tile");
    constexpr int TS = Cfg::TS, TC = Cfg::TC;
    constexpr int NLOC = 16 * TC;  // a lane's channels of one sample row (half of the wave's WC)
    typedef CoreSel<DT, Cfg, RING> Sel;
    typedef TileParams<Cfg::BC> Par;
    static_assert(Cfg::WAVES_C * Cfg::BS * 8 <= Sel::SMEM, "partials fit in LDS");
    __shared__ __attribute__((aligned(1024))) unsigned char smem[Sel::SMEM + Par::BYTES];
    float *par = reinterpret_cast<float *>(smem + Sel::SMEM);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int lr = lane & 31;
    const int h = lane >> 5;
    const int wsI = wave / Cfg::WAVES_C;
    const int wcI = wave % Cfg::WAVES_C;
    const int ws0 = wsI * Cfg::WS;
    const int wc0 = wcI * Cfg::WC;
    int tm, tn;
    tile_coords<8>(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * Cfg::BS;
    const int n0 = tn * Cfg::BC;

    // b_lin and b_add only (gamma/beta belong to the second kernel)
    Par::stage(par, b_lin, b_add, b_add, b_add, n0, N, tid, Cfg::NT);
    __syncthreads();

    f32x16 acc[TS][TC];
#pragma unroll
    for (int tc = 0; tc < TC; ++tc)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const f32x4 bl = Par::get(par, 0, wc0 + 32 * tc + 8 * q + 4 * h);
#pragma unroll
            for (int ts = 0; ts < TS; ++ts)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[ts][tc][4 * q + j] = bl[j];
        }
    Sel::type::run(x, W, M, N, K, m0, n0, smem, tid, wc0, ws0, lr, h, acc);

    // Swish, then the external bias; per-lane two-pass statistics over the
    // lane's NLOC channels of each sample row, merged with lane^32 (equal
    // counts): the wave's WC channels of that row
    float mean[TS], m2[TS];
#pragma unroll
    for (int ts = 0; ts < TS; ++ts) {
        float sum = 0.f;
#pragma unroll
        for (int tc = 0; tc < TC; ++tc)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f32x4 ba = Par::get(par, 1, wc0 + 32 * tc + 8 * q + 4 * h);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float u = swish(acc[ts][tc][4 * q + j]) + ba[j];
                    acc[ts][tc][4 * q + j] = u;
                    sum += u;
                }
            }
        const float mu = sum * (1.0f / NLOC);
        float q2 = 0.f;
#pragma unroll
        for (int tc = 0; tc < TC; ++tc)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float d = acc[ts][tc][r] - mu;
                q2 += d * d;
            }
        mean[ts] = mu;
        m2[ts] = q2;
        merge_halves(mean[ts], m2[ts], (float)NLOC);
    }

    // the tile's waves along channels, in wave order (equal counts WC)
    float2 *red = reinterpret_cast<float2 *>(smem);   // [WAVES_C][BS]
    __syncthreads();   // the main loop's last LDS reads are done
    if (h == 0) {
#pragma unroll
        for (int ts = 0; ts < TS; ++ts)
            red[wcI * Cfg::BS + ws0 + 32 * ts + lr] = make_float2(mean[ts], m2[ts]);
    }
    __syncthreads();
    if (wcI == 0 && h == 0) {
#pragma unroll
        for (int ts = 0; ts < TS; ++ts) {
            const int srow = ws0 + 32 * ts + lr;
            float mu = red[srow].x, q2 = red[srow].y;
#pragma unroll
            for (int j = 1; j < Cfg::WAVES_C; ++j) {
                const float2 o = red[j * Cfg::BS + srow];
                const float d = o.x - mu;
                mu = mu + d * (1.0f / (float)(j + 1));
                q2 = q2 + o.y + d * d * ((float)Cfg::WC * (float)j / (float)(j + 1));
            }
            const int row = m0 + srow;
            if (row < M) part[(size_t)row * (size_t)tiles_n + tn] = make_float2(mu, q2);
        }
    }

    // u to `out`: through the waves' LDS blocks (whole row segments per store)
    // when they fit in the ring, else directly (N % 256 == 0: no ragged columns)
    constexpr bool STAGED = Cfg::WC >= 64 && Cfg::WC <= 256 &&
                            (Cfg::NT / 64) * (32 * Cfg::WC * 4) <= Sel::SMEM;
    if constexpr (STAGED) {
        __syncthreads();   // the partials area is read before the blocks reuse it
#pragma unroll
        for (int ts = 0; ts < TS; ++ts) {
            typedef BlockStore<Cfg::WC> BS_;
            BS_::store(smem + wave * BS_::BYTES, lane,
                       [&](int tc, int q) {
                           f32x4 v;
#pragma unroll
                           for (int j = 0; j < 4; ++j) v[j] = acc[ts][tc][4 * q + j];
                           return v;
                       },
                       out, N, M, m0 + ws0 + 32 * ts, n0 + wc0);
        }
    } else {
#pragma unroll
        for (int ts = 0; ts < TS; ++ts) {
            const int m = m0 + ws0 + 32 * ts + lr;
            if (m >= M) continue;
#pragma unroll
            for (int tc = 0; tc < TC; ++tc)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    f32x4 v;
#pragma unroll
                    for (int j = 0; j < 4; ++j) v[j] = acc[ts][tc][4 * q + j];
                    *reinterpret_cast<f32x4 *>(out + (size_t)m * (size_t)N + n0 + wc0 + 32 * tc +
                                               8 * q + 4 * h) = v;
                }
        }
    }
}

// Kernel 2: one wave per (row, group) of C = tiles_per_group * TILE channels.
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
