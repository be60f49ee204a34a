// lgn_fused.hpp -- the fused kernel: MFMA GEMM tile, then bias, Swish, bias,
// per-(row, group) statistics, normalisation and affine, all on chip, and one
// write of the output tile.
//
// Forward (POPCORNBENCH "Kimi-K2.6 l2_p37", problem statement): linear with
// its own bias, Swish sigmoid(z)*z, add the external per-channel bias, then
// GroupNorm over contiguous channel groups (population variance, eps inside
// the square root) with per-channel gamma/beta.
//
// Statistics.  For every (sample, group) each lane first reduces the values it
// holds with a local two-pass (sum -> local mean -> local sum of squared
// deviations); partial (mean, M2) pairs are then combined with the pairwise
// update of Chan, Golub and LeVeque -- across the two lane halves (lane^32),
// and, when a group is wider than one wave's channel span, across the waves
// through LDS.  Every merge is between equal counts or in a fixed order, so
// all lanes of a group obtain bitwise identical statistics and the output is
// deterministic.
#pragma once

#include "lgn_device.hpp"

namespace lgn {

// CG = channels per group (power of two, 8 .. 1024).  The tile's channel
// span BC is a multiple of CG, so every group lies inside one workgroup.
template <class DT, class Cfg, int CG>
__global__ __launch_bounds__(Cfg::NT) void lgn_fused_kernel(
    const typename dt_traits<DT>::storage *__restrict__ x,
    const typename dt_traits<DT>::storage *__restrict__ W, const float *__restrict__ b_lin,
    const float *__restrict__ b_add, const float *__restrict__ gamma,
    const float *__restrict__ beta, int M, int K, int N, float eps, float *__restrict__ out,
    int tiles_m, int tiles_n) {
    static_assert(Cfg::BC % CG == 0, "groups must not straddle workgroup tiles");
    constexpr int TS = Cfg::TS, TC = Cfg::TC;
    // Values of one (sample, group) held by one lane, and segments per lane.
    constexpr int SPAN = CG < Cfg::WC ? CG : Cfg::WC;   // channels of a group inside one wave
    constexpr int NLOC = SPAN / 2;                       // ... inside one lane
    constexpr int NSEG = (TC * 16) / NLOC;
    constexpr int WPG = CG > Cfg::WC ? CG / Cfg::WC : 1; // waves per group
    static_assert(CG >= 8 && (CG & (CG - 1)) == 0, "CG: power of two >= 8");
    static_assert(WPG == 1 || NSEG == 1, "a cross-wave group fills the wave's channel span");
    static_assert(WPG <= Cfg::WAVES_C, "group wider than the tile");

    __shared__ __attribute__((aligned(16))) unsigned char smem[2 * Cfg::STAGE_BYTES];

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

    f32x16 acc[TS][TC];
    GemmCore<DT, Cfg>::run(x, W, M, N, K, m0, n0, smem, tid, wc0, ws0, lr, h, acc);

    // ---- bias, Swish, bias (in registers) ----
#pragma unroll
    for (int tc = 0; tc < TC; ++tc) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int c = n0 + wc0 + 32 * tc + 8 * q + 4 * h;
            float bl[4] = {0.f, 0.f, 0.f, 0.f}, ba[4] = {0.f, 0.f, 0.f, 0.f};
            if (c < N) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    bl[j] = b_lin[c + j];
                    ba[j] = b_add[c + j];
                }
            }
#pragma unroll
            for (int ts = 0; ts < TS; ++ts)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[ts][tc][4 * q + j] = swish(acc[ts][tc][4 * q + j] + bl[j]) + ba[j];
        }
    }

    // ---- per-lane local statistics and the lane-half merge ----
    float mean[TS][NSEG], m2[TS][NSEG];
#pragma unroll
    for (int ts = 0; ts < TS; ++ts) {
#pragma unroll
        for (int s = 0; s < NSEG; ++s) {
            float sum = 0.f;
#pragma unroll
            for (int f = s * NLOC; f < (s + 1) * NLOC; ++f) sum += acc[ts][f / 16][f % 16];
            const float mu = sum * (1.0f / NLOC);
            float q2 = 0.f;
#pragma unroll
            for (int f = s * NLOC; f < (s + 1) * NLOC; ++f) {
                const float d = acc[ts][f / 16][f % 16] - mu;
                q2 += d * d;
            }
            mean[ts][s] = mu;
            m2[ts][s] = q2;
            merge_halves(mean[ts][s], m2[ts][s], (float)NLOC);
        }
    }

    // ---- groups wider than a wave: merge the waves' partials through LDS ----
    if constexpr (WPG > 1) {
        static_assert(Cfg::WAVES_C * Cfg::BS * 8 <= 2 * Cfg::STAGE_BYTES, "partials fit in LDS");
        float2 *part = reinterpret_cast<float2 *>(smem);   // [WAVES_C][BS]
        __syncthreads();   // the main loop's last LDS reads are done
        if (h == 0) {
#pragma unroll
            for (int ts = 0; ts < TS; ++ts)
                part[wcI * Cfg::BS + ws0 + 32 * ts + lr] = make_float2(mean[ts][0], m2[ts][0]);
        }
        __syncthreads();
        const int first = (wcI / WPG) * WPG;
#pragma unroll
        for (int ts = 0; ts < TS; ++ts) {
            const int srow = ws0 + 32 * ts + lr;
            float2 p = part[first * Cfg::BS + srow];
            float mu = p.x, q2 = p.y;
#pragma unroll
            for (int j = 1; j < WPG; ++j) {
                const float2 o = part[(first + j) * Cfg::BS + srow];
                // counts: j*WC so far, WC incoming
                const float d = o.x - mu;
                mu = mu + d * (1.0f / (float)(j + 1));
                q2 = q2 + o.y + d * d * ((float)Cfg::WC * (float)j / (float)(j + 1));
            }
            mean[ts][0] = mu;
            m2[ts][0] = q2;
        }
    }

    // ---- normalise, affine, one 16-byte store per 4 channels ----
    float rstd[TS][NSEG];
#pragma unroll
    for (int ts = 0; ts < TS; ++ts)
#pragma unroll
        for (int s = 0; s < NSEG; ++s)
            rstd[ts][s] = __builtin_amdgcn_rsqf(m2[ts][s] * (1.0f / CG) + eps);

#pragma unroll
    for (int tc = 0; tc < TC; ++tc) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int c = n0 + wc0 + 32 * tc + 8 * q + 4 * h;
            if (c >= N) continue;
            float g[4], bt[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                g[j] = gamma[c + j];
                bt[j] = beta[c + j];
            }
#pragma unroll
            for (int ts = 0; ts < TS; ++ts) {
                const int m = m0 + ws0 + 32 * ts + lr;
                if (m >= M) continue;
                const int s = (tc * 16 + 4 * q) / NLOC;
                f32x4 y;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    y[j] = (acc[ts][tc][4 * q + j] - mean[ts][s]) * rstd[ts][s] * g[j] + bt[j];
                *reinterpret_cast<f32x4 *>(out + (size_t)m * (size_t)N + c) = y;
            }
        }
    }
}

}  // namespace lgn
