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

// Per-channel vectors of the tile, staged once into LDS: [4][BC] floats
// (b_lin, b_add, gamma, beta); channels past N read as 0.
template <int BC>
struct TileParams {
    static constexpr int BYTES = 4 * BC * 4;
    static __device__ __forceinline__ void stage(float *lds, const float *__restrict__ b_lin,
                                                 const float *__restrict__ b_add,
                                                 const float *__restrict__ gamma,
                                                 const float *__restrict__ beta, int n0, int N,
                                                 int tid, int nt) {
        for (int i = tid; i < BC; i += nt) {
            const int n = n0 + i;
            const bool ok = n < N;
            lds[i] = ok ? b_lin[n] : 0.f;
            lds[BC + i] = ok ? b_add[n] : 0.f;
            lds[2 * BC + i] = ok ? gamma[n] : 0.f;
            lds[3 * BC + i] = ok ? beta[n] : 0.f;
        }
    }
    // 4 consecutive channels starting at tile channel c (c % 4 == 0) of vector v.
    static __device__ __forceinline__ f32x4 get(const float *lds, int v, int c) {
        return *reinterpret_cast<const f32x4 *>(lds + v * BC + c);
    }
};

// CG = channels per group (power of two, 8 .. 1024).  The tile's channel
// span BC is a multiple of CG, so every group lies inside one workgroup.
// RING selects the GEMM core (0: register-staged, any K; >= 2: LDS DMA ring).
// WIDE (groups wider than the tile; CG is then the wave's channel span WC):
// instead of normalising, the kernel writes u = Swish(z) + b_add to `out` and,
// per row and WC-channel span, the (mean, M2) of those WC values to
// wide_part[row * (N / WC) + span]; a second kernel merges a group's spans and
// normalises.  The epilogue keeps the per-sample-tile order of the normal
// path: statistics, then that sample tile's stores.
template <class DT, class Cfg, int CG, int RING, bool WIDE = false>
__global__ __launch_bounds__(Cfg::NT) __attribute__((amdgpu_waves_per_eu(Cfg::OCC)))
void lgn_fused_kernel(
    const typename dt_traits<DT>::storage *__restrict__ x,
    const typename dt_traits<DT>::storage *__restrict__ W, const float *__restrict__ b_lin,
    const float *__restrict__ b_add, const float *__restrict__ gamma,
    const float *__restrict__ beta, int M, int K, int N, float eps, float *__restrict__ out,
    int tiles_m, int tiles_n, float2 *__restrict__ wide_part) {
    static_assert(Cfg::BC % CG == 0, "groups must not straddle workgroup tiles");
    static_assert(!WIDE || CG == Cfg::WC, "the wide mode reduces each wave's channel span");
    constexpr int TS = Cfg::TS, TC = Cfg::TC;
    // Values of one (sample, group) held by one lane, and segments per lane.
    constexpr int SPAN = CG < Cfg::WC ? CG : Cfg::WC;   // channels of a group inside one wave
    constexpr int NLOC = SPAN / 2;                       // ... inside one lane
    constexpr int NSEG = (TC * 16) / NLOC;
    constexpr int WPG = CG > Cfg::WC ? CG / Cfg::WC : 1; // waves per group
    static_assert(CG >= 8 && (CG & (CG - 1)) == 0, "CG: power of two >= 8");
    static_assert(WPG == 1 || NSEG == 1, "a cross-wave group fills the wave's channel span");
    static_assert(WPG <= Cfg::WAVES_C, "group wider than the tile");

    typedef CoreSel<DT, Cfg, RING> Sel;
    typedef TileParams<Cfg::BC> Par;
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
    tile_coords<Cfg::GM>(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * Cfg::BS;
    const int n0 = tn * Cfg::BC;

    Par::stage(par, b_lin, b_add, gamma, beta, n0, N, tid, Cfg::NT);
    __syncthreads();

    // Accumulators start at the linear bias of their channel.
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

    // ---- Swish, then the external bias (in registers) ----
    auto activate = [&](int ts) {
#pragma unroll
        for (int tc = 0; tc < TC; ++tc)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f32x4 ba = Par::get(par, 1, wc0 + 32 * tc + 8 * q + 4 * h);
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[ts][tc][4 * q + j] = swish(acc[ts][tc][4 * q + j]) + ba[j];
            }
    };
    // ---- per-lane local statistics of segment s, merged with lane^32 ----
    auto local_stats = [&](int ts, int s, float &mean, float &m2) {
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
        mean = mu;
        m2 = q2;
        merge_halves(mean, m2, (float)NLOC);
    };
    // ---- normalise, affine, store ----
    //   y = (u - mean) * rstd * gamma + beta = fma(fma(u, rstd, -mean*rstd), gamma, beta)
    // Stores go through the wave's LDS block (whole row segments per
    // instruction) when the blocks of all waves fit in the ring, else direct.
    constexpr bool STAGED = Cfg::WC >= 64 && Cfg::WC <= 256 &&
                            (Cfg::NT / 64) * (32 * Cfg::WC * 4) <= Sel::SMEM;
    auto normalise = [&](int ts, int tc, int q, const float *rstd, const float *nmr) {
        f32x4 y;
        if constexpr (WIDE) {   // u itself: the second kernel normalises
#pragma unroll
            for (int j = 0; j < 4; ++j) y[j] = acc[ts][tc][4 * q + j];
        } else {
            const int ct = wc0 + 32 * tc + 8 * q + 4 * h;
            const int s = (tc * 16 + 4 * q) / NLOC;
            const f32x4 g = Par::get(par, 2, ct);
            const f32x4 bt = Par::get(par, 3, ct);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                y[j] = __builtin_fmaf(__builtin_fmaf(acc[ts][tc][4 * q + j], rstd[s], nmr[s]),
                                      g[j], bt[j]);
        }
        return y;
    };
    auto finish = [&](int ts, const float *rstd, const float *nmr) {
        if constexpr (STAGED) {
            // the final output is streamed; u of the wide mode is re-read by the second kernel
            typedef BlockStore<Cfg::WC, !WIDE> BS_;
            BS_::store(smem + wave * BS_::BYTES, lane,
                       [&](int tc, int q) { return normalise(ts, tc, q, rstd, nmr); }, out, N, M,
                       m0 + ws0 + 32 * ts, n0 + wc0);
        } else {
            const int m = m0 + ws0 + 32 * ts + lr;
#pragma unroll
            for (int tc = 0; tc < TC; ++tc)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int ct = wc0 + 32 * tc + 8 * q + 4 * h;
                    const f32x4 y = normalise(ts, tc, q, rstd, nmr);
                    if (m < M && n0 + ct < N)
                        *reinterpret_cast<f32x4 *>(out + (size_t)m * (size_t)N + n0 + ct) = y;
                }
        }
    };

    if constexpr (WPG == 1) {
        // every group inside this wave: one sample tile at a time
        if constexpr (STAGED) __syncthreads();   // all waves are done with the ring
#pragma unroll
        for (int ts = 0; ts < TS; ++ts) {
            activate(ts);
            float rstd[NSEG], nmr[NSEG];
#pragma unroll
            for (int s = 0; s < NSEG; ++s) {
                float mean, m2;
                local_stats(ts, s, mean, m2);
                rstd[s] = __builtin_amdgcn_rsqf(m2 * (1.0f / CG) + eps);
                nmr[s] = -mean * rstd[s];
                if constexpr (WIDE) {
                    const int row = m0 + ws0 + 32 * ts + lr;
                    if (h == 0 && row < M)
                        wide_part[(size_t)row * (size_t)(N / Cfg::WC) + (n0 + wc0) / Cfg::WC] =
                            make_float2(mean, m2);
                }
            }
            finish(ts, rstd, nmr);
        }
    } else {
        // groups span WPG waves: merge the waves' partials through LDS
        static_assert(Cfg::WAVES_C * Cfg::BS * 8 <= Sel::SMEM, "partials fit in LDS");
        float mean[TS], m2[TS];
#pragma unroll
        for (int ts = 0; ts < TS; ++ts) {
            activate(ts);
            local_stats(ts, 0, mean[ts], m2[ts]);
        }
        float2 *part = reinterpret_cast<float2 *>(smem);   // [WAVES_C][BS]
        __syncthreads();   // the main loop's last LDS reads are done
        if (h == 0) {
#pragma unroll
            for (int ts = 0; ts < TS; ++ts)
                part[wcI * Cfg::BS + ws0 + 32 * ts + lr] = make_float2(mean[ts], m2[ts]);
        }
        __syncthreads();
        const int first = (wcI / WPG) * WPG;
        float rstd[TS], nmr[TS];
#pragma unroll
        for (int ts = 0; ts < TS; ++ts) {
            const int srow = ws0 + 32 * ts + lr;
            const float2 p = part[first * Cfg::BS + srow];
            float mu = p.x, q2 = p.y;
#pragma unroll
            for (int j = 1; j < WPG; ++j) {
                const float2 o = part[(first + j) * Cfg::BS + srow];
                // counts: j*WC so far, WC incoming
                const float d = o.x - mu;
                mu = mu + d * (1.0f / (float)(j + 1));
                q2 = q2 + o.y + d * d * ((float)Cfg::WC * (float)j / (float)(j + 1));
            }
            rstd[ts] = __builtin_amdgcn_rsqf(q2 * (1.0f / CG) + eps);
            nmr[ts] = -mu * rstd[ts];

        }
        if constexpr (STAGED) __syncthreads();   // partials read before the block area is reused
#pragma unroll
        for (int ts = 0; ts < TS; ++ts) finish(ts, &rstd[ts], &nmr[ts]);
    }
}

}  // namespace lgn
