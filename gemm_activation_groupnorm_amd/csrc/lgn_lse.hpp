// lgn_lse.hpp -- the second method: Linear, then logsumexp over all output
// features of a row, then LeakyReLU (slope 0.01) twice and the exact GELU
// twice on that scalar (POPCORNBENCH "Kimi-K2.6 l2_p64", problem statement;
// the two-stage cross-tile reduction is the one the transcript sketches for
// its GEMM epilogue: per-block partial max / partial sum, then a small kernel).
//
// Kernel 1 runs the MFMA GEMM core on a BS x BC tile and reduces, for every
// sample row of the tile, its BC values z to a partial (max, sum exp(z - max))
// -- in registers per lane, with lane^32, then across the waves of the tile
// through LDS, always in a fixed order -- and writes that pair to
// part[row][tile column].  Kernel 2 (one wave per row) merges a row's
// partials in a fixed order and applies the scalar activations.  No M x N
// intermediate is written.
#pragma once

#include "lgn_device.hpp"

namespace lgn {

// e^v on the hardware exp2.
__device__ __forceinline__ float lse_exp(float v) {
    return __builtin_amdgcn_exp2f(v * 1.4426950408889634f);
}

// (m, s) <- merge of (m, s) and (om, os); an empty partial is (-inf, 0).
// The first operand's terms are added first, so a fixed call order gives a
// fixed result.
__device__ __forceinline__ void lse_merge(float &m, float &s, float om, float os) {
    const float mx = fmaxf(m, om);
    if (mx == -__builtin_inff()) return;   // both empty
    s = s * lse_exp(m - mx) + os * lse_exp(om - mx);
    m = mx;
}

// Kernel 1.  part is [M][tiles_n] (max, sum) pairs.
template <class DT, class Cfg, int RING>
__global__ __launch_bounds__(Cfg::NT) __attribute__((amdgpu_waves_per_eu(Cfg::OCC)))
void lgn_lse_partial_kernel(const typename dt_traits<DT>::storage *__restrict__ x,
                            const typename dt_traits<DT>::storage *__restrict__ W,
                            const float *__restrict__ b, int M, int K, int N,
                            float2 *__restrict__ part, int tiles_m, int tiles_n) {
    typedef CoreSel<DT, Cfg, RING> Sel;
    constexpr int TS = Cfg::TS, TC = Cfg::TC;
    static_assert(Cfg::WAVES_C * Cfg::BS * 8 <= Sel::SMEM, "partials fit in LDS");
    __shared__ __attribute__((aligned(1024))) unsigned char smem[Sel::SMEM];
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

    // accumulators start at the bias of their channel (channels past N: 0,
    // and they are left out of the reduction below)
    f32x16 acc[TS][TC];
#pragma unroll
    for (int tc = 0; tc < TC; ++tc)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int c = n0 + wc0 + 32 * tc + 8 * q + 4 * h;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float bv = c < N ? b[c + j] : 0.f;
#pragma unroll
                for (int ts = 0; ts < TS; ++ts) acc[ts][tc][4 * q + j] = bv;
            }
        }
    Sel::type::run(x, W, M, N, K, m0, n0, smem, tid, wc0, ws0, lr, h, acc);

    // per lane and sample row: max, then the shifted sum, over the lane's
    // valid channels (N % 4 == 0, so a 4-channel chunk is all in or all out)
    float pm[TS], ps[TS];
#pragma unroll
    for (int ts = 0; ts < TS; ++ts) {
        float mx = -__builtin_inff();
#pragma unroll
        for (int tc = 0; tc < TC; ++tc)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (n0 + wc0 + 32 * tc + 8 * q + 4 * h < N)
#pragma unroll
                    for (int j = 0; j < 4; ++j) mx = fmaxf(mx, acc[ts][tc][4 * q + j]);
        float s = 0.f;
        if (mx != -__builtin_inff()) {
#pragma unroll
            for (int tc = 0; tc < TC; ++tc)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if (n0 + wc0 + 32 * tc + 8 * q + 4 * h < N)
#pragma unroll
                        for (int j = 0; j < 4; ++j) s += lse_exp(acc[ts][tc][4 * q + j] - mx);
        }
        // merge with lane^32, lower half first on both lanes (same bits)
        const float om = __shfl_xor(mx, 32);
        const float os = __shfl_xor(s, 32);
        float m_lo = h == 0 ? mx : om, s_lo = h == 0 ? s : os;
        lse_merge(m_lo, s_lo, h == 0 ? om : mx, h == 0 ? os : s);
        pm[ts] = m_lo;
        ps[ts] = s_lo;
    }

    // across the waves of the tile's channel span, in wave order
    float2 *red = reinterpret_cast<float2 *>(smem);   // [WAVES_C][BS]
    __syncthreads();   // the main loop's last LDS reads are done
    if (h == 0) {
#pragma unroll
        for (int ts = 0; ts < TS; ++ts)
            red[wcI * Cfg::BS + ws0 + 32 * ts + lr] = make_float2(pm[ts], ps[ts]);
    }
    __syncthreads();
    if (wcI == 0 && h == 0) {
#pragma unroll
        for (int ts = 0; ts < TS; ++ts) {
            const int srow = ws0 + 32 * ts + lr;
            float m = red[srow].x, s = red[srow].y;
#pragma unroll
            for (int j = 1; j < Cfg::WAVES_C; ++j) {
                const float2 o = red[j * Cfg::BS + srow];
                lse_merge(m, s, o.x, o.y);
            }
            const int row = m0 + srow;
            if (row < M) part[(size_t)row * (size_t)tiles_n + tn] = make_float2(m, s);
        }
    }
}

__device__ __forceinline__ float leaky_relu_001(float v) { return v > 0.f ? v : 0.01f * v; }

// Exact GELU, v * Phi(v) with Phi(v) = (1 + erf(v / sqrt 2)) / 2.
__device__ __forceinline__ float gelu_erf(float v) {
    return v * (0.5f * (1.0f + erff(v * 0.70710678118654752f)));
}

// Kernel 2: one wave per row.  Lane t < tiles_n holds the row's partial of
// channel tile t (lanes t, t+64, ... for more than 64 tiles, merged in tile
// order); an xor butterfly then merges the lanes, each pair in lower-lane-
// first order, so that both lanes of a pair hold the same bits and lane 0
// ends with the merge of every tile in a fixed order.
__global__ __launch_bounds__(256) void lgn_lse_finish_kernel(const float2 *__restrict__ part,
                                                             int M, int tiles_n,
                                                             float *__restrict__ out) {
    const int lane = threadIdx.x & 63;
    const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= M) return;   // whole wave leaves together
    const float2 *p = part + (size_t)row * (size_t)tiles_n;
    float m = -__builtin_inff(), s = 0.f;
    for (int t = lane; t < tiles_n; t += 64) lse_merge(m, s, p[t].x, p[t].y);
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const float om = __shfl_xor(m, off);
        const float os = __shfl_xor(s, off);
        const bool lower = (lane & off) == 0;
        float a_m = lower ? m : om, a_s = lower ? s : os;
        lse_merge(a_m, a_s, lower ? om : m, lower ? os : s);
        m = a_m;
        s = a_s;
    }
    if (lane == 0) {
        // s >= 1: the row maximum contributes e^0
        const float l = m + __builtin_amdgcn_logf(s) * 0.69314718055994531f;
        float v = leaky_relu_001(leaky_relu_001(l));
        out[row] = gelu_erf(gelu_erf(v));
    }
}

}  // namespace lgn
