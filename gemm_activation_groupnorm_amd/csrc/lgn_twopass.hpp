// lgn_twopass.hpp -- the two-pass ablation: kernel 1 is the MFMA GEMM with
// the linear bias, writing z to a workspace; kernel 2 is one elementwise +
// GroupNorm pass over z.  This is the structure the transcript settles on
// (a library GEMM, then a fused Swish/bias/GroupNorm tail kernel working on
// the GEMM output in place), rebuilt for gfx950.
#pragma once

#include "lgn_device.hpp"

namespace lgn {

// z[m, n] = sum_k x[m,k] W[n,k] + b_lin[n], fp32, [M, N] row-major.
// RING selects the GEMM core (0: register-staged, any K; >= 2: LDS DMA ring).
template <class DT, class Cfg, int RING>
__global__ __launch_bounds__(Cfg::NT) __attribute__((amdgpu_waves_per_eu(Cfg::OCC)))
void lgn_gemm_bias_kernel(
    const typename dt_traits<DT>::storage *__restrict__ x,
    const typename dt_traits<DT>::storage *__restrict__ W, const float *__restrict__ b_lin,
    int M, int K, int N, float *__restrict__ z, int tiles_m, int tiles_n) {
    typedef CoreSel<DT, Cfg, RING> Sel;
    __shared__ __attribute__((aligned(1024))) unsigned char smem[Sel::SMEM];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int lr = lane & 31;
    const int h = lane >> 5;
    const int ws0 = (wave / Cfg::WAVES_C) * Cfg::WS;
    const int wc0 = (wave % Cfg::WAVES_C) * Cfg::WC;
    int tm, tn;
    tile_coords<Cfg::GM>(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * Cfg::BS;
    const int n0 = tn * Cfg::BC;

    // accumulators start at the linear bias of their channel
    f32x16 acc[Cfg::TS][Cfg::TC];
#pragma unroll
    for (int tc = 0; tc < Cfg::TC; ++tc)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int c = n0 + wc0 + 32 * tc + 8 * q + 4 * h;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float bl = c < N ? b_lin[c + j] : 0.f;
#pragma unroll
                for (int ts = 0; ts < Cfg::TS; ++ts) acc[ts][tc][4 * q + j] = bl;
            }
        }
    Sel::type::run(x, W, M, N, K, m0, n0, smem, tid, wc0, ws0, lr, h, acc);

    constexpr bool STAGED = Cfg::WC >= 64 && Cfg::WC <= 256 &&
                            (Cfg::NT / 64) * (32 * Cfg::WC * 4) <= Sel::SMEM;
    if constexpr (STAGED) {
        typedef BlockStore<Cfg::WC> BS_;
        __syncthreads();   // all waves are done with the ring
#pragma unroll
        for (int ts = 0; ts < Cfg::TS; ++ts)
            BS_::store(smem + wave * BS_::BYTES, lane,
                       [&](int tc, int q) {
                           f32x4 v;
#pragma unroll
                           for (int j = 0; j < 4; ++j) v[j] = acc[ts][tc][4 * q + j];
                           return v;
                       },
                       z, N, M, m0 + ws0 + 32 * ts, n0 + wc0);
    } else {
#pragma unroll
        for (int tc = 0; tc < Cfg::TC; ++tc) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int c = n0 + wc0 + 32 * tc + 8 * q + 4 * h;
                if (c >= N) continue;
#pragma unroll
                for (int ts = 0; ts < Cfg::TS; ++ts) {
                    const int m = m0 + ws0 + 32 * ts + lr;
                    if (m >= M) continue;
                    f32x4 v;
#pragma unroll
                    for (int j = 0; j < 4; ++j) v[j] = acc[ts][tc][4 * q + j];
                    *reinterpret_cast<f32x4 *>(z + (size_t)m * (size_t)N + c) = v;
                }
            }
        }
    }
}

// Epilogue, vectorised: a group of CG = 4*LPG*V channels is handled by LPG
// lanes holding V float4 chunks each, of two rows at once: unit q = (row
// pair rp, group g), q = rp*G + g, covers rows 2rp and 2rp+1 (only 2rp when
// it is the last row), and one wave covers 64/LPG consecutive units.  One
// load of b_add, gamma and beta serves both rows.  Statistics per row: a
// per-lane local two-pass, then an xor-butterfly of equal-count Chan merges
// inside each LPG-lane segment.  In place (out == z) is safe: every value is
// read before the unit's outputs are written, by the same lane.  One wave
// per workgroup: more, smaller workgroups keep more of the HBM stream in
// flight.  Against one row per lane (bitwise the same output) the two-row
// form measured 0.183 -> 0.178 ms (64-channel groups, 32768 x 4096) and
// 0.199 -> 0.185 ms (1024-channel groups, 16384 x 8192).
template <int LPG, int V>
__global__ __launch_bounds__(64) void lgn_gn_epilogue_vec_kernel(
    const float *z, const float *__restrict__ b_add, const float *__restrict__ gamma,
    const float *__restrict__ beta, long long M, int G, float eps, float *out) {
    constexpr int CG = 4 * LPG * V;
    constexpr int UPW = 64 / LPG;   // units per wave
    const int lane = threadIdx.x & 63;
    const long long units = (M + 1) / 2 * G;
    const long long q = (long long)blockIdx.x * UPW + lane / LPG;
    const int j = lane % LPG;
    const bool live = q < units;
    const long long rp = live ? q / G : 0;
    const int g = live ? (int)(q % G) : 0;
    const bool two = live && 2 * rp + 1 < M;
    const size_t base0 = ((size_t)(2 * rp) * G + g) * CG;
    const size_t base1 = two ? base0 + (size_t)G * CG : base0;   // a lone row reads itself twice

    f32x4 u[2][V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
        const int cc = 4 * (j + LPG * v);
        f32x4 a = {0.f, 0.f, 0.f, 0.f}, b = {0.f, 0.f, 0.f, 0.f};
        if (live) {
            a = *reinterpret_cast<const f32x4 *>(z + base0 + cc);
            b = *reinterpret_cast<const f32x4 *>(z + base1 + cc);
            const int ch = g * CG + cc;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float ba = b_add[ch + e];
                a[e] = swish(a[e]) + ba;
                b[e] = swish(b[e]) + ba;
            }
        }
        u[0][v] = a;
        u[1][v] = b;
    }
    float mean[2], rstd[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        float sum = 0.f;
#pragma unroll
        for (int v = 0; v < V; ++v)
#pragma unroll
            for (int e = 0; e < 4; ++e) sum += u[r][v][e];
        float mn = sum * (1.0f / (4 * V));
        float m2 = 0.f;
#pragma unroll
        for (int v = 0; v < V; ++v)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float d = u[r][v][e] - mn;
                m2 += d * d;
            }
        float n = (float)(4 * V);
#pragma unroll
        for (int off = 1; off < LPG; off <<= 1) {
            const float om = __shfl_xor(mn, off);
            const float om2 = __shfl_xor(m2, off);
            const float d = mn - om;
            mn = (mn + om) * 0.5f;
            m2 = (m2 + om2) + d * d * (0.5f * n);
            n *= 2.0f;
        }
        mean[r] = mn;
        rstd[r] = __builtin_amdgcn_rsqf(m2 * (1.0f / CG) + eps);
    }
    if (!live) return;
#pragma unroll
    for (int v = 0; v < V; ++v) {
        const int cc = 4 * (j + LPG * v);
        const int ch = g * CG + cc;
        f32x4 y0, y1;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float ga = gamma[ch + e], be = beta[ch + e];
            y0[e] = (u[0][v][e] - mean[0]) * rstd[0] * ga + be;
            y1[e] = (u[1][v][e] - mean[1]) * rstd[1] * ga + be;
        }
        *reinterpret_cast<f32x4 *>(out + base0 + cc) = y0;
        if (two) *reinterpret_cast<f32x4 *>(out + base1 + cc) = y1;
    }
}

// Epilogue for a group width CG not of the form 4*LPG*V: the vectorised
// kernel's layout in slots of EW consecutive channels (EW = 4, a float4, when
// CG % 4 == 0; 2 when CG % 2 == 0; else 1), with the slots past the group's
// F = CG/EW masked
// off (LPG >= F when V == 1, else LPG = 64 and 64*V >= F), for R rows per
// lane: unit q = (block of R rows, group g), q = rb*G + g, one load of b_add,
// gamma and beta serving the R rows.  A lane's count of values varies (0 for
// a lane with no slot), so the merges across the LPG lanes carry counts:
// Chan's update, lower lane first, so both lanes of a pair hold the same bits.
template <int LPG, int V, int R, int EW>
__global__ __launch_bounds__(64) void lgn_gn_epilogue_masked_kernel(
    const float *z, const float *__restrict__ b_add, const float *__restrict__ gamma,
    const float *__restrict__ beta, long long M, int G, int CG, float eps, float *out) {
    static_assert(EW == 1 || EW == 2 || EW == 4, "slots of one, two or four floats");
    constexpr int UPW = 64 / LPG;   // units per wave
    const int lane = threadIdx.x & 63;
    const long long units = (M + R - 1) / R * G;
    const long long q = (long long)blockIdx.x * UPW + lane / LPG;
    const int j = lane % LPG;
    const bool live = q < units;
    const long long r0 = live ? (long long)R * (q / G) : 0;
    const int g = live ? (int)(q % G) : 0;
    const int F = CG / EW;
    size_t base[R];
    bool valid[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        valid[r] = live && r0 + r < M;
        base[r] = ((size_t)(valid[r] ? r0 + r : r0) * G + g) * CG;   // a missing row reads row r0
    }
    auto load = [&](const float *p, float (&d)[EW]) {
        if constexpr (EW == 4) {
            const f32x4 t = *reinterpret_cast<const f32x4 *>(p);
#pragma unroll
            for (int e = 0; e < 4; ++e) d[e] = t[e];
        } else if constexpr (EW == 2) {
            const float2 t = *reinterpret_cast<const float2 *>(p);
            d[0] = t.x;
            d[1] = t.y;
        } else {
            d[0] = *p;
        }
    };

    float u[R][V][EW];
    float sum[R], n = 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r) sum[r] = 0.f;
#pragma unroll
    for (int v = 0; v < V; ++v) {
        const int f = j + LPG * v;
        const bool in = live && f < F;
        float ba[EW];
#pragma unroll
        for (int e = 0; e < EW; ++e) ba[e] = 0.f;
        if (in) {
            const int ch = g * CG + EW * f;
#pragma unroll
            for (int e = 0; e < EW; ++e) ba[e] = b_add[ch + e];
            n += (float)EW;
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            float val[EW];
#pragma unroll
            for (int e = 0; e < EW; ++e) val[e] = 0.f;
            if (in) {
                load(z + base[r] + EW * f, val);
#pragma unroll
                for (int e = 0; e < EW; ++e) val[e] = swish(val[e]) + ba[e];
            }
#pragma unroll
            for (int e = 0; e < EW; ++e) {
                u[r][v][e] = val[e];
                sum[r] += val[e];
            }
        }
    }
    float mean[R], rstd[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        float mn = n > 0.f ? sum[r] / n : 0.f;
        float m2 = 0.f, cnt = n;
#pragma unroll
        for (int v = 0; v < V; ++v)
            if (j + LPG * v < F) {
#pragma unroll
                for (int e = 0; e < EW; ++e) {
                    const float d = u[r][v][e] - mn;
                    m2 += d * d;
                }
            }
#pragma unroll
        for (int off = 1; off < LPG; off <<= 1) {
            const float om = __shfl_xor(mn, off), om2 = __shfl_xor(m2, off),
                        on = __shfl_xor(cnt, off);
            const bool lower = (lane & off) == 0;
            const float am = lower ? mn : om, am2 = lower ? m2 : om2, an = lower ? cnt : on;
            const float bm = lower ? om : mn, bm2 = lower ? om2 : m2, bn = lower ? on : cnt;
            const float nt = an + bn;
            if (bn == 0.f) {
                mn = am;
                m2 = am2;
            } else if (an == 0.f) {
                mn = bm;
                m2 = bm2;
            } else {
                const float d = bm - am;
                const float fr = bn / nt;
                mn = am + d * fr;
                m2 = am2 + bm2 + d * d * (an * fr);
            }
            cnt = nt;
        }
        mean[r] = mn;
        rstd[r] = __builtin_amdgcn_rsqf(m2 / (float)CG + eps);
    }
    if (!live) return;
#pragma unroll
    for (int v = 0; v < V; ++v) {
        const int f = j + LPG * v;
        if (f < F) {
            const int ch = g * CG + EW * f;
            float ga[EW], be[EW];
#pragma unroll
            for (int e = 0; e < EW; ++e) {
                ga[e] = gamma[ch + e];
                be[e] = beta[ch + e];
            }
#pragma unroll
            for (int r = 0; r < R; ++r) {
                if (!valid[r]) continue;
                if constexpr (EW == 4) {
                    f32x4 y;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        y[e] = (u[r][v][e] - mean[r]) * rstd[r] * ga[e] + be[e];
                    *reinterpret_cast<f32x4 *>(out + base[r] + 4 * f) = y;
                } else if constexpr (EW == 2) {
                    *reinterpret_cast<float2 *>(out + base[r] + 2 * f) =
                        make_float2((u[r][v][0] - mean[r]) * rstd[r] * ga[0] + be[0],
                                    (u[r][v][1] - mean[r]) * rstd[r] * ga[1] + be[1]);
                } else {
                    out[base[r] + f] = (u[r][v][0] - mean[r]) * rstd[r] * ga[0] + be[0];
                }
            }
        }
    }
}

// Epilogue, any channel count: one wave per (row, group), three passes over
// the group (sum; sum of squared deviations from the mean; normalise), each
// an xor-butterfly sum over the wave.  Used for groups wider than the masked
// kernel covers (2048 slots: 8192 channels when C % 4 == 0, 4096 when C % 2
// == 0, else 2048).
__global__ __launch_bounds__(64) void lgn_gn_epilogue_generic_kernel(
    const float *z, const float *__restrict__ b_add, const float *__restrict__ gamma,
    const float *__restrict__ beta, long long pairs, int G, int CG, float eps, float *out) {
    const int lane = threadIdx.x & 63;
    const long long p = blockIdx.x;
    const int g = (int)(p % G);
    const size_t base = (size_t)p * CG;
    float sum = 0.f;
    for (int c = lane; c < CG; c += 64) sum += swish(z[base + c]) + b_add[g * CG + c];
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) sum += __shfl_xor(sum, off);
    const float mean = sum / (float)CG;
    float ss = 0.f;
    for (int c = lane; c < CG; c += 64) {
        const float d = swish(z[base + c]) + b_add[g * CG + c] - mean;
        ss += d * d;
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) ss += __shfl_xor(ss, off);
    const float rstd = __builtin_amdgcn_rsqf(ss / (float)CG + eps);
    for (int c = lane; c < CG; c += 64) {
        const float uu = swish(z[base + c]) + b_add[g * CG + c];
        out[base + c] = (uu - mean) * rstd * gamma[g * CG + c] + beta[g * CG + c];
    }
}

}  // namespace lgn
