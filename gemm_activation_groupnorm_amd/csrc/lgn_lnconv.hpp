// lgn_lnconv.hpp -- the fourth method: a pre-norm dilated convolution block
// (POPCORNBENCH transcript "Kimi-K2.6 l2_p5", problem statement and its
// derivation of the convolution's indices) on x [B][C][L]:
//
//   per sample b, over all C*L values: mean, population variance
//   h = (x - mean) / sqrt(var + eps) * ln_w[c][p] + ln_b[c][p]     ln_w, ln_b [C][L]
//   g = GELU(h)                                (exact, or the tanh form)
//   out[b][co][j] = conv_b[co] + x[b][co][j] + sum_ci sum_{t<3} W[co][ci][t] * g[ci][j - d + t*d]
//   g = 0 outside [0, L)                       (kernel 3, dilation d, zero padding d)
//
// The normalisation sits before the contraction, so it cannot be an
// epilogue: its statistics come from a first pass (the spatial GroupNorm's
// stats kernel without the Swish, one group of C*L values per sample), and
// LayerNorm + GELU are applied to the activation tiles while they are staged
// into LDS for the convolution.
//
// The convolution is an implicit GEMM on fp32 MFMA (v_mfma_f32_32x32x2_f32):
//   D[co][j] = sum_{k = (t, ci)} Wt[t][ci][co] * g[ci][j - d + t*d]
// operand A = weights (M = output channels), operand B = activations (N =
// positions), K = 3 taps x C input channels.  In the 32x32 accumulator a lane
// then holds one position and 16 output channels, so each store instruction
// writes 32 consecutive positions of one channel row.
#pragma once

#include "lgn_sgh.hpp"

namespace lgn {

constexpr int kLcKc = 16;         // input channels per stage (K = 3 * 16 per stage)
constexpr int kLcMaxHalo = 16;    // largest dilation handled (halo rounded up to 4)

// Workgroup tile: CO output channels x POS positions; waves of 64 channels x
// WPOS positions, (CO / 64) x (POS / WPOS) of them.
template <int CO_, int POS_, int WPOS_>
struct LcTile {
    static constexpr int CO = CO_, POS = POS_, WPOS = WPOS_;
    static constexpr int WAVES_C = CO / 64, WAVES_P = POS / WPOS;
    static constexpr int NT = 64 * WAVES_C * WAVES_P;
    static constexpr int TP = WPOS / 32;                       // 32-position MFMA tiles per wave
    static constexpr int GP = POS + 2 * kLcMaxHalo;            // LDS pitch of an activation row
    static constexpr int WF4 = 3 * kLcKc * CO / 4 / NT;        // weight float4s per thread
    static constexpr int GF4 = 3;                              // activation float4s per thread
    static_assert(WF4 == 6, "six weight float4s per thread and stage");
};
typedef LcTile<128, 128, 64> LcSmall;    // 4 waves of 64 x 64
typedef LcTile<256, 256, 128> LcLarge;   // 8 waves of 64 x 128

// W [co][ci][t] -> Wt [t][ci][co]: the weights as K-major rows of output
// channels, so a stage's weight slab is read with 16-byte loads.
__global__ __launch_bounds__(256) void lgn_conv_wpack_kernel(const float *__restrict__ w, int C,
                                                             float *__restrict__ wt) {
    const long long e = (long long)blockIdx.x * 256 + threadIdx.x;
    const long long n = 3LL * C * C;
    if (e >= n) return;
    const int co = (int)(e % C);
    const long long r = e / C;
    const int ci = (int)(r % C);
    const int t = (int)(r / C);
    wt[e] = w[((size_t)co * C + ci) * 3 + t];
}

// GELU of the activations, while they are staged for the convolution.  The
// fp32 MFMA does not issue alongside VALU work, so every instruction here
// takes time from the matrix unit; the library erff / tanhf cost about 35
// instructions each, these forms about 15 and 7.
//
// Exact form v * Phi(v) = 0.5 v (1 + erf(v / sqrt 2)), with erf after
// Abramowitz & Stegun, Handbook of Mathematical Functions, formula 7.1.26:
//   erf(z) = 1 - (a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5) exp(-z^2),
//   t = 1 / (1 + p z), z >= 0, |error| <= 1.5e-7,
// so that 1 + erf(z) = 2 - Q for z >= 0 and Q for z < 0, Q = poly(t) e^{-z^2}
// taken at |z|.  Tanh form 0.5 v (1 + tanh(u)), u = sqrt(2/pi) (v + 0.044715
// v^3), with tanh(u) = 1 - 2 / (1 + e^{2u}) (e^{2u} overflowing to +inf gives 1).
template <bool TANH>
__device__ __forceinline__ float lc_gelu(float v) {
    if constexpr (TANH) {
        const float u = 0.7978845608028654f * (v + 0.044715f * v * v * v);
        const float e = __builtin_amdgcn_exp2f(u * 2.8853900817779268f);   // e^{2u}
        return 0.5f * v * (2.0f - 2.0f * __builtin_amdgcn_rcpf(1.0f + e));
    } else {
        const float z = __builtin_fabsf(v) * 0.7071067811865476f;
        const float t = __builtin_amdgcn_rcpf(__builtin_fmaf(0.3275911f, z, 1.0f));
        float poly = __builtin_fmaf(t, 1.061405429f, -1.453152027f);
        poly = __builtin_fmaf(t, poly, 1.421413741f);
        poly = __builtin_fmaf(t, poly, -0.284496736f);
        poly = __builtin_fmaf(t, poly, 0.254829592f);
        poly *= t;
        // e^{-z^2} = 2^{-v^2 log2(e) / 2}
        const float q = poly * __builtin_amdgcn_exp2f(v * v * -0.7213475204444817f);
        return 0.5f * v * (v >= 0.0f ? 2.0f - q : q);
    }
}

// The convolution with LayerNorm + GELU applied while staging.  Grid: one
// workgroup per (sample, position tile, channel tile), samples fastest; the
// hardware id is remapped so each XCD gets a contiguous run.
// part[b * parts + p] = (mean, M2) of chunk p (kSghChunk values) of sample b.
// H = the staged halo: the dilation rounded up to a multiple of 4 (<= kLcMaxHalo).
// Requires C % Tile::CO == 0, L % 4 == 0, 1 <= d <= H <= 16; out must not overlap x.
// The next stage's weights and activations are loaded at the top of a stage
// and written to the other LDS buffer in three parts, one after each tap's
// MFMAs, so that their LayerNorm + GELU arithmetic runs under the MFMAs.
template <class Tile, bool TANH, int H>
__global__ __launch_bounds__(Tile::NT) void lgn_lnconv_kernel(
    const float *__restrict__ x, const float *__restrict__ ln_w, const float *__restrict__ ln_b,
    const float *__restrict__ wt, const float *__restrict__ conv_b,
    const float2 *__restrict__ part, int C, int L, int d, int parts, float eps,
    int tiles_l, int tiles_c, float *__restrict__ out) {
    constexpr int CO = Tile::CO, POS = Tile::POS, NT = Tile::NT, TP = Tile::TP;
    constexpr int WF4 = Tile::WF4, GF4 = Tile::GF4, GP = Tile::GP;
    static_assert(H % 4 == 0 && H >= 4 && H <= kLcMaxHalo, "halo: 4, 8, 12 or 16");
    constexpr int win4 = (POS + 2 * H) / 4;   // float4s per staged activation row
    constexpr int gtot = kLcKc * win4;
    static_assert(gtot > (GF4 - 1) * NT && gtot <= GF4 * NT, "three activation float4s per thread");
    // weight rows: odd rows have their 32-float halves swapped (column ^ 32),
    // so the two lane halves of a read (rows 2k, 2k+1) hit disjoint banks
    __shared__ __attribute__((aligned(16))) float ws[2][3 * kLcKc][CO];
    __shared__ __attribute__((aligned(16))) float gs[2][kLcKc][GP];
    __shared__ float red[3 * (NT / 64)];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int i = lane & 31, h = lane >> 5;
    const int wc = wave % Tile::WAVES_C, wp = wave / Tile::WAVES_C;

    const int nblocks = gridDim.x;
    int t_id = blockIdx.x;
    if ((nblocks & 7) == 0) t_id = (blockIdx.x & 7) * (nblocks >> 3) + (blockIdx.x >> 3);
    // samples fastest: the workgroups resident on one XCD at a time cover the
    // same positions of different samples, so ln_w / ln_b windows (shared by
    // every sample) and the weights are re-read from that XCD's L2
    const int nb_ = nblocks / (tiles_c * tiles_l);
    const int b = t_id % nb_;
    const int rest = t_id / nb_;
    const int ct = rest % tiles_c;
    const int lt = rest / tiles_c;
    const int co0 = ct * CO;
    const int j0 = lt * POS;

    // ---- the sample's statistics from its chunk partials, in a fixed order ----
    const long long n = (long long)C * L;
    float mean = 0.f, m2 = 0.f, cnt = 0.f;
    for (int t = tid; t < parts; t += NT) {
        const long long ctn = n - (long long)t * kSghChunk;
        const float2 q = part[(size_t)b * parts + t];
        chan_merge(mean, m2, cnt, q.x, q.y, (float)(ctn < kSghChunk ? ctn : kSghChunk));
    }
    block_merge<NT / 64>(mean, m2, cnt, red);
    const float rstd = __builtin_amdgcn_rsqf(m2 / (float)n + eps);
    const float nmr = -mean * rstd;

    const float *xb = x + (size_t)b * C * L;

    f32x4 rw[WF4];
    f32x4 rx[GF4], rg[GF4], rb[GF4];

    // Buffer loads: per-thread byte offsets fixed for the whole loop, the
    // stage's channel offset in a scalar register or in the descriptor's
    // base.  A raw buffer (stride 0) returns 0 for an offset at or beyond its
    // size, so the halo loads that fall outside the sample (the left halo of
    // channel 0, the right halo of the last channel) read 0 and touch no
    // memory.  0x00020000 is the gfx9 descriptor word for 32-bit data.  The
    // API keeps C * L below 2^29 and C at most 8192, so every offset fits 31
    // bits.
    const __amdgpu_buffer_rsrc_t rs_w =
        __builtin_amdgcn_make_buffer_rsrc((void *)wt, (short)0, 3 * C * C * 4, 0x00020000);
    int vo_w[WF4], vo_g[GF4];
#pragma unroll
    for (int q = 0; q < WF4; ++q) {
        const int f = tid + q * NT;
        const int row = f / (CO / 4), col4 = f % (CO / 4);
        const int t = row / kLcKc, cl = row % kLcKc;
        vo_w[q] = 4 * ((t * C + cl) * C + co0 + 4 * col4);
    }
#pragma unroll
    for (int q = 0; q < GF4; ++q) {
        const int f = tid + q * NT;
        const int cl = f / win4, col4 = f - cl * win4;
        vo_g[q] = 4 * (cl * L + j0 - H + 4 * col4);
    }
    auto load_stage = [&](int s) {
        const int c0 = s * kLcKc;
#pragma unroll
        for (int q = 0; q < WF4; ++q)
            rw[q] = __builtin_bit_cast(
                f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs_w, vo_w[q], 4 * c0 * C, 0));
        // the activation buffers start at this stage's first channel and end
        // at the sample's last one, so every halo load outside them reads 0
        const size_t cs = (size_t)c0 * L;
        const int rem = (C - c0) * L * 4;
        const __amdgpu_buffer_rsrc_t rs_x =
            __builtin_amdgcn_make_buffer_rsrc((void *)(xb + cs), (short)0, rem, 0x00020000);
        const __amdgpu_buffer_rsrc_t rs_g =
            __builtin_amdgcn_make_buffer_rsrc((void *)(ln_w + cs), (short)0, rem, 0x00020000);
        const __amdgpu_buffer_rsrc_t rs_b =
            __builtin_amdgcn_make_buffer_rsrc((void *)(ln_b + cs), (short)0, rem, 0x00020000);
#pragma unroll
        for (int q = 0; q < GF4; ++q) {
            const int f = tid + q * NT;
            if (f < gtot) {
                rx[q] = __builtin_bit_cast(
                    f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs_x, vo_g[q], 0, 0));
                rg[q] = __builtin_bit_cast(
                    f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs_g, vo_g[q], 0, 0));
                rb[q] = __builtin_bit_cast(
                    f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs_b, vo_g[q], 0, 0));
            }
        }
    };
    // registers -> LDS buffer `buf`, LayerNorm + GELU on the way; 0 outside [0, L).
    // Part 0: weight float4s 0-2; part 1: weight float4s 3-5 and activation
    // float4 0; part 2: activation float4s 1-2 (all of them: part -1).
    auto store_stage = [&](int buf, int which) {
#pragma unroll
        for (int q = 0; q < WF4; ++q) {
            if (which >= 0 && which != (q < 3 ? 0 : 1)) continue;
            const int f = tid + q * NT;
            const int row = f / (CO / 4);
            *reinterpret_cast<f32x4 *>(&ws[buf][row][(4 * (f % (CO / 4))) ^ (32 * (row & 1))]) =
                rw[q];
        }
#pragma unroll
        for (int q = 0; q < GF4; ++q) {
            if (which >= 0 && which != (q == 0 ? 1 : 2)) continue;
            const int f = tid + q * NT;
            const int cl = f / win4, col4 = f - cl * win4;
            const int p = j0 - H + 4 * col4;
            if (f < gtot) {
                f32x4 g = {0.f, 0.f, 0.f, 0.f};
                if (p >= 0 && p < L) {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        g[e] = lc_gelu<TANH>(
                            __builtin_fmaf(__builtin_fmaf(rx[q][e], rstd, nmr), rg[q][e], rb[q][e]));
                }
                *reinterpret_cast<f32x4 *>(&gs[buf][cl][4 * col4]) = g;
            }
        }
    };

    f32x16 acc[2][TP];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int c = 0; c < TP; ++c)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][c][r] = 0.f;

    const int stages = C / kLcKc;
    load_stage(0);
    store_stage(0, -1);
    __syncthreads();
    for (int s = 0; s < stages; ++s) {
        const int buf = s & 1;
        const bool more = s + 1 < stages;
        if (more) load_stage(s + 1);
#pragma unroll
        for (int t = 0; t < 3; ++t) {
            const int shift = H + (t - 1) * d;
#pragma unroll
            for (int kk = 0; kk < kLcKc / 2; ++kk) {
                const int kr = 2 * kk + h;
                float av[2], bv[TP];
#pragma unroll
                for (int tc = 0; tc < 2; ++tc)
                    av[tc] = ws[buf][t * kLcKc + kr][(wc * 64 + 32 * tc + i) ^ (32 * h)];
#pragma unroll
                for (int tp = 0; tp < TP; ++tp)
                    bv[tp] = gs[buf][kr][shift + wp * Tile::WPOS + 32 * tp + i];
#pragma unroll
                for (int tc = 0; tc < 2; ++tc)
#pragma unroll
                    for (int tp = 0; tp < TP; ++tp)
                        acc[tc][tp] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[tc], bv[tp],
                                                                          acc[tc][tp], 0, 0, 0);
            }
            if (more) store_stage(buf ^ 1, t);
        }
        __syncthreads();
    }

    // ---- epilogue: + conv bias + the input itself, one store per value ----
#pragma unroll
    for (int tc = 0; tc < 2; ++tc)
#pragma unroll
        for (int tp = 0; tp < TP; ++tp) {
            const int pos = j0 + wp * Tile::WPOS + 32 * tp + i;
            if (pos < L) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int co = co0 + wc * 64 + 32 * tc + 8 * (r >> 2) + 4 * h + (r & 3);
                    const size_t o = ((size_t)b * C + co) * L + pos;
                    out[o] = acc[tc][tp][r] + conv_b[co] + x[o];
                }
            }
        }
}

}  // namespace lgn
