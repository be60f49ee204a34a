// lgn_sgh.hpp -- the third method: the tail after a 3-D transposed
// convolution (POPCORNBENCH "Kimi-K2.6 l2_p60", problem statement): Swish,
// then GroupNorm over a group's channels and every spatial position of one
// sample (population variance, eps inside the square root, per-channel
// weight and bias), then HardSwish v * clamp(v + 3, 0, 6) / 6.
//
// y is [Nb][C][S] (S = D*H*W flattened).  A group (n, g) is the contiguous
// slab of L = (C/G)*S elements starting at (n*C + g*C/G)*S.  The work is
// bound by HBM traffic, not arithmetic: each slab is cut into chunks of
// kSghChunk elements, one workgroup per chunk, and two kernels run:
//   stats: each chunk's (mean, M2) -- per thread an exact two-pass over the
//          64 values it holds in registers, then Chan merges with counts
//          across the wave (xor butterfly, lower lane first) and the four
//          waves (LDS, in wave order) -- into the workspace;
//   apply: every workgroup merges its group's chunk partials in the same
//          fixed order (so all of a group's workgroups agree bit for bit),
//          then writes hardswish(fma(swish(y), rstd*gamma, beta - mean*rstd*gamma)).
// Loads are dwords, lane-contiguous (a wave reads 256 consecutive bytes):
// slabs start on arbitrary element boundaries when S is odd.
#pragma once

#include "lgn_device.hpp"

namespace lgn {

constexpr int kSghThreads = 256;
constexpr int kSghPerThread = 64;
constexpr int kSghChunk = kSghThreads * kSghPerThread;   // elements per workgroup

// Chan et al. pairwise merge of (mean, M2) over counts na and nb; `a` first.
__device__ __forceinline__ void chan_merge(float &mean, float &m2, float &n, float mb, float m2b,
                                           float nb) {
    const float nt = n + nb;
    if (nb == 0.f) return;
    if (n == 0.f) {
        mean = mb;
        m2 = m2b;
        n = nb;
        return;
    }
    const float d = mb - mean;
    const float f = nb / nt;
    mean = mean + d * f;
    m2 = m2 + m2b + d * d * (n * f);
    n = nt;
}

// Merge across the wave (xor butterfly, lower lane's partial first in each
// pair, so both lanes of a pair hold the same bits), then across the block's
// waves through LDS in wave order.  Every thread returns the block's result.
__device__ __forceinline__ void block_merge(float &mean, float &m2, float &n, float *red) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const float om = __shfl_xor(mean, off), om2 = __shfl_xor(m2, off), on = __shfl_xor(n, off);
        const bool lower = (lane & off) == 0;
        float a_m = lower ? mean : om, a_m2 = lower ? m2 : om2, a_n = lower ? n : on;
        chan_merge(a_m, a_m2, a_n, lower ? om : mean, lower ? om2 : m2, lower ? on : n);
        mean = a_m;
        m2 = a_m2;
        n = a_n;
    }
    if (lane == 0) {
        red[3 * wave] = mean;
        red[3 * wave + 1] = m2;
        red[3 * wave + 2] = n;
    }
    __syncthreads();
    mean = red[0];
    m2 = red[1];
    n = red[2];
#pragma unroll
    for (int w = 1; w < kSghThreads / 64; ++w) chan_merge(mean, m2, n, red[3 * w], red[3 * w + 1], red[3 * w + 2]);
}

// Stats kernel: grid = groups * parts.  part[group * parts + p] = (mean, M2).
__global__ __launch_bounds__(kSghThreads) void lgn_sgh_stats_kernel(
    const float *__restrict__ y, int C, long long S, int G, int parts, float2 *__restrict__ part) {
    __shared__ float red[3 * (kSghThreads / 64)];
    const int tid = threadIdx.x;
    const long long gi = blockIdx.x / parts;   // n * G + g
    const int p = blockIdx.x % parts;
    const long long n = gi / G, g = gi % G;
    const long long cg = C / G;
    const long long L = cg * S;
    const size_t base = (size_t)(n * C + g * cg) * (size_t)S;
    const long long c0 = (long long)p * kSghChunk;
    const int cnt = (int)(L - c0 < kSghChunk ? L - c0 : kSghChunk);
    const float *src = y + base + c0;

    float v[kSghPerThread];
    int mine = 0;
#pragma unroll
    for (int k = 0; k < kSghPerThread; ++k) {
        const int e = tid + k * kSghThreads;
        v[k] = e < cnt ? swish(src[e]) : 0.f;
        mine += e < cnt ? 1 : 0;
    }
    float sum = 0.f;
#pragma unroll
    for (int k = 0; k < kSghPerThread; ++k) sum += v[k];
    const float nf = (float)mine;
    float mean = mine ? sum / nf : 0.f;
    float m2 = 0.f;
#pragma unroll
    for (int k = 0; k < kSghPerThread; ++k) {
        const float d = v[k] - mean;
        m2 += tid + k * kSghThreads < cnt ? d * d : 0.f;
    }
    float nn = nf;
    block_merge(mean, m2, nn, red);
    if (tid == 0) part[blockIdx.x] = make_float2(mean, m2);
}

// Apply kernel: same grid; out may be y itself (each element is read and
// then written by the same thread).
__global__ __launch_bounds__(kSghThreads) void lgn_sgh_apply_kernel(
    const float *y, const float *__restrict__ gamma, const float *__restrict__ beta, int C,
    long long S, int G, int parts, float eps, const float2 *__restrict__ part, float *out) {
    __shared__ float red[3 * (kSghThreads / 64)];
    const int tid = threadIdx.x;
    const long long gi = blockIdx.x / parts;
    const int p = blockIdx.x % parts;
    const long long n = gi / G, g = gi % G;
    const long long cg = C / G;
    const long long L = cg * S;
    const size_t base = (size_t)(n * C + g * cg) * (size_t)S;

    // the group's statistics from its chunk partials, in a fixed order
    float mean = 0.f, m2 = 0.f, cntf = 0.f;
    for (int t = tid; t < parts; t += kSghThreads) {
        const long long ct = L - (long long)t * kSghChunk;
        const float2 q = part[gi * parts + t];
        chan_merge(mean, m2, cntf, q.x, q.y, (float)(ct < kSghChunk ? ct : kSghChunk));
    }
    block_merge(mean, m2, cntf, red);
    const float rstd = __builtin_amdgcn_rsqf(m2 / (float)L + eps);

    const long long c0 = (long long)p * kSghChunk;
    const int cnt = (int)(L - c0 < kSghChunk ? L - c0 : kSghChunk);
    const float *src = y + base + c0;
    float *dst = out + base + c0;
    // channel of this thread's first element, then advanced incrementally
    long long rel = c0 + tid;
    long long ch = rel / S;
    long long off = rel - ch * S;
    for (int e = tid; e < cnt; e += kSghThreads) {
        const int c = (int)(g * cg + ch);
        const float a = rstd * gamma[c];
        const float b = beta[c] - mean * a;
        const float t = __builtin_fmaf(swish(src[e]), a, b);
        const float r = fminf(fmaxf(t + 3.0f, 0.0f), 6.0f);
        dst[e] = t * r * (1.0f / 6.0f);
        off += kSghThreads;
        while (off >= S) {
            off -= S;
            ++ch;
        }
    }
}

}  // namespace lgn
