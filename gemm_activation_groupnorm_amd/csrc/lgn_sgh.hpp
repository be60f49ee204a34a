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
// Accesses are 16 bytes per lane over the 16-byte-aligned body of each chunk
// (slabs start on arbitrary element boundaries when S is odd, so up to 3
// elements at each end are done one by one); each wave owns a contiguous
// 16 KiB span of the body, and each thread issues all of its loads before
// using any, so they are in flight together.
#pragma once

#include "lgn_device.hpp"

namespace lgn {

constexpr int kSghThreads = 256;
constexpr int kSghPerThread = 64;
constexpr int kSghChunk = kSghThreads * kSghPerThread;   // elements per workgroup
// The single-pass kernel serves groups of at most this many chunks (4 Mi
// elements); larger groups take the two-kernel path.
constexpr int kSghOnePassMaxParts = 256;

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
// WAVES waves through LDS (red: 3 * WAVES floats) in wave order.  Every thread
// of the block must call it; every thread returns the block's result.
template <int WAVES = kSghThreads / 64>
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
    for (int w = 1; w < WAVES; ++w) chan_merge(mean, m2, n, red[3 * w], red[3 * w + 1], red[3 * w + 2]);
}

// A chunk [start, end) of absolute element indices, split for 16-byte
// accesses: a head [start, a0) of < 4 elements up to the first multiple of 4,
// a body [a0, a1) of whole float4s, and a tail [a1, end) of < 4 elements.
// y and out are 16-byte aligned.  Both boundaries are clamped into the chunk,
// so a chunk that holds no whole float4 is a head and a tail of < 4 each
// (at most 3 + 3 elements then), and every element is covered exactly once.
struct SghSplit {
    long long start, a0, a1, end;
    __device__ __forceinline__ SghSplit(long long s, long long e) : start(s), end(e) {
        const long long up = (s + 3) & ~3LL;
        a0 = up < e ? up : e;
        const long long dn = e & ~3LL;
        a1 = dn > a0 ? dn : a0;
    }
    __device__ __forceinline__ int body4() const { return (int)((a1 - a0) >> 2); }
    // edge element handled by thread t (head: t < 4, tail: 64 <= t < 68), or -1
    __device__ __forceinline__ long long edge(int t) const {
        if (t < 4) return start + t < a0 ? start + t : -1;
        if (t >= 64 && t < 68) return a1 + (t - 64) < end ? a1 + (t - 64) : -1;
        return -1;
    }
};

constexpr int kSghVec = kSghPerThread / 4;   // float4s per thread per chunk

// Body float4 k of thread tid.  Each wave owns one contiguous span of
// kSghVec * 64 float4s (16 KiB) and walks it 1 KiB per k.  Against the four
// waves interleaving over the whole 64 KiB chunk this moved a 1 GiB copy from
// 5.13 to 5.60 TB/s and the single pass at 128 x 16 x 31 x 63 x 63 from
// 0.418 to 0.390 ms: the fewer DRAM pages a wave touches at once, the better.
__device__ __forceinline__ int sgh_f4(int tid, int k) {
    return (tid >> 6) * (kSghVec * 64) + k * 64 + (tid & 63);
}

// Loads this thread's share of the chunk [sp.start, sp.end) of y and forms
// the chunk's (mean, M2) of f(y), f = Swish (SWISH) or the identity.  On
// return v holds f of the thread's body float4s (0 past the body), ei / ev
// the thread's edge element and f of it (ei = -1, ev = 0 if none), and every
// thread of the block holds the chunk's moments: per thread an exact
// two-pass over its values, then the block merge.  Every thread must call it.
template <bool SWISH>
__device__ __forceinline__ void sgh_chunk_moments(const float *__restrict__ y, const SghSplit &sp,
                                                  f32x4 (&v)[kSghVec], long long &ei, float &ev,
                                                  float &mean, float &m2, float *red) {
    const int tid = threadIdx.x;
    const int nb4 = sp.body4();
    const f32x4 *body = reinterpret_cast<const f32x4 *>(y + sp.a0);
#pragma unroll
    for (int k = 0; k < kSghVec; ++k) {
        const int f = sgh_f4(tid, k);
        v[k] = f < nb4 ? body[f] : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    ei = sp.edge(tid);
    ev = ei >= 0 ? (SWISH ? swish(y[ei]) : y[ei]) : 0.f;
    float sum = ei >= 0 ? ev : 0.f;
    int mine = ei >= 0 ? 1 : 0;
#pragma unroll
    for (int k = 0; k < kSghVec; ++k) {
        const bool ok = sgh_f4(tid, k) < nb4;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[k][j] = ok ? (SWISH ? swish(v[k][j]) : v[k][j]) : 0.f;
            sum += v[k][j];
        }
        mine += ok ? 4 : 0;
    }
    const float nf = (float)mine;
    mean = mine ? sum / nf : 0.f;
    m2 = ei >= 0 ? (ev - mean) * (ev - mean) : 0.f;
#pragma unroll
    for (int k = 0; k < kSghVec; ++k) {
        const bool ok = sgh_f4(tid, k) < nb4;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float d = v[k][j] - mean;
            m2 += ok ? d * d : 0.f;
        }
    }
    float nn = nf;
    block_merge(mean, m2, nn, red);
}

// The same (mean, M2) of Swish(y) as sgh_chunk_moments<true> (the same
// per-thread values in the same order, so bitwise the same result) without
// holding the chunk in registers: the thread's float4s are read once for the
// sum and once more for the squared deviations.  For the single-pass
// kernel's fallback, where register room matters more than reads.
__device__ __forceinline__ void sgh_chunk_moments_lean(const float *__restrict__ y,
                                                       const SghSplit &sp, float &mean,
                                                       float &m2, float *red) {
    const int tid = threadIdx.x;
    const int nb4 = sp.body4();
    const f32x4 *body = reinterpret_cast<const f32x4 *>(y + sp.a0);
    const long long ei = sp.edge(tid);
    const float ev = ei >= 0 ? swish(y[ei]) : 0.f;
    float sum = ei >= 0 ? ev : 0.f;
    int mine = ei >= 0 ? 1 : 0;
#pragma unroll 1
    for (int k = 0; k < kSghVec; ++k) {
        const bool ok = sgh_f4(tid, k) < nb4;
        const f32x4 w = ok ? body[sgh_f4(tid, k)] : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; ++j) sum += ok ? swish(w[j]) : 0.f;
        mine += ok ? 4 : 0;
    }
    const float nf = (float)mine;
    mean = mine ? sum / nf : 0.f;
    m2 = ei >= 0 ? (ev - mean) * (ev - mean) : 0.f;
#pragma unroll 1
    for (int k = 0; k < kSghVec; ++k) {
        const bool ok = sgh_f4(tid, k) < nb4;
        const f32x4 w = ok ? body[sgh_f4(tid, k)] : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float d = (ok ? swish(w[j]) : 0.f) - mean;
            m2 += ok ? d * d : 0.f;
        }
    }
    float nn = nf;
    block_merge(mean, m2, nn, red);
}

// Chunk p of group gi: the group is the contiguous slab of L = cg * S
// elements starting at base = (n * C + g * cg) * S.
struct SghChunkPos {
    long long base, L;
    SghSplit sp;
    __device__ __forceinline__ SghChunkPos(long long gi, int p, int C, long long S, int G)
        : base(0), L(0), sp(0, 0) {
        const long long n = gi / G, g = gi % G;
        const long long cg = C / G;
        L = cg * S;
        base = (n * C + g * cg) * S;
        const long long c0 = (long long)p * kSghChunk;
        const long long cnt = L - c0 < kSghChunk ? L - c0 : kSghChunk;
        sp = SghSplit(base + c0, base + c0 + cnt);
    }
};

// Stats kernel: grid = (groups of this round) * parts, starting at group
// g_first.  part[group * parts + p] = (mean, M2) of Swish(y), or of y itself
// with SWISH = false (the LayerNorm statistics of the conv block: one group of
// C*L values per sample).
template <bool SWISH = true>
__global__ __launch_bounds__(kSghThreads) void lgn_sgh_stats_kernel(
    const float *__restrict__ y, int C, long long S, int G, int parts, long long g_first,
    float2 *__restrict__ part) {
    __shared__ float red[3 * (kSghThreads / 64)];
    const long long gi = g_first + blockIdx.x / parts;   // n * G + g
    const int p = blockIdx.x % parts;
    const SghChunkPos pos(gi, p, C, S, G);
    f32x4 v[kSghVec];
    long long ei;
    float ev, mean, m2;
    sgh_chunk_moments<SWISH>(y, pos.sp, v, ei, ev, mean, m2, red);
    if (threadIdx.x == 0) part[gi * parts + p] = make_float2(mean, m2);
}

// The group's statistics from its chunk partials q(t), t = 0 .. parts-1, in a
// fixed order (thread t % 256 merges t, t + 256, ...; then the block merge),
// so every workgroup of a group obtains bitwise the same (mean, M2).
template <class PartOf>
__device__ __forceinline__ void sgh_group_moments(PartOf &&part_of, int parts, long long L,
                                                  float &mean, float &m2, float *red) {
    float cntf = 0.f;
    mean = 0.f;
    m2 = 0.f;
    for (int t = threadIdx.x; t < parts; t += kSghThreads) {
        const long long ct = L - (long long)t * kSghChunk;
        const float2 q = part_of(t);
        chan_merge(mean, m2, cntf, q.x, q.y, (float)(ct < kSghChunk ? ct : kSghChunk));
    }
    block_merge(mean, m2, cntf, red);
}

// Per-channel (a, b) of the group's channels into LDS: a = rstd * gamma,
// b = beta - mean * a, with one spare entry ("next channel" past the end).
// Ends with a barrier.
template <int MAXCG>
__device__ __forceinline__ void sgh_coefficients(float mean, float m2, long long L, float eps,
                                                 const float *__restrict__ gamma,
                                                 const float *__restrict__ beta, long long g,
                                                 int cg, float *coef_a, float *coef_b) {
    const float rstd = __builtin_amdgcn_rsqf(m2 / (float)L + eps);
    for (int c = threadIdx.x; c <= cg; c += kSghThreads) {
        const int cc = c < cg ? c : cg - 1;
        const float a = rstd * gamma[g * cg + cc];
        coef_a[c] = a;
        coef_b[c] = beta[g * cg + cc] - mean * a;
    }
    __syncthreads();
}

// Writes hardswish(fma(s, a[c], b[c])) for this thread's Swish values s (the
// body float4s and the edge element) of the chunk, c the channel of each
// element.  The channel index is advanced incrementally per float4, with the
// coefficients of the current channel and the next one in registers (a
// float4 crosses at most one channel boundary when S >= 4).  Stores are
// non-temporal: nothing reads the output again.
__device__ __forceinline__ void sgh_store(const SghChunkPos &pos, long long S, int cg,
                                          const f32x4 (&s)[kSghVec], long long ei, float sev,
                                          const float *coef_a, const float *coef_b, float *out) {
    const int tid = threadIdx.x;
    const SghSplit &sp = pos.sp;
    const long long base = pos.base;
    const int nb4 = sp.body4();
    auto act = [](float t) {
        const float r = fminf(fmaxf(t + 3.0f, 0.0f), 6.0f);
        return t * r * (1.0f / 6.0f);
    };
    if (ei >= 0) {
        const int c = (int)((ei - base) / S);
        __builtin_nontemporal_store(act(__builtin_fmaf(sev, coef_a[c], coef_b[c])), &out[ei]);
    }
    f32x4 *obody = reinterpret_cast<f32x4 *>(out + sp.a0);
    long long r = sp.a0 - base + 4LL * sgh_f4(tid, 0);   // group-relative index of this thread's float4
    long long ch = r / S;
    long long off = r - ch * S;
    int cc = ch < cg ? (int)ch : cg;
    float a0 = coef_a[cc], b0 = coef_b[cc], a1 = coef_a[cc < cg ? cc + 1 : cg],
          b1 = coef_b[cc < cg ? cc + 1 : cg];
#pragma unroll
    for (int k = 0; k < kSghVec; ++k) {
        const int f = sgh_f4(tid, k);
        f32x4 o;
        if (S >= 4) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const bool nxt = off + j >= S;
                o[j] = act(__builtin_fmaf(s[k][j], nxt ? a1 : a0, nxt ? b1 : b0));
            }
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                long long cj = ch + (off + j) / S;
                const int ci = cj < cg ? (int)cj : cg;
                o[j] = act(__builtin_fmaf(s[k][j], coef_a[ci], coef_b[ci]));
            }
        }
        if (f < nb4) __builtin_nontemporal_store(o, &obody[f]);
        off += 4 * 64;
        if (off >= S) {
            while (off >= S) {
                off -= S;
                ++ch;
            }
            cc = ch < cg ? (int)ch : cg;
            a0 = coef_a[cc];
            b0 = coef_b[cc];
            a1 = coef_a[cc < cg ? cc + 1 : cg];
            b1 = coef_b[cc < cg ? cc + 1 : cg];
        }
    }
}

// Apply kernel: same grid, walked from the last chunk to the first; out may
// be y itself (each element is read and then written by the same thread).
// Every workgroup merges its group's chunk partials in the same fixed order,
// so all of a group's workgroups agree bit for bit.
template <int MAXCG>
__global__ __launch_bounds__(kSghThreads) void lgn_sgh_apply_kernel(
    const float *y, const float *__restrict__ gamma, const float *__restrict__ beta, int C,
    long long S, int G, int parts, long long g_first, float eps, const float2 *__restrict__ part,
    float *out) {
    __shared__ float red[3 * (kSghThreads / 64)];
    __shared__ float coef_a[MAXCG + 1], coef_b[MAXCG + 1];
    const int tid = threadIdx.x;
    // Last chunk first: the stats pass has just read the end of y, the part
    // the MALL still holds when this pass starts.  The stores of out are
    // non-temporal so that they do not displace it.  (At 128 x 16 x 123039
    // fp32: 0.560 ms -> 0.549 ms reversed, 0.547 ms streamed, 0.525 ms both.)
    const unsigned bid = gridDim.x - 1 - blockIdx.x;
    const long long gi = g_first + bid / parts;
    const int p = bid % parts;
    const SghChunkPos pos(gi, p, C, S, G);
    const SghSplit &sp = pos.sp;
    const int nb4 = sp.body4();
    const f32x4 *body = reinterpret_cast<const f32x4 *>(y + sp.a0);

    f32x4 v[kSghVec];
#pragma unroll
    for (int k = 0; k < kSghVec; ++k) {
        const int f = sgh_f4(tid, k);
        v[k] = f < nb4 ? body[f] : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const long long ei = sp.edge(tid);
    const float ev = ei >= 0 ? y[ei] : 0.f;

    float mean, m2;
    sgh_group_moments([&](int t) { return part[gi * parts + t]; }, parts, pos.L, mean, m2, red);
    sgh_coefficients<MAXCG>(mean, m2, pos.L, eps, gamma, beta, gi % G, C / G, coef_a, coef_b);
#pragma unroll
    for (int k = 0; k < kSghVec; ++k)
#pragma unroll
        for (int j = 0; j < 4; ++j) v[k][j] = swish(v[k][j]);
    sgh_store(pos, S, C / G, v, ei, swish(ev), coef_a, coef_b, out);
}

// Single-pass form (out must not overlap y): grid = groups * parts, one
// workgroup per chunk, group by group in blockIdx order.  Workgroups are
// dealt to the 8 XCDs in turn, so a group's chunks spread over all of them
// and the whole GPU holds about 32 groups at a time (4 channels x 31 x 63 x
// 63 each): only the group being dispatched at the moment waits long.
// (Keeping each group on one XCD instead left about 4 groups per XCD in
// flight and measured 0.548 ms against 0.415 ms at 128 x 16 x 31 x 63 x 63.
// Placement decides speed only.)
//
// A workgroup loads its chunk once and keeps the Swish values in registers.
// It publishes the chunk's (mean, M2) as ONE 64-bit atomic store into
// part[], whose entries the clear kernel has set to kSghEmpty beforehand, so
// the value itself says whether it has arrived: no counter, and no fence
// ordering a store before another (an agent-scope release would write back
// the XCD's L2 for every chunk).  Thread t then polls entry t of its group
// with device-coherent loads until it has arrived, the group's partials are
// merged in the same fixed order as the apply kernel, and the chunk is
// written.  y is read once instead of twice.
//
// The wait is bounded: should an entry not arrive within spin_limit polls,
// the workgroup computes every chunk's (mean, M2) of its group itself from y,
// with the arithmetic and per-thread order of that chunk's own workgroup
// (sgh_chunk_moments_lean), so it obtains bitwise the same statistics.
// Every wait therefore ends, and the output is the same either way (and
// equal to the two-kernel path's).  y is never written by this kernel, so
// reading any chunk of it is always safe.
constexpr unsigned long long kSghEmpty = 0x7fbadbad7fbadbadULL;   // a NaN pair

__device__ __forceinline__ unsigned long long sgh_pack(float mean, float m2) {
    return (unsigned long long)__float_as_uint(mean) |
           ((unsigned long long)__float_as_uint(m2) << 32);
}

// Occupancy: 4 waves per SIMD (128 VGPRs); the MAXCG = 8192 instance's 66 KiB
// of LDS allows 2 workgroups per CU, so it asks for 2.
template <int MAXCG>
__global__ __launch_bounds__(kSghThreads)
__attribute__((amdgpu_waves_per_eu(MAXCG > 1024 ? 2 : 4)))
void lgn_sgh_onepass_kernel(
    const float *__restrict__ y, const float *__restrict__ gamma,
    const float *__restrict__ beta, int C, long long S, int G, int parts, float eps,
    unsigned long long *__restrict__ part, int spin_limit,
    float *__restrict__ out) {
    __shared__ float red[3 * (kSghThreads / 64)];
    __shared__ float coef_a[MAXCG + 1], coef_b[MAXCG + 1];
    __shared__ float2 own[kSghOnePassMaxParts];
    __shared__ int missing;
    const long long gi = blockIdx.x / parts;
    const int p = blockIdx.x % parts;
    const SghChunkPos pos(gi, p, C, S, G);

    f32x4 v[kSghVec];
    long long ei;
    float ev, mean, m2;
    sgh_chunk_moments<true>(y, pos.sp, v, ei, ev, mean, m2, red);

    unsigned long long *gpart = part + gi * parts;
    if (threadIdx.x == 0) {
        missing = 0;
        __hip_atomic_store(&gpart[p], sgh_pack(mean, m2), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    // entry t of the group: thread t polls it (parts <= kSghOnePassMaxParts = kSghThreads)
    unsigned long long q = kSghEmpty;
    if ((int)threadIdx.x < parts) {
        int polls = 0;
        q = __hip_atomic_load(&gpart[threadIdx.x], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        while (q == kSghEmpty && polls < spin_limit) {
            __builtin_amdgcn_s_sleep(8);
            ++polls;
            q = __hip_atomic_load(&gpart[threadIdx.x], __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
        }
        if (q == kSghEmpty) missing = 1;
    }
    __syncthreads();
    if (!missing) {
        sgh_group_moments(
            [&](int t) {
                (void)t;   // thread t holds entry t (t < parts)
                return make_float2(__uint_as_float((unsigned)q), __uint_as_float((unsigned)(q >> 32)));
            },
            parts, pos.L, mean, m2, red);
    } else {
        // bounded wait ran out: form each chunk's partial here, as its own
        // workgroup does
        for (int t = 0; t < parts; ++t) {
            const SghChunkPos pt(gi, t, C, S, G);
            float wm, wm2;
            sgh_chunk_moments_lean(y, pt.sp, wm, wm2, red);
            if (threadIdx.x == 0) own[t] = make_float2(wm, wm2);
            __syncthreads();   // red is reused by the next chunk's merge
        }
        sgh_group_moments([&](int t) { return own[t]; }, parts, pos.L, mean, m2, red);
    }
    sgh_coefficients<MAXCG>(mean, m2, pos.L, eps, gamma, beta, gi % G, C / G, coef_a, coef_b);
    sgh_store(pos, S, C / G, v, ei, ev, coef_a, coef_b, out);
}

}  // namespace lgn
