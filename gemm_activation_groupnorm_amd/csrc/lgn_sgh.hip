// Swish -> spatial GroupNorm -> HardSwish: launchers of the stats and apply
// kernels.
#include "lgn_launch.hpp"
#include "lgn_sgh.hpp"

namespace lgn {

long long sgh_parts(long long group_elems) {
    return (group_elems + kSghChunk - 1) / kSghChunk;
}

template <int MAXCG>
static hipError_t launch_apply(long long blocks, const float *y, const float *gamma,
                               const float *beta, int C, long long S, int G, int parts,
                               float eps, const float2 *part, float *out, hipStream_t stream) {
    return launch_kernel(lgn_sgh_apply_kernel<MAXCG>, dim3((unsigned)blocks), dim3(kSghThreads),
                         stream, y, gamma, beta, C, S, G, parts, 0LL, eps, part, out);
}

// Sets every (mean, M2) entry of the single-pass kernel to "not arrived".
__global__ __launch_bounds__(256) void lgn_sgh_clear_kernel(unsigned long long *__restrict__ part,
                                                            long long n) {
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i < n) part[i] = kSghEmpty;
}

template <int MAXCG>
static hipError_t launch_onepass(long long blocks, const float *y,
                                 const float *gamma, const float *beta, int C, long long S,
                                 int G, int parts, float eps, unsigned long long *part, float *out,
                                 hipStream_t stream) {
    hipError_t e = launch_kernel(lgn_sgh_clear_kernel, dim3((unsigned)((blocks + 255) / 256)),
                                 dim3(256), stream, part, blocks);
    if (e != hipSuccess) return e;
    return launch_kernel(lgn_sgh_onepass_kernel<MAXCG>, dim3((unsigned)blocks),
                         dim3(kSghThreads), stream, y, gamma, beta, C, S, G, parts, eps, part,
                         g_sgh_spin_limit.load(std::memory_order_relaxed), out);
}

size_t sgh_workspace_bytes(int Nb, int C, long long S, int G) {
    const long long L = (long long)(C / G) * S;
    // one (mean, M2) pair per chunk of every group
    return (size_t)Nb * (size_t)G * (size_t)sgh_parts(L) * 2 * sizeof(float);
}

// Out of place with at most kSghOnePassMaxParts chunks per group: the
// single-pass kernel (y read once).  Otherwise one stats pass over all
// groups, then one apply pass (in place allowed).  (Cutting the groups into
// rounds small enough for the apply pass to re-read them from the MALL
// measured slower at every round size tried: 24 to 160 MB per round.)
hipError_t launch_swish_gn_hardswish_f32(const float *y, const float *gamma, const float *beta,
                                         int Nb, int C, long long S, int G, float eps, float *out,
                                         void *workspace, hipStream_t stream) {
    const int cg = C / G;
    const long long parts = sgh_parts((long long)cg * S);
    const long long groups = (long long)Nb * G;
    const long long blocks = groups * parts;
    if (blocks > 0x7fffffffLL || parts > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    if (cg > 8192) return hipErrorInvalidValue;   // rejected by the API before any launch
    float2 *part = reinterpret_cast<float2 *>(workspace);
    const long long n = groups * cg * S;
    const bool overlap = out < y + n && y < out + n;
    if (!overlap && parts <= kSghOnePassMaxParts) {
        unsigned long long *slots = reinterpret_cast<unsigned long long *>(workspace);
        if (cg <= 64)
            return launch_onepass<64>(blocks, y, gamma, beta, C, S, G, (int)parts, eps,
                                      slots, out, stream);
        if (cg <= 1024)
            return launch_onepass<1024>(blocks, y, gamma, beta, C, S, G, (int)parts,
                                        eps, slots, out, stream);
        return launch_onepass<8192>(blocks, y, gamma, beta, C, S, G, (int)parts, eps,
                                    slots, out, stream);
    }
    hipError_t e = launch_kernel(lgn_sgh_stats_kernel<true>, dim3((unsigned)blocks), dim3(kSghThreads),
                                 stream, y, C, S, G, (int)parts, 0LL, part);
    if (e != hipSuccess) return e;
    const float2 *cpart = part;
    if (cg <= 64)
        return launch_apply<64>(blocks, y, gamma, beta, C, S, G, (int)parts, eps, cpart, out,
                                stream);
    if (cg <= 1024)
        return launch_apply<1024>(blocks, y, gamma, beta, C, S, G, (int)parts, eps, cpart, out,
                                  stream);
    return launch_apply<8192>(blocks, y, gamma, beta, C, S, G, (int)parts, eps, cpart, out,
                              stream);
}

}  // namespace lgn
