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

// One stats pass over all groups, then one apply pass.  (Cutting the groups
// into rounds small enough for the apply pass to re-read them from the MALL
// measured slower at every round size tried: 24 to 160 MB per round.)
hipError_t launch_swish_gn_hardswish_f32(const float *y, const float *gamma, const float *beta,
                                         int Nb, int C, long long S, int G, float eps, float *out,
                                         void *workspace, hipStream_t stream) {
    const int cg = C / G;
    const long long parts = sgh_parts((long long)cg * S);
    const long long blocks = (long long)Nb * G * parts;
    if (blocks > 0x7fffffffLL || parts > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    if (cg > 8192) return hipErrorInvalidValue;   // rejected by the API before any launch
    float2 *part = reinterpret_cast<float2 *>(workspace);
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
