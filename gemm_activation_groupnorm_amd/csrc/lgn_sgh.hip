// Swish -> spatial GroupNorm -> HardSwish: launchers of the stats and apply
// kernels.
#include "lgn_launch.hpp"
#include "lgn_sgh.hpp"

namespace lgn {

long long sgh_parts(long long group_elems) {
    return (group_elems + kSghChunk - 1) / kSghChunk;
}

hipError_t launch_swish_gn_hardswish_f32(const float *y, const float *gamma, const float *beta,
                                         int Nb, int C, long long S, int G, float eps, float *out,
                                         void *workspace, hipStream_t stream) {
    const long long parts = sgh_parts((long long)(C / G) * S);
    const long long blocks = (long long)Nb * G * parts;
    if (blocks > 0x7fffffffLL || parts > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    float2 *part = reinterpret_cast<float2 *>(workspace);
    hipError_t e = launch_kernel(lgn_sgh_stats_kernel, dim3((unsigned)blocks), dim3(kSghThreads),
                                 stream, y, C, S, G, (int)parts, part);
    if (e != hipSuccess) return e;
    return launch_kernel(lgn_sgh_apply_kernel, dim3((unsigned)blocks), dim3(kSghThreads), stream,
                         y, gamma, beta, C, S, G, (int)parts, eps, (const float2 *)part, out);
}

}  // namespace lgn
