// LayerNorm -> GELU -> dilated Conv1d -> + input: launchers of the weight
// packing, statistics and convolution kernels.
#include "lgn_launch.hpp"
#include "lgn_lnconv.hpp"

namespace lgn {

size_t lnconv_wt_bytes(int C) {
    return ((size_t)3 * C * C * sizeof(float) + 255) & ~(size_t)255;
}

// Workspace: Wt [3][C][C] (256-byte padded), then B * parts (mean, M2) pairs.
hipError_t launch_ln_gelu_conv1d_f32(const float *x, const float *ln_w, const float *ln_b,
                                     const float *conv_w, const float *conv_b, int B, int C,
                                     int L, int dilation, float eps, int gelu_tanh, float *out,
                                     void *workspace, hipStream_t stream) {
    const long long n = (long long)C * L;
    const long long parts = sgh_parts(n);
    const int tiles_l = (L + kLcPos - 1) / kLcPos;
    const int tiles_c = C / kLcCo;
    const long long blocks = (long long)B * tiles_l * tiles_c;
    const long long stat_blocks = (long long)B * parts;
    if (blocks > 0x7fffffffLL || stat_blocks > 0x7fffffffLL || parts > 0x7fffffffLL)
        return hipErrorInvalidConfiguration;
    float *wt = reinterpret_cast<float *>(workspace);
    float2 *part = reinterpret_cast<float2 *>(reinterpret_cast<char *>(workspace) +
                                              lnconv_wt_bytes(C));
    const long long nw = 3LL * C * C;
    hipError_t e = launch_kernel(lgn_conv_wpack_kernel, dim3((unsigned)((nw + 255) / 256)),
                                 dim3(256), stream, conv_w, C, wt);
    if (e != hipSuccess) return e;
    // per-sample statistics: one group of C * L values per sample, no Swish
    e = launch_kernel(lgn_sgh_stats_kernel<false>, dim3((unsigned)stat_blocks), dim3(kSghThreads),
                      stream, x, C, (long long)L, 1, (int)parts, 0LL, part);
    if (e != hipSuccess) return e;
    const int H = (dilation + 3) & ~3;
    if (gelu_tanh)
        return launch_kernel(lgn_lnconv_kernel<true>, dim3((unsigned)blocks), dim3(kLcThreads),
                             stream, x, ln_w, ln_b, (const float *)wt, conv_b,
                             (const float2 *)part, C, L, dilation, H, (int)parts, eps, tiles_l,
                             tiles_c, out);
    return launch_kernel(lgn_lnconv_kernel<false>, dim3((unsigned)blocks), dim3(kLcThreads),
                         stream, x, ln_w, ln_b, (const float *)wt, conv_b, (const float2 *)part,
                         C, L, dilation, H, (int)parts, eps, tiles_l, tiles_c, out);
}

}  // namespace lgn
