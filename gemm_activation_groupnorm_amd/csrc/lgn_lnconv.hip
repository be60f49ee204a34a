// LayerNorm -> GELU -> dilated Conv1d -> + input: launchers of the weight
// packing, statistics and convolution kernels.
#include "lgn_launch.hpp"
#include "lgn_lnconv.hpp"

namespace lgn {

size_t lnconv_wt_bytes(int C) {
    return ((size_t)3 * C * C * sizeof(float) + 255) & ~(size_t)255;
}

template <class Tile, bool TANH, int H>
static hipError_t launch_conv(const float *x, const float *ln_w, const float *ln_b,
                              const float *wt, const float *conv_b, const float2 *part, int B,
                              int C, int L, int dilation, int parts, float eps, float *out,
                              hipStream_t stream) {
    const int tiles_l = (L + Tile::POS - 1) / Tile::POS;
    const int tiles_c = C / Tile::CO;
    const long long blocks = (long long)B * tiles_l * tiles_c;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    return launch_kernel(lgn_lnconv_kernel<Tile, TANH, H>, dim3((unsigned)blocks),
                         dim3(Tile::NT), stream, x, ln_w, ln_b, wt, conv_b, part, C, L, dilation,
                         parts, eps, tiles_l, tiles_c, out);
}

template <class Tile>
static hipError_t launch_conv_any(const float *x, const float *ln_w, const float *ln_b,
                                  const float *wt, const float *conv_b, const float2 *part, int B,
                                  int C, int L, int dilation, int parts, float eps, int gelu_tanh,
                                  float *out, hipStream_t stream) {
    const int H = (dilation + 3) & ~3;
    switch (H * 2 + (gelu_tanh ? 1 : 0)) {
#define LGN_LC(HH, T)                                                                          \
    case HH * 2 + T:                                                                           \
        return launch_conv<Tile, T != 0, HH>(x, ln_w, ln_b, wt, conv_b, part, B, C, L, dilation, \
                                             parts, eps, out, stream);
        LGN_LC(4, 0) LGN_LC(4, 1) LGN_LC(8, 0) LGN_LC(8, 1)
        LGN_LC(12, 0) LGN_LC(12, 1) LGN_LC(16, 0) LGN_LC(16, 1)
#undef LGN_LC
        default: return hipErrorInvalidValue;   // dilation > 16: rejected by the API
    }
}

// Workspace: Wt [3][C][C] (256-byte padded), then B * parts (mean, M2) pairs.
// The 256 x 256 tile serves C % 256 == 0, the 128 x 128 tile any other C % 128 == 0.
hipError_t launch_ln_gelu_conv1d_f32(const float *x, const float *ln_w, const float *ln_b,
                                     const float *conv_w, const float *conv_b, int B, int C,
                                     int L, int dilation, float eps, int gelu_tanh, float *out,
                                     void *workspace, hipStream_t stream) {
    const long long n = (long long)C * L;
    const long long parts = sgh_parts(n);
    const long long stat_blocks = (long long)B * parts;
    if (stat_blocks > 0x7fffffffLL || parts > 0x7fffffffLL) return hipErrorInvalidConfiguration;
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
    if (C % LcLarge::CO == 0)
        return launch_conv_any<LcLarge>(x, ln_w, ln_b, wt, conv_b, part, B, C, L, dilation,
                                        (int)parts, eps, gelu_tanh, out, stream);
    return launch_conv_any<LcSmall>(x, ln_w, ln_b, wt, conv_b, part, B, C, L, dilation,
                                    (int)parts, eps, gelu_tanh, out, stream);
}

}  // namespace lgn
