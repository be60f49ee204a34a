// Linear -> logsumexp -> LeakyReLU x2 -> GELU x2: launchers of the partial
// (GEMM + per-tile row reduction) and finish kernels.
#include "lgn_launch.hpp"
#include "lgn_lse.hpp"

namespace lgn {

template <class DT, class Cfg, int RING>
static hipError_t launch_lse_partial_cfg(const typename dt_traits<DT>::storage *x,
                                         const typename dt_traits<DT>::storage *W,
                                         const float *b, int M, int K, int N, float2 *part,
                                         hipStream_t stream) {
    static_assert(Cfg::BC == kLseTileChannels, "partials are laid out per 256-channel tile");
    const int tiles_m = (M + Cfg::BS - 1) / Cfg::BS;
    const int tiles_n = (N + Cfg::BC - 1) / Cfg::BC;
    const long long blocks = (long long)tiles_m * tiles_n;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    return launch_kernel(lgn_lse_partial_kernel<DT, Cfg, RING>, dim3((unsigned)blocks),
                         dim3(Cfg::NT), stream, x, W, b, M, K, N, part, tiles_m, tiles_n);
}

// 128 x 256 tiles of 4 waves (128 x 64 each): at the transcript's shape
// (1024 x 8192 outputs) that is 256 workgroups, each running the whole K.
// The 4-stage LDS DMA ring (96 KiB) also keeps the dispatcher from placing
// two workgroups on one CU while another CU idles.  K not a multiple of the
// stage depth takes the register-staged core.
template <class DT>
static hipError_t launch_lse(const typename dt_traits<DT>::storage *x,
                             const typename dt_traits<DT>::storage *W, const float *b, int M,
                             int K, int N, float *out, void *workspace, hipStream_t stream) {
    typedef TileCfg<DT, 128, kLseTileChannels, 1, 4, 64, 1> Cfg;
    float2 *part = reinterpret_cast<float2 *>(workspace);
    const hipError_t e =
        K % Cfg::BK == 0 ? launch_lse_partial_cfg<DT, Cfg, 4>(x, W, b, M, K, N, part, stream)
                         : launch_lse_partial_cfg<DT, Cfg, 0>(x, W, b, M, K, N, part, stream);
    if (e != hipSuccess) return e;
    const int tiles_n = (N + kLseTileChannels - 1) / kLseTileChannels;
    return launch_kernel(lgn_lse_finish_kernel, dim3((unsigned)((M + 3) / 4)), dim3(256),
                         stream, part, M, tiles_n, out);
}

hipError_t launch_linear_lse_f32(const float *x, const float *W, const float *b, int M, int K,
                                 int N, float *out, void *workspace, hipStream_t stream) {
    return launch_lse<f32_t>(x, W, b, M, K, N, out, workspace, stream);
}

hipError_t launch_linear_lse_bf16(const uint16_t *x, const uint16_t *W, const float *b, int M,
                                  int K, int N, float *out, void *workspace, hipStream_t stream) {
    return launch_lse<bf16_t>(x, W, b, M, K, N, out, workspace, stream);
}

}  // namespace lgn
