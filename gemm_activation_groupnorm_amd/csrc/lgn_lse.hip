// Linear -> logsumexp -> LeakyReLU x2 -> GELU x2: launchers of the partial
// (GEMM + per-tile row reduction) and finish kernels.
#include "lgn_launch.hpp"
#include "lgn_lse.hpp"

#include <type_traits>

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

// 128 x 256 tiles: at the transcript's shape (1024 x 8192 outputs) that is
// 256 workgroups, each running the whole K, and an LDS ring large enough to
// keep the dispatcher from placing two workgroups on one CU while another
// idles.
//   fp32: 4 waves of 128 x 64, 4-stage ring of 64-byte rows (96 KiB).
//   bf16: 8 waves of 64 x 64, 3-stage ring of 128-byte rows (whole cache
//         lines, 144 KiB) with the mid-stage barrier; at 1024 x 8192 x 8192
//         0.127-0.128 ms against 0.134-0.139 ms for the fp32 tile's
//         64-byte rows, bitwise the same output.  K that is a multiple of 32
//         but not of 64 keeps the 64-byte rows.
// K not a multiple of any stage depth takes the register-staged core.
template <class DT>
static hipError_t launch_lse(const typename dt_traits<DT>::storage *x,
                             const typename dt_traits<DT>::storage *W, const float *b, int M,
                             int K, int N, float *out, void *workspace, hipStream_t stream) {
    typedef TileCfg<DT, 128, kLseTileChannels, 1, 4, 64, 1> Cfg;
    typedef TileCfg<DT, 128, kLseTileChannels, 2, 4, 128, 2, 2, 1> Wide;
    constexpr bool BF = std::is_same<DT, bf16_t>::value;
    float2 *part = reinterpret_cast<float2 *>(workspace);
    const hipError_t e =
        BF && K % Wide::BK == 0
            ? launch_lse_partial_cfg<DT, Wide, 3>(x, W, b, M, K, N, part, stream)
        : K % Cfg::BK == 0 ? launch_lse_partial_cfg<DT, Cfg, 4>(x, W, b, M, K, N, part, stream)
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
