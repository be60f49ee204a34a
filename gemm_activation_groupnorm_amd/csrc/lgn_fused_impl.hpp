// lgn_fused_impl.hpp -- tile configuration table of the fused kernel and its
// launcher, shared by the fp32 and bf16 instantiation units.
#pragma once

#include "lgn_fused.hpp"
#include "lgn_launch.hpp"

namespace lgn {

// Tile per channel-per-group count CG (BS samples x BC channels, waves
// along samples x channels, LDS row bytes):
//   CG <= 64  : 128 x 128, 2 x 2 waves of 64 x 64        (group inside a wave)
//   CG == 128 : 128 x 128, 4 x 1 waves of 32 x 128       (group inside a wave)
//   CG == 256 : 128 x 256, 2 x 2 waves of 64 x 128       (2 waves per group)
//   CG == 512 :  64 x 512, 1 x 4 waves of 64 x 128       (4 waves per group)
//   CG == 1024:  64 x 1024, 1 x 8 waves of 64 x 128      (8 waves per group)
template <class DT, class Cfg, int CG>
hipError_t launch_fused_cfg(const typename dt_traits<DT>::storage *x,
                            const typename dt_traits<DT>::storage *W, const float *b_lin,
                            const float *b_add, const float *gamma, const float *beta, int M,
                            int K, int N, float eps, float *out, hipStream_t stream) {
    const int tiles_m = (M + Cfg::BS - 1) / Cfg::BS;
    const int tiles_n = (N + Cfg::BC - 1) / Cfg::BC;
    const long long blocks = (long long)tiles_m * tiles_n;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    return launch_kernel(lgn_fused_kernel<DT, Cfg, CG>, dim3((unsigned)blocks), dim3(Cfg::NT),
                         stream, x, W, b_lin, b_add, gamma, beta, M, K, N, eps, out, tiles_m,
                         tiles_n);
}

template <class DT>
hipError_t launch_fused(const typename dt_traits<DT>::storage *x,
                        const typename dt_traits<DT>::storage *W, const float *b_lin,
                        const float *b_add, const float *gamma, const float *beta, int M, int K,
                        int N, int G, float eps, float *out, hipStream_t stream) {
    constexpr int RB = 128;
    typedef TileCfg<DT, 128, 128, 2, 2, RB> C64;
    typedef TileCfg<DT, 128, 128, 4, 1, RB> C128;
    typedef TileCfg<DT, 128, 256, 2, 2, 64> C256;
    typedef TileCfg<DT, 64, 512, 1, 4, 64> C512;
    typedef TileCfg<DT, 64, 1024, 1, 8, 64> C1024;
    const int cg = N / G;
    switch (cg) {
        case 8: return launch_fused_cfg<DT, C64, 8>(x, W, b_lin, b_add, gamma, beta, M, K, N, eps, out, stream);
        case 16: return launch_fused_cfg<DT, C64, 16>(x, W, b_lin, b_add, gamma, beta, M, K, N, eps, out, stream);
        case 32: return launch_fused_cfg<DT, C64, 32>(x, W, b_lin, b_add, gamma, beta, M, K, N, eps, out, stream);
        case 64: return launch_fused_cfg<DT, C64, 64>(x, W, b_lin, b_add, gamma, beta, M, K, N, eps, out, stream);
        case 128: return launch_fused_cfg<DT, C128, 128>(x, W, b_lin, b_add, gamma, beta, M, K, N, eps, out, stream);
        case 256: return launch_fused_cfg<DT, C256, 256>(x, W, b_lin, b_add, gamma, beta, M, K, N, eps, out, stream);
        case 512: return launch_fused_cfg<DT, C512, 512>(x, W, b_lin, b_add, gamma, beta, M, K, N, eps, out, stream);
        case 1024: return launch_fused_cfg<DT, C1024, 1024>(x, W, b_lin, b_add, gamma, beta, M, K, N, eps, out, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace lgn
