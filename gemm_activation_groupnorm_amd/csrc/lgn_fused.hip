// lgn_fused.hip -- tile configuration table of the fused kernel, its
// launcher, and the fp32 (v_mfma_f32_32x32x2_f32) and bf16
// (v_mfma_f32_32x32x16_bf16) entry points behind lgn_forward_f32/_bf16.

#include "lgn_fused.hpp"
#include "lgn_launch.hpp"

#include <type_traits>

namespace lgn {

// Tiles per channel-per-group count CG, for K a multiple of the stage depth
// (LDS DMA ring) -- BS samples x BC channels, waves along samples x channels:
//   CG <= 64  : 256 x 256, 2 x 4 waves of 128 x 64; bf16: ring of 4 with the
//               mid-stage barrier schedule; fp32: ring of 3
//   CG == 128 : fp32: 128 x 256, 2 x 2 waves of 64 x 128, ring of 3 (4.01 ms
//               against 4.71 ms on 256 x 128 tiles of 4 x 1 waves at 16384 x
//               2048 x 8192, output bitwise the same);
//               bf16: the CG <= 64 tile, 2 waves per group
//   CG == 256 : fp32: 128 x 256, 2 x 2 waves of 64 x 128 (2 waves per group), ring of 3;
//               bf16: the CG <= 64 tile, 4 waves per group
//   CG == 512 : fp32: 64 x 512, 1 x 4 waves of 64 x 128 (4 waves per group), ring of 3;
//               bf16: 128 x 512, 2 x 4 waves of 64 x 128, ring of 3
//   CG == 1024:  64 x 1024, 1 x 8 waves of 64 x 128 (8 waves per group), ring of 2;
//                fp32 with the simple schedule (fragments read right before their MFMAs)
//                and bands of 16 sample tiles
// and register-staged tiles for any other K.  (For fp32 inputs with CG >= 512
// and K a positive multiple of 16, lgn_forward_f32 runs the two-kernel form
// instead: see fused_f32_runs_two_kernels.)
template <class DT, class Cfg, int CG, int RING>
hipError_t launch_fused_cfg(const typename dt_traits<DT>::storage *x,
                            const typename dt_traits<DT>::storage *W, const float *b_lin,
                            const float *b_add, const float *gamma, const float *beta, int M,
                            int K, int N, float eps, float *out, hipStream_t stream) {
    const int tiles_m = (M + Cfg::BS - 1) / Cfg::BS;
    const int tiles_n = (N + Cfg::BC - 1) / Cfg::BC;
    const long long blocks = (long long)tiles_m * tiles_n;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    return launch_kernel(lgn_fused_kernel<DT, Cfg, CG, RING>, dim3((unsigned)blocks),
                         dim3(Cfg::NT), stream, x, W, b_lin, b_add, gamma, beta, M, K, N, eps,
                         out, tiles_m, tiles_n, (float2 *)nullptr);
}

// The LDS DMA ring needs K to be a multiple of its stage depth; any other K
// takes the register-staged core (zero-filled K tail).
template <class DT, class Fast, int RING, class Slow, int CG>
hipError_t launch_fused_pick(const typename dt_traits<DT>::storage *x,
                             const typename dt_traits<DT>::storage *W, const float *b_lin,
                             const float *b_add, const float *gamma, const float *beta, int M,
                             int K, int N, float eps, float *out, hipStream_t stream) {
    if (K % Fast::BK == 0)
        return launch_fused_cfg<DT, Fast, CG, RING>(x, W, b_lin, b_add, gamma, beta, M, K, N, eps,
                                                    out, stream);
    return launch_fused_cfg<DT, Slow, CG, 0>(x, W, b_lin, b_add, gamma, beta, M, K, N, eps, out,
                                             stream);
}

template <class DT>
hipError_t launch_fused(const typename dt_traits<DT>::storage *x,
                        const typename dt_traits<DT>::storage *W, const float *b_lin,
                        const float *b_add, const float *gamma, const float *beta, int M, int K,
                        int N, int G, float eps, float *out, hipStream_t stream) {
    // register-staged fallbacks (any K)
    typedef TileCfg<DT, 128, 128, 2, 2, 128, 2> S64;
    typedef TileCfg<DT, 128, 128, 4, 1, 128> S128;
    typedef TileCfg<DT, 128, 256, 2, 2, 64> S256;
    typedef TileCfg<DT, 64, 512, 1, 4, 64> S512;
    typedef TileCfg<DT, 64, 1024, 1, 8, 32> S1024;
    // LDS DMA ring tiles (K % BK == 0)
    // fp32: end-of-stage barrier, ring of 3; bf16 (16x shorter stages):
    // mid-stage barrier, ring of 4, two sample tiles of MFMAs ahead of reads
    typedef typename std::conditional<std::is_same<DT, bf16_t>::value,
                                      TileCfg<DT, 256, 256, 2, 4, 64, 2, 2, 2>,
                                      TileCfg<DT, 256, 256, 2, 4, 64, 2>>::type F64;
    constexpr int R64 = std::is_same<DT, bf16_t>::value ? 4 : 3;
    // bf16 keeps the 256 x 256 tile up to CG = 256 (groups then span 2 or 4
    // waves, merged through LDS); fp32 measured faster on the narrower tiles
    constexpr bool BF = std::is_same<DT, bf16_t>::value;
    typedef typename std::conditional<BF, F64, TileCfg<DT, 128, 256, 2, 2, 64>>::type F128;
    typedef typename std::conditional<BF, F64, TileCfg<DT, 128, 256, 2, 2, 64>>::type F256;
    constexpr int R128 = BF ? 4 : 3;
    typedef typename std::conditional<BF, TileCfg<DT, 128, 512, 2, 4, 64, 2>,
                                      TileCfg<DT, 64, 512, 1, 4, 64>>::type F512;
    // fp32: simple schedule, bands of 16 sample tiles (the same time as bands
    // of 8 at 16384 x 2048 x 8192, with 1.61 GB fetched beyond L2 per launch
    // instead of 2.42 GB); bf16: fragments read under the MFMAs
    typedef typename std::conditional<BF, TileCfg<DT, 64, 1024, 1, 8, 64, 1, 1>,
                                      TileCfg<DT, 64, 1024, 1, 8, 64, 1, 0, 1, 16>>::type F1024;
    const int cg = N / G;
#define LGN_CASE(C, FAST, RING, SLOW)                                                            \
    case C:                                                                                     \
        return launch_fused_pick<DT, FAST, RING, SLOW, C>(x, W, b_lin, b_add, gamma, beta, M, K, \
                                                          N, eps, out, stream);
    switch (cg) {
        LGN_CASE(8, F64, R64, S64)
        LGN_CASE(16, F64, R64, S64)
        LGN_CASE(32, F64, R64, S64)
        LGN_CASE(64, F64, R64, S64)
        LGN_CASE(128, F128, R128, S128)
        LGN_CASE(256, F256, R128, S256)
        LGN_CASE(512, F512, 3, S512)
        LGN_CASE(1024, F1024, 2, S1024)
        default: return hipErrorInvalidValue;
    }
#undef LGN_CASE
}

hipError_t launch_fused_f32(const float *x, const float *W, const float *b_lin,
                            const float *b_add, const float *gamma, const float *beta, int M,
                            int K, int N, int G, float eps, float *out, hipStream_t stream) {
    return launch_fused<f32_t>(x, W, b_lin, b_add, gamma, beta, M, K, N, G, eps, out, stream);
}

hipError_t launch_fused_bf16(const uint16_t *x, const uint16_t *W, const float *b_lin,
                             const float *b_add, const float *gamma, const float *beta, int M,
                             int K, int N, int G, float eps, float *out, hipStream_t stream) {
    return launch_fused<bf16_t>(x, W, b_lin, b_add, gamma, beta, M, K, N, G, eps, out, stream);
}

}  // namespace lgn
