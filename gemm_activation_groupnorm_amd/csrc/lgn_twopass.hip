// Two-pass ablation: GEMM + linear bias into a workspace, then the
// elementwise + GroupNorm epilogue.
#include "lgn_launch.hpp"
#include "lgn_twopass.hpp"

#include <type_traits>

namespace lgn {

template <class DT, class Cfg, int RING>
static hipError_t launch_gemm_bias_cfg(const typename dt_traits<DT>::storage *x,
                                       const typename dt_traits<DT>::storage *W,
                                       const float *b_lin, int M, int K, int N, float *z,
                                       hipStream_t stream) {
    const int tiles_m = (M + Cfg::BS - 1) / Cfg::BS;
    const int tiles_n = (N + Cfg::BC - 1) / Cfg::BC;
    const long long blocks = (long long)tiles_m * tiles_n;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    return launch_kernel(lgn_gemm_bias_kernel<DT, Cfg, RING>, dim3((unsigned)blocks),
                         dim3(Cfg::NT), stream, x, W, b_lin, M, K, N, z, tiles_m, tiles_n);
}

// The fused kernel's 256 x 256 tile (8 waves of 128 x 64; fp32: ring of 3,
// bf16: ring of 4 with the mid-stage barrier) when K is a multiple of its
// stage depth, else the register-staged core.  The GEMM-only kernel measured
// 1.94-2.55 ms (fp32) and 0.311 ms (bf16) on this tile at 32768 x 1024 x
// 4096, against 2.23-2.34 ms and 0.351 ms on 256 x 128 tiles of 4 waves;
// z is bitwise the same.
template <class DT>
static hipError_t launch_gemm_bias(const typename dt_traits<DT>::storage *x,
                                   const typename dt_traits<DT>::storage *W, const float *b_lin,
                                   int M, int K, int N, float *z, hipStream_t stream) {
    constexpr bool BF = std::is_same<DT, bf16_t>::value;
    typedef typename std::conditional<BF, TileCfg<DT, 256, 256, 2, 4, 64, 2, 2, 2>,
                                      TileCfg<DT, 256, 256, 2, 4, 64, 2>>::type Fast;
    typedef TileCfg<DT, 128, 128, 2, 2, 128, 2> Slow;
    constexpr int RING = BF ? 4 : 3;
    if (K % Fast::BK == 0)
        return launch_gemm_bias_cfg<DT, Fast, RING>(x, W, b_lin, M, K, N, z, stream);
    return launch_gemm_bias_cfg<DT, Slow, 0>(x, W, b_lin, M, K, N, z, stream);
}

hipError_t launch_gemm_bias_f32(const float *x, const float *W, const float *b_lin, int M,
                                int K, int N, float *z, hipStream_t stream) {
    return launch_gemm_bias<f32_t>(x, W, b_lin, M, K, N, z, stream);
}

hipError_t launch_gemm_bias_bf16(const uint16_t *x, const uint16_t *W, const float *b_lin,
                                 int M, int K, int N, float *z, hipStream_t stream) {
    return launch_gemm_bias<bf16_t>(x, W, b_lin, M, K, N, z, stream);
}

template <int LPG, int V>
static hipError_t launch_vec(const float *z, const float *b_add, const float *gamma,
                             const float *beta, int M, int G, float eps, float *out,
                             hipStream_t stream) {
    // one wave per workgroup, 64/LPG units (row pair, group) per wave
    constexpr long long per_block = 64 / LPG;
    const long long units = ((long long)M + 1) / 2 * G;
    const long long blocks = (units + per_block - 1) / per_block;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    return launch_kernel(lgn_gn_epilogue_vec_kernel<LPG, V>, dim3((unsigned)blocks), dim3(64),
                         stream, z, b_add, gamma, beta, (long long)M, G, eps, out);
}

hipError_t launch_gn_epilogue(const float *z, const float *b_add, const float *gamma,
                              const float *beta, int M, int N, int G, float eps, float *out,
                              hipStream_t stream) {
    const int cg = N / G;
    const long long pairs = (long long)M * G;
    switch (cg) {
        case 4: return launch_vec<1, 1>(z, b_add, gamma, beta, M, G, eps, out, stream);
        case 8: return launch_vec<2, 1>(z, b_add, gamma, beta, M, G, eps, out, stream);
        case 16: return launch_vec<4, 1>(z, b_add, gamma, beta, M, G, eps, out, stream);
        case 32: return launch_vec<8, 1>(z, b_add, gamma, beta, M, G, eps, out, stream);
        case 64: return launch_vec<16, 1>(z, b_add, gamma, beta, M, G, eps, out, stream);
        case 128: return launch_vec<32, 1>(z, b_add, gamma, beta, M, G, eps, out, stream);
        case 256: return launch_vec<64, 1>(z, b_add, gamma, beta, M, G, eps, out, stream);
        case 512: return launch_vec<64, 2>(z, b_add, gamma, beta, M, G, eps, out, stream);
        case 1024: return launch_vec<64, 4>(z, b_add, gamma, beta, M, G, eps, out, stream);
        default: {
            if (pairs > 0x7fffffffLL) return hipErrorInvalidConfiguration;
            return launch_kernel(lgn_gn_epilogue_generic_kernel, dim3((unsigned)pairs), dim3(64),
                                 stream, z, b_add, gamma, beta, pairs, G, cg, eps, out);
        }
    }
}

}  // namespace lgn
