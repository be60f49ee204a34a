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

template <int LPG, int V, int R, int EW>
static hipError_t launch_masked(const float *z, const float *b_add, const float *gamma,
                                const float *beta, int M, int G, int cg, float eps, float *out,
                                hipStream_t stream) {
    // one wave per workgroup, 64/LPG units (R rows, group) per wave
    constexpr long long per_block = 64 / LPG;
    const long long units = ((long long)M + R - 1) / R * G;
    const long long blocks = (units + per_block - 1) / per_block;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    return launch_kernel(lgn_gn_epilogue_masked_kernel<LPG, V, R, EW>, dim3((unsigned)blocks),
                         dim3(64), stream, z, b_add, gamma, beta, (long long)M, G, cg, eps, out);
}

// Group widths not of the form 4*LPG*V, in slots of EW channels (F = cg/EW
// slots per group, at most 2048): the masked kernel with the fewest lanes
// (F <= 64) or the fewest slots per lane (above) that cover the group, two
// rows per lane except for float4 slots above 64 per group and for 32 slots
// per lane.  Two rows per
// lane measured about 10 % faster at 48, 96 and 200 channels and 2.5 %
// slower at 768 (float4 slots).  Two-float slots against one-float slots:
// 0.676 -> 0.362 ms at 50 channels, 0.408 -> 0.317 ms at 250 (32768 rows).
template <int EW>
static hipError_t launch_masked_any(const float *z, const float *b_add, const float *gamma,
                                    const float *beta, int M, int G, int cg, float eps,
                                    float *out, hipStream_t stream) {
    const int F = cg / EW;
#define LGN_MASKED(LPG, V, R) \
    launch_masked<LPG, V, R, EW>(z, b_add, gamma, beta, M, G, cg, eps, out, stream)
    if (F <= 2) return LGN_MASKED(2, 1, 2);
    if (F <= 4) return LGN_MASKED(4, 1, 2);
    if (F <= 8) return LGN_MASKED(8, 1, 2);
    if (F <= 16) return LGN_MASKED(16, 1, 2);
    if (F <= 32) return LGN_MASKED(32, 1, 2);
    if (F <= 64) return LGN_MASKED(64, 1, 2);
    constexpr int RB = EW == 4 ? 1 : 2;
    if (F <= 128) return LGN_MASKED(64, 2, RB);
    if (F <= 256) return LGN_MASKED(64, 4, RB);
    if (F <= 512) return LGN_MASKED(64, 8, RB);
    if (F <= 1024) return LGN_MASKED(64, 16, RB);
    return LGN_MASKED(64, 32, 1);
#undef LGN_MASKED
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
            if (cg % 4 == 0 && cg <= 8192)
                return launch_masked_any<4>(z, b_add, gamma, beta, M, G, cg, eps, out, stream);
            if (cg % 4 != 0 && cg % 2 == 0 && cg <= 4096)
                return launch_masked_any<2>(z, b_add, gamma, beta, M, G, cg, eps, out, stream);
            if (cg % 2 != 0 && cg <= 2048)
                return launch_masked_any<1>(z, b_add, gamma, beta, M, G, cg, eps, out, stream);
            if (pairs > 0x7fffffffLL) return hipErrorInvalidConfiguration;
            return launch_kernel(lgn_gn_epilogue_generic_kernel, dim3((unsigned)pairs), dim3(64),
                                 stream, z, b_add, gamma, beta, pairs, G, cg, eps, out);
        }
    }
}

}  // namespace lgn
