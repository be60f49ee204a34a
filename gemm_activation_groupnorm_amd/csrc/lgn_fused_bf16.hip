// Fused kernel instantiations, bf16 operands (v_mfma_f32_32x32x16_bf16).
#include "lgn_fused_impl.hpp"

namespace lgn {
hipError_t launch_fused_bf16(const uint16_t *x, const uint16_t *W, const float *b_lin,
                             const float *b_add, const float *gamma, const float *beta, int M,
                             int K, int N, int G, float eps, float *out, hipStream_t stream) {
    return launch_fused<bf16_t>(x, W, b_lin, b_add, gamma, beta, M, K, N, G, eps, out, stream);
}
}  // namespace lgn
