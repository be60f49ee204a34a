// Fused kernel instantiations, fp32 operands (v_mfma_f32_32x32x2_f32).
#include "lgn_fused_impl.hpp"

namespace lgn {
hipError_t launch_fused_f32(const float *x, const float *W, const float *b_lin,
                            const float *b_add, const float *gamma, const float *beta, int M,
                            int K, int N, int G, float eps, float *out, hipStream_t stream) {
    return launch_fused<f32_t>(x, W, b_lin, b_add, gamma, beta, M, K, N, G, eps, out, stream);
}
}  // namespace lgn
