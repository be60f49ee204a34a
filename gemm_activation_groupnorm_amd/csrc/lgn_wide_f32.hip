// fp32 instantiation of the wide-group forward.
#include "lgn_wide_impl.hpp"

namespace lgn {

hipError_t launch_wide_f32(const float *x, const float *W, const float *b_lin, const float *b_add,
                           const float *gamma, const float *beta, int M, int K, int N, int G,
                           float eps, float *out, void *workspace, hipStream_t stream) {
    return launch_wide<f32_t>(x, W, b_lin, b_add, gamma, beta, M, K, N, G, eps, out, workspace,
                              stream);
}

}  // namespace lgn
