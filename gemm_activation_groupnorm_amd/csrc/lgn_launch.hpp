// lgn_launch.hpp -- host-side launchers of the kernel instantiations.  Each
// returns the HIP error of the launch; argument validation has been done by
// the caller (lgn_api.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <tuple>

namespace lgn {

// Failure injection for the error-path tests (lgn_testing_fail_launches):
// while fail_launches > 0, each launch decrements it and returns
// fail_error instead of launching.
inline std::atomic<int> g_fail_launches{0};
inline std::atomic<int> g_fail_error{0};

inline bool take_injected_failure(hipError_t &e) {
    int n = g_fail_launches.load(std::memory_order_relaxed);
    while (n > 0) {
        if (g_fail_launches.compare_exchange_weak(n, n - 1, std::memory_order_relaxed)) {
            e = (hipError_t)g_fail_error.load(std::memory_order_relaxed);
            return true;
        }
    }
    return false;
}

// Launches `kernel` with hipLaunchKernel and returns that call's own status
// (not a sticky error left by some earlier runtime call).  Arguments are
// converted to the kernel's parameter types first.
template <typename... KArgs, typename... Args>
hipError_t launch_kernel(void (*kernel)(KArgs...), dim3 grid, dim3 block, hipStream_t stream,
                         Args... args) {
    static_assert(sizeof...(KArgs) == sizeof...(Args), "argument count");
    hipError_t injected;
    if (take_injected_failure(injected)) return injected;
    std::tuple<KArgs...> packed(args...);
    void *argv[sizeof...(KArgs) > 0 ? sizeof...(KArgs) : 1];
    std::apply([&](auto &...e) {
        int i = 0;
        ((argv[i++] = (void *)&e), ...);
    }, packed);
    return hipLaunchKernel((const void *)kernel, grid, block, argv, 0, stream);
}

// Channel-per-group counts the fused kernel is instantiated for.
inline bool fused_cg_supported(int cg) {
    return cg == 8 || cg == 16 || cg == 32 || cg == 64 || cg == 128 || cg == 256 ||
           cg == 512 || cg == 1024;
}

// fp32 inputs with 512 or 1024 channels per group: the fused kernel's tile is
// then at most 64 samples tall (a taller one's fp32 accumulators would not fit
// a CU's register file), so it reads W again for every 64 rows.  Two kernels
// in place on `out` -- the GEMM on the 256 x 256 tile writing z, then the
// GroupNorm epilogue -- measured as fast or faster at every M (2048 to 16384)
// and K (1024 to 4096) tried: 3-8 % for 512 channels, up to 7 % for 1024 when
// K >= 2048.  The 256 x 256 tile needs K a multiple of its 16-element stage.
inline bool fused_f32_runs_two_kernels(int K, int cg) {
    return cg >= 512 && K >= 16 && K % 16 == 0;
}
// bf16 inputs: the single kernel wins at K = 1024 (by up to 19 %), the two
// kernels at 1024 channels per group once K >= 2048 (3-22 % at M = 2048 to
// 16384); 512-channel groups are mixed and keep the single kernel.  The bf16
// 256 x 256 tile's stage is 32 elements.
inline bool fused_bf16_runs_two_kernels(int K, int cg) {
    return cg == 1024 && K >= 2048 && K % 32 == 0;
}

hipError_t launch_fused_f32(const float *x, const float *W, const float *b_lin,
                            const float *b_add, const float *gamma, const float *beta, int M,
                            int K, int N, int G, float eps, float *out, hipStream_t stream);
hipError_t launch_fused_bf16(const uint16_t *x, const uint16_t *W, const float *b_lin,
                             const float *b_add, const float *gamma, const float *beta, int M,
                             int K, int N, int G, float eps, float *out, hipStream_t stream);

// Groups wider than one tile (C = N/G a multiple of 256): the workspace
// holds one (mean, M2) float pair per row and per 64 channels.
hipError_t launch_wide_f32(const float *x, const float *W, const float *b_lin, const float *b_add,
                           const float *gamma, const float *beta, int M, int K, int N, int G,
                           float eps, float *out, void *workspace, hipStream_t stream);
hipError_t launch_wide_bf16(const uint16_t *x, const uint16_t *W, const float *b_lin,
                            const float *b_add, const float *gamma, const float *beta, int M,
                            int K, int N, int G, float eps, float *out, void *workspace,
                            hipStream_t stream);
// The library-held scratch that replaces that workspace in the entry point
// that allocates nothing: its size, and its device address on the current
// device (looked up on the first call on each device).
constexpr size_t kWideScratchBytes = (size_t)32 << 20;
hipError_t wide_scratch_address(void **addr);

// Linear -> logsumexp -> LeakyReLU x2 -> GELU x2.  The workspace holds one
// (max, sum) float pair per row and per tile of this many channels.
constexpr int kLseTileChannels = 256;
hipError_t launch_linear_lse_f32(const float *x, const float *W, const float *b, int M, int K,
                                 int N, float *out, void *workspace, hipStream_t stream);
hipError_t launch_linear_lse_bf16(const uint16_t *x, const uint16_t *W, const float *b, int M,
                                  int K, int N, float *out, void *workspace, hipStream_t stream);

// Swish -> spatial GroupNorm -> HardSwish.  The workspace holds one
// (mean, M2) float pair per chunk of kSghChunk elements of every group.
long long sgh_parts(long long group_elems);
size_t sgh_workspace_bytes(int Nb, int C, long long S, int G);
// Polls of the single-pass kernel's bounded wait before it forms the group's
// statistics itself (lgn_testing_set_sgh_spin_limit).
constexpr int kSghSpinLimit = 1 << 16;
inline std::atomic<int> g_sgh_spin_limit{kSghSpinLimit};

// LayerNorm -> GELU -> dilated Conv1d -> + input (C % 128 == 0, L % 4 == 0,
// dilation 1..16).  The workspace holds the packed weights
// (lnconv_wt_bytes(C)) followed by the per-sample statistics partials.
size_t lnconv_wt_bytes(int C);
hipError_t launch_ln_gelu_conv1d_f32(const float *x, const float *ln_w, const float *ln_b,
                                     const float *conv_w, const float *conv_b, int B, int C,
                                     int L, int dilation, float eps, int gelu_tanh, float *out,
                                     void *workspace, hipStream_t stream);
hipError_t launch_swish_gn_hardswish_f32(const float *y, const float *gamma, const float *beta,
                                         int Nb, int C, long long S, int G, float eps, float *out,
                                         void *workspace, hipStream_t stream);

hipError_t launch_gemm_bias_f32(const float *x, const float *W, const float *b_lin, int M,
                                int K, int N, float *z, hipStream_t stream);
hipError_t launch_gemm_bias_bf16(const uint16_t *x, const uint16_t *W, const float *b_lin,
                                 int M, int K, int N, float *z, hipStream_t stream);
hipError_t launch_gn_epilogue(const float *z, const float *b_add, const float *gamma,
                              const float *beta, int M, int N, int G, float eps, float *out,
                              hipStream_t stream);

}  // namespace lgn
