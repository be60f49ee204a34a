// lgn_api.hip -- the C ABI of liblgn.so (declared in include/lgn.h):
// argument validation (host only, before any HIP call), the gfx950 device
// check, and dispatch to the kernel launchers.
#include "lgn.h"

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <atomic>

#include "lgn_launch.hpp"

namespace {

enum Dtype { DT_F32 = 0, DT_BF16 = 1 };

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// Sizes, eps and pointers.  Returns LGN_OK, LGN_ERR_INVALID_ARG or
// LGN_ERR_UNSUPPORTED; makes no HIP call.
lgn_status validate(int dtype, const void *x, const void *W, const float *b_lin,
                    const float *b_add, const float *gamma, const float *beta, int M, int K, int N,
                    int G, float eps, const float *out) {
    if (M < 0 || K < 0 || N < 1 || G < 1) return LGN_ERR_INVALID_ARG;
    if (N % G != 0) return LGN_ERR_INVALID_ARG;
    if (!(eps > 0.0f) || !isfinite(eps)) return LGN_ERR_INVALID_ARG;
    if (M == 0) return LGN_OK;   // empty batch: nothing is read or written
    if (!b_lin || !b_add || !gamma || !beta || !out) return LGN_ERR_INVALID_ARG;
    if (K > 0 && (!x || !W)) return LGN_ERR_INVALID_ARG;
    const int epc = dtype == DT_F32 ? 4 : 8;   // elements per 16-byte load
    if (K % epc != 0 || N % 4 != 0) return LGN_ERR_UNSUPPORTED;
    if (!aligned(x, 16) || !aligned(W, 16) || !aligned(out, 16)) return LGN_ERR_UNSUPPORTED;
    if (!aligned(b_lin, 4) || !aligned(b_add, 4) || !aligned(gamma, 4) || !aligned(beta, 4))
        return LGN_ERR_UNSUPPORTED;
    return LGN_OK;
}

// The HIP error behind the last LGN_ERR_HIP returned on this thread.
thread_local hipError_t g_last_hip = hipSuccess;

lgn_status from_hip(hipError_t e) {
    if (e == hipSuccess) return LGN_OK;
    g_last_hip = e;
    return LGN_ERR_HIP;
}

// Per-device cache of "is this a gfx950": 0 unknown, 1 yes, 2 no.
constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_ok[kMaxDevices];

bool is_gfx950(const char *arch) { return strncmp(arch, "gfx950", 6) == 0; }

// Architecture name set by lgn_testing_set_arch (empty: query the device).
char g_arch_override[64];
std::atomic<bool> g_arch_overridden{false};

lgn_status check_device() {
    if (g_arch_overridden.load(std::memory_order_acquire))
        return is_gfx950(g_arch_override) ? LGN_OK : LGN_ERR_UNSUPPORTED;
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return from_hip(e);
    if (dev < 0) return from_hip(hipErrorInvalidDevice);
    if (dev < kMaxDevices) {
        const int c = g_arch_ok[dev].load(std::memory_order_relaxed);
        if (c == 1) return LGN_OK;
        if (c == 2) return LGN_ERR_UNSUPPORTED;
    }
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return from_hip(e);
    const bool ok = is_gfx950(prop.gcnArchName);
    if (dev < kMaxDevices) g_arch_ok[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
    return ok ? LGN_OK : LGN_ERR_UNSUPPORTED;
}

template <int DT, class T>
lgn_status forward_fused(const T *x, const T *W, const float *b_lin, const float *b_add,
                         const float *gamma, const float *beta, int M, int K, int N, int G,
                         float eps, float *out, hipStream_t stream) {
    lgn_status s = validate(DT, x, W, b_lin, b_add, gamma, beta, M, K, N, G, eps, out);
    if (s != LGN_OK || M == 0) return s;
    if (!lgn::fused_cg_supported(N / G)) return LGN_ERR_UNSUPPORTED;
    s = check_device();
    if (s != LGN_OK) return s;
    if (DT == DT_F32 ? lgn::fused_f32_runs_two_kernels(K, N / G)
                     : lgn::fused_bf16_runs_two_kernels(K, N / G)) {
        // z = x W^T + b_lin into out on the 256 x 256 GEMM tile, then the
        // GroupNorm epilogue in place
        hipError_t e = DT == DT_F32
                           ? lgn::launch_gemm_bias_f32((const float *)x, (const float *)W, b_lin,
                                                       M, K, N, out, stream)
                           : lgn::launch_gemm_bias_bf16((const uint16_t *)x, (const uint16_t *)W,
                                                        b_lin, M, K, N, out, stream);
        if (e != hipSuccess) return from_hip(e);
        return from_hip(lgn::launch_gn_epilogue(out, b_add, gamma, beta, M, N, G, eps, out,
                                                stream));
    }
    if (DT == DT_F32)
        return from_hip(lgn::launch_fused_f32((const float *)x, (const float *)W, b_lin, b_add,
                                              gamma, beta, M, K, N, G, eps, out, stream));
    return from_hip(lgn::launch_fused_bf16((const uint16_t *)x, (const uint16_t *)W, b_lin,
                                           b_add, gamma, beta, M, K, N, G, eps, out, stream));
}

template <int DT, class T>
lgn_status forward_twopass(const T *x, const T *W, const float *b_lin, const float *b_add,
                           const float *gamma, const float *beta, int M, int K, int N, int G,
                           float eps, float *out, void *workspace, size_t ws_bytes,
                           hipStream_t stream) {
    lgn_status s = validate(DT, x, W, b_lin, b_add, gamma, beta, M, K, N, G, eps, out);
    if (s != LGN_OK || M == 0) return s;
    if (!workspace || ws_bytes < lgn_twopass_workspace_bytes(M, N)) return LGN_ERR_INVALID_ARG;
    if (!aligned(workspace, 16)) return LGN_ERR_UNSUPPORTED;
    s = check_device();
    if (s != LGN_OK) return s;
    float *z = (float *)workspace;
    hipError_t e = DT == DT_F32
                       ? lgn::launch_gemm_bias_f32((const float *)x, (const float *)W, b_lin, M,
                                                   K, N, z, stream)
                       : lgn::launch_gemm_bias_bf16((const uint16_t *)x, (const uint16_t *)W,
                                                    b_lin, M, K, N, z, stream);
    if (e != hipSuccess) return from_hip(e);
    return from_hip(lgn::launch_gn_epilogue(z, b_add, gamma, beta, M, N, G, eps, out, stream));
}

template <int DT, class T>
lgn_status forward_wide(const T *x, const T *W, const float *b_lin, const float *b_add,
                        const float *gamma, const float *beta, int M, int K, int N, int G,
                        float eps, float *out, void *workspace, size_t ws_bytes,
                        hipStream_t stream) {
    lgn_status s = validate(DT, x, W, b_lin, b_add, gamma, beta, M, K, N, G, eps, out);
    if (s != LGN_OK || M == 0) return s;
    if ((N / G) % 256 != 0) return LGN_ERR_UNSUPPORTED;
    if (!aligned(gamma, 16) || !aligned(beta, 16)) return LGN_ERR_UNSUPPORTED;
    if (!workspace || ws_bytes < lgn_wide_workspace_bytes(M, N)) return LGN_ERR_INVALID_ARG;
    if (!aligned(workspace, 8)) return LGN_ERR_UNSUPPORTED;
    s = check_device();
    if (s != LGN_OK) return s;
    if (DT == DT_F32)
        return from_hip(lgn::launch_wide_f32((const float *)x, (const float *)W, b_lin, b_add,
                                             gamma, beta, M, K, N, G, eps, out, workspace,
                                             stream));
    return from_hip(lgn::launch_wide_bf16((const uint16_t *)x, (const uint16_t *)W, b_lin, b_add,
                                          gamma, beta, M, K, N, G, eps, out, workspace, stream));
}

// The wide forward with the library's own scratch in place of the caller's
// workspace: no allocation of any kind (for callers that cannot allocate).
lgn_status forward_wide_noalloc(const float *x, const float *W, const float *b_lin,
                                const float *b_add, const float *gamma, const float *beta,
                                int M, int K, int N, int G, float eps, float *out,
                                hipStream_t stream) {
    lgn_status s = validate(DT_F32, x, W, b_lin, b_add, gamma, beta, M, K, N, G, eps, out);
    if (s != LGN_OK || M == 0) return s;
    if ((N / G) % 256 != 0) return LGN_ERR_UNSUPPORTED;
    if (!aligned(gamma, 16) || !aligned(beta, 16)) return LGN_ERR_UNSUPPORTED;
    if (lgn_wide_workspace_bytes(M, N) > lgn::kWideScratchBytes) return LGN_ERR_TOO_LARGE;
    s = check_device();
    if (s != LGN_OK) return s;
    void *ws = nullptr;
    hipError_t e = lgn::wide_scratch_address(&ws);
    if (e != hipSuccess) return from_hip(e);
    return from_hip(lgn::launch_wide_f32(x, W, b_lin, b_add, gamma, beta, M, K, N, G, eps, out,
                                         ws, stream));
}

template <int DT, class T>
lgn_status linear_lse(const T *x, const T *W, const float *b, int M, int K, int N, float *out,
                      void *workspace, size_t ws_bytes, hipStream_t stream) {
    if (M < 0 || K < 0 || N < 1) return LGN_ERR_INVALID_ARG;
    if (M == 0) return LGN_OK;   // empty batch: nothing is read or written
    if (!b || !out || !workspace) return LGN_ERR_INVALID_ARG;
    if (K > 0 && (!x || !W)) return LGN_ERR_INVALID_ARG;
    if (ws_bytes < lgn_lse_workspace_bytes(M, N)) return LGN_ERR_INVALID_ARG;
    const int epc = DT == DT_F32 ? 4 : 8;
    if (K % epc != 0 || N % 4 != 0) return LGN_ERR_UNSUPPORTED;
    if (!aligned(x, 16) || !aligned(W, 16) || !aligned(b, 4) || !aligned(out, 4) ||
        !aligned(workspace, 8))
        return LGN_ERR_UNSUPPORTED;
    lgn_status s = check_device();
    if (s != LGN_OK) return s;
    if (DT == DT_F32)
        return from_hip(lgn::launch_linear_lse_f32((const float *)x, (const float *)W, b, M, K,
                                                   N, out, workspace, stream));
    return from_hip(lgn::launch_linear_lse_bf16((const uint16_t *)x, (const uint16_t *)W, b, M,
                                                K, N, out, workspace, stream));
}

}  // namespace

extern "C" {

lgn_status lgn_forward_f32(const float *x, const float *W, const float *b_lin,
                           const float *b_add, const float *gamma, const float *beta, int M,
                           int K, int N, int G, float eps, float *out, hipStream_t stream) {
    return forward_fused<DT_F32>(x, W, b_lin, b_add, gamma, beta, M, K, N, G, eps, out, stream);
}

lgn_status lgn_forward_bf16(const lgn_bf16 *x, const lgn_bf16 *W, const float *b_lin,
                            const float *b_add, const float *gamma, const float *beta, int M,
                            int K, int N, int G, float eps, float *out, hipStream_t stream) {
    return forward_fused<DT_BF16>(x, W, b_lin, b_add, gamma, beta, M, K, N, G, eps, out, stream);
}

int lgn_fused_supported(int dtype, int M, int K, int N, int G) {
    if (dtype != DT_F32 && dtype != DT_BF16) return 0;
    if (M < 0 || K < 0 || N < 1 || G < 1 || N % G != 0) return 0;
    const int epc = dtype == DT_F32 ? 4 : 8;
    if (K % epc != 0 || N % 4 != 0) return 0;
    return lgn::fused_cg_supported(N / G) ? 1 : 0;
}

size_t lgn_twopass_workspace_bytes(int M, int N) {
    if (M <= 0 || N <= 0) return 0;
    return (size_t)M * (size_t)N * sizeof(float);
}

lgn_status lgn_forward_twopass_f32(const float *x, const float *W, const float *b_lin,
                                   const float *b_add, const float *gamma, const float *beta,
                                   int M, int K, int N, int G, float eps, float *out,
                                   void *workspace, size_t workspace_bytes, hipStream_t stream) {
    return forward_twopass<DT_F32>(x, W, b_lin, b_add, gamma, beta, M, K, N, G, eps, out,
                                   workspace, workspace_bytes, stream);
}

lgn_status lgn_forward_twopass_bf16(const lgn_bf16 *x, const lgn_bf16 *W, const float *b_lin,
                                    const float *b_add, const float *gamma, const float *beta,
                                    int M, int K, int N, int G, float eps, float *out,
                                    void *workspace, size_t workspace_bytes, hipStream_t stream) {
    return forward_twopass<DT_BF16>(x, W, b_lin, b_add, gamma, beta, M, K, N, G, eps, out,
                                    workspace, workspace_bytes, stream);
}

size_t lgn_wide_workspace_bytes(int M, int N) {
    if (M <= 0 || N <= 0) return 0;
    return (size_t)M * (size_t)((N + 63) / 64) * 2 * sizeof(float);
}

lgn_status lgn_forward_wide_f32(const float *x, const float *W, const float *b_lin,
                                const float *b_add, const float *gamma, const float *beta, int M,
                                int K, int N, int G, float eps, float *out, void *workspace,
                                size_t workspace_bytes, hipStream_t stream) {
    return forward_wide<DT_F32>(x, W, b_lin, b_add, gamma, beta, M, K, N, G, eps, out, workspace,
                                workspace_bytes, stream);
}

lgn_status lgn_forward_wide_bf16(const lgn_bf16 *x, const lgn_bf16 *W, const float *b_lin,
                                 const float *b_add, const float *gamma, const float *beta, int M,
                                 int K, int N, int G, float eps, float *out, void *workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
    return forward_wide<DT_BF16>(x, W, b_lin, b_add, gamma, beta, M, K, N, G, eps, out, workspace,
                                 workspace_bytes, stream);
}

lgn_status lgn_forward_wide_f32_noalloc(const float *x, const float *W, const float *b_lin,
                                        const float *b_add, const float *gamma,
                                        const float *beta, int M, int K, int N, int G, float eps,
                                        float *out, hipStream_t stream) {
    static_assert(lgn::kWideScratchBytes == LGN_WIDE_NOALLOC_SCRATCH_BYTES, "header limit");
    return forward_wide_noalloc(x, W, b_lin, b_add, gamma, beta, M, K, N, G, eps, out, stream);
}

size_t lgn_lse_workspace_bytes(int M, int N) {
    if (M <= 0 || N <= 0) return 0;
    const size_t tiles = ((size_t)N + lgn::kLseTileChannels - 1) / lgn::kLseTileChannels;
    return (size_t)M * tiles * 2 * sizeof(float);
}

lgn_status lgn_linear_lse_f32(const float *x, const float *W, const float *b, int M, int K,
                              int N, float *out, void *workspace, size_t workspace_bytes,
                              hipStream_t stream) {
    return linear_lse<DT_F32>(x, W, b, M, K, N, out, workspace, workspace_bytes, stream);
}

lgn_status lgn_linear_lse_bf16(const lgn_bf16 *x, const lgn_bf16 *W, const float *b, int M,
                               int K, int N, float *out, void *workspace, size_t workspace_bytes,
                               hipStream_t stream) {
    return linear_lse<DT_BF16>(x, W, b, M, K, N, out, workspace, workspace_bytes, stream);
}

size_t lgn_sgh_workspace_bytes(int Nb, int C, long long S, int G) {
    if (Nb <= 0 || C <= 0 || S <= 0 || G <= 0 || C % G != 0) return 0;
    const long long L = (long long)(C / G) * S;
    if (L > 0x7fffffffLL) return 0;
    return lgn::sgh_workspace_bytes(Nb, C, S, G);
}

size_t lgn_lnconv_workspace_bytes(int B, int C, int L) {
    if (B <= 0 || C <= 0 || L <= 0) return 0;
    const long long parts = lgn::sgh_parts((long long)C * L);
    return lgn::lnconv_wt_bytes(C) + (size_t)B * (size_t)parts * 2 * sizeof(float);
}

lgn_status lgn_ln_gelu_conv1d_f32(const float *x, const float *ln_w, const float *ln_b,
                                  const float *conv_w, const float *conv_b, int B, int C, int L,
                                  int dilation, float eps, int gelu_tanh, float *out,
                                  void *workspace, size_t workspace_bytes, hipStream_t stream) {
    if (B < 0 || C < 1 || L < 1 || dilation < 1) return LGN_ERR_INVALID_ARG;
    if (!(eps > 0.0f) || !isfinite(eps)) return LGN_ERR_INVALID_ARG;
    if (B == 0) return LGN_OK;   // empty batch: nothing is read or written
    if (!x || !ln_w || !ln_b || !conv_w || !conv_b || !out || !workspace)
        return LGN_ERR_INVALID_ARG;
    if (out == x) return LGN_ERR_INVALID_ARG;   // the convolution reads neighbours of x
    if (C % 128 != 0 || L % 4 != 0 || dilation > 16) return LGN_ERR_UNSUPPORTED;
    // the convolution addresses a sample and the packed weights with 32-bit
    // byte offsets
    if ((long long)C * L >= (1LL << 29) || C > 8192) return LGN_ERR_UNSUPPORTED;
    if (workspace_bytes < lgn_lnconv_workspace_bytes(B, C, L)) return LGN_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(ln_w, 16) || !aligned(ln_b, 16) || !aligned(out, 16) ||
        !aligned(workspace, 16) || !aligned(conv_w, 4) || !aligned(conv_b, 4))
        return LGN_ERR_UNSUPPORTED;
    lgn_status s = check_device();
    if (s != LGN_OK) return s;
    return from_hip(lgn::launch_ln_gelu_conv1d_f32(x, ln_w, ln_b, conv_w, conv_b, B, C, L,
                                                   dilation, eps, gelu_tanh, out, workspace,
                                                   stream));
}

lgn_status lgn_swish_gn_hardswish_f32(const float *y, const float *gamma, const float *beta,
                                      int Nb, int C, long long S, int G, float eps, float *out,
                                      void *workspace, size_t workspace_bytes,
                                      hipStream_t stream) {
    if (Nb < 0 || C < 1 || S < 1 || G < 1 || C % G != 0) return LGN_ERR_INVALID_ARG;
    if (!(eps > 0.0f) || !isfinite(eps)) return LGN_ERR_INVALID_ARG;
    if (Nb == 0) return LGN_OK;   // empty batch: nothing is read or written
    if ((long long)(C / G) * S > 0x7fffffffLL || C / G > 8192) return LGN_ERR_UNSUPPORTED;
    if (!y || !gamma || !beta || !out || !workspace) return LGN_ERR_INVALID_ARG;
    if (workspace_bytes < lgn_sgh_workspace_bytes(Nb, C, S, G)) return LGN_ERR_INVALID_ARG;
    if (!aligned(y, 16) || !aligned(out, 16) || !aligned(gamma, 4) || !aligned(beta, 4) ||
        !aligned(workspace, 8))
        return LGN_ERR_UNSUPPORTED;
    lgn_status s = check_device();
    if (s != LGN_OK) return s;
    return from_hip(lgn::launch_swish_gn_hardswish_f32(y, gamma, beta, Nb, C, S, G, eps, out,
                                                       workspace, stream));
}

const char *lgn_status_string(lgn_status s) {
    switch (s) {
        case LGN_OK: return "LGN_OK: success";
        case LGN_ERR_INVALID_ARG:
            return "LGN_ERR_INVALID_ARG: null pointer, bad size, N % G != 0, eps not > 0 and "
                   "finite, or workspace too small";
        case LGN_ERR_UNSUPPORTED:
            return "LGN_ERR_UNSUPPORTED: device is not gfx950, or shape/alignment not covered "
                   "(16-byte aligned x/W/out, N % 4 == 0, K % 4 (fp32) or K % 8 (bf16) == 0; "
                   "fused: N/G a power of two in 8..1024)";
        case LGN_ERR_HIP: return "LGN_ERR_HIP: a HIP runtime call or kernel launch failed";
        case LGN_ERR_TOO_LARGE:
            return "LGN_ERR_TOO_LARGE: the call needs more scratch than the no-allocation entry "
                   "point holds (LGN_WIDE_NOALLOC_SCRATCH_BYTES)";
        default: return "unknown lgn_status";
    }
}

const char *lgn_version(void) { return "0.1.0"; }

const char *lgn_last_hip_error_string(void) {
    return g_last_hip == hipSuccess ? "no HIP error" : hipGetErrorString(g_last_hip);
}

void lgn_testing_set_arch(const char *arch) {
    if (!arch) {
        g_arch_overridden.store(false, std::memory_order_release);
        return;
    }
    g_arch_overridden.store(false, std::memory_order_release);
    strncpy(g_arch_override, arch, sizeof(g_arch_override) - 1);
    g_arch_override[sizeof(g_arch_override) - 1] = '\0';
    g_arch_overridden.store(true, std::memory_order_release);
}

void lgn_testing_set_sgh_spin_limit(int polls) {
    lgn::g_sgh_spin_limit.store(polls < 0 ? lgn::kSghSpinLimit : polls,
                                std::memory_order_relaxed);
}

void lgn_testing_fail_launches(int hip_error, int count) {
    if (count <= 0 || hip_error == (int)hipSuccess) {
        lgn::g_fail_launches.store(0, std::memory_order_relaxed);
        return;
    }
    lgn::g_fail_error.store(hip_error, std::memory_order_relaxed);
    lgn::g_fail_launches.store(count, std::memory_order_relaxed);
}

}  // extern "C"
