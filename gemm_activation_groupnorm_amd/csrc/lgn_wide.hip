// lgn_wide.hip -- launcher of the wide-group forward (groups wider than one
// workgroup tile) and its fp32 and bf16 entry points.

#include "lgn_launch.hpp"
#include "lgn_wide.hpp"

#include <atomic>
#include <mutex>
#include <type_traits>

namespace lgn {

// Scratch of the no-allocation entry point (lgn_forward_wide_f32_noalloc):
// the per-(row, 64-channel span) (mean, M2) partials that the other wide
// entry points keep in the caller's workspace.  Every GPU the library runs on
// holds its own copy for the life of the process; every call on one GPU
// shares it.  Host code never passes `scratch` itself to a kernel (on the
// host it only names the symbol): it passes the device address that
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[kWideScratchBytes];

namespace {
constexpr int kScratchDevices = 64;
std::atomic<void *> g_scratch_addr[kScratchDevices];
std::mutex g_scratch_mu;
}  // namespace

hipError_t wide_scratch_address(void **addr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
    void *p = g_scratch_addr[dev].load(std::memory_order_acquire);
    if (!p) {
        // first call on this device, with the device current: look the
        // symbol up once and keep its address
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_addr[dev].load(std::memory_order_relaxed);
        if (!p) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            if (!p) return hipErrorInvalidSymbol;
            g_scratch_addr[dev].store(p, std::memory_order_release);
        }
    }
    *addr = p;
    return hipSuccess;
}

// Kernel 1 is the fused kernel's 256 x 256 tile (same core and schedules as
// its C <= 64 case) in WIDE mode; K not a multiple of the stage depth takes
// the register-staged core on a 128 x 256 tile (also 64-channel wave spans).
template <class DT>
hipError_t launch_wide(const typename dt_traits<DT>::storage *x,
                       const typename dt_traits<DT>::storage *W, const float *b_lin,
                       const float *b_add, const float *gamma, const float *beta, int M, int K,
                       int N, int G, float eps, float *out, void *workspace,
                       hipStream_t stream) {
    typedef typename std::conditional<std::is_same<DT, bf16_t>::value,
                                      TileCfg<DT, 256, 256, 2, 4, 64, 2, 2, 2>,
                                      TileCfg<DT, 256, 256, 2, 4, 64, 2>>::type Fast;
    constexpr int RING = std::is_same<DT, bf16_t>::value ? 4 : 3;
    typedef TileCfg<DT, 128, 256, 2, 4, 64, 2> Slow;
    float2 *part = reinterpret_cast<float2 *>(workspace);
    const int tiles_n = N / 256;
    hipError_t e;
    if (K % Fast::BK == 0) {
        const int tiles_m = (M + Fast::BS - 1) / Fast::BS;
        e = launch_kernel(lgn_fused_kernel<DT, Fast, kWideSpan, RING, true>,
                          dim3((unsigned)((long long)tiles_m * tiles_n)), dim3(Fast::NT), stream,
                          x, W, b_lin, b_add, gamma, beta, M, K, N, eps, out, tiles_m, tiles_n,
                          part);
    } else {
        const int tiles_m = (M + Slow::BS - 1) / Slow::BS;
        e = launch_kernel(lgn_fused_kernel<DT, Slow, kWideSpan, 0, true>,
                          dim3((unsigned)((long long)tiles_m * tiles_n)), dim3(Slow::NT), stream,
                          x, W, b_lin, b_add, gamma, beta, M, K, N, eps, out, tiles_m, tiles_n,
                          part);
    }
    if (e != hipSuccess) return e;
    // one wave per (pair of rows, group)
    const long long waves = ((long long)M + kWideNormRows - 1) / kWideNormRows * G;
    if (waves > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    return launch_kernel(lgn_wide_norm_kernel<kWideSpan>, dim3((unsigned)waves), dim3(64), stream,
                         (const float2 *)part, gamma, beta, (long long)M, G, (N / G) / kWideSpan,
                         N / kWideSpan, eps, out);
}

hipError_t launch_wide_f32(const float *x, const float *W, const float *b_lin, const float *b_add,
                           const float *gamma, const float *beta, int M, int K, int N, int G,
                           float eps, float *out, void *workspace, hipStream_t stream) {
    return launch_wide<f32_t>(x, W, b_lin, b_add, gamma, beta, M, K, N, G, eps, out, workspace,
                              stream);
}

hipError_t launch_wide_bf16(const uint16_t *x, const uint16_t *W, const float *b_lin,
                            const float *b_add, const float *gamma, const float *beta, int M,
                            int K, int N, int G, float eps, float *out, void *workspace,
                            hipStream_t stream) {
    return launch_wide<bf16_t>(x, W, b_lin, b_add, gamma, beta, M, K, N, G, eps, out, workspace,
                               stream);
}

}  // namespace lgn
