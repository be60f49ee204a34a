// mfma_ceiling.hip -- measures the sustained dense MFMA rate of this GPU and
// the shader clock it runs at, for zero and for random operands.
//
// The MI355X is power-limited under a full MFMA load: how much power an MFMA
// draws depends on how its operand bits toggle, and the clock follows.  A
// roofline peak quoted from the data sheet assumes the top clock; this probe
// shows the clock and the MFMA rate that operands like a real workload's
// actually get.  Each lane keeps 8 A and 8 B operand registers (read once
// from a buffer of bf16 or fp32 values) and feeds a different pair to every
// MFMA, on 8 independent accumulators per wave, 2 waves per SIMD.  The clock
// is the ratio of the shader-clock counter (s_memtime) to the 100 MHz
// real-time counter (s_memrealtime) over each workgroup's run.
//
// Output: one JSON object per line (dtype, operands, ms, TFLOP/s, GHz).
// Not part of liblgn.so; built next to it by gemm_activation_groupnorm_amd.build.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>
#include <vector>

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaveLanes = 64;
constexpr int kThreads = 256;
constexpr int kSrcBlocks = 64;                            // distinct operand sets
constexpr size_t kVecs = (size_t)kSrcBlocks * kThreads * 16;   // u32x4 per buffer

template <bool BF16>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void mfma_loop(const u32x4 *src, float *out, int iters, unsigned long long *clk) {
    const int tid = threadIdx.x;
    const unsigned long long t0 = __builtin_amdgcn_s_memtime();
    const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
    const size_t base = ((size_t)(blockIdx.x % kSrcBlocks) * kThreads + tid) * 16;
    u32x4 a[8], b[8];
    for (int i = 0; i < 8; ++i) {
        a[i] = src[base + i];
        b[i] = src[base + 8 + i];
    }
    f32x16 acc[8];
    for (int i = 0; i < 8; ++i)
        for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const u32x4 av = a[(i + j) & 7], bv = b[(3 * i + j) & 7];
                if constexpr (BF16) {
                    acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        __builtin_bit_cast(bf16x8, av), __builtin_bit_cast(bf16x8, bv), acc[i], 0,
                        0, 0);
                } else {
                    acc[i] = __builtin_amdgcn_mfma_f32_32x32x2f32(__builtin_bit_cast(float, av[0]),
                                                                  __builtin_bit_cast(float, bv[0]),
                                                                  acc[i], 0, 0, 0);
                }
            }
    }
    float s = 0.f;
    for (int i = 0; i < 8; ++i)
        for (int r = 0; r < 16; ++r) s += acc[i][r];
    out[(size_t)blockIdx.x * kThreads + tid] = s;
    const unsigned long long t1 = __builtin_amdgcn_s_memtime();
    const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
    if (tid == 0) {
        clk[2 * blockIdx.x] = t1 - t0;
        clk[2 * blockIdx.x + 1] = r1 - r0;
    }
}

static uint16_t to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    u += 0x7fff + ((u >> 16) & 1);
    return (uint16_t)(u >> 16);
}

#define CHECK(x)                                                                         \
    do {                                                                                 \
        hipError_t e_ = (x);                                                             \
        if (e_ != hipSuccess) {                                                          \
            fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
            return 1;                                                                    \
        }                                                                                \
    } while (0)

int main() {
    const int wgs = 2048;
    u32x4 *src;
    float *out;
    unsigned long long *clk;
    CHECK(hipMalloc(&src, kVecs * sizeof(u32x4)));
    CHECK(hipMalloc(&out, (size_t)wgs * kThreads * sizeof(float)));
    CHECK(hipMalloc(&clk, (size_t)wgs * 2 * sizeof(unsigned long long)));
    std::mt19937 gen(1);
    std::normal_distribution<float> nd(0.f, 1.f);
    hipEvent_t e0, e1;
    CHECK(hipEventCreate(&e0));
    CHECK(hipEventCreate(&e1));
    for (int bf16 = 1; bf16 >= 0; --bf16) {
        for (int random = 0; random < 2; ++random) {
            std::vector<uint32_t> h(kVecs * 4);
            for (size_t i = 0; i < h.size(); ++i) {
                if (bf16) {
                    const uint32_t lo = random ? to_bf16(nd(gen)) : 0u;
                    const uint32_t hi = random ? to_bf16(nd(gen)) : 0u;
                    h[i] = lo | (hi << 16);
                } else {
                    const float f = random ? nd(gen) : 0.f;
                    memcpy(&h[i], &f, 4);
                }
            }
            CHECK(hipMemcpy(src, h.data(), kVecs * sizeof(u32x4), hipMemcpyHostToDevice));
            const int iters = bf16 ? 200 : 40;
            auto launch = [&] {
                if (bf16)
                    hipLaunchKernelGGL(mfma_loop<true>, dim3(wgs), dim3(kThreads), 0, 0, src, out,
                                       iters, clk);
                else
                    hipLaunchKernelGGL(mfma_loop<false>, dim3(wgs), dim3(kThreads), 0, 0, src, out,
                                       iters, clk);
            };
            for (int w = 0; w < 10; ++w) launch();   // let the clocks settle under load
            CHECK(hipGetLastError());
            CHECK(hipDeviceSynchronize());
            float best = 1e30f;
            for (int rep = 0; rep < 5; ++rep) {
                CHECK(hipEventRecord(e0));
                launch();
                CHECK(hipEventRecord(e1));
                CHECK(hipEventSynchronize(e1));
                float ms;
                CHECK(hipEventElapsedTime(&ms, e0, e1));
                if (ms < best) best = ms;
            }
            std::vector<unsigned long long> hc((size_t)wgs * 2);
            CHECK(hipMemcpy(hc.data(), clk, hc.size() * sizeof(unsigned long long),
                            hipMemcpyDeviceToHost));
            double sc = 0, sr = 0;
            for (int i = 0; i < wgs; ++i) {
                sc += (double)hc[2 * i];
                sr += (double)hc[2 * i + 1];
            }
            const double ghz = sc / (sr / 100e6) / 1e9;
            const double flop_per_mfma = bf16 ? 32.0 * 32 * 16 * 2 : 32.0 * 32 * 2 * 2;
            const double flops = (double)wgs * (kThreads / kWaveLanes) * iters * 64 * flop_per_mfma;
            printf("{\"dtype\": \"%s\", \"operands\": \"%s\", \"ms\": %.4f, \"tflops\": %.1f, "
                   "\"shader_clock_ghz\": %.3f}\n",
                   bf16 ? "bf16" : "f32", random ? "random N(0,1)" : "zeros", best,
                   flops / best / 1e9, ghz);
            fflush(stdout);
        }
    }
    CHECK(hipFree(src));
    CHECK(hipFree(out));
    CHECK(hipFree(clk));
    return 0;
}
