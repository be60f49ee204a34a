// lds_bandwidth.hip -- measures the LDS read bandwidth of one compute unit
// (bytes per shader clock per CU) with 16-byte reads (ds_read_b128), the
// instruction the GEMM cores read their MFMA fragments with.
//
// Each workgroup of 512 threads fills 64 KiB of LDS, then every wave issues
// groups of 8 independent ds_read_b128 whose addresses move on every
// iteration (so no read can be hoisted), 16 consecutive lanes covering 256
// contiguous bytes (all banks, no conflict).  The values are folded into a
// few registers with XOR so the reads stay live.  Two workgroups per CU
// (16 waves) keep the LDS busy.  Bytes per clock per CU = bytes read / (CUs
// x seconds x shader clock); the clock is the ratio of s_memtime to the
// 100 MHz s_memrealtime over each workgroup's run.
//
// Output: one JSON object (ms, bytes, GB/s, shader clock, bytes per clock per CU).
// Not part of liblgn.so; built next to it by gemm_activation_groupnorm_amd.build.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <vector>

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 512;
constexpr int kEntries = 4096;   // u32x4 entries: 64 KiB of LDS per workgroup

__global__ __launch_bounds__(kThreads) void lds_read_loop(int iters, u32x4 *out,
                                                          unsigned long long *clk) {
    __shared__ u32x4 buf[kEntries];
    const int tid = threadIdx.x;
    for (int e = tid; e < kEntries; e += kThreads)
        buf[e] = u32x4{(unsigned)e, (unsigned)(e * 3), (unsigned)(e ^ 0x55), (unsigned)(e + 7)};
    __syncthreads();
    const unsigned long long t0 = __builtin_amdgcn_s_memtime();
    const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
    const int lane = tid & 63, wave = tid >> 6;
    u32x4 acc[4] = {};
    int base = wave * 512 + lane;
    for (int it = 0; it < iters; ++it) {
        u32x4 v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = buf[(base + 64 * j) & (kEntries - 1)];
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j & 3] ^= v[j];
        base += 512 + 64;
    }
    out[(size_t)blockIdx.x * kThreads + tid] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
    const unsigned long long t1 = __builtin_amdgcn_s_memtime();
    const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
    if (tid == 0) {
        clk[2 * blockIdx.x] = t1 - t0;
        clk[2 * blockIdx.x + 1] = r1 - r0;
    }
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
    int dev = 0, cus = 0;
    CHECK(hipGetDevice(&dev));
    CHECK(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev));
    const int wgs = cus * 2 * 8;   // two resident per CU, eight rounds
    const int iters = 4000;
    u32x4 *out;
    unsigned long long *clk;
    CHECK(hipMalloc(&out, (size_t)wgs * kThreads * sizeof(u32x4)));
    CHECK(hipMalloc(&clk, (size_t)wgs * 2 * sizeof(unsigned long long)));
    hipEvent_t e0, e1;
    CHECK(hipEventCreate(&e0));
    CHECK(hipEventCreate(&e1));
    for (int w = 0; w < 5; ++w)
        hipLaunchKernelGGL(lds_read_loop, dim3(wgs), dim3(kThreads), 0, 0, iters, out, clk);
    CHECK(hipGetLastError());
    CHECK(hipDeviceSynchronize());
    float best = 1e30f;
    for (int rep = 0; rep < 5; ++rep) {
        CHECK(hipEventRecord(e0));
        hipLaunchKernelGGL(lds_read_loop, dim3(wgs), dim3(kThreads), 0, 0, iters, out, clk);
        CHECK(hipEventRecord(e1));
        CHECK(hipEventSynchronize(e1));
        float ms;
        CHECK(hipEventElapsedTime(&ms, e0, e1));
        if (ms < best) best = ms;
    }
    std::vector<unsigned long long> hc((size_t)wgs * 2);
    CHECK(hipMemcpy(hc.data(), clk, hc.size() * sizeof(unsigned long long), hipMemcpyDeviceToHost));
    double sc = 0, sr = 0;
    for (int i = 0; i < wgs; ++i) {
        sc += (double)hc[2 * i];
        sr += (double)hc[2 * i + 1];
    }
    const double ghz = sc / (sr / 100e6) / 1e9;
    const double bytes = (double)wgs * kThreads * iters * 8 * 16;
    const double gbps = bytes / (best * 1e-3) / 1e9;
    printf("{\"probe\": \"lds_read_b128\", \"cus\": %d, \"ms\": %.4f, \"bytes\": %.4g, "
           "\"gb_per_s\": %.1f, \"shader_clock_ghz\": %.3f, \"bytes_per_clk_per_cu\": %.1f}\n",
           cus, best, bytes, gbps, ghz, gbps * 1e9 / (cus * ghz * 1e9));
    fflush(stdout);
    CHECK(hipFree(out));
    CHECK(hipFree(clk));
    return 0;
}
