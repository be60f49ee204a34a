// l2_feed.hip -- measures how fast global -> LDS DMA (global_load_lds_dwordx4)
// can feed one CU when each load instruction's 64 lanes cover 16 rows x 64
// bytes (LDS rows of 64 bytes) or 8 rows x 128 bytes (rows of 128 bytes).
//
// The GEMM cores stage a 512-row operand panel per workgroup (256 W rows and
// 256 x rows, K-contiguous, 2048 bytes per row for K = 1024 in bf16) one
// K-slice at a time.  With 64-byte rows a slice uses half of every 128-byte
// line and the other half is fetched one slice later; with 128-byte rows
// every line is used whole by one instruction.  This probe streams the same
// panel shape with either row width (for 64-byte rows also with the two
// slices of each line issued back to back) and a fixed number of bytes in
// flight per workgroup, without barriers and without MFMAs, and reports the
// delivered operand bytes per shader clock per CU.  Two data placements:
// "resident" (every workgroup reads the same 1 MiB panel, so all but the
// first reads hit L2) and "spread" (workgroup b reads panel b % 64 of a
// 64 MiB buffer, like the x tiles of the fused kernel).
//
// Output: one JSON object per line.
// Not part of liblgn.so; built next to it by gemm_activation_groupnorm_amd.build.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <vector>

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void gbl_void_t;

constexpr int kThreads = 512;                // 8 waves
constexpr int kRows = 512;                   // panel rows
constexpr int kRowBytes = 2048;              // K = 1024 bf16
constexpr size_t kPanel = (size_t)kRows * kRowBytes;
constexpr int kPanels = 64;

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
    asm volatile("" ::: "memory");
}

// ROWB: bytes of each row per K-slice (64 or 128).  WIN: slices in flight
// per wave.  LDS holds two slots of one slice each; slices in flight beyond
// two land in slots whose contents nobody reads (a bandwidth probe).
// PAIR (64-byte rows): slices 2j and 2j+1, which share every 128-byte line,
// are issued together, block by block, so both halves of a line are
// requested back to back.
template <int ROWB, int WIN, bool PAIR = false>
__global__ __launch_bounds__(kThreads) void feed(const unsigned char *src, int spread, int passes,
                                                 unsigned long long *clk) {
    constexpr int SLICE = kRows * ROWB;          // bytes per K-slice
    constexpr int NB = SLICE / 1024;             // 1 KiB blocks per slice
    constexpr int BPW = NB / (kThreads / 64);    // blocks per wave per slice
    constexpr int SLICES = kRowBytes / ROWB;
    static_assert((WIN - 1) * BPW < 64, "vmcnt range");
    __shared__ __attribute__((aligned(1024))) unsigned char lds[2 * SLICE];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const unsigned long long t0 = __builtin_amdgcn_s_memtime();
    const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
    const unsigned char *panel = src + (spread ? (size_t)(blockIdx.x % kPanels) * kPanel : 0);
    const unsigned char *lsrc[BPW];
#pragma unroll
    for (int j = 0; j < BPW; ++j) {
        const int o = (wave * BPW + j) * 1024 + 16 * lane;
        lsrc[j] = panel + (size_t)(o / ROWB) * kRowBytes + (o % ROWB);
    }
    for (int p = 0; p < passes; ++p) {
        if constexpr (PAIR) {
            static_assert(WIN >= 2 && SLICES % 2 == 0, "pairs of slices");
            for (int s = 0; s < SLICES; s += 2) {
#pragma unroll
                for (int j = 0; j < BPW; ++j) {
                    __builtin_amdgcn_global_load_lds((gbl_void_t *)(lsrc[j] + s * ROWB),
                                                     (lds_void_t *)(lds + (wave * BPW + j) * 1024),
                                                     16, 0, 0);
                    __builtin_amdgcn_global_load_lds(
                        (gbl_void_t *)(lsrc[j] + (s + 1) * ROWB),
                        (lds_void_t *)(lds + SLICE + (wave * BPW + j) * 1024), 16, 0, 0);
                }
                wait_vmcnt<(WIN - 2) * BPW>();
            }
            continue;
        }
        for (int s = 0; s < SLICES; ++s) {
            unsigned char *slot = lds + (s & 1) * SLICE;
#pragma unroll
            for (int j = 0; j < BPW; ++j)
                __builtin_amdgcn_global_load_lds((gbl_void_t *)(lsrc[j] + s * ROWB),
                                                 (lds_void_t *)(slot + (wave * BPW + j) * 1024),
                                                 16, 0, 0);
            wait_vmcnt<(WIN - 1) * BPW>();
        }
    }
    wait_vmcnt<0>();
    __syncthreads();
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

template <int ROWB, int WIN, bool PAIR = false>
static int run(const unsigned char *src, unsigned long long *clk, int spread) {
    const int wgs = 256;        // one workgroup per CU (LDS-limited)
    const int passes = 64;
    hipEvent_t e0, e1;
    CHECK(hipEventCreate(&e0));
    CHECK(hipEventCreate(&e1));
    auto launch = [&] {
        hipLaunchKernelGGL((feed<ROWB, WIN, PAIR>), dim3(wgs), dim3(kThreads), 0, 0, src, spread,
                           passes, clk);
    };
    for (int w = 0; w < 5; ++w) launch();
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
    const double bytes_per_wg = (double)passes * kPanel;
    const double ghz = sc / (sr / 100e6) / 1e9;
    printf("{\"row_bytes\": %d, \"paired\": %s, \"in_flight_kib\": %d, \"placement\": \"%s\", \"ms\": %.4f, "
           "\"tb_per_s\": %.2f, \"bytes_per_clk_per_cu\": %.1f, \"shader_clock_ghz\": %.3f}\n",
           ROWB, PAIR ? "true" : "false", WIN * kRows * ROWB / 1024, spread ? "spread" : "resident", best,
           bytes_per_wg * wgs / best / 1e9, bytes_per_wg / (sc / wgs), ghz);
    fflush(stdout);
    CHECK(hipEventDestroy(e0));
    CHECK(hipEventDestroy(e1));
    return 0;
}

int main() {
    unsigned char *src;
    unsigned long long *clk;
    CHECK(hipMalloc(&src, kPanel * kPanels));
    CHECK(hipMemset(src, 0x3c, kPanel * kPanels));
    CHECK(hipMalloc(&clk, 256 * 2 * sizeof(unsigned long long)));
    for (int spread = 0; spread < 2; ++spread) {
        if (run<64, 2>(src, clk, spread) || run<64, 3>(src, clk, spread) ||
            run<64, 4>(src, clk, spread) || run<64, 2, true>(src, clk, spread) ||
            run<64, 4, true>(src, clk, spread) || run<128, 1>(src, clk, spread) ||
            run<128, 2>(src, clk, spread))
            return 1;
    }
    CHECK(hipFree(src));
    CHECK(hipFree(clk));
    return 0;
}
