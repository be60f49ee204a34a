/*
 * lgn.h -- C ABI of liblgn.so: fused Linear -> Swish -> +bias -> GroupNorm
 * on AMD Instinct MI355X (gfx950), its two-pass and wide-group forms, plus
 * Linear -> logsumexp -> LeakyReLU x2 -> GELU x2, Swish -> spatial GroupNorm
 * -> HardSwish and LayerNorm -> GELU -> dilated Conv1d -> + input (declared
 * further down).
 *
 * The operation (POPCORNBENCH transcript "Kimi-K2.6 l2_p37", problem
 * statement and the passages fixing the forward order):
 *
 *   z[m,n] = sum_k x[m,k] * W[n,k] + b_lin[n]        nn.Linear, W is [N,K]
 *   u[m,n] = z[m,n] * sigmoid(z[m,n]) + b_add[n]      Swish, then the bias
 *   for each row m and group g of C = N/G contiguous channels:
 *       mu  = mean of u[m, gC .. gC+C-1]
 *       var = population variance (divide by C) of the same values
 *   y[m,n] = (u[m,n] - mu) / sqrt(var + eps) * gamma[n] + beta[n]
 *
 * Layouts: x [M,K], W [N,K], out [M,N], all dense row-major with no stride
 * arguments; b_lin, b_add, gamma, beta are [N] fp32; out is always fp32.
 *
 * Ownership: every pointer is DEVICE memory owned by the caller, on the
 * device that is current when the call is made.  The library allocates and
 * frees nothing (lgn_forward_wide_f32_noalloc uses a fixed array the library
 * holds per device instead of a workspace; see there).  `out` must not overlap any input.  The two-pass workspace
 * may be the same buffer as `out` (it is then overwritten in place) but must
 * not overlap any input.
 *
 * Execution: every call enqueues its kernels on `stream` and returns without
 * waiting; results are visible after the caller synchronises the stream.
 * Calls keep no state between them except a per-device cache of the device
 * architecture (and the no-allocation entry point's array), so concurrent
 * calls on different streams are safe, except overlapping calls of
 * lgn_forward_wide_f32_noalloc on one device.  Output is bitwise reproducible
 * run to run: every reduction has a fixed order, and the only atomics publish
 * partial statistics (Swish -> spatial GroupNorm), never accumulate.
 *
 * Errors: calls return an lgn_status.  Argument errors are detected before any
 * HIP call and nothing is launched.  Faults inside a kernel surface at the
 * caller's synchronisation, as for any HIP kernel.
 */
#ifndef LGN_H
#define LGN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int lgn_status;
enum {
    LGN_OK = 0,
    LGN_ERR_INVALID_ARG = 1, /* null pointer, bad size, N % G != 0, eps not > 0 and finite,
                                workspace too small */
    LGN_ERR_UNSUPPORTED = 2, /* device is not gfx950, or a shape/alignment outside what the
                                kernels cover (see each entry point) */
    LGN_ERR_HIP = 3,         /* a HIP runtime call or kernel launch failed */
    LGN_ERR_TOO_LARGE = 4    /* the no-allocation entry point's scratch is too small for
                                the call */
};

/* Raw bfloat16 bits: the upper 16 bits of an IEEE binary32. */
typedef uint16_t lgn_bf16;

/* Shape rules common to the GroupNorm entry points:
 *   M >= 0 (M == 0 launches nothing and returns LGN_OK), K >= 0, N >= 1,
 *   G >= 1, N % G == 0, eps > 0 and finite.
 *   Pointers may be NULL only when the array they address is empty
 *   (x when M*K == 0, W when K == 0).
 *   128-bit paths: x, W and out must be 16-byte aligned, N % 4 == 0, and
 *   K % 4 == 0 (fp32 inputs) or K % 8 == 0 (bf16 inputs); otherwise
 *   LGN_ERR_UNSUPPORTED.  b_lin, b_add, gamma, beta need 4-byte alignment. */

/* Fused forward, fp32 x and W, fp32 MFMA with fp32 accumulate.
 * One kernel: MFMA GEMM tile, then bias, Swish, bias, group statistics,
 * normalisation and affine in registers, and one write of `out`.
 * Covers channel-per-group counts C = N/G that are powers of two from 8 to
 * 1024; other C return LGN_ERR_UNSUPPORTED (the two-pass entry point covers
 * every C).
 * Exception, for speed: with C = 512 or 1024 and K a positive multiple of 16,
 * the call runs two kernels in place on `out` instead (the GEMM writes
 * x W^T + b_lin into `out`, then one pass applies Swish, b_add, the group
 * statistics and the affine).  A single-kernel tile holding whole groups that
 * wide can be at most 64 samples tall -- a taller one's fp32 accumulators
 * would not fit a compute unit's registers -- so it reads W again for every
 * 64 rows, and the two kernels measured as fast or faster at every shape
 * tried.  The result is the same up to rounding; `out` is written twice. */
lgn_status lgn_forward_f32(const float *x, const float *W,
                           const float *b_lin, const float *b_add,
                           const float *gamma, const float *beta,
                           int M, int K, int N, int G, float eps,
                           float *out, hipStream_t stream);

/* Same as lgn_forward_f32 with x and W in bfloat16 (bf16 MFMA, fp32
 * accumulate); biases, gamma, beta and out stay fp32.  The two-kernel
 * exception applies here to C = 1024 with K >= 2048 and a multiple of 32
 * only: for bf16 the single kernel is faster at smaller K and at C = 512. */
lgn_status lgn_forward_bf16(const lgn_bf16 *x, const lgn_bf16 *W,
                            const float *b_lin, const float *b_add,
                            const float *gamma, const float *beta,
                            int M, int K, int N, int G, float eps,
                            float *out, hipStream_t stream);

/* Whether the fused entry point covers this shape (1) or not (0), for dtype
 * 0 = fp32 inputs, 1 = bf16 inputs.  Pure host logic; no HIP call. */
int lgn_fused_supported(int dtype, int M, int K, int N, int G);

/* Two-pass ablation (the transcript's adopted design: GEMM, then one fused
 * elementwise + GroupNorm kernel).  Kernel 1 writes z = x.W^T + b_lin as fp32
 * [M,N] into `workspace`; kernel 2 reads z, applies Swish, b_add, the group
 * statistics and the affine, and writes `out`.  `workspace` must hold
 * lgn_twopass_workspace_bytes(M, N) bytes, be 16-byte aligned, and may be the
 * same pointer as `out`.  Covers every C = N/G. */
size_t lgn_twopass_workspace_bytes(int M, int N);

lgn_status lgn_forward_twopass_f32(const float *x, const float *W,
                                   const float *b_lin, const float *b_add,
                                   const float *gamma, const float *beta,
                                   int M, int K, int N, int G, float eps,
                                   float *out, void *workspace, size_t workspace_bytes,
                                   hipStream_t stream);

lgn_status lgn_forward_twopass_bf16(const lgn_bf16 *x, const lgn_bf16 *W,
                                    const float *b_lin, const float *b_add,
                                    const float *gamma, const float *beta,
                                    int M, int K, int N, int G, float eps,
                                    float *out, void *workspace, size_t workspace_bytes,
                                    hipStream_t stream);

/* ---- Second method: Linear -> logsumexp -> LeakyReLU x2 -> GELU x2 ----
 * (POPCORNBENCH transcript "Kimi-K2.6 l2_p64", problem statement: logsumexp
 * over the output features of each row, LeakyReLU with negative slope 0.01
 * applied twice, then the exact GELU v * Phi(v), Phi the standard normal CDF,
 * applied twice.)  One fp32 scalar per row:
 *
 *   z[m,n]  = sum_k x[m,k] * W[n,k] + b[n]              nn.Linear, W is [N,K]
 *   l[m]    = log(sum_n exp(z[m,n]))
 *   out[m]  = gelu(gelu(leaky(leaky(l[m]))))
 *
 * Layouts: x [M,K], W [N,K] dense row-major; b [N] fp32; out [M] fp32.
 * Kernel 1 runs the MFMA GEMM on 256-channel tiles and writes, per row and
 * tile, the pair (max, sum of exp(z - max)) into `workspace`; kernel 2 merges
 * a row's pairs in tile order and applies the activations.  `workspace` must
 * hold lgn_lse_workspace_bytes(M, N) bytes (8 per row per 256-channel tile),
 * be 8-byte aligned and overlap nothing else; its contents on entry do not
 * matter.  Shape rules: M >= 0 (M == 0 is a no-op), K >= 0, N >= 1; x and W
 * 16-byte aligned, N % 4 == 0, K % 4 == 0 (fp32) or K % 8 == 0 (bf16), else
 * LGN_ERR_UNSUPPORTED.  Results are bitwise reproducible. */
size_t lgn_lse_workspace_bytes(int M, int N);

lgn_status lgn_linear_lse_f32(const float *x, const float *W, const float *b,
                              int M, int K, int N, float *out,
                              void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Same with x and W in bfloat16 (bf16 MFMA, fp32 accumulate). */
lgn_status lgn_linear_lse_bf16(const lgn_bf16 *x, const lgn_bf16 *W, const float *b,
                               int M, int K, int N, float *out,
                               void *workspace, size_t workspace_bytes, hipStream_t stream);

/* ---- Third method: Swish -> spatial GroupNorm -> HardSwish ----
 * (POPCORNBENCH transcript "Kimi-K2.6 l2_p60", the tail after its 3-D
 * transposed convolution: Swish, then GroupNorm whose statistics run over a
 * group's channels AND every spatial position of one sample, then
 * HardSwish v * clamp(v + 3, 0, 6) / 6.)
 *
 *   s[n,c,i]   = y[n,c,i] * sigmoid(y[n,c,i])         y is [Nb, C, S] fp32,
 *                                                     S = D*H*W flattened
 *   per sample n and group g of C/G contiguous channels, over those channels
 *   and all S positions: mean, population variance var
 *   out[n,c,i] = hardswish((s - mean) / sqrt(var + eps) * gamma[c] + beta[c])
 *
 * Layouts: y and out [Nb][C][S] dense (NCDHW); gamma, beta [C] fp32.  `out`
 * may be `y` itself (in place) but must not overlap it otherwise.  Out of
 * place, with groups of at most 256 chunks of 16384 elements, one kernel
 * reads y once: each workgroup holds its chunk, publishes the chunk's
 * statistics, waits (bounded) for the rest of its group and writes its chunk.
 * In place or with larger groups, two kernels: per-chunk statistics into
 * `workspace`, then the apply pass.  Both give bitwise the same output.
 * `workspace` must hold lgn_sgh_workspace_bytes(Nb, C, S, G) bytes (8 per
 * 16384-element chunk of every group), be 8-byte aligned and overlap nothing
 * else.  Rules: Nb >= 0 (0 is a no-op), C >= 1, S >= 1, G >= 1, C % G == 0,
 * eps > 0 and finite; a group of (C/G)*S elements must fit in 2^31 - 1 and
 * C/G must not exceed 8192, else LGN_ERR_UNSUPPORTED.  y and out need 16-byte
 * alignment, gamma and beta 4-byte.  Results are bitwise reproducible. */
size_t lgn_sgh_workspace_bytes(int Nb, int C, long long S, int G);

lgn_status lgn_swish_gn_hardswish_f32(const float *y, const float *gamma, const float *beta,
                                      int Nb, int C, long long S, int G, float eps,
                                      float *out, void *workspace, size_t workspace_bytes,
                                      hipStream_t stream);

/* ---- Fourth method: LayerNorm -> GELU -> dilated Conv1d -> + input ----
 * (POPCORNBENCH transcript "Kimi-K2.6 l2_p5", problem statement and its
 * derivation of the convolution's indices: a pre-norm dilated convolution
 * block on x [B, C, L].)
 *
 *   per sample b, over all C*L values of x[b]: mean, population variance var
 *   h[c][p] = (x[b][c][p] - mean) / sqrt(var + eps) * ln_w[c][p] + ln_b[c][p]
 *   g = GELU(h): exact v*Phi(v) (gelu_tanh = 0, nn.GELU's default) or the tanh
 *       form 0.5 v (1 + tanh(sqrt(2/pi) (v + 0.044715 v^3))) (gelu_tanh != 0)
 *   out[b][co][j] = conv_b[co] + x[b][co][j]
 *                 + sum_ci sum_{t=0..2} conv_w[co][ci][t] * g[ci][j - d + t*d]
 *   with g = 0 at positions outside [0, L) (Conv1d, kernel 3, dilation d,
 *   zero padding d on both sides, so the output has length L).
 *
 * Layouts: x and out [B][C][L], ln_w and ln_b [C][L], conv_w [C][C][3]
 * (out, in, tap), conv_b [C], all fp32 and dense.  `out` must not overlap any
 * input (the call rejects out == x).  Three kernels on `stream`: the weights
 * are packed into `workspace`, the per-sample statistics go there too, then
 * the convolution applies LayerNorm + GELU while staging its input tiles.
 * `workspace` must hold lgn_lnconv_workspace_bytes(B, C, L) bytes, be 16-byte
 * aligned and overlap nothing else.  Rules: B >= 0 (0 is a no-op), C >= 1,
 * L >= 1, dilation >= 1, eps > 0 and finite, else LGN_ERR_INVALID_ARG;
 * C % 128, L % 4, dilation > 16, C > 8192, C*L >= 2^29 (one sample and the
 * packed weights are addressed with 32-bit byte offsets) or x, ln_w, ln_b,
 * out not 16-byte aligned give LGN_ERR_UNSUPPORTED.  Results are bitwise
 * reproducible. */
size_t lgn_lnconv_workspace_bytes(int B, int C, int L);

lgn_status lgn_ln_gelu_conv1d_f32(const float *x, const float *ln_w, const float *ln_b,
                                  const float *conv_w, const float *conv_b,
                                  int B, int C, int L, int dilation, float eps, int gelu_tanh,
                                  float *out, void *workspace, size_t workspace_bytes,
                                  hipStream_t stream);

/* Groups wider than one workgroup tile: the same forward as lgn_forward_f32
 * (POPCORNBENCH transcript "Kimi-K2.6 l2_p37", problem statement and forward
 * order) for C = N/G a multiple of 256, up to LayerNorm over all N when G = 1.
 * The statistics then cross workgroups and take the two-stage form (per-block
 * partials, then a light second pass) that the "Kimi-K2.6 l2_p64" transcript
 * plans for its row reduction wider than one block: kernel 1 runs the fused GEMM
 * tile, bias, Swish and bias, writes u = Swish(z) + b_add to `out` and, per
 * row and 64 channels, the partial (mean, M2) into `workspace`; kernel 2
 * merges each (row, group)'s partials in a fixed order and normalises `out`
 * in place.  `workspace` must hold lgn_wide_workspace_bytes(M, N) bytes (8
 * per row per 64 channels), be 8-byte aligned and overlap nothing else.
 * Rules as for lgn_forward_f32, plus (N/G) % 256 == 0 and 16-byte aligned
 * gamma and beta, else LGN_ERR_UNSUPPORTED. */
size_t lgn_wide_workspace_bytes(int M, int N);

lgn_status lgn_forward_wide_f32(const float *x, const float *W,
                                const float *b_lin, const float *b_add,
                                const float *gamma, const float *beta,
                                int M, int K, int N, int G, float eps,
                                float *out, void *workspace, size_t workspace_bytes,
                                hipStream_t stream);

lgn_status lgn_forward_wide_bf16(const lgn_bf16 *x, const lgn_bf16 *W,
                                 const float *b_lin, const float *b_add,
                                 const float *gamma, const float *beta,
                                 int M, int K, int N, int G, float eps,
                                 float *out, void *workspace, size_t workspace_bytes,
                                 hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * forward as lgn_forward_wide_f32, with the (mean, M2) partials kept in a
 * scratch array that the library holds for the life of the process instead of
 * a caller workspace.  The call allocates nothing (no hipMalloc, no library
 * allocation); the caller still passes x, W, the vectors and out.
 *
 * Limit: the call needs lgn_wide_workspace_bytes(M, N) (8 bytes per row per
 * 64 channels) of scratch; above LGN_WIDE_NOALLOC_SCRATCH_BYTES (32 MiB, for
 * example M * N up to 2^31 elements) it returns LGN_ERR_TOO_LARGE before any
 * HIP call.  Every GPU the library runs on holds its own copy of the scratch
 * (32 MiB of device memory each), and every call on one GPU shares it: calls
 * that overlap in time on one GPU (different streams, or threads) race on it
 * and give wrong results; serialise them.  The scratch needs no clearing:
 * each call writes every partial before reading it.  Other rules, errors and
 * results (bitwise equal to lgn_forward_wide_f32 on the same inputs) as for
 * lgn_forward_wide_f32. */
#define LGN_WIDE_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

lgn_status lgn_forward_wide_f32_noalloc(const float *x, const float *W,
                                        const float *b_lin, const float *b_add,
                                        const float *gamma, const float *beta,
                                        int M, int K, int N, int G, float eps,
                                        float *out, hipStream_t stream);

/* Static, NUL-terminated description of a status code. */
const char *lgn_status_string(lgn_status s);

/* Library version as "major.minor.patch". */
const char *lgn_version(void);

/* Text of the HIP error behind the last LGN_ERR_HIP returned on the calling
 * thread ("no HIP error" if none).  Static storage; do not free. */
const char *lgn_last_hip_error_string(void);

/* ---- Failure-path hooks, for tests of the error paths above ----
 * They let a test reach LGN_ERR_UNSUPPORTED (wrong device) and LGN_ERR_HIP
 * (failed launch) without another GPU and without a faulty kernel.  Both are
 * process-wide and not synchronised with calls running on other threads:
 * set them while no entry point is in flight.
 *
 * lgn_testing_set_arch: while `arch` is non-NULL, every entry point's device
 * check compares this architecture name (for example "gfx942") instead of
 * querying the current device, and makes no HIP call for it; a name that does
 * not start with "gfx950" then yields LGN_ERR_UNSUPPORTED.  The string is
 * copied (at most 63 characters).  NULL restores the device query.
 *
 * lgn_testing_fail_launches: the next `count` kernel launches made by the
 * library return `hip_error` (a hipError_t value other than hipSuccess)
 * instead of launching, so the entry point returns LGN_ERR_HIP and
 * lgn_last_hip_error_string() names that error.  count <= 0 clears it.
 *
 * lgn_testing_set_sgh_spin_limit: the number of polls the single-pass
 * spatial GroupNorm kernel makes for the rest of its group before it forms
 * the group's statistics itself (bitwise the same result, by another route);
 * 0 takes that route at once, a negative value restores the default. */
void lgn_testing_set_arch(const char *arch);
void lgn_testing_fail_launches(int hip_error, int count);
void lgn_testing_set_sgh_spin_limit(int polls);

#ifdef __cplusplus
}
#endif

#endif /* LGN_H */
