// lgn_device.hpp -- device building blocks for gfx950 (CDNA4, wave64).
//
// The GEMM core computes the transposed tile  Z^T = W . x^T  with
// v_mfma_f32_32x32x2_f32 (fp32 inputs) or v_mfma_f32_32x32x16_bf16 (bf16
// inputs): the MFMA "A" operand is a 32-row slab of W (32 channels) and the
// "B" operand a 32-row slab of x (32 samples).  In the 32x32 accumulator a
// lane then holds ONE sample (lane % 32) and 16 channels,
//     channel(r, h) = 8*(r/4) + 4*h + (r%4),   r = 0..15, h = lane / 32,
// so a GroupNorm group of contiguous channels sits mostly inside one lane's
// registers: the statistics need in-register sums, one exchange with lane^32
// and, only for groups wider than a wave's channel span, one LDS merge.
// Registers r = 4q..4q+3 are 4 contiguous channels -> one 16-byte store.
//
// Both operands are K-contiguous in memory (x is [M,K], W is [N,K], the
// nn.Linear layout) and are staged through LDS in rows of ROWB bytes with a
// 16-byte-chunk XOR swizzle, so that the 16 lanes of one LDS phase (16 rows,
// same logical chunk) hit 16 distinct 16-byte bank groups of gfx950's
// 64 x 4-byte banks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lgn {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

struct f32_t {};   // tag: fp32 operands
struct bf16_t {};  // tag: bf16 operands (raw uint16 storage)

template <class DT> struct dt_traits;
template <> struct dt_traits<f32_t> {
    typedef float storage;
    static constexpr int bytes = 4;
};
template <> struct dt_traits<bf16_t> {
    typedef uint16_t storage;
    static constexpr int bytes = 2;
};

// ---------------------------------------------------------------- tiles ----
// BS samples x BC channels per workgroup; WAVES_S x WAVES_C waves; each wave
// owns WS x WC = (32*TS) x (32*TC) of the tile.  ROWB bytes of K per LDS row.
// OCC = waves per SIMD the kernel must fit (register budget 512/OCC per
// lane, accumulators included).  PIPE selects the LDS DMA core's schedule:
//   0: each chunk pair's fragments are read right before its MFMAs;
//   1: the next chunk pair's fragments are read under the current MFMAs, one
//      barrier at the end of each stage;
//   2: as 1, with the barrier before the stage's last chunk pair, so that the
//      next stage's first reads hide under that whole chunk pair (needs a
//      ring of at least 3 stages and an even number of chunk pairs).
// EARLY (PIPE >= 1) = sample tiles whose MFMAs are issued before those reads
// (0: reads first).  GM = sample tiles per band of the tile order (tile_coords).
template <class DT, int BS_, int BC_, int WAVES_S_, int WAVES_C_, int ROWB_, int OCC_ = 1,
          int PIPE_ = 1, int EARLY_ = 1, int GM_ = 8>
struct TileCfg {
    static constexpr int GM = GM_;
    static constexpr int BS = BS_, BC = BC_, WAVES_S = WAVES_S_, WAVES_C = WAVES_C_;
    static constexpr int ROWB = ROWB_;
    static constexpr int OCC = OCC_;
    static constexpr bool PIPE = PIPE_ != 0;
    static constexpr int SCHED = PIPE_;
    static constexpr int EARLY = EARLY_;
    static constexpr int NT = 64 * WAVES_S * WAVES_C;
    static constexpr int WS = BS / WAVES_S, WC = BC / WAVES_C;
    static constexpr int TS = WS / 32, TC = WC / 32;
    static constexpr int EB = dt_traits<DT>::bytes;
    static constexpr int EPC = 16 / EB;               // elements per 16-byte chunk
    static constexpr int CPR = ROWB / 16;             // chunks per LDS row
    static constexpr int BK = CPR * EPC;              // K elements per stage
    static constexpr int ROWS = BS + BC;              // W rows first, then x rows
    static constexpr int CHUNKS = ROWS * CPR;
    static constexpr int CPT = (CHUNKS + NT - 1) / NT;
    static constexpr int STAGE_BYTES = ROWS * ROWB;
    static constexpr int RPW = 256 / ROWB;            // rows per 256-byte bank window
    static_assert(WS % 32 == 0 && WC % 32 == 0, "wave tile must be whole 32x32 MFMA tiles");
    static_assert(ROWB == 32 || ROWB == 64 || ROWB == 128, "LDS row of 32, 64 or 128 bytes");
    static_assert(NT % CPR == 0, "every thread keeps one chunk column");
    static_assert((BC * CPR) % NT == 0 || CHUNKS % NT == 0 || true, "");
};

// Physical 16-byte chunk of logical chunk c in LDS row r.
template <class Cfg>
__device__ __forceinline__ int swz(int r, int c) {
    return c ^ ((r / Cfg::RPW) % Cfg::CPR);
}

// --------------------------------------------------------------- MFMA ----
template <class DT> struct Mfma;

template <> struct Mfma<f32_t> {
    // One 16-byte fragment per operand = 4 K-steps of v_mfma_f32_32x32x2_f32.
    // Lane half h feeds K slot h of each step with the k = 4h + kk element of
    // the 8-wide K chunk; A and B use the same assignment, so the pair of
    // steps kk covers the chunk exactly once.
    static __device__ __forceinline__ void run(f32x16 &acc, u32x4 a, u32x4 b) {
        f32x4 af = __builtin_bit_cast(f32x4, a);
        f32x4 bf = __builtin_bit_cast(f32x4, b);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(af[0], bf[0], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(af[1], bf[1], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(af[2], bf[2], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(af[3], bf[3], acc, 0, 0, 0);
    }
};

template <> struct Mfma<bf16_t> {
    // One 16-byte fragment = 8 bf16 = the lane's K slice of one
    // v_mfma_f32_32x32x16_bf16.
    static __device__ __forceinline__ void run(f32x16 &acc, u32x4 a, u32x4 b) {
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                      __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
    }
};

// ----------------------------------------------------------- GEMM core ----
// Adds to acc[ts][tc] (32 samples x 32 channels each; the caller sets the
// initial value) the products of the workgroup tile at (m0, n0) over K.  Global -> register prefetch of the
// next stage overlaps the MFMAs of the current one; two LDS stages, one
// barrier per stage.  Rows past M or N and K past the end load as zeros.
template <class DT, class Cfg>
struct GemmCore {
    typedef typename dt_traits<DT>::storage T;

    static __device__ __forceinline__ void load_global(const T *__restrict__ x,
                                                       const T *__restrict__ W, int M, int N,
                                                       int K, int m0, int n0, int k0, int tid,
                                                       u32x4 (&pref)[Cfg::CPT]) {
#pragma unroll
        for (int i = 0; i < Cfg::CPT; ++i) {
            const int idx = tid + i * Cfg::NT;
            u32x4 v = {0u, 0u, 0u, 0u};
            if (Cfg::CHUNKS % Cfg::NT == 0 || idx < Cfg::CHUNKS) {
                const int r = idx / Cfg::CPR;
                const int c = idx % Cfg::CPR;
                const int k = k0 + c * Cfg::EPC;
                if (r < Cfg::BC) {
                    const int n = n0 + r;
                    if (n < N && k < K)
                        v = *reinterpret_cast<const u32x4 *>(W + (size_t)n * (size_t)K + k);
                } else {
                    const int m = m0 + (r - Cfg::BC);
                    if (m < M && k < K)
                        v = *reinterpret_cast<const u32x4 *>(x + (size_t)m * (size_t)K + k);
                }
            }
            pref[i] = v;
        }
    }

    static __device__ __forceinline__ void store_lds(unsigned char *stage, int tid,
                                                     const u32x4 (&pref)[Cfg::CPT]) {
#pragma unroll
        for (int i = 0; i < Cfg::CPT; ++i) {
            const int idx = tid + i * Cfg::NT;
            if (Cfg::CHUNKS % Cfg::NT == 0 || idx < Cfg::CHUNKS) {
                const int r = idx / Cfg::CPR;
                const int c = idx % Cfg::CPR;
                *reinterpret_cast<u32x4 *>(stage + r * Cfg::ROWB + 16 * swz<Cfg>(r, c)) = pref[i];
            }
        }
    }

    // Fragments of chunk pair cp: lane half h reads logical chunk 2*cp + h of
    // its W row (a) and x row (b).  wc0 / ws0: first channel / sample of this
    // wave inside the tile.
    static __device__ __forceinline__ void load_frags(const unsigned char *stage, int cp, int wc0,
                                                      int ws0, int lr, int h, u32x4 (&a)[Cfg::TC],
                                                      u32x4 (&b)[Cfg::TS]) {
        const int c = 2 * cp + h;
#pragma unroll
        for (int tc = 0; tc < Cfg::TC; ++tc) {
            const int r = wc0 + 32 * tc + lr;
            a[tc] = *reinterpret_cast<const u32x4 *>(stage + r * Cfg::ROWB + 16 * swz<Cfg>(r, c));
        }
#pragma unroll
        for (int ts = 0; ts < Cfg::TS; ++ts) {
            const int r = Cfg::BC + ws0 + 32 * ts + lr;
            b[ts] = *reinterpret_cast<const u32x4 *>(stage + r * Cfg::ROWB + 16 * swz<Cfg>(r, c));
        }
    }

    // MFMAs of sample tiles [T0, T1) against all channel tiles.
    template <int T0 = 0, int T1 = Cfg::TS>
    static __device__ __forceinline__ void mfma_block(const u32x4 (&a)[Cfg::TC],
                                                      const u32x4 (&b)[Cfg::TS],
                                                      f32x16 (&acc)[Cfg::TS][Cfg::TC]) {
#pragma unroll
        for (int ts = T0; ts < T1; ++ts)
#pragma unroll
            for (int tc = 0; tc < Cfg::TC; ++tc) Mfma<DT>::run(acc[ts][tc], a[tc], b[ts]);
    }

    // All MFMAs of one LDS stage.  Fragments are double-buffered in registers:
    // the reads of chunk pair cp+1 are issued before the MFMAs of cp, and a
    // scheduling barrier keeps the compiler from sinking them back next to
    // their use, so LDS latency hides under MFMA work.
    static __device__ __forceinline__ void compute_stage(const unsigned char *stage, int wc0,
                                                         int ws0, int lr, int h,
                                                         f32x16 (&acc)[Cfg::TS][Cfg::TC]) {
        constexpr int CP = Cfg::CPR / 2;
        u32x4 a0[Cfg::TC], b0[Cfg::TS], a1[Cfg::TC], b1[Cfg::TS];
        load_frags(stage, 0, wc0, ws0, lr, h, a0, b0);
#pragma unroll
        for (int cp = 0; cp < CP; ++cp) {
            if (cp % 2 == 0) {
                if (cp + 1 < CP) load_frags(stage, cp + 1, wc0, ws0, lr, h, a1, b1);
                __builtin_amdgcn_sched_barrier(0);
                mfma_block(a0, b0, acc);
            } else {
                if (cp + 1 < CP) load_frags(stage, cp + 1, wc0, ws0, lr, h, a0, b0);
                __builtin_amdgcn_sched_barrier(0);
                mfma_block(a1, b1, acc);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    static __device__ __forceinline__ void run(const T *__restrict__ x, const T *__restrict__ W,
                                               int M, int N, int K, int m0, int n0,
                                               unsigned char *smem, int tid, int wc0, int ws0,
                                               int lr, int h, f32x16 (&acc)[Cfg::TS][Cfg::TC]) {

        const int KT = (K + Cfg::BK - 1) / Cfg::BK;
        if (KT == 0) return;
        u32x4 pref[Cfg::CPT];
        load_global(x, W, M, N, K, m0, n0, 0, tid, pref);
        store_lds(smem, tid, pref);
        __syncthreads();
        for (int kt = 0; kt < KT; ++kt) {
            unsigned char *cur = smem + (kt & 1) * Cfg::STAGE_BYTES;
            unsigned char *nxt = smem + ((kt + 1) & 1) * Cfg::STAGE_BYTES;
            const bool more = kt + 1 < KT;
            if (more) load_global(x, W, M, N, K, m0, n0, (kt + 1) * Cfg::BK, tid, pref);
            compute_stage(cur, wc0, ws0, lr, h, acc);
            if (more) store_lds(nxt, tid, pref);
            __syncthreads();
        }
    }
};

// --------------------------------------------- GEMM core, LDS DMA ring ----
// Same contract as GemmCore, for K a multiple of the stage depth BK.
// Operands go global -> LDS directly (global_load_lds_dwordx4: each lane's
// 16 bytes land at the wave-uniform LDS base + 16 * lane), so no registers
// hold staged data and STAGES-1 stages are in flight while one is consumed.
// The swizzle is applied on the global side: the lane that fills physical
// chunk p of LDS row r fetches logical chunk p ^ f(r).  Rows past M or N are
// clamped to the last row (their results are never stored).
//
// Synchronisation, one barrier per stage.  Before it a wave waits (vmcnt) for
// its own DMA share of the stage about to be read and has consumed, with its
// MFMAs, every fragment of the slot about to be refilled; after it, the whole
// stage is visible and the slot is free for every wave.  The schedules differ
// in where the barrier sits (end of stage, or before its last chunk pair) and
// so in how many stages the refill runs ahead.
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void gbl_void_t;

__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

// s_waitcnt vmcnt(n) with expcnt/lgkmcnt left alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    compiler_fence();
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
    compiler_fence();
}

__device__ __forceinline__ void block_barrier() {
    compiler_fence();
    __builtin_amdgcn_s_barrier();
    compiler_fence();
}

template <class DT, class Cfg, int STAGES>
struct GemmCoreDMA {
    static constexpr int EARLY = Cfg::EARLY;
    typedef typename dt_traits<DT>::storage T;
    static constexpr int NW = Cfg::NT / 64;
    static constexpr int NB = Cfg::STAGE_BYTES / 1024;   // 1 KiB blocks per stage
    static constexpr int BPW = (NB + NW - 1) / NW;       // blocks per wave per stage
    static constexpr int ROWS_PER_BLOCK = 1024 / Cfg::ROWB;
    static_assert(Cfg::STAGE_BYTES % 1024 == 0, "whole 1 KiB blocks per stage");
    static_assert((Cfg::BC * Cfg::ROWB) % 1024 == 0, "W and x rows never share a block");
    static_assert(STAGES >= 2 && STAGES <= 4, "ring depth");
    static_assert((STAGES - 2) * BPW < 64, "vmcnt range");
    static constexpr int SMEM_BYTES = STAGES * Cfg::STAGE_BYTES;

    // Block j of a wave.  When the blocks do not divide evenly, the spare
    // loads of the last waves repeat block NB-1: the same bytes to the same
    // LDS location, so every wave issues exactly BPW loads per stage and the
    // vmcnt arithmetic is the same for all waves.
    static __device__ __forceinline__ int block_of(int wave, int j) {
        const int b = wave * BPW + j;
        return b < NB ? b : NB - 1;
    }

    // Per-lane source pointer (k = 0) of each block this wave fills.
    static __device__ __forceinline__ void setup(const T *__restrict__ x, const T *__restrict__ W,
                                                 int M, int N, int K, int m0, int n0, int wave,
                                                 int lane, const unsigned char *(&src)[BPW]) {
#pragma unroll
        for (int j = 0; j < BPW; ++j) {
            const int b = block_of(wave, j);
            const int o = b * 1024 + 16 * lane;
            const int r = o / Cfg::ROWB;
            const int p = (o % Cfg::ROWB) / 16;
            const int c = swz<Cfg>(r, p);   // XOR swizzle is its own inverse
            const T *row;
            if (b * ROWS_PER_BLOCK < Cfg::BC) {
                int n = n0 + r;
                n = n < N ? n : N - 1;
                row = W + (size_t)n * (size_t)K;
            } else {
                int m = m0 + (r - Cfg::BC);
                m = m < M ? m : M - 1;
                row = x + (size_t)m * (size_t)K;
            }
            src[j] = reinterpret_cast<const unsigned char *>(row + c * Cfg::EPC);
        }
    }

    static __device__ __forceinline__ void issue(unsigned char *smem, int slot, int wave, int kt,
                                                 const unsigned char *const (&src)[BPW]) {
        const size_t koff = (size_t)kt * (Cfg::BK * Cfg::EB);
#pragma unroll
        for (int j = 0; j < BPW; ++j) {
            unsigned char *dst = smem + slot * Cfg::STAGE_BYTES + block_of(wave, j) * 1024;
            __builtin_amdgcn_global_load_lds((gbl_void_t *)(src[j] + koff), (lds_void_t *)dst, 16,
                                             0, 0);
        }
    }

    struct Frags {
        u32x4 a[Cfg::TC];
        u32x4 b[Cfg::TS];
    };

    // Chunk pair CPI of stage kt: `cur` holds its fragments, `nxt` receives
    // the next ones (recursion keeps every buffer binding compile-time).
    template <int CPI, bool HANDOVER, bool ISSUE, int AFTER>
    static __device__ __forceinline__ void cp_step(unsigned char *smem, int kt, int KT, int wave,
                                                   int wc0,
                                                   int ws0, int lr, int h,
                                                   const unsigned char *const (&src)[BPW],
                                                   Frags &cur, Frags &nxt,
                                                   f32x16 (&acc)[Cfg::TS][Cfg::TC]) {
        typedef GemmCore<DT, Cfg> C;
        constexpr int CP = Cfg::CPR / 2;
        if constexpr (CPI + 1 < CP) {
            // first MFMAs of this chunk pair, then the next pair's reads (their
            // registers are free by now), then the remaining MFMAs
            const unsigned char *stage = smem + (kt % STAGES) * Cfg::STAGE_BYTES;
            C::template mfma_block<0, EARLY>(cur.a, cur.b, acc);
            __builtin_amdgcn_sched_barrier(0);
            C::load_frags(stage, CPI + 1, wc0, ws0, lr, h, nxt.a, nxt.b);
            __builtin_amdgcn_sched_barrier(0);
            C::template mfma_block<EARLY, Cfg::TS>(cur.a, cur.b, acc);
            __builtin_amdgcn_sched_barrier(0);
            cp_step<CPI + 1, HANDOVER, ISSUE, AFTER>(smem, kt, KT, wave, wc0, ws0, lr, h, src, nxt,
                                                     cur, acc);
        } else {
            constexpr int HALF = Cfg::TS / 2 > 0 ? Cfg::TS / 2 : 1;
            C::template mfma_block<0, HALF>(cur.a, cur.b, acc);
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (HANDOVER) {
                compiler_fence();
                __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
                wait_vmcnt<AFTER * BPW>();
                block_barrier();
                // next stage's first reads before the DMA issue: they gate the MFMAs
                C::load_frags(smem + ((kt + 1) % STAGES) * Cfg::STAGE_BYTES, 0, wc0, ws0, lr, h,
                              nxt.a, nxt.b);
                if constexpr (ISSUE)
                    issue(smem, kt % STAGES, wave, kt + STAGES < KT ? kt + STAGES : KT - 1, src);
            }
            __builtin_amdgcn_sched_barrier(0);
            C::template mfma_block<HALF, Cfg::TS>(cur.a, cur.b, acc);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // Schedule 2, chunk pair CPI of stage kt.  The barrier sits before the
    // last chunk pair: by then this wave's MFMAs have consumed every fragment
    // of stage kt-1 (so, past the barrier, that slot is free for every wave)
    // and, after the vmcnt wait, its DMA share of stage kt+1 has landed (so,
    // past the barrier, all of stage kt+1 is visible).  The last chunk pair
    // then reads stage kt+1's first fragments and refills the slot of stage
    // kt-1 with stage kt+STAGES-1 under its own MFMAs.  No LDS read is waited
    // for at the barrier: the reads in flight there are of stage kt.
    template <int CPI>
    static __device__ __forceinline__ void mb_step(unsigned char *smem, int kt, int KT, int wave,
                                                   int wc0, int ws0, int lr, int h,
                                                   const unsigned char *const (&src)[BPW],
                                                   Frags &cur, Frags &nxt,
                                                   f32x16 (&acc)[Cfg::TS][Cfg::TC]) {
        typedef GemmCore<DT, Cfg> C;
        constexpr int CP = Cfg::CPR / 2;
        C::template mfma_block<0, EARLY>(cur.a, cur.b, acc);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (CPI + 1 < CP) {
            C::load_frags(smem + (kt % STAGES) * Cfg::STAGE_BYTES, CPI + 1, wc0, ws0, lr, h,
                          nxt.a, nxt.b);
            __builtin_amdgcn_sched_barrier(0);
            C::template mfma_block<EARLY, Cfg::TS>(cur.a, cur.b, acc);
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (CPI + 2 == CP) {
                wait_vmcnt<(STAGES - 3) * BPW>();
                block_barrier();
            }
            mb_step<CPI + 1>(smem, kt, KT, wave, wc0, ws0, lr, h, src, nxt, cur, acc);
        } else {
            C::load_frags(smem + ((kt + 1) % STAGES) * Cfg::STAGE_BYTES, 0, wc0, ws0, lr, h,
                          nxt.a, nxt.b);
            const int ns = kt + STAGES - 1;
            __builtin_amdgcn_sched_barrier(0);
            mfma_with_refill<EARLY, Cfg::TS>(cur, acc, smem, ns % STAGES, wave,
                                             ns < KT ? ns : KT - 1, src);
        }
    }

    // MFMAs of sample tiles [T0, T1) with the refill of one stage spread over
    // them: DMA block j is issued after the j-th MFMA (blocks left over after
    // the last MFMA follow it).  Issued as one burst between MFMA blocks, the
    // DMA instructions held up the wave's next MFMAs; spread out, the main
    // loop of the bf16 256 x 256 tile takes 6-7 % fewer cycles.
    template <int T0, int T1>
    static __device__ __forceinline__ void mfma_with_refill(const Frags &f,
                                                            f32x16 (&acc)[Cfg::TS][Cfg::TC],
                                                            unsigned char *smem, int slot, int wave,
                                                            int kt,
                                                            const unsigned char *const (&src)[BPW]) {
        const size_t koff = (size_t)kt * (Cfg::BK * Cfg::EB);
        unsigned char *base = smem + slot * Cfg::STAGE_BYTES;
        constexpr int NM = (T1 - T0) * Cfg::TC;
#pragma unroll
        for (int i = 0; i < NM; ++i) {
            Mfma<DT>::run(acc[T0 + i / Cfg::TC][i % Cfg::TC], f.a[i % Cfg::TC], f.b[T0 + i / Cfg::TC]);
            __builtin_amdgcn_sched_barrier(0);
            if (i < BPW)
                __builtin_amdgcn_global_load_lds((gbl_void_t *)(src[i] + koff),
                                                 (lds_void_t *)(base + block_of(wave, i) * 1024),
                                                 16, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int j = NM; j < BPW; ++j)
            __builtin_amdgcn_global_load_lds((gbl_void_t *)(src[j] + koff),
                                             (lds_void_t *)(base + block_of(wave, j) * 1024), 16,
                                             0, 0);
        __builtin_amdgcn_sched_barrier(0);
    }

    // Schedule 2 main loop.  The prologue fills STAGES-1 slots; iteration kt
    // issues stage kt+STAGES-1 (clamped to the last stage past the end, into
    // a slot no later stage reads), so before the barrier of stage kt the
    // loads of stages kt+2 .. kt+STAGES-2 may still be in flight.  The reads
    // of "stage KT" in the last iteration fetch a slot nobody uses.
    static __device__ __forceinline__ void run_midbar(const T *__restrict__ x,
                                                      const T *__restrict__ W, int M, int N, int K,
                                                      int m0, int n0, unsigned char *smem, int tid,
                                                      int wc0, int ws0, int lr, int h,
                                                      f32x16 (&acc)[Cfg::TS][Cfg::TC]) {
        static_assert(STAGES >= 3, "schedule 2 refills the slot of the previous stage");
        static_assert(Cfg::CPR / 2 >= 2 && (Cfg::CPR / 2) % 2 == 0,
                      "schedule 2: an even number of chunk pairs per stage");
        const int KT = K / Cfg::BK;
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
        const unsigned char *src[BPW];
        setup(x, W, M, N, K, m0, n0, wave, lane, src);
#pragma unroll
        for (int s = 0; s < STAGES - 1; ++s) issue(smem, s, wave, s < KT ? s : KT - 1, src);
        wait_vmcnt<(STAGES - 2) * BPW>();
        block_barrier();
        Frags fa, fb;
        GemmCore<DT, Cfg>::load_frags(smem, 0, wc0, ws0, lr, h, fa.a, fa.b);
        for (int kt = 0; kt < KT; ++kt)
            mb_step<0>(smem, kt, KT, wave, wc0, ws0, lr, h, src, fa, fb, acc);
        wait_vmcnt<0>();   // no DMA may land in LDS after the main loop
    }

    template <bool HANDOVER, bool ISSUE, int AFTER>
    static __device__ __forceinline__ void stage_body(unsigned char *smem, int kt, int KT, int wave,
                                                      int wc0, int ws0, int lr, int h,
                                                      const unsigned char *const (&src)[BPW],
                                                      Frags &fa, Frags &fb,
                                                      f32x16 (&acc)[Cfg::TS][Cfg::TC]) {
        cp_step<0, HANDOVER, ISSUE, AFTER>(smem, kt, KT, wave, wc0, ws0, lr, h, src, fa, fb, acc);
    }

    // Simple schedule: per stage, wait for it, barrier, issue stage
    // kt+STAGES-1 into the slot of stage kt-1, then read-and-MFMA each chunk
    // pair.  Stage indices past the end are clamped as in run().
    static __device__ __forceinline__ void run_simple(const T *__restrict__ x,
                                                      const T *__restrict__ W, int M, int N, int K,
                                                      int m0, int n0, unsigned char *smem, int tid,
                                                      int wc0, int ws0, int lr, int h,
                                                      f32x16 (&acc)[Cfg::TS][Cfg::TC]) {
        typedef GemmCore<DT, Cfg> C;
        const int KT = K / Cfg::BK;
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
        const unsigned char *src[BPW];
        setup(x, W, M, N, K, m0, n0, wave, lane, src);
#pragma unroll
        for (int s = 0; s < STAGES - 1; ++s) issue(smem, s, wave, s < KT ? s : KT - 1, src);
        for (int kt = 0; kt < KT; ++kt) {
            wait_vmcnt<(STAGES - 2) * BPW>();
            block_barrier();
            const int nk = kt + STAGES - 1;
            issue(smem, nk % STAGES, wave, nk < KT ? nk : KT - 1, src);
            const unsigned char *stage = smem + (kt % STAGES) * Cfg::STAGE_BYTES;
#pragma unroll
            for (int cp = 0; cp < Cfg::CPR / 2; ++cp) {
                u32x4 a[Cfg::TC], b[Cfg::TS];
                C::load_frags(stage, cp, wc0, ws0, lr, h, a, b);
                C::mfma_block(a, b, acc);
            }
        }
        wait_vmcnt<0>();
    }

    static __device__ __forceinline__ void run(const T *__restrict__ x, const T *__restrict__ W,
                                               int M, int N, int K, int m0, int n0,
                                               unsigned char *smem, int tid, int wc0, int ws0,
                                               int lr, int h, f32x16 (&acc)[Cfg::TS][Cfg::TC]) {
        constexpr int CP = Cfg::CPR / 2;
        const int KT = K / Cfg::BK;
        if (KT == 0) return;
        if constexpr (!Cfg::PIPE) {
            run_simple(x, W, M, N, K, m0, n0, smem, tid, wc0, ws0, lr, h, acc);
            return;
        } else if constexpr (Cfg::SCHED == 2) {
            run_midbar(x, W, M, N, K, m0, n0, smem, tid, wc0, ws0, lr, h, acc);
            return;
        }
        // wave index as a scalar: the DMA's LDS base (M0) is then computed on
        // the scalar unit
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
        const unsigned char *src[BPW];
        setup(x, W, M, N, K, m0, n0, wave, lane, src);
        // Every iteration issues exactly one stage, so the vmcnt arithmetic is
        // the same everywhere: stage indices past the end are clamped to the
        // last stage (L2-resident by then) and land in the slot just freed,
        // which no later stage uses.
#pragma unroll
        for (int s = 0; s < STAGES; ++s)
            issue(smem, s, wave, s < KT ? s : KT - 1, src);
        wait_vmcnt<(STAGES - 1) * BPW>();
        block_barrier();
        Frags fa, fb;
        GemmCore<DT, Cfg>::load_frags(smem, 0, wc0, ws0, lr, h, fa.a, fa.b);
        if constexpr (CP % 2 == 0) {
            // an even number of chunk pairs leaves the next stage's first
            // fragments back in `fa`
            for (int kt = 0; kt + 1 < KT; ++kt)
                stage_body<true, true, STAGES - 2>(smem, kt, KT, wave, wc0, ws0, lr, h, src, fa,
                                                   fb, acc);
            stage_body<false, false, 0>(smem, KT - 1, KT, wave, wc0, ws0, lr, h, src, fa, fb, acc);
        } else {
            // an odd number leaves them in `fb`: alternate the roles
            int kt = 0;
            for (; kt + 2 < KT; kt += 2) {
                stage_body<true, true, STAGES - 2>(smem, kt, KT, wave, wc0, ws0, lr, h, src, fa,
                                                   fb, acc);
                stage_body<true, true, STAGES - 2>(smem, kt + 1, KT, wave, wc0, ws0, lr, h, src,
                                                   fb, fa, acc);
            }
            if (KT - kt == 2) {
                stage_body<true, true, STAGES - 2>(smem, kt, KT, wave, wc0, ws0, lr, h, src, fa,
                                                   fb, acc);
                stage_body<false, false, 0>(smem, kt + 1, KT, wave, wc0, ws0, lr, h, src, fb, fa,
                                            acc);
            } else {
                stage_body<false, false, 0>(smem, kt, KT, wave, wc0, ws0, lr, h, src, fa, fb,
                                            acc);
            }
        }
        wait_vmcnt<0>();   // no DMA may land in LDS after the main loop
    }
};

// Core selector: RING == 0 is the register-staged GemmCore (two LDS stages,
// any K); RING >= 2 is the LDS DMA ring of that depth (K % BK == 0).
template <class DT, class Cfg, int RING>
struct CoreSel {
    typedef GemmCoreDMA<DT, Cfg, RING> type;
    static constexpr int SMEM = RING * Cfg::STAGE_BYTES;
};
template <class DT, class Cfg>
struct CoreSel<DT, Cfg, 0> {
    typedef GemmCore<DT, Cfg> type;
    static constexpr int SMEM = 2 * Cfg::STAGE_BYTES;
};

// ------------------------------------------------- staged block store ----
// A lane holds 16-byte pieces of 32 different output rows (the MFMA
// accumulator layout), so a direct store writes 32 bytes per row per
// instruction.  Instead the wave writes its 32-row x WC-channel block to a
// private LDS area (16-byte chunks XOR-swizzled by the row's low 4 bits:
// conflict-free both ways for rows of 64..256 channels) and reads it back
// row by row, so each store instruction writes WC*4 contiguous bytes per row.
// value(tc, q) gives the lane's 4 channels 32*tc + 8*q + 4*h .. +3 of its row.
// STREAM: non-temporal stores, for output nothing in the kernel reads again:
// the lines then do not displace the GEMM operands cached in L2 and the MALL.
template <int WC, bool STREAM = false>
struct BlockStore {
    static_assert(WC >= 64 && WC <= 256, "block rows of 64..256 channels");
    static constexpr int BYTES = 32 * WC * 4;
    static constexpr int CPRW = WC / 4;   // 16-byte chunks per block row
    static constexpr int RPI = 64 / CPRW; // block rows per store instruction
    template <class F>
    static __device__ __forceinline__ void store(unsigned char *blk, int lane, F &&value,
                                                 float *__restrict__ out, int N, int M,
                                                 int row0, int col0) {
        const int lr = lane & 31, h = lane >> 5;
#pragma unroll
        for (int tc = 0; tc < WC / 32; ++tc)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int chunk = 8 * tc + 2 * q + h;
                *reinterpret_cast<f32x4 *>(blk + lr * (CPRW * 16) + 16 * (chunk ^ (lr & 15))) =
                    value(tc, q);
            }
        // one base address per lane; block row i*RPI lies i*RPI*N floats further on
        const int r0 = lane / CPRW, chunk = lane % CPRW;
        float *base = out + (size_t)(row0 + r0) * (size_t)N + (col0 + 4 * chunk);
        auto put = [&](f32x4 *dst, const f32x4 &y) {
            if constexpr (STREAM)
                __builtin_nontemporal_store(y, dst);
            else
                *dst = y;
        };
        auto get = [&](int i) {
            const int row = RPI * i + r0;
            return *reinterpret_cast<const f32x4 *>(blk + row * (CPRW * 16) +
                                                    16 * (chunk ^ (row & 15)));
        };
        if (row0 + 32 <= M && col0 + WC <= N) {
            // the whole block lies inside out (the wave-uniform common case): no checks
#pragma unroll
            for (int i = 0; i < 32 / RPI; ++i)
                put(reinterpret_cast<f32x4 *>(base + (size_t)(i * RPI) * (size_t)N), get(i));
        } else {
            const bool col_ok = col0 + 4 * chunk < N;
#pragma unroll
            for (int i = 0; i < 32 / RPI; ++i)
                if (col_ok && row0 + RPI * i + r0 < M)
                    put(reinterpret_cast<f32x4 *>(base + (size_t)(i * RPI) * (size_t)N), get(i));
        }
    }
};

// ------------------------------------------------------ tile schedule ----
// Workgroups are dispatched round-robin over the 8 XCDs (each with its own
// L2).  Remap the hardware id so that each XCD receives a contiguous run of
// logical tiles, then walk tiles in column-major order inside bands of
// GROUP_M sample-tiles, so that the workgroups resident on one XCD at the
// same time share x rows and W rows through that XCD's L2.
template <int GROUP_M>
__device__ __forceinline__ void tile_coords(int bid, int nblocks, int tiles_m, int tiles_n,
                                            int &tm, int &tn) {
    int t = bid;
    if ((nblocks & 7) == 0) t = (bid & 7) * (nblocks >> 3) + (bid >> 3);
    const int per_band = GROUP_M * tiles_n;
    const int band = t / per_band;
    const int first_m = band * GROUP_M;
    const int rem = tiles_m - first_m;
    const int gsize = rem < GROUP_M ? rem : GROUP_M;
    const int local = t - band * per_band;
    tm = first_m + local % gsize;
    tn = local / gsize;
}

// ------------------------------------------------------- elementwise ----
// Swish with unit slope: v * sigmoid(v), sigmoid(v) = 1 / (1 + e^-v), with
// e^-v = 2^(-v*log2 e) on the hardware exp2 and a hardware reciprocal.  For
// v -> -inf, e^-v -> +inf and the reciprocal -> 0, so the result -> -0.
__device__ __forceinline__ float swish(float v) {
    const float e = __builtin_amdgcn_exp2f(v * -1.4426950408889634f);
    return v * __builtin_amdgcn_rcpf(1.0f + e);
}

// Merge of two equal-count partial statistics (count n each) held by this
// lane and by lane^32.  Written symmetrically so that both lanes obtain
// bitwise identical results.
__device__ __forceinline__ void merge_halves(float &mean, float &m2, float n) {
    const float om = __shfl_xor(mean, 32);
    const float om2 = __shfl_xor(m2, 32);
    const float d = mean - om;
    mean = (mean + om) * 0.5f;
    m2 = (m2 + om2) + d * d * (0.5f * n);
}

}  // namespace lgn
