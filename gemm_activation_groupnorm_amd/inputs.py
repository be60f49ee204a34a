"""Seeded synthetic inputs for the fused Linear -> Swish -> +bias -> GroupNorm path.

This module only draws random numbers and rounds them to the storage type; it
holds none of the method's arithmetic.  The tests feed the same arrays to the
CPU oracle and to the HIP library; the benchmark uses it for its workload.

Value distributions follow the transcript's problem (an nn.Linear with
PyTorch's default uniform(-1/sqrt(K), 1/sqrt(K)) init for weight and bias, an
external per-channel bias, and GroupNorm gamma/beta), perturbed so that every
term of the forward is exercised:

    x      ~ x_scale * N(0, 1)
    W      ~ U(-1/sqrt(K), 1/sqrt(K))          [N, K], nn.Linear layout
    b_lin  ~ U(-1/sqrt(K), 1/sqrt(K))          [N]
    b_add  ~ 0.02 * N(0, 1)                    [N]
    gamma  ~ 1 + 0.1 * N(0, 1)                 [N]
    beta   ~ 0.1 * N(0, 1)                     [N]

Draw order x, W, b_lin, b_add, gamma, beta from numpy's PCG64
(``default_rng(seed)``), in float64, then rounded to float32 (round to nearest
even).  For the bf16 workload x and W are further rounded from float32 to
bfloat16 (round to nearest even); both sides then see the same bf16 values.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    M: int
    K: int
    N: int
    G: int
    dtype: str          # "f32" or "bf16": storage type of x and W
    seed: int
    eps: float = 1e-5
    x_scale: float = 1.0

    @property
    def channels_per_group(self) -> int:
        return self.N // self.G

    @property
    def flops(self) -> int:
        """GEMM flops, 2*M*N*K (the epilogue is not counted)."""
        return 2 * self.M * self.N * self.K


# The five workloads: tiny, small, the transcript's own shape in fp32 and in
# bf16, and a wide-group shape (1024 channels per group).
WORKLOADS = [
    Workload("tiny_f32", 64, 32, 128, 8, "f32", 0),
    Workload("small_f32", 1024, 256, 1024, 16, "f32", 1),
    Workload("m32768_k1024_n4096_g64_f32", 32768, 1024, 4096, 64, "f32", 2),
    Workload("m32768_k1024_n4096_g64_bf16", 32768, 1024, 4096, 64, "bf16", 3),
    Workload("m16384_k2048_n8192_g8_f32", 16384, 2048, 8192, 8, "f32", 4, x_scale=2.0),
]


# Groups wider than one workgroup tile: LayerNorm over all 8192 channels of
# the wide-group shape (the forward's G = 1 case).
WIDE_WORKLOADS = [
    Workload("m16384_k2048_n8192_g1_f32", 16384, 2048, 8192, 1, "f32", 8, x_scale=2.0),
]

# The second method (Linear -> logsumexp -> LeakyReLU x2 -> GELU x2) at the
# shape of its transcript: batch 1024, 8192 input and 8192 output features.
# It uses x, W and b_lin (as the linear bias) of the same draw; G is unused.
LSE_WORKLOADS = [
    Workload("m1024_k8192_n8192_lse_f32", 1024, 8192, 8192, 1, "f32", 5),
    Workload("m1024_k8192_n8192_lse_bf16", 1024, 8192, 8192, 1, "bf16", 6),
]


@dataclasses.dataclass(frozen=True)
class SghWorkload:
    """Swish -> spatial GroupNorm -> HardSwish on y [Nb, C, D, H, W]."""
    name: str
    Nb: int
    C: int
    D: int
    H: int
    W: int
    G: int
    seed: int
    eps: float = 1e-5

    @property
    def S(self) -> int:
        return self.D * self.H * self.W

    @property
    def elements(self) -> int:
        return self.Nb * self.C * self.S


# The third method at its transcript's shape: the output of a 3-D transposed
# convolution (batch 128, 16 channels, 31 x 63 x 63) in 4 groups.
SGH_WORKLOADS = [
    SghWorkload("n128_c16_d31_h63_w63_g4_sgh_f32", 128, 16, 31, 63, 63, 4, 7),
]


def make_sgh_inputs(Nb: int, C: int, S: int, seed: int) -> Dict[str, np.ndarray]:
    """y [Nb, C, S] ~ N(0, 1), gamma ~ 1 + 0.1 N(0, 1), beta ~ 0.1 N(0, 1) [C];
    drawn in that order in float64 from default_rng(seed), rounded to float32."""
    rng = np.random.default_rng(seed)
    y = rng.standard_normal((Nb, C, S)).astype(np.float32)
    gamma = (1.0 + 0.1 * rng.standard_normal(C)).astype(np.float32)
    beta = (0.1 * rng.standard_normal(C)).astype(np.float32)
    return dict(y=y, gamma=gamma, beta=beta)


@dataclasses.dataclass(frozen=True)
class LnConvWorkload:
    """LayerNorm over [C, L] -> GELU -> Conv1d (kernel 3, dilation d, padding d)
    -> + input, on x [B, C, L]."""
    name: str
    B: int
    C: int
    L: int
    dilation: int
    seed: int
    eps: float = 1e-5
    gelu_tanh: bool = False

    @property
    def flops(self) -> int:
        """Convolution flops, 2 * B * L * C_out * (C_in * 3)."""
        return 2 * self.B * self.L * self.C * self.C * 3


# The fourth method at its transcript's shape: batch 32, 256 channels, 4096
# positions, dilation 4; the GELU of nn.GELU() (exact).
LNCONV_WORKLOADS = [
    LnConvWorkload("b32_c256_l4096_d4_lnconv_f32", 32, 256, 4096, 4, 9),
]


def make_lnconv_inputs(B: int, C: int, L: int, seed: int) -> Dict[str, np.ndarray]:
    """x [B, C, L] ~ N(0, 1); ln_w ~ 1 + 0.1 N(0, 1), ln_b ~ 0.1 N(0, 1) [C, L];
    conv_w [C, C, 3] and conv_b [C] ~ U(-1/sqrt(3C), 1/sqrt(3C)) (nn.Conv1d's
    default bound); drawn in that order in float64 from default_rng(seed),
    rounded to float32."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, C, L)).astype(np.float32)
    ln_w = (1.0 + 0.1 * rng.standard_normal((C, L))).astype(np.float32)
    ln_b = (0.1 * rng.standard_normal((C, L))).astype(np.float32)
    bound = 1.0 / np.sqrt(3.0 * C)
    conv_w = rng.uniform(-bound, bound, (C, C, 3)).astype(np.float32)
    conv_b = rng.uniform(-bound, bound, C).astype(np.float32)
    return dict(x=x, ln_w=ln_w, ln_b=ln_b, conv_w=conv_w, conv_b=conv_b)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); uint16 bits.

    Inputs are finite by construction, so NaN handling is not needed."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    rounding = np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))
    return ((u + rounding) >> np.uint64(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def make_inputs(M: int, K: int, N: int, seed: int, dtype: str = "f32",
                x_scale: float = 1.0) -> Dict[str, np.ndarray]:
    """Draw one input set.

    Returns float32 arrays ``x, W, b_lin, b_add, gamma, beta``.  For
    ``dtype == "bf16"`` also ``x_bf16, W_bf16`` (uint16 bit patterns) and
    ``x, W`` hold the float32 widening of exactly those bf16 values.
    """
    rng = np.random.default_rng(seed)
    bound = 1.0 / np.sqrt(K) if K > 0 else 0.0
    x = (rng.standard_normal((M, K)) * x_scale).astype(np.float32)
    W = rng.uniform(-bound, bound, (N, K)).astype(np.float32)
    b_lin = rng.uniform(-bound, bound, N).astype(np.float32)
    b_add = (rng.standard_normal(N) * 0.02).astype(np.float32)
    gamma = (1.0 + 0.1 * rng.standard_normal(N)).astype(np.float32)
    beta = (0.1 * rng.standard_normal(N)).astype(np.float32)
    out = dict(x=x, W=W, b_lin=b_lin, b_add=b_add, gamma=gamma, beta=beta)
    if dtype == "bf16":
        xb = f32_to_bf16_bits(x)
        Wb = f32_to_bf16_bits(W)
        out.update(x_bf16=xb, W_bf16=Wb, x=bf16_bits_to_f32(xb), W=bf16_bits_to_f32(Wb))
    elif dtype != "f32":
        raise ValueError("dtype must be 'f32' or 'bf16'")
    return out


def workload_inputs(w: Workload) -> Dict[str, np.ndarray]:
    return make_inputs(w.M, w.K, w.N, w.seed, w.dtype, w.x_scale)


def get_workload(name_or_index) -> Workload:
    if isinstance(name_or_index, int):
        return WORKLOADS[name_or_index]
    for w in WORKLOADS + WIDE_WORKLOADS + LSE_WORKLOADS:
        if w.name == name_or_index:
            return w
    raise KeyError(name_or_index)


def sample_rows(M: int, count: int, seed: int = 12345) -> np.ndarray:
    """Sorted, distinct row indices that always include the first and last row."""
    count = min(count, M)
    rng = np.random.default_rng(seed)
    rows = set([0, M - 1])
    rest = rng.choice(M, size=count, replace=False)
    for r in rest:
        if len(rows) >= count:
            break
        rows.add(int(r))
    return np.array(sorted(rows), dtype=np.int64)
