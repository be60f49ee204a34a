"""GPU parity on a seeded sweep of random shapes: group widths from 1 to ~1200
channels with every divisibility (powers of two, multiples of 4, even, odd),
ragged row counts, K down to 0.  Each shape runs through the two-pass entry
point (every group width), and through the fused one where it takes the
shape; both against the fp64 oracle on every element."""
import numpy as np
import pytest
import torch

from gemm_activation_groupnorm_amd import lgn
from gpu_helpers import TOL, case, log, max_err, oracle_rows, run, to_device

pytestmark = pytest.mark.gpu


def _shapes(n=24, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        G = int(rng.choice([1, 2, 3, 4, 5, 6, 7, 8, 10, 12, 16, 20, 32, 64]))
        C = int(rng.integers(1, 1200))
        N = G * C
        if N % 4 or N > 12288:
            continue
        M = int(rng.integers(1, 70))
        K = int(rng.choice([0, 4, 8, 16, 24, 40, 64, 96]))
        out.append((M, K, N, G))
    return out


SHAPES = _shapes()
# bf16 inputs need K % 8 == 0
CASES = [(s, dt) for s in SHAPES for dt in ("f32", "bf16") if dt == "f32" or s[1] % 8 == 0]


@pytest.mark.parametrize("shape, dtype", CASES, ids=lambda c: c if isinstance(c, str) else
                         "M%d_K%d_N%d_G%d" % c)
def test_random_shape(shape, dtype):
    M, K, N, G = shape
    inp = case(M, K, N, G, 3000 + M + K + N + G, dtype)
    ref = oracle_rows(inp, G, 1e-5)
    dev = to_device(inp, dtype)
    variants = ["twopass"]
    if lgn.lgn_fused_supported(0 if dtype == "f32" else 1, M, K, N, G):
        variants.append("fused")
    for v in variants:
        log("random case M=%d K=%d N=%d G=%d (C=%d) %s %s" % (M, K, N, G, N // G, dtype, v))
        y = run(dev, M, K, N, G, 1e-5, dtype, v)
        torch.cuda.synchronize()
        err = max_err(y.cpu().numpy(), ref)
        assert err <= TOL[dtype], "%s: max abs err %.3e" % (v, err)
