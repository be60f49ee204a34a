"""GPU parity at the full workload sizes, on EVERY output element.

Each full-size workload runs through every entry point that covers it (the
fused kernel, the two-pass ablation and, for groups of a multiple of 256
channels, the wide-group path); the fp64 oracle is computed once per chunk of
rows and every element of every output is compared with it.  The log gives
max abs, mean abs and the count above the tolerance (2e-4 for fp32 inputs,
3e-2 for bf16 inputs); a single element above it fails the test, which a
sampled-row comparison could miss (a race that corrupts a few values shows
as a large max with a near-zero mean).

Also here: the edge cases of the fused epilogue (groups of zero and of tiny
variance, where the 1/sqrt(eps) ~ 316 factor amplifies any rounding of the
mean, and Swish driven deep into both tails), and bitwise run-to-run and
row-split equality at the full sizes, where the tile remap over the 8 XCDs and
the DMA ring's clamps are active.
"""
import numpy as np
import pytest
import torch

from gemm_activation_groupnorm_amd import lgn
from gemm_activation_groupnorm_amd.inputs import WORKLOADS, WIDE_WORKLOADS, workload_inputs
from gpu_helpers import TOL, case, compare_all_rows, log, oracle_rows, run, to_device

pytestmark = pytest.mark.gpu


def run_wide(dev, M, K, N, G, eps, dtype):
    out = torch.empty((M, N), dtype=torch.float32, device="cuda")
    nb = lgn.lgn_wide_workspace_bytes(M, N)
    ws = torch.empty(max(1, nb // 4), dtype=torch.float32, device="cuda")
    fn = lgn.lgn_forward_wide_f32 if dtype == "f32" else lgn.lgn_forward_wide_bf16
    lgn.check(fn(dev["x"], dev["W"], dev["b_lin"], dev["b_add"], dev["gamma"], dev["beta"], M, K,
                 N, G, eps, out, ws, nb))
    return out


def _outputs(w, inp, variants):
    dev = to_device(inp, w.dtype)
    outs = {}
    for v in variants:
        log("workload %s variant=%s (full size)" % (w.name, v))
        if v == "wide":
            y = run_wide(dev, w.M, w.K, w.N, w.G, w.eps, w.dtype)
        else:
            y = run(dev, w.M, w.K, w.N, w.G, w.eps, w.dtype, v)
        torch.cuda.synchronize()
        outs[v] = y.cpu().numpy()
        del y
    del dev
    torch.cuda.empty_cache()
    return outs


def _check_all(w, inp, outs):
    stats = compare_all_rows(outs, lambda r0, r1: oracle_rows(inp, w.G, w.eps, slice(r0, r1)),
                             w.M, TOL[w.dtype])
    for v, s in stats.items():
        log("  %s/%s: %s" % (w.name, v, s))
    for v, s in stats.items():
        assert s.n == w.M * w.N
        assert s.max <= TOL[w.dtype], "%s/%s: %s" % (w.name, v, s)


@pytest.mark.parametrize("wi", [2, 3, 4], ids=lambda i: WORKLOADS[i].name)
def test_full_size_every_element(wi):
    w = WORKLOADS[wi]
    variants = ["fused", "twopass"] + (["wide"] if (w.N // w.G) % 256 == 0 else [])
    inp = workload_inputs(w)
    _check_all(w, inp, _outputs(w, inp, variants))


@pytest.mark.parametrize("wi", range(len(WIDE_WORKLOADS)), ids=lambda i: WIDE_WORKLOADS[i].name)
def test_wide_groups_full_size_every_element(wi):
    w = WIDE_WORKLOADS[wi]
    inp = workload_inputs(w)
    # G = 1: only the wide path and the two-pass ablation cover 8192-channel groups
    _check_all(w, inp, _outputs(w, inp, ["wide", "twopass"]))


# ---- edge cases of the fused epilogue ----

EDGE_SHAPES = [(300, 64, 512, 8), (257, 128, 1024, 16), (130, 96, 2048, 2), (96, 64, 1024, 1)]


def _fused_like(dev, M, K, N, G, dtype):
    """Outputs of every entry point covering (N/G), for the edge cases."""
    outs = {"twopass": run(dev, M, K, N, G, 1e-5, dtype, "twopass")}
    if lgn.lgn_fused_supported(0 if dtype == "f32" else 1, M, K, N, G):
        outs["fused"] = run(dev, M, K, N, G, 1e-5, dtype, "fused")
    if (N // G) % 256 == 0:
        outs["wide"] = run_wide(dev, M, K, N, G, 1e-5, dtype)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in outs.items()}


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", EDGE_SHAPES, ids=lambda s: "M%d_K%d_N%d_G%d" % s)
def test_zero_variance_groups_give_beta(shape, dtype):
    # W = 0 and b_lin = 0 make z = 0 and Swish(0) = 0, and b_add constant
    # inside each group then makes every group constant: its variance is 0,
    # so y = beta exactly in the oracle and up to eps^-1/2 times the rounding
    # of the mean on the GPU
    M, K, N, G = shape
    log("zero-variance case M=%d K=%d N=%d G=%d dtype=%s" % (M, K, N, G, dtype))
    inp = case(M, K, N, G, 61, dtype)
    for k in ("W", "W_bf16"):
        if k in inp:
            inp[k][:] = 0
    inp["b_lin"][:] = 0
    inp["b_add"][:] = np.repeat(np.linspace(-0.7, 1.3, G), N // G).astype(np.float32)
    ref = oracle_rows(inp, G, 1e-5)
    assert np.array_equal(ref, np.broadcast_to(inp["beta"].astype(np.float64), (M, N)))
    for v, y in _fused_like(to_device(inp, dtype), M, K, N, G, dtype).items():
        err = float(np.max(np.abs(y.astype(np.float64) - ref)))
        log("  %s: max abs err %.3e" % (v, err))
        assert err <= TOL["f32"], v   # the GEMM contributes exact zeros: fp32 bar for both


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", EDGE_SHAPES, ids=lambda s: "M%d_K%d_N%d_G%d" % s)
def test_tiny_variance_groups(shape, dtype):
    # W scaled down by 1e-3: each group's variance (~1e-9) sits far below
    # eps, so rstd ~ 316 multiplies every rounding error of u and the mean
    M, K, N, G = shape
    log("tiny-variance case M=%d K=%d N=%d G=%d dtype=%s" % (M, K, N, G, dtype))
    inp = case(M, K, N, G, 62, "f32")
    inp["W"] = (inp["W"] * np.float32(1e-3)).astype(np.float32)
    inp["b_lin"] = (inp["b_lin"] * np.float32(1e-3)).astype(np.float32)
    if dtype == "bf16":
        from gemm_activation_groupnorm_amd.inputs import bf16_bits_to_f32, f32_to_bf16_bits
        for k in ("x", "W"):
            inp[k + "_bf16"] = f32_to_bf16_bits(inp[k])
            inp[k] = bf16_bits_to_f32(inp[k + "_bf16"])
    ref = oracle_rows(inp, G, 1e-5)
    for v, y in _fused_like(to_device(inp, dtype), M, K, N, G, dtype).items():
        err = float(np.max(np.abs(y.astype(np.float64) - ref)))
        log("  %s: max abs err %.3e" % (v, err))
        assert err <= TOL[dtype], v


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", EDGE_SHAPES, ids=lambda s: "M%d_K%d_N%d_G%d" % s)
def test_saturated_swish(shape, dtype):
    # x scaled by 60 spreads z over about +-100: Swish(z) underflows to -0 for
    # z << 0 (exp(-z) overflows to inf in fp32 below about -88.7, where the
    # sigmoid's two textbook forms part ways) and equals z to fp32 precision
    # for z >> 0
    M, K, N, G = shape
    log("saturated-Swish case M=%d K=%d N=%d G=%d dtype=%s" % (M, K, N, G, dtype))
    inp = case(M, K, N, G, 63, dtype, x_scale=60.0)
    import oracle
    zz = oracle.linear(inp["x"], inp["W"], inp["b_lin"])
    assert zz.min() < -90.0 and zz.max() > 90.0, (zz.min(), zz.max())
    ref = oracle_rows(inp, G, 1e-5)
    for v, y in _fused_like(to_device(inp, dtype), M, K, N, G, dtype).items():
        err = float(np.max(np.abs(y.astype(np.float64) - ref)))
        log("  %s: max abs err %.3e" % (v, err))
        assert err <= TOL[dtype], v


# ---- bitwise determinism at the full sizes ----

@pytest.mark.parametrize("variant", ["fused", "twopass"])
@pytest.mark.parametrize("wi", [2, 3, 4], ids=lambda i: WORKLOADS[i].name)
def test_full_size_bitwise_deterministic_and_row_split(wi, variant):
    w = WORKLOADS[wi]
    log("determinism workload %s variant=%s" % (w.name, variant))
    inp = workload_inputs(w)
    dev = to_device(inp, w.dtype)
    y1 = run(dev, w.M, w.K, w.N, w.G, w.eps, w.dtype, variant)
    y2 = run(dev, w.M, w.K, w.N, w.G, w.eps, w.dtype, variant)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2), "run-to-run difference"
    del y2
    # split at a row that is not a multiple of any tile height, so every
    # sample tile of the second call starts at a different row
    h = w.M // 2 + 37
    ya = run(dict(dev, x=dev["x"][:h].contiguous()), h, w.K, w.N, w.G, w.eps, w.dtype, variant)
    assert torch.equal(ya, y1[:h]), "row split changes the first part"
    del ya
    yb = run(dict(dev, x=dev["x"][h:].contiguous()), w.M - h, w.K, w.N, w.G, w.eps, w.dtype,
             variant)
    torch.cuda.synchronize()
    assert torch.equal(yb, y1[h:]), "row split changes the second part"
