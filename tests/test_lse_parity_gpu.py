"""GPU parity of Linear -> logsumexp -> LeakyReLU x2 -> GELU x2 (through the C
ABI) against the fp64 oracle.  Tolerances as for the GroupNorm path: 2e-4 max
abs for fp32 inputs, 3e-2 for bf16 inputs (the oracle then runs on the same
bf16 values, widened exactly)."""
import numpy as np
import pytest
import torch

import oracle
from gemm_activation_groupnorm_amd import lgn
from gemm_activation_groupnorm_amd.inputs import LSE_WORKLOADS, make_inputs
from gpu_helpers import TOL, ErrStats, log, to_device

pytestmark = pytest.mark.gpu


def run_lse(dev, M, K, N, dtype, out=None, stream=None):
    if out is None:
        out = torch.empty(M, dtype=torch.float32, device="cuda")
    nb = lgn.lgn_lse_workspace_bytes(M, N)
    ws = torch.empty(max(1, nb // 4), dtype=torch.float32, device="cuda")
    fn = lgn.lgn_linear_lse_f32 if dtype == "f32" else lgn.lgn_linear_lse_bf16
    lgn.check(fn(dev["x"], dev["W"], dev["b_lin"], M, K, N, out, ws, nb, stream=stream))
    return out


def oracle_lse(inp, rows=None):
    x = inp["x"] if rows is None else inp["x"][rows]
    return oracle.linear_lse_forward(x, inp["W"], inp["b_lin"], return_lse=True)


def _err(y, ref):
    assert np.all(np.isfinite(y)), "non-finite GPU output"
    return float(np.max(np.abs(y.astype(np.float64) - ref))) if y.size else 0.0


SHAPES = [
    # M,   K,   N
    (64, 32, 256),       # one channel tile
    (130, 40, 300),      # ragged channel tile; K off the fp32/bf16 stage depth
    (1, 64, 4),          # a single row of 4 outputs
    (257, 128, 1280),    # ragged sample tile, 5 channel tiles
    (33, 0, 100),        # K = 0: z is the bias
    (100, 16, 12),       # fewer channels than one wave's span
    (300, 96, 1000),
    (70, 256, 8192),     # the transcript's feature count
    (129, 192, 520),     # bf16: three 64-deep stages (the ring's depth), ragged tiles
    (200, 640, 2048),    # bf16: ten 64-deep stages
]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "M%d_K%d_N%d" % s)
def test_lse_shapes(shape, dtype):
    M, K, N = shape
    log("lse case M=%d K=%d N=%d dtype=%s" % (M, K, N, dtype))
    if dtype == "bf16" and K % 8:
        pytest.skip("bf16 needs K % 8 == 0")
    inp = make_inputs(M, K, N, 500 + M + K + N, dtype)
    y = run_lse(to_device(inp, dtype), M, K, N, dtype)
    torch.cuda.synchronize()
    ref, _ = oracle_lse(inp)
    err = _err(y.cpu().numpy(), ref)
    log("  max abs err %.3e" % err)
    assert err <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shift", [-200.0, -12.0, 6.0, 200.0])
def test_lse_activation_branches(shift, dtype):
    # a bias far below 0 makes every logsumexp negative (both LeakyReLUs then
    # scale it by 0.01 and the GELUs see small negative values); far above,
    # the activations are close to the identity.  At +-200 every exp of an
    # unshifted z overflows (or underflows) in fp32: only the max-shifted
    # partials and their merge keep the result finite and exact
    M, K, N = 96, 64, 512
    inp = make_inputs(M, K, N, 77, dtype)
    inp["b_lin"] = (inp["b_lin"] + np.float32(shift)).astype(np.float32)
    y = run_lse(to_device(inp, dtype), M, K, N, dtype)
    torch.cuda.synchronize()
    ref, lse = oracle_lse(inp)
    assert np.all(lse < 0) if shift < 0 else np.all(lse > 0)
    assert _err(y.cpu().numpy(), ref) <= TOL[dtype]


@pytest.mark.parametrize("wi", range(len(LSE_WORKLOADS)))
def test_lse_full_size_every_row(wi):
    w = LSE_WORKLOADS[wi]
    log("lse workload %s" % w.name)
    inp = make_inputs(w.M, w.K, w.N, w.seed, w.dtype, w.x_scale)
    y = run_lse(to_device(inp, w.dtype), w.M, w.K, w.N, w.dtype)
    torch.cuda.synchronize()
    ref, _ = oracle_lse(inp)
    st = ErrStats(TOL[w.dtype])
    st.add(y.cpu().numpy(), ref)
    log("  every row: %s" % st)
    assert st.n == w.M and st.max <= TOL[w.dtype]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_lse_deterministic_and_row_split(dtype):
    M, K, N = 513, 128, 4096
    inp = make_inputs(M, K, N, 88, dtype)
    dev = to_device(inp, dtype)
    y1 = run_lse(dev, M, K, N, dtype)
    y2 = run_lse(dev, M, K, N, dtype)
    h = 200
    ya = run_lse(dict(dev, x=dev["x"][:h].contiguous()), h, K, N, dtype)
    yb = run_lse(dict(dev, x=dev["x"][h:].contiguous()), M - h, K, N, dtype)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2), "run-to-run difference"
    assert torch.equal(torch.cat([ya, yb]), y1), "row split changes results"


def test_lse_side_stream_and_empty_batch():
    M, K, N = 40, 32, 640
    inp = make_inputs(M, K, N, 9, "f32")
    dev = to_device(inp, "f32")
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        y = run_lse(dev, M, K, N, "f32", stream=s)
    s.synchronize()
    ref, _ = oracle_lse(inp)
    assert _err(y.cpu().numpy(), ref) <= TOL["f32"]
    assert lgn.lgn_linear_lse_f32(None, dev["W"], dev["b_lin"], 0, K, N, None, None, 0) == \
        lgn.LGN_OK
