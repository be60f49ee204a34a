"""GPU parity of the wide-group forward (groups spanning several 256-channel
tiles, down to LayerNorm over all N) through the C ABI, against the fp64
oracle; tolerances as for the fused path (2e-4 fp32, 3e-2 bf16)."""
import numpy as np
import pytest
import torch

from gemm_activation_groupnorm_amd import lgn
from gemm_activation_groupnorm_amd.inputs import WORKLOADS, workload_inputs
from gpu_helpers import TOL, case, log, max_err, oracle_rows, run, to_device

pytestmark = pytest.mark.gpu


def run_wide(dev, M, K, N, G, eps, dtype, out=None):
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device="cuda")
    nb = lgn.lgn_wide_workspace_bytes(M, N)
    ws = torch.empty(max(1, nb // 4), dtype=torch.float32, device="cuda")
    fn = lgn.lgn_forward_wide_f32 if dtype == "f32" else lgn.lgn_forward_wide_bf16
    lgn.check(fn(dev["x"], dev["W"], dev["b_lin"], dev["b_add"], dev["gamma"], dev["beta"], M, K,
                 N, G, eps, out, ws, nb))
    return out


SHAPES = [
    # M,   K,   N,    G     (channels per group)
    (300, 64, 512, 1),      # 512: LayerNorm over the row, 2 tiles
    (257, 128, 1024, 1),    # 1024, ragged sample tile
    (130, 40, 768, 1),      # 768, K off the stage depth (register-staged core)
    (1, 32, 2048, 2),       # 1024, a single row
    (520, 96, 4096, 2),     # 2048
    (64, 0, 512, 2),        # K = 0: the linear layer is its bias
    (33, 256, 8192, 1),     # LayerNorm over 8192 channels
]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "M%d_K%d_N%d_G%d" % s)
def test_wide_shapes(shape, dtype):
    M, K, N, G = shape
    log("wide case M=%d K=%d N=%d G=%d dtype=%s" % (M, K, N, G, dtype))
    if dtype == "bf16" and K % 8:
        pytest.skip("bf16 needs K % 8 == 0")
    inp = case(M, K, N, G, 900 + M + K + N + G, dtype)
    y = run_wide(to_device(inp, dtype), M, K, N, G, 1e-5, dtype)
    torch.cuda.synchronize()
    err = max_err(y.cpu().numpy(), oracle_rows(inp, G, 1e-5))
    log("  max abs err %.3e" % err)
    assert err <= TOL[dtype]


def test_wide_matches_fused_on_the_wide_group_shape():
    # C = 1024 is covered by both entry points: same values up to rounding
    # (their parity against the oracle on every element is in the full-size tests)
    w = WORKLOADS[4]
    inp = workload_inputs(w)
    dev = to_device(inp, w.dtype)
    a = run_wide(dev, w.M, w.K, w.N, w.G, w.eps, w.dtype)
    b = run(dev, w.M, w.K, w.N, w.G, w.eps, w.dtype, "fused")
    torch.cuda.synchronize()
    assert float((a - b).abs().max()) <= TOL["f32"]


def test_wide_deterministic_and_row_split():
    M, K, N, G = 777, 64, 2048, 1
    inp = case(M, K, N, G, 44)
    dev = to_device(inp, "f32")
    y1 = run_wide(dev, M, K, N, G, 1e-5, "f32")
    y2 = run_wide(dev, M, K, N, G, 1e-5, "f32")
    h = 300
    ya = run_wide(dict(dev, x=dev["x"][:h].contiguous()), h, K, N, G, 1e-5, "f32")
    yb = run_wide(dict(dev, x=dev["x"][h:].contiguous()), M - h, K, N, G, 1e-5, "f32")
    torch.cuda.synchronize()
    assert torch.equal(y1, y2), "run-to-run difference"
    assert torch.equal(torch.cat([ya, yb]), y1), "row split changes results"


@pytest.mark.parametrize("M", [131, 132])
def test_wide_no_writes_outside_output_or_workspace(M):
    # The normalise kernel takes rows in pairs: with an odd M the last pair
    # has one row, and nothing past row M-1 may be written.
    K, N, G = 64, 512, 2
    log("wide bounds case M=%d K=%d N=%d G=%d" % (M, K, N, G))
    inp = case(M, K, N, G, 45)
    dev = to_device(inp, "f32")
    pad = 4096
    buf = torch.full((M * N + 2 * pad,), 12345.0, dtype=torch.float32, device="cuda")
    nb = lgn.lgn_wide_workspace_bytes(M, N)
    wsbuf = torch.full((nb // 4 + 2 * pad,), 12345.0, dtype=torch.float32, device="cuda")
    lgn.check(lgn.lgn_forward_wide_f32(dev["x"], dev["W"], dev["b_lin"], dev["b_add"],
                                       dev["gamma"], dev["beta"], M, K, N, G, 1e-5,
                                       buf.data_ptr() + pad * 4, wsbuf.data_ptr() + pad * 4, nb))
    torch.cuda.synchronize()
    assert bool((buf[:pad] == 12345.0).all()) and bool((buf[pad + M * N:] == 12345.0).all())
    assert bool((wsbuf[:pad] == 12345.0).all()) and bool((wsbuf[pad + nb // 4:] == 12345.0).all())
    y = buf[pad:pad + M * N].view(M, N).cpu().numpy()
    assert max_err(y, oracle_rows(inp, G, 1e-5)) <= TOL["f32"]
