"""GPU parity of LayerNorm -> GELU -> dilated Conv1d -> + input (through the C
ABI) against the fp64 oracle; max abs error <= 2e-4 (fp32 data, fp32 MFMA
accumulation over K = 3 * C terms)."""
import numpy as np
import pytest
import torch

import oracle
from gemm_activation_groupnorm_amd import lgn
from gemm_activation_groupnorm_amd.inputs import LNCONV_WORKLOADS, make_lnconv_inputs
from gpu_helpers import TOL, compare_all_rows, log

pytestmark = pytest.mark.gpu


def dev(inp):
    return {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in inp.items()}


def run_lnconv(d, B, C, L, dil, eps=1e-5, tanh=False, out=None, stream=None):
    if out is None:
        out = torch.empty((B, C, L), dtype=torch.float32, device="cuda")
    nb = lgn.lgn_lnconv_workspace_bytes(B, C, L)
    ws = torch.empty(max(1, nb // 4), dtype=torch.float32, device="cuda")
    lgn.check(lgn.lgn_ln_gelu_conv1d_f32(d["x"], d["ln_w"], d["ln_b"], d["conv_w"], d["conv_b"],
                                         B, C, L, dil, eps, tanh, out, ws, nb, stream=stream))
    return out


def _err(y, ref):
    assert np.all(np.isfinite(y)), "non-finite GPU output"
    return float(np.max(np.abs(y.astype(np.float64) - ref))) if y.size else 0.0


SHAPES = [
    # B, C,   L,    dilation, tanh GELU
    (2, 128, 256, 4, False),     # two position tiles, one channel tile
    (3, 256, 200, 4, False),     # ragged last position tile, two channel tiles
    (1, 128, 12, 3, True),       # L shorter than the halo; dilation rounded up to 4
    (2, 128, 132, 16, False),    # largest dilation, 4 positions in the last tile
    (1, 384, 64, 1, True),       # dilation 1, three channel tiles
    (2, 128, 4, 2, False),       # a single float4 of positions
    (1, 256, 256, 5, False),     # dilation 5 (halo 8); 64K values = four stats chunks
    (1, 8192, 64, 16, False),    # the largest C: 805 MB of packed weights, 32-bit offsets
                                 # near their bound; the position tile larger than L
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B%d_C%d_L%d_d%d_tanh%d" % s)
def test_lnconv_shapes(shape):
    B, C, L, dil, tanh = shape
    log("lnconv case B=%d C=%d L=%d d=%d tanh=%d" % shape)
    inp = make_lnconv_inputs(B, C, L, 900 + B + C + L + dil)
    out = run_lnconv(dev(inp), B, C, L, dil, tanh=tanh)
    torch.cuda.synchronize()
    ref = oracle.ln_gelu_conv1d(inp["x"], inp["ln_w"], inp["ln_b"], inp["conv_w"], inp["conv_b"],
                                dil, 1e-5, gelu_tanh=tanh)
    err = _err(out.cpu().numpy(), ref)
    log("  max abs err %.3e" % err)
    assert err <= TOL["f32"]


def test_lnconv_zero_weights_give_bias_plus_input_exactly():
    B, C, L, dil = 2, 128, 136, 4
    inp = make_lnconv_inputs(B, C, L, 77)
    inp["conv_w"] = np.zeros_like(inp["conv_w"])
    out = run_lnconv(dev(inp), B, C, L, dil)
    torch.cuda.synchronize()
    want = (inp["conv_b"][None, :, None] + inp["x"]).astype(np.float32)
    assert np.array_equal(out.cpu().numpy(), want)


def test_lnconv_constant_sample():
    # variance 0: the normalised values are 0 and g = GELU(ln_b) (rstd = 1/sqrt(eps))
    B, C, L, dil = 2, 256, 260, 3
    inp = make_lnconv_inputs(B, C, L, 81)
    inp["x"][1] = 0.75
    out = run_lnconv(dev(inp), B, C, L, dil)
    torch.cuda.synchronize()
    ref = oracle.ln_gelu_conv1d(inp["x"], inp["ln_w"], inp["ln_b"], inp["conv_w"], inp["conv_b"],
                                dil, 1e-5)
    err = _err(out.cpu().numpy(), ref)
    log("  constant sample: max abs err %.3e" % err)
    assert err <= TOL["f32"]


def test_lnconv_deterministic_and_side_stream():
    B, C, L, dil = 2, 256, 512, 4
    inp = make_lnconv_inputs(B, C, L, 78)
    d = dev(inp)
    a = run_lnconv(d, B, C, L, dil)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        b = run_lnconv(d, B, C, L, dil, stream=s)
    s.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_lnconv_sample_split_matches_whole_batch():
    B, C, L, dil = 4, 128, 384, 4
    inp = make_lnconv_inputs(B, C, L, 79)
    d = dev(inp)
    whole = run_lnconv(d, B, C, L, dil)
    part = {k: v for k, v in d.items()}
    part["x"] = d["x"][2:].contiguous()
    tail = run_lnconv(part, 2, C, L, dil)
    torch.cuda.synchronize()
    assert torch.equal(whole[2:], tail)


@pytest.mark.parametrize("tanh", [False, True])
def test_lnconv_full_size_every_element(tanh):
    w = LNCONV_WORKLOADS[0]
    log("lnconv full size %s tanh=%d" % (w.name, tanh))
    inp = make_lnconv_inputs(w.B, w.C, w.L, w.seed)
    out = run_lnconv(dev(inp), w.B, w.C, w.L, w.dilation, w.eps, tanh=tanh)
    torch.cuda.synchronize()
    y = out.cpu().numpy()
    del out
    # whole samples at a time (the LayerNorm statistics span a sample), every element
    stats = compare_all_rows(
        {"lnconv": y},
        lambda b0, b1: oracle.ln_gelu_conv1d(inp["x"][b0:b1], inp["ln_w"], inp["ln_b"],
                                             inp["conv_w"], inp["conv_b"], w.dilation, w.eps,
                                             gelu_tanh=tanh),
        w.B, TOL["f32"], chunk=16)
    log("  every element: %s" % stats["lnconv"])
    assert stats["lnconv"].n == w.B * w.C * w.L and stats["lnconv"].max <= TOL["f32"]
