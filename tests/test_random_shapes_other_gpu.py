"""GPU parity on seeded sweeps of random shapes for the entry points other
than the GroupNorm forward: the wide-group path (group widths a multiple of
256), the Linear -> logsumexp method, the spatial GroupNorm tail (single pass
and in place) and the conv block, each within its documented limits and
against the fp64 oracle on every element."""
import numpy as np
import pytest
import torch

import oracle
from gemm_activation_groupnorm_amd import lgn
from gemm_activation_groupnorm_amd.inputs import make_inputs, make_lnconv_inputs, make_sgh_inputs
from gpu_helpers import TOL, case, log, max_err, oracle_rows, to_device

pytestmark = pytest.mark.gpu


def _dev(inp):
    return {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in inp.items()}


def _ws(nb):
    return torch.empty(max(1, nb // 4), dtype=torch.float32, device="cuda")


def _draw(n, seed, pick):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        s = pick(rng)
        if s is not None:
            out.append(s)
    return out


def _wide(rng):
    G = int(rng.choice([1, 2, 3, 4, 6, 8]))
    C = 256 * int(rng.integers(1, 9))
    if G * C > 12288:
        return None
    return (int(rng.integers(1, 90)), int(rng.choice([0, 8, 24, 64, 96])), G * C, G)


def _lse(rng):
    return (int(rng.integers(1, 300)), int(rng.choice([0, 8, 16, 40, 64, 128, 200])),
            4 * int(rng.integers(1, 1200)))


def _sgh(rng):
    G = int(rng.choice([1, 2, 3, 4, 8]))
    C = G * int(rng.integers(1, 9))
    return (int(rng.integers(1, 4)), C, int(rng.integers(1, 40000)), G)


def _lnc(rng):
    return (int(rng.integers(1, 4)), 128 * int(rng.integers(1, 4)), 4 * int(rng.integers(1, 300)),
            int(rng.integers(1, 17)), bool(rng.integers(0, 2)))


WIDE = _draw(10, 11, _wide)
LSE = _draw(12, 12, _lse)
SGH = _draw(12, 13, _sgh)
LNC = _draw(10, 14, _lnc)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", WIDE, ids=lambda s: "M%d_K%d_N%d_G%d" % s)
def test_wide_random(shape, dtype):
    M, K, N, G = shape
    log("random wide M=%d K=%d N=%d G=%d %s" % (M, K, N, G, dtype))
    inp = case(M, K, N, G, 4000 + M + K + N, dtype)
    dev = to_device(inp, dtype)
    out = torch.empty((M, N), dtype=torch.float32, device="cuda")
    nb = lgn.lgn_wide_workspace_bytes(M, N)
    fn = lgn.lgn_forward_wide_f32 if dtype == "f32" else lgn.lgn_forward_wide_bf16
    lgn.check(fn(dev["x"], dev["W"], dev["b_lin"], dev["b_add"], dev["gamma"], dev["beta"], M, K,
                 N, G, 1e-5, out, _ws(nb), nb))
    torch.cuda.synchronize()
    assert max_err(out.cpu().numpy(), oracle_rows(inp, G, 1e-5)) <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", LSE, ids=lambda s: "M%d_K%d_N%d" % s)
def test_lse_random(shape, dtype):
    M, K, N = shape
    log("random lse M=%d K=%d N=%d %s" % (M, K, N, dtype))
    inp = make_inputs(M, K, N, 4100 + M + K + N, dtype)
    dev = to_device(inp, dtype)
    out = torch.empty(M, dtype=torch.float32, device="cuda")
    nb = lgn.lgn_lse_workspace_bytes(M, N)
    fn = lgn.lgn_linear_lse_f32 if dtype == "f32" else lgn.lgn_linear_lse_bf16
    lgn.check(fn(dev["x"], dev["W"], dev["b_lin"], M, K, N, out, _ws(nb), nb))
    torch.cuda.synchronize()
    ref = oracle.linear_lse_forward(inp["x"], inp["W"], inp["b_lin"])
    assert max_err(out.cpu().numpy(), ref) <= TOL[dtype]


@pytest.mark.parametrize("in_place", [False, True])
@pytest.mark.parametrize("shape", SGH, ids=lambda s: "Nb%d_C%d_S%d_G%d" % s)
def test_spatial_groupnorm_random(shape, in_place):
    Nb, C, S, G = shape
    log("random sgh Nb=%d C=%d S=%d G=%d in_place=%d" % (Nb, C, S, G, in_place))
    inp = make_sgh_inputs(Nb, C, S, 4200 + Nb + C + S + G)
    d = _dev(inp)
    out = d["y"] if in_place else torch.empty_like(d["y"])
    nb = lgn.lgn_sgh_workspace_bytes(Nb, C, S, G)
    lgn.check(lgn.lgn_swish_gn_hardswish_f32(d["y"], d["gamma"], d["beta"], Nb, C, S, G, 1e-5, out,
                                             _ws(nb), nb))
    torch.cuda.synchronize()
    ref = oracle.swish_gn_hardswish(inp["y"], inp["gamma"], inp["beta"], G, 1e-5)
    assert max_err(out.cpu().numpy(), ref) <= TOL["f32"]


@pytest.mark.parametrize("shape", LNC, ids=lambda s: "B%d_C%d_L%d_d%d_tanh%d" % s)
def test_conv_block_random(shape):
    B, C, L, dil, tanh = shape
    log("random conv B=%d C=%d L=%d d=%d tanh=%d" % shape)
    inp = make_lnconv_inputs(B, C, L, 4300 + B + C + L + dil)
    d = _dev(inp)
    out = torch.empty_like(d["x"])
    nb = lgn.lgn_lnconv_workspace_bytes(B, C, L)
    lgn.check(lgn.lgn_ln_gelu_conv1d_f32(d["x"], d["ln_w"], d["ln_b"], d["conv_w"], d["conv_b"],
                                         B, C, L, dil, 1e-5, tanh, out, _ws(nb), nb))
    torch.cuda.synchronize()
    ref = oracle.ln_gelu_conv1d(inp["x"], inp["ln_w"], inp["ln_b"], inp["conv_w"], inp["conv_b"],
                                dil, 1e-5, gelu_tanh=tanh)
    assert max_err(out.cpu().numpy(), ref) <= TOL["f32"]
