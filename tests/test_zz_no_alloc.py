"""The entry point that allocates nothing (lgn_forward_wide_f32_noalloc),
through the C ABI, against the workspace entry point lgn_forward_wide_f32 on
the same inputs.  Both run the same kernels, so the outputs must be bitwise
equal; the first call fills the library's scratch to its limit and the
second, smaller call must not see anything the first one left there."""
import numpy as np
import pytest
import torch

from gemm_activation_groupnorm_amd import lgn
from gpu_helpers import TOL, case, log, max_err, oracle_rows, to_device

pytestmark = pytest.mark.gpu


def _wide(dev, M, K, N, G, eps=1e-5):
    out = torch.empty((M, N), dtype=torch.float32, device="cuda")
    nb = lgn.lgn_wide_workspace_bytes(M, N)
    ws = torch.empty(max(1, nb // 4), dtype=torch.float32, device="cuda")
    lgn.check(lgn.lgn_forward_wide_f32(dev["x"], dev["W"], dev["b_lin"], dev["b_add"],
                                       dev["gamma"], dev["beta"], M, K, N, G, eps, out, ws, nb))
    return out


def _noalloc(dev, M, K, N, G, eps=1e-5):
    out = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    lgn.check(lgn.lgn_forward_wide_f32_noalloc(dev["x"], dev["W"], dev["b_lin"], dev["b_add"],
                                               dev["gamma"], dev["beta"], M, K, N, G, eps, out))
    return out


# the first call needs exactly the whole scratch (16384 rows x 16384 channels:
# 8 bytes per row per 64 channels = 32 MiB); the second is smaller, with
# groups of another width
CALLS = [(16384, 64, 16384, 4, 11), (777, 128, 2048, 1, 12)]


def test_noalloc_two_calls_match_the_workspace_entry_point():
    assert lgn.lgn_wide_workspace_bytes(CALLS[0][0], CALLS[0][2]) == \
        lgn.WIDE_NOALLOC_SCRATCH_BYTES
    for M, K, N, G, seed in CALLS:
        log("no-alloc case M=%d K=%d N=%d G=%d" % (M, K, N, G))
        inp = case(M, K, N, G, seed)
        dev = to_device(inp, "f32")
        got = _noalloc(dev, M, K, N, G)
        ref = _wide(dev, M, K, N, G)
        torch.cuda.synchronize()
        assert bool(torch.isfinite(got).all()), "elements left unwritten"
        assert torch.equal(got, ref), "differs from lgn_forward_wide_f32"
        rows = np.unique(np.array([0, 1, M // 2, M - 2, M - 1]))
        err = max_err(got[torch.from_numpy(rows).cuda()].cpu().numpy(),
                      oracle_rows(inp, G, 1e-5, rows))
        log("  bitwise equal to the workspace entry point; max abs err vs oracle %.3e" % err)
        assert err <= TOL["f32"]
        del got, ref, dev
        torch.cuda.empty_cache()
