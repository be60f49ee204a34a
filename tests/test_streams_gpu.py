"""Every entry point except the no-allocation one keeps no state between calls
(scratch memory comes from the caller), so calls enqueued on different streams
at once, which the GPU may run overlapped, must give bitwise the outputs of the
same calls made one at a time.  Each call here has its own stream, output and
workspace; all of them are enqueued before any is waited for."""
import numpy as np
import pytest
import torch

from gemm_activation_groupnorm_amd import lgn
from gemm_activation_groupnorm_amd.inputs import make_inputs, make_lnconv_inputs, make_sgh_inputs
from gpu_helpers import DEV, log, to_device

pytestmark = pytest.mark.gpu


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _ws(nb):
    return torch.empty(max(1, nb // 4), dtype=torch.float32, device=DEV)


def _calls():
    """(name, out, call(stream)) for one call of each entry point."""
    calls = []
    M, K, N = 1024, 256, 2048
    for dtype in ("f32", "bf16"):
        d = to_device(make_inputs(M, K, N, 51, dtype), dtype)
        for G, name in ((32, "fused C64"), (2, "fused C1024")):
            args = (d["x"], d["W"], d["b_lin"], d["b_add"], d["gamma"], d["beta"], M, K, N, G, 1e-5)
            out = torch.empty((M, N), dtype=torch.float32, device=DEV)
            fn = lgn.lgn_forward_f32 if dtype == "f32" else lgn.lgn_forward_bf16
            calls.append(("%s %s" % (name, dtype), out,
                          lambda s, fn=fn, args=args, out=out: lgn.check(fn(*args, out, stream=s))))
        args = (d["x"], d["W"], d["b_lin"], d["b_add"], d["gamma"], d["beta"], M, K, N, 64, 1e-5)
        out = torch.empty((M, N), dtype=torch.float32, device=DEV)
        ws, nb = _ws(lgn.lgn_twopass_workspace_bytes(M, N)), lgn.lgn_twopass_workspace_bytes(M, N)
        fn = lgn.lgn_forward_twopass_f32 if dtype == "f32" else lgn.lgn_forward_twopass_bf16
        calls.append(("twopass %s" % dtype, out, lambda s, fn=fn, args=args, out=out, ws=ws, nb=nb:
                      lgn.check(fn(*args, out, ws, nb, stream=s))))
        args = (d["x"], d["W"], d["b_lin"], d["b_add"], d["gamma"], d["beta"], M, K, N, 1, 1e-5)
        out = torch.empty((M, N), dtype=torch.float32, device=DEV)
        nb = lgn.lgn_wide_workspace_bytes(M, N)
        ws = _ws(nb)
        fn = lgn.lgn_forward_wide_f32 if dtype == "f32" else lgn.lgn_forward_wide_bf16
        calls.append(("wide %s" % dtype, out, lambda s, fn=fn, args=args, out=out, ws=ws, nb=nb:
                      lgn.check(fn(*args, out, ws, nb, stream=s))))
        out = torch.empty((M,), dtype=torch.float32, device=DEV)
        nb = lgn.lgn_lse_workspace_bytes(M, N)
        ws = _ws(nb)
        fn = lgn.lgn_linear_lse_f32 if dtype == "f32" else lgn.lgn_linear_lse_bf16
        calls.append(("lse %s" % dtype, out, lambda s, fn=fn, d=d, out=out, ws=ws, nb=nb:
                      lgn.check(fn(d["x"], d["W"], d["b_lin"], M, K, N, out, ws, nb, stream=s))))
    Nb, C, S, G = 4, 16, 40000, 4
    t = {k: _dev(v) for k, v in make_sgh_inputs(Nb, C, S, 52).items()}
    out = torch.empty_like(t["y"])
    nb = lgn.lgn_sgh_workspace_bytes(Nb, C, S, G)
    ws = _ws(nb)
    calls.append(("spatial groupnorm", out, lambda s, t=t, out=out, ws=ws, nb=nb: lgn.check(
        lgn.lgn_swish_gn_hardswish_f32(t["y"], t["gamma"], t["beta"], Nb, C, S, G, 1e-5, out, ws,
                                       nb, stream=s))))
    B, Cc, L, dil = 4, 256, 1024, 4
    t2 = {k: _dev(v) for k, v in make_lnconv_inputs(B, Cc, L, 53).items()}
    out = torch.empty_like(t2["x"])
    nb = lgn.lgn_lnconv_workspace_bytes(B, Cc, L)
    ws = _ws(nb)
    calls.append(("conv block", out, lambda s, t=t2, out=out, ws=ws, nb=nb: lgn.check(
        lgn.lgn_ln_gelu_conv1d_f32(t["x"], t["ln_w"], t["ln_b"], t["conv_w"], t["conv_b"], B, Cc,
                                   L, dil, 1e-5, 0, out, ws, nb, stream=s))))
    return calls


def test_all_entry_points_at_once_on_separate_streams():
    calls = _calls()
    alone = []
    for name, out, call in calls:
        log("stream case %s: alone" % name)
        out.fill_(float("nan"))
        call(torch.cuda.current_stream())
        torch.cuda.synchronize()
        alone.append(out.clone())
        assert torch.isfinite(alone[-1]).all(), name
    for rep in range(3):
        log("stream case: all %d calls at once, repetition %d" % (len(calls), rep))
        for _, out, _ in calls:
            out.fill_(float("nan"))
        torch.cuda.synchronize()
        streams = [torch.cuda.Stream() for _ in calls]
        for (_, _, call), s in zip(calls, streams):
            call(s)
        torch.cuda.synchronize()
        for (name, out, _), want in zip(calls, alone):
            assert torch.equal(out, want), "%s: differs when run beside the others" % name
