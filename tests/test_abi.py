"""The C ABI without a GPU: the library loads, exports every symbol that
include/lgn.h declares, and rejects bad arguments before any HIP call."""
import math
import os
import re

import pytest

from gemm_activation_groupnorm_amd import lgn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
A = 1 << 20          # a 16-byte aligned fake device address; never dereferenced
GOOD = dict(M=64, K=32, N=128, G=8, eps=1e-5)


def declared_symbols():
    text = open(os.path.join(ROOT, "include", "lgn.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lgn_[a-z0-9_]+)\s*\(", text)))


def test_header_and_binding_agree():
    assert declared_symbols() == sorted(lgn.EXPORTS)


@pytest.mark.parametrize("name", declared_symbols())
def test_library_exports_symbol(name):
    assert hasattr(lgn._lib, name)


def test_status_strings_and_version():
    for s in (lgn.LGN_OK, lgn.LGN_ERR_INVALID_ARG, lgn.LGN_ERR_UNSUPPORTED, lgn.LGN_ERR_HIP):
        assert lgn.lgn_status_string(s).startswith(
            ["LGN_OK", "LGN_ERR_INVALID_ARG", "LGN_ERR_UNSUPPORTED", "LGN_ERR_HIP"][s])
    assert lgn.lgn_status_string(99) == "unknown lgn_status"
    assert re.fullmatch(r"\d+\.\d+\.\d+", lgn.lgn_version())


def test_workspace_bytes():
    assert lgn.lgn_twopass_workspace_bytes(32768, 4096) == 32768 * 4096 * 4
    assert lgn.lgn_twopass_workspace_bytes(0, 16) == 0
    assert lgn.lgn_twopass_workspace_bytes(-1, 16) == 0


def test_fused_supported():
    F32, BF16 = lgn.DTYPE_F32, lgn.DTYPE_BF16
    assert lgn.lgn_fused_supported(F32, 32768, 1024, 4096, 64)
    assert lgn.lgn_fused_supported(BF16, 32768, 1024, 4096, 64)
    assert lgn.lgn_fused_supported(F32, 16384, 2048, 8192, 8)
    assert lgn.lgn_fused_supported(F32, 64, 32, 128, 8)
    for cg in (8, 16, 32, 64, 128, 256, 512, 1024):
        assert lgn.lgn_fused_supported(F32, 5, 8, 4 * cg, 4)
    assert not lgn.lgn_fused_supported(F32, 64, 32, 96, 8)       # 12 channels per group
    assert not lgn.lgn_fused_supported(F32, 64, 32, 2048, 1)     # 2048 per group
    assert not lgn.lgn_fused_supported(BF16, 64, 12, 128, 8)     # K % 8 != 0 for bf16
    assert lgn.lgn_fused_supported(F32, 64, 12, 128, 8)          # K % 4 == 0 is fine for fp32
    assert not lgn.lgn_fused_supported(F32, 64, 32, 128, 3)      # N % G != 0
    assert not lgn.lgn_fused_supported(2, 64, 32, 128, 8)        # unknown dtype


def _call(fn, **kw):
    a = dict(x=A, W=A, b_lin=A, b_add=A, gamma=A, beta=A, out=A, **GOOD)
    a.update(kw)
    args = [a["x"], a["W"], a["b_lin"], a["b_add"], a["gamma"], a["beta"], a["M"], a["K"], a["N"],
            a["G"], a["eps"], a["out"]]
    if "twopass" in fn.__name__:
        args += [a.get("ws", A), a.get("ws_bytes", 1 << 40)]
    return fn(*args, stream=0)


FNS = [lgn.lgn_forward_f32, lgn.lgn_forward_bf16, lgn.lgn_forward_twopass_f32,
       lgn.lgn_forward_twopass_bf16]
INVALID = [
    dict(M=-1), dict(K=-1), dict(N=0), dict(G=0), dict(G=-2), dict(N=128, G=3),
    dict(eps=0.0), dict(eps=-1e-5), dict(eps=math.nan), dict(eps=math.inf),
    dict(b_lin=None), dict(b_add=None), dict(gamma=None), dict(beta=None), dict(out=None),
    dict(x=None), dict(W=None),
]
UNSUPPORTED = [dict(K=6), dict(N=126, G=2), dict(x=A + 4), dict(W=A + 8), dict(out=A + 4),
               dict(gamma=A + 2)]


@pytest.mark.parametrize("fn", FNS, ids=lambda f: f.__name__)
@pytest.mark.parametrize("bad", INVALID, ids=lambda d: ",".join("%s=%s" % i for i in d.items()))
def test_invalid_arguments(fn, bad):
    assert _call(fn, **bad) == lgn.LGN_ERR_INVALID_ARG


@pytest.mark.parametrize("fn", FNS, ids=lambda f: f.__name__)
@pytest.mark.parametrize("bad", UNSUPPORTED, ids=lambda d: ",".join("%s=%s" % i for i in d.items()))
def test_unsupported_shapes(fn, bad):
    assert _call(fn, **bad) == lgn.LGN_ERR_UNSUPPORTED


@pytest.mark.parametrize("fn", [lgn.lgn_forward_f32, lgn.lgn_forward_bf16], ids=lambda f: f.__name__)
def test_fused_rejects_uncovered_group_width(fn):
    assert _call(fn, N=96, G=8) == lgn.LGN_ERR_UNSUPPORTED


@pytest.mark.parametrize("fn", [lgn.lgn_forward_twopass_f32, lgn.lgn_forward_twopass_bf16],
                         ids=lambda f: f.__name__)
def test_twopass_workspace_checks(fn):
    need = lgn.lgn_twopass_workspace_bytes(GOOD["M"], GOOD["N"])
    assert _call(fn, ws=None) == lgn.LGN_ERR_INVALID_ARG
    assert _call(fn, ws_bytes=need - 1) == lgn.LGN_ERR_INVALID_ARG
    assert _call(fn, ws=A + 4, ws_bytes=need) == lgn.LGN_ERR_UNSUPPORTED


@pytest.mark.parametrize("fn", FNS, ids=lambda f: f.__name__)
def test_empty_batch_is_a_no_op(fn):
    # M == 0 returns before any HIP call, with null data pointers
    assert _call(fn, M=0, x=None, out=None, ws=None, ws_bytes=0) == lgn.LGN_OK


def test_binding_rejects_non_contiguous_tensor():
    import torch
    t = torch.zeros(8, 8).t()
    with pytest.raises(ValueError):
        lgn._ptr(t, "f32")
    with pytest.raises(ValueError):
        lgn._ptr(torch.zeros(4, dtype=torch.float64), "f32")


# ---- Linear -> logsumexp -> LeakyReLU x2 -> GELU x2 ----

LSE_FNS = [lgn.lgn_linear_lse_f32, lgn.lgn_linear_lse_bf16]
LSE_GOOD = dict(M=64, K=32, N=300)


def _call_lse(fn, **kw):
    a = dict(x=A, W=A, b=A, out=A, ws=A, ws_bytes=1 << 40, **LSE_GOOD)
    a.update(kw)
    return fn(a["x"], a["W"], a["b"], a["M"], a["K"], a["N"], a["out"], a["ws"], a["ws_bytes"],
              stream=0)


def test_lse_workspace_bytes():
    # one (max, sum) float pair per row and per 256-channel tile
    assert lgn.lgn_lse_workspace_bytes(1024, 8192) == 1024 * 32 * 8
    assert lgn.lgn_lse_workspace_bytes(3, 257) == 3 * 2 * 8
    assert lgn.lgn_lse_workspace_bytes(3, 256) == 3 * 1 * 8
    assert lgn.lgn_lse_workspace_bytes(0, 16) == 0
    assert lgn.lgn_lse_workspace_bytes(5, 0) == 0


LSE_INVALID = [dict(M=-1), dict(K=-1), dict(N=0), dict(b=None), dict(out=None), dict(ws=None),
               dict(x=None), dict(W=None), dict(ws_bytes=lgn.lgn_lse_workspace_bytes(64, 300) - 1)]
LSE_UNSUPPORTED = [dict(K=6), dict(N=302), dict(x=A + 4), dict(W=A + 8), dict(b=A + 2),
                   dict(out=A + 2), dict(ws=A + 4)]


@pytest.mark.parametrize("fn", LSE_FNS, ids=lambda f: f.__name__)
@pytest.mark.parametrize("bad", LSE_INVALID, ids=lambda d: ",".join("%s=%s" % i for i in d.items()))
def test_lse_invalid_arguments(fn, bad):
    assert _call_lse(fn, **bad) == lgn.LGN_ERR_INVALID_ARG


@pytest.mark.parametrize("fn", LSE_FNS, ids=lambda f: f.__name__)
@pytest.mark.parametrize("bad", LSE_UNSUPPORTED,
                         ids=lambda d: ",".join("%s=%s" % i for i in d.items()))
def test_lse_unsupported_shapes(fn, bad):
    assert _call_lse(fn, **bad) == lgn.LGN_ERR_UNSUPPORTED


@pytest.mark.parametrize("fn", LSE_FNS, ids=lambda f: f.__name__)
def test_lse_empty_batch_is_a_no_op(fn):
    assert _call_lse(fn, M=0, x=None, out=None, ws=None, ws_bytes=0) == lgn.LGN_OK


# ---- Swish -> spatial GroupNorm -> HardSwish ----

SGH_GOOD = dict(Nb=2, C=16, S=123039, G=4, eps=1e-5)


def _call_sgh(**kw):
    a = dict(y=A, gamma=A, beta=A, out=A, ws=A, ws_bytes=1 << 40, **SGH_GOOD)
    a.update(kw)
    return lgn.lgn_swish_gn_hardswish_f32(a["y"], a["gamma"], a["beta"], a["Nb"], a["C"], a["S"],
                                          a["G"], a["eps"], a["out"], a["ws"], a["ws_bytes"],
                                          stream=0)


def test_sgh_workspace_bytes():
    # one (mean, M2) float pair per 16384-element chunk of each group
    parts = -(-4 * 123039 // 16384)
    assert lgn.lgn_sgh_workspace_bytes(128, 16, 123039, 4) == 128 * 4 * parts * 8
    assert lgn.lgn_sgh_workspace_bytes(1, 4, 1, 4) == 4 * 1 * 8
    assert lgn.lgn_sgh_workspace_bytes(0, 4, 10, 2) == 0
    assert lgn.lgn_sgh_workspace_bytes(2, 6, 10, 4) == 0          # C % G != 0
    assert lgn.lgn_sgh_workspace_bytes(1, 2, 1 << 31, 1) == 0     # group past 2^31 - 1


SGH_INVALID = [dict(Nb=-1), dict(C=0), dict(S=0), dict(G=0), dict(C=16, G=3), dict(eps=0.0),
               dict(eps=math.nan), dict(y=None), dict(gamma=None), dict(beta=None),
               dict(out=None), dict(ws=None), dict(ws_bytes=lgn.lgn_sgh_workspace_bytes(
                   2, 16, 123039, 4) - 1)]
SGH_UNSUPPORTED = [dict(y=A + 4), dict(out=A + 8), dict(gamma=A + 2), dict(ws=A + 4),
                   dict(C=4, G=1, S=1 << 30), dict(C=16384, G=1, S=4)]


@pytest.mark.parametrize("bad", SGH_INVALID, ids=lambda d: ",".join("%s=%s" % i for i in d.items()))
def test_sgh_invalid_arguments(bad):
    assert _call_sgh(**bad) == lgn.LGN_ERR_INVALID_ARG


@pytest.mark.parametrize("bad", SGH_UNSUPPORTED,
                         ids=lambda d: ",".join("%s=%s" % i for i in d.items()))
def test_sgh_unsupported(bad):
    assert _call_sgh(**bad) == lgn.LGN_ERR_UNSUPPORTED


def test_sgh_empty_batch_is_a_no_op():
    assert _call_sgh(Nb=0, y=None, out=None, ws=None, ws_bytes=0) == lgn.LGN_OK


# ---- groups wider than one tile ----

WIDE_FNS = [lgn.lgn_forward_wide_f32, lgn.lgn_forward_wide_bf16]


def _call_wide(fn, **kw):
    a = dict(x=A, W=A, b_lin=A, b_add=A, gamma=A, beta=A, out=A, ws=A, ws_bytes=1 << 40,
             M=64, K=32, N=1024, G=2, eps=1e-5)
    a.update(kw)
    return fn(a["x"], a["W"], a["b_lin"], a["b_add"], a["gamma"], a["beta"], a["M"], a["K"],
              a["N"], a["G"], a["eps"], a["out"], a["ws"], a["ws_bytes"], stream=0)


def test_wide_workspace_bytes():
    assert lgn.lgn_wide_workspace_bytes(16384, 8192) == 16384 * 128 * 8
    assert lgn.lgn_wide_workspace_bytes(3, 512) == 3 * 8 * 8
    assert lgn.lgn_wide_workspace_bytes(0, 512) == 0


@pytest.mark.parametrize("fn", WIDE_FNS, ids=lambda f: f.__name__)
@pytest.mark.parametrize("bad", [dict(M=-1), dict(N=1024, G=3), dict(eps=0.0), dict(ws=None),
                                 dict(ws_bytes=64 * 16 * 8 - 1), dict(gamma=None), dict(x=None)],
                         ids=lambda d: ",".join("%s=%s" % i for i in d.items()))
def test_wide_invalid_arguments(fn, bad):
    assert _call_wide(fn, **bad) == lgn.LGN_ERR_INVALID_ARG


@pytest.mark.parametrize("fn", WIDE_FNS, ids=lambda f: f.__name__)
@pytest.mark.parametrize("bad", [dict(N=1024, G=8), dict(N=768, G=2), dict(gamma=A + 4),
                                 dict(beta=A + 8), dict(ws=A + 4), dict(K=6), dict(x=A + 4)],
                         ids=lambda d: ",".join("%s=%s" % i for i in d.items()))
def test_wide_unsupported(fn, bad):
    assert _call_wide(fn, **bad) == lgn.LGN_ERR_UNSUPPORTED


@pytest.mark.parametrize("fn", WIDE_FNS, ids=lambda f: f.__name__)
def test_wide_empty_batch_is_a_no_op(fn):
    assert _call_wide(fn, M=0, x=None, out=None, ws=None, ws_bytes=0) == lgn.LGN_OK


# ---- LayerNorm -> GELU -> dilated Conv1d -> + input ----

LNC_GOOD = dict(B=2, C=256, L=4096, d=4, eps=1e-5, tanh=0)


def _call_lnc(**kw):
    a = dict(x=A, ln_w=A, ln_b=A, conv_w=A, conv_b=A, out=A + 4096, ws=A, ws_bytes=1 << 40,
             **LNC_GOOD)
    a.update(kw)
    return lgn.lgn_ln_gelu_conv1d_f32(a["x"], a["ln_w"], a["ln_b"], a["conv_w"], a["conv_b"],
                                      a["B"], a["C"], a["L"], a["d"], a["eps"], a["tanh"],
                                      a["out"], a["ws"], a["ws_bytes"], stream=0)


def test_lnconv_workspace_bytes():
    # packed weights 3*C*C floats (256-byte padded), then one (mean, M2) pair
    # per 16384-value chunk of each sample
    assert lgn.lgn_lnconv_workspace_bytes(32, 256, 4096) == 3 * 256 * 256 * 4 + 32 * 64 * 8
    assert lgn.lgn_lnconv_workspace_bytes(1, 128, 4) == 3 * 128 * 128 * 4 + 1 * 1 * 8
    assert lgn.lgn_lnconv_workspace_bytes(0, 128, 4) == 0


LNC_INVALID = [dict(B=-1), dict(C=0), dict(L=0), dict(d=0), dict(eps=0.0), dict(eps=math.inf),
               dict(x=None), dict(ln_w=None), dict(ln_b=None), dict(conv_w=None),
               dict(conv_b=None), dict(out=None), dict(ws=None), dict(out=A),
               dict(ws_bytes=lgn.lgn_lnconv_workspace_bytes(2, 256, 4096) - 1)]
LNC_UNSUPPORTED = [dict(C=192), dict(L=4094), dict(d=17), dict(x=A + 4), dict(ln_w=A + 8),
                   dict(ln_b=A + 4), dict(out=A + 4100), dict(ws=A + 8), dict(conv_w=A + 2),
                   dict(C=1 << 16, L=1 << 16), dict(C=1 << 14, L=1 << 15),
                   dict(C=8320, L=4)]


@pytest.mark.parametrize("bad", LNC_INVALID, ids=lambda d: ",".join("%s=%s" % i for i in d.items()))
def test_lnconv_invalid_arguments(bad):
    assert _call_lnc(**bad) == lgn.LGN_ERR_INVALID_ARG


@pytest.mark.parametrize("bad", LNC_UNSUPPORTED,
                         ids=lambda d: ",".join("%s=%s" % i for i in d.items()))
def test_lnconv_unsupported(bad):
    assert _call_lnc(**bad) == lgn.LGN_ERR_UNSUPPORTED


def test_lnconv_empty_batch_is_a_no_op():
    assert _call_lnc(B=0, x=None, out=None, ws=None, ws_bytes=0) == lgn.LGN_OK


# ---- the binding's own checks: device, size (before any C call) ----

def _host_args(M=6, K=8, N=16, short=None):
    """CPU tensors of the forward's sizes; `short` names one to make 1 element short."""
    import torch
    sizes = dict(x=M * K, W=N * K, b_lin=N, b_add=N, gamma=N, beta=N, out=M * N)
    if short:
        sizes[short] -= 1
    return {k: torch.zeros(v, dtype=torch.float32) for k, v in sizes.items()}


@pytest.mark.parametrize("short", [None, "x", "W", "b_lin", "b_add", "gamma", "beta", "out"])
@pytest.mark.parametrize("fn", [lgn.lgn_forward_f32, lgn.lgn_forward_twopass_f32,
                                lgn.lgn_forward_wide_f32], ids=lambda f: f.__name__)
def test_binding_checks_sizes_then_device(fn, short):
    import torch
    M, K, N, G = 6, 8, 16, 2
    a = _host_args(M, K, N, short)
    args = [a["x"], a["W"], a["b_lin"], a["b_add"], a["gamma"], a["beta"], M, K, N, G, 1e-5,
            a["out"]]
    if fn is not lgn.lgn_forward_f32:
        args += [torch.zeros(M * N), M * N * 4]
    # an undersized tensor is named before anything else; a right-sized host
    # tensor is refused because it is not device memory
    with pytest.raises(ValueError, match="holds" if short else "on the GPU"):
        fn(*args, stream=0)


def test_binding_checks_workspace_bytes():
    import torch
    M, K, N, G = 6, 8, 16, 2
    a = _host_args(M, K, N)
    with pytest.raises(ValueError, match="holds 16 bytes, the call addresses 384"):
        lgn.lgn_forward_twopass_f32(a["x"], a["W"], a["b_lin"], a["b_add"], a["gamma"], a["beta"],
                                    M, K, N, G, 1e-5, a["out"], torch.zeros(4), M * N * 4,
                                    stream=0)


def test_binding_checks_other_entry_points():
    import torch
    z = lambda n: torch.zeros(n)
    with pytest.raises(ValueError, match="holds"):
        lgn.lgn_linear_lse_f32(z(6 * 8), z(16 * 8), z(16), 6, 8, 16, z(5), z(100), 400, stream=0)
    with pytest.raises(ValueError, match="holds"):
        lgn.lgn_swish_gn_hardswish_f32(z(2 * 4 * 9 - 1), z(4), z(4), 2, 4, 9, 2, 1e-5, z(72),
                                       z(100), 400, stream=0)
    with pytest.raises(ValueError, match="holds"):
        lgn.lgn_ln_gelu_conv1d_f32(z(2 * 128 * 8), z(128 * 8), z(128 * 8), z(128 * 128 * 3 - 1),
                                   z(128), 2, 128, 8, 1, 1e-5, 0, z(2 * 128 * 8), z(10), 40,
                                   stream=0)
    with pytest.raises(ValueError, match="on the GPU"):
        lgn.lgn_linear_lse_f32(z(6 * 8), z(16 * 8), z(16), 6, 8, 16, z(6), z(100), 400, stream=0)


# ---- failure paths: wrong device architecture, failed launch ----

HIP_ERROR_LAUNCH_FAILURE = 719   # hipErrorLaunchFailure


@pytest.fixture
def arch_override():
    yield lgn.lgn_testing_set_arch
    lgn.lgn_testing_set_arch(None)
    lgn.lgn_testing_fail_launches(0, 0)


def _all_entry_points():
    """(name, call) for every compute entry point, with valid shapes and fake addresses."""
    calls = [(f.__name__, (lambda f=f: _call(f))) for f in FNS]
    calls += [(f.__name__, (lambda f=f: _call_lse(f))) for f in LSE_FNS]
    calls += [(f.__name__, (lambda f=f: f(A, A, A, A, A, A, 64, 32, 512, 2, 1e-5, A, A, 1 << 40,
                                           stream=0)))
              for f in (lgn.lgn_forward_wide_f32, lgn.lgn_forward_wide_bf16)]
    calls.append(("lgn_swish_gn_hardswish_f32",
                  lambda: lgn.lgn_swish_gn_hardswish_f32(A, A, A, 2, 16, 1000, 4, 1e-5, A, A,
                                                         1 << 40, stream=0)))
    calls.append(("lgn_ln_gelu_conv1d_f32",
                  lambda: lgn.lgn_ln_gelu_conv1d_f32(A, A, A, A, A, 2, 128, 64, 4, 1e-5, 0,
                                                     A + 1024, A, 1 << 40, stream=0)))
    return calls


@pytest.mark.parametrize("name,call", _all_entry_points(), ids=lambda v: v if isinstance(v, str) else "")
def test_other_device_architecture_is_unsupported(arch_override, name, call):
    # the device check compares the injected name and makes no HIP call
    arch_override("gfx942")
    assert call() == lgn.LGN_ERR_UNSUPPORTED
    arch_override("gfx90a:sramecc+:xnack-")
    assert call() == lgn.LGN_ERR_UNSUPPORTED


@pytest.mark.parametrize("name,call", _all_entry_points(), ids=lambda v: v if isinstance(v, str) else "")
def test_failed_launch_maps_to_hip_error(arch_override, name, call):
    # the device check passes (injected gfx950) and the first kernel launch
    # reports hipErrorLaunchFailure instead of launching: nothing reaches a GPU
    arch_override("gfx950:sramecc+:xnack-")
    lgn.lgn_testing_fail_launches(HIP_ERROR_LAUNCH_FAILURE, 1000)
    assert call() == lgn.LGN_ERR_HIP
    text = lgn.lgn_last_hip_error_string()
    assert text != "no HIP error" and text
    with pytest.raises(lgn.LgnError, match="LGN_ERR_HIP"):
        lgn.check(lgn.LGN_ERR_HIP)


def test_failure_injection_counts_down(arch_override):
    arch_override("gfx950")
    lgn.lgn_testing_fail_launches(HIP_ERROR_LAUNCH_FAILURE, 2)
    assert _call(lgn.lgn_forward_f32) == lgn.LGN_ERR_HIP
    assert _call(lgn.lgn_forward_bf16) == lgn.LGN_ERR_HIP
    lgn.lgn_testing_fail_launches(0, 0)
    # cleared: an argument error is still reported before any launch
    assert _call(lgn.lgn_forward_f32, M=-1) == lgn.LGN_ERR_INVALID_ARG


# ---- the entry point that allocates nothing ----

def _call_noalloc(**kw):
    a = dict(x=A, W=A, b_lin=A, b_add=A, gamma=A, beta=A, out=A, M=64, K=32, N=512, G=2,
             eps=1e-5)
    a.update(kw)
    return lgn.lgn_forward_wide_f32_noalloc(a["x"], a["W"], a["b_lin"], a["b_add"], a["gamma"],
                                            a["beta"], a["M"], a["K"], a["N"], a["G"], a["eps"],
                                            a["out"], stream=0)


def test_noalloc_limit_matches_header():
    text = open(os.path.join(ROOT, "include", "lgn.h")).read()
    m = re.search(r"#define LGN_WIDE_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == lgn.WIDE_NOALLOC_SCRATCH_BYTES


def test_noalloc_rejects_calls_beyond_its_scratch():
    # 8 bytes per row per 64 channels: 32768 x 16384 needs 64 MiB > 32 MiB
    need = lgn.lgn_wide_workspace_bytes(32768, 16384)
    assert need > lgn.WIDE_NOALLOC_SCRATCH_BYTES
    assert _call_noalloc(M=32768, N=16384, G=16) == lgn.LGN_ERR_TOO_LARGE
    # the largest row count that fits at N = 16384
    fit = lgn.WIDE_NOALLOC_SCRATCH_BYTES // (16384 // 64 * 8)
    assert lgn.lgn_wide_workspace_bytes(fit, 16384) == lgn.WIDE_NOALLOC_SCRATCH_BYTES
    assert _call_noalloc(M=fit + 1, N=16384, G=16) == lgn.LGN_ERR_TOO_LARGE
    assert lgn.lgn_status_string(lgn.LGN_ERR_TOO_LARGE).startswith("LGN_ERR_TOO_LARGE")


@pytest.mark.parametrize("bad", INVALID, ids=lambda d: ",".join("%s=%s" % i for i in d.items()))
def test_noalloc_invalid_arguments(bad):
    kw = dict(bad)
    if kw.get("N") == 128 and kw.get("G") == 3:
        kw = dict(N=512, G=3)
    assert _call_noalloc(**kw) == lgn.LGN_ERR_INVALID_ARG


def test_noalloc_unsupported_and_empty(arch_override):
    assert _call_noalloc(N=384, G=3) == lgn.LGN_ERR_UNSUPPORTED       # 128-channel groups
    assert _call_noalloc(K=6) == lgn.LGN_ERR_UNSUPPORTED
    assert _call_noalloc(gamma=A + 4) == lgn.LGN_ERR_UNSUPPORTED
    assert _call_noalloc(M=0, x=None, out=None) == lgn.LGN_OK
    arch_override("gfx942")
    assert _call_noalloc() == lgn.LGN_ERR_UNSUPPORTED


def test_header_compiles_as_c_and_links(tmp_path):
    """include/lgn.h from a plain C99 program linked against liblgn.so: the
    host helpers and argument checks answer without a GPU."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no gcc")
    pkg = os.path.dirname(lgn.LIB_PATH)
    exe = str(tmp_path / "c_abi_check")
    cmd = [gcc, "-std=c99", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
           os.path.join(ROOT, "tests", "c_abi_check.c"), "-L", pkg, "-llgn",
           "-Wl,-rpath," + pkg, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr


def test_header_compiles_as_cxx_and_links(tmp_path):
    """The same C program built as C++17 (the header's extern "C" block), linked
    against liblgn.so: the names resolve without C++ mangling."""
    import shutil
    import subprocess
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("no g++")
    pkg = os.path.dirname(lgn.LIB_PATH)
    exe = str(tmp_path / "cxx_abi_check")
    cmd = [gxx, "-x", "c++", "-std=c++17", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
           os.path.join(ROOT, "tests", "c_abi_check.c"), "-x", "none", "-L", pkg, "-llgn",
           "-Wl,-rpath," + pkg, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
