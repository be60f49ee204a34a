"""ctypes binding of liblgn.so, entry point for entry point (include/lgn.h).

Argument marshalling only: every array argument may be a torch tensor on the
GPU (dense, of the dtype the C signature names) or a raw device address
(int); ``stream`` may be a ``torch.cuda.Stream``, a raw ``hipStream_t``
(int) or ``None`` for torch's current stream.  Each call returns the C
status code unchanged; ``check(status)`` turns a non-zero code into
``LgnError``.  Nothing here computes: the forward runs in liblgn.so's HIP
kernels, and importing this module fails loudly if the library is missing.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "liblgn.so")

LGN_OK = 0
LGN_ERR_INVALID_ARG = 1
LGN_ERR_UNSUPPORTED = 2
LGN_ERR_HIP = 3
LGN_ERR_TOO_LARGE = 4
# scratch held by the library for lgn_forward_wide_f32_noalloc (include/lgn.h)
WIDE_NOALLOC_SCRATCH_BYTES = 32 << 20

DTYPE_F32 = 0
DTYPE_BF16 = 1

# Every symbol include/lgn.h declares.
EXPORTS = (
    "lgn_forward_f32",
    "lgn_forward_bf16",
    "lgn_fused_supported",
    "lgn_twopass_workspace_bytes",
    "lgn_forward_twopass_f32",
    "lgn_forward_twopass_bf16",
    "lgn_wide_workspace_bytes",
    "lgn_forward_wide_f32",
    "lgn_forward_wide_bf16",
    "lgn_forward_wide_f32_noalloc",
    "lgn_lse_workspace_bytes",
    "lgn_linear_lse_f32",
    "lgn_linear_lse_bf16",
    "lgn_sgh_workspace_bytes",
    "lgn_swish_gn_hardswish_f32",
    "lgn_lnconv_workspace_bytes",
    "lgn_ln_gelu_conv1d_f32",
    "lgn_status_string",
    "lgn_version",
    "lgn_last_hip_error_string",
    "lgn_testing_set_arch",
    "lgn_testing_fail_launches",
    "lgn_testing_set_sgh_spin_limit",
)


class LgnError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        msg = "lgn status %d: %s" % (status, lgn_status_string(status))
        if status == LGN_ERR_HIP:
            msg += " (%s)" % lgn_last_hip_error_string()
        super().__init__(msg)


def _load():
    # PyTorch ships its own HIP runtime under the same SONAME
    # (libamdhip64.so.7).  Loading torch first makes liblgn.so bind to that
    # already-loaded runtime, so the process has ONE HIP runtime and torch's
    # streams and allocations are valid handles for the library.  Loaded the
    # other way round, two runtimes would coexist and the second one may not
    # see the device.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(LIB_PATH):
        raise ImportError("liblgn.so not built at %s; run "
                          "`python -m gemm_activation_groupnorm_amd.build`" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    fwd = [vp, vp, vp, vp, vp, vp, i, i, i, i, f, vp, vp]
    two = [vp, vp, vp, vp, vp, vp, i, i, i, i, f, vp, vp, sz, vp]
    lse = [vp, vp, vp, i, i, i, vp, vp, sz, vp]
    for name, args, res in (
        ("lgn_forward_f32", fwd, i),
        ("lgn_forward_bf16", fwd, i),
        ("lgn_fused_supported", [i, i, i, i, i], i),
        ("lgn_twopass_workspace_bytes", [i, i], sz),
        ("lgn_forward_twopass_f32", two, i),
        ("lgn_forward_twopass_bf16", two, i),
        ("lgn_wide_workspace_bytes", [i, i], sz),
        ("lgn_forward_wide_f32", two, i),
        ("lgn_forward_wide_bf16", two, i),
        ("lgn_forward_wide_f32_noalloc", fwd, i),
        ("lgn_lse_workspace_bytes", [i, i], sz),
        ("lgn_linear_lse_f32", lse, i),
        ("lgn_linear_lse_bf16", lse, i),
        ("lgn_sgh_workspace_bytes", [i, i, ctypes.c_longlong, i], sz),
        ("lgn_swish_gn_hardswish_f32",
         [vp, vp, vp, i, i, ctypes.c_longlong, i, f, vp, vp, sz, vp], i),
        ("lgn_lnconv_workspace_bytes", [i, i, i], sz),
        ("lgn_ln_gelu_conv1d_f32", [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, vp, sz, vp], i),
        ("lgn_status_string", [i], ctypes.c_char_p),
        ("lgn_version", [], ctypes.c_char_p),
        ("lgn_last_hip_error_string", [], ctypes.c_char_p),
        ("lgn_testing_set_arch", [ctypes.c_char_p], None),
        ("lgn_testing_fail_launches", [i, i], None),
        ("lgn_testing_set_sgh_spin_limit", [i], None),
    ):
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


_lib = _load()


def _check(a, want: Optional[str], need: int) -> None:
    """Checks one array argument: a tensor must be dense, of dtype ``want``
    ("f32", "bf16", or None for a workspace of any dtype) and hold at least
    ``need`` elements (bytes when ``want`` is None), so that the kernels never
    address past its end.  An int is a raw device address and is not checked."""
    if a is None or isinstance(a, int):
        return
    import torch
    if not isinstance(a, torch.Tensor):
        raise TypeError("expected a torch.Tensor or an int address, got %r" % type(a))
    if not a.is_contiguous():
        raise ValueError("tensor arguments must be contiguous (dense row-major)")
    if want == "f32" and a.dtype != torch.float32:
        raise ValueError("expected float32, got %s" % a.dtype)
    if want == "bf16" and a.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise ValueError("expected bfloat16 (or 16-bit raw bits), got %s" % a.dtype)
    have = a.numel() * a.element_size() if want is None else a.numel()
    if have < need:
        raise ValueError("tensor holds %d %s, the call addresses %d"
                         % (have, "bytes" if want is None else "elements", need))


def _ptrs(*specs):
    """Addresses of the array arguments, given as (array, want, need) triples.

    Every array is checked (see _check) before any is converted; then every
    tensor must be GPU memory, since the kernels dereference the address."""
    for a, want, need in specs:
        _check(a, want, need)
    out = []
    for a, _, _ in specs:
        if a is None or isinstance(a, int):
            out.append(a)
            continue
        if not a.is_cuda:
            raise ValueError("tensor arguments must be on the GPU, got device %s" % a.device)
        out.append(a.data_ptr() if a.numel() > 0 else None)
    return out


def _ptr(a, want: Optional[str], need: int = 0) -> Optional[int]:
    """Address of one array argument (see _ptrs)."""
    return _ptrs((a, want, need))[0]


def _n(*dims) -> int:
    """Element count of an array of these dimensions (0 if any is negative)."""
    r = 1
    for d in dims:
        if d < 0:
            return 0
        r *= d
    return r


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _fwd(dt, x, W, b_lin, b_add, gamma, beta, M, K, N, out, *workspace):
    """Checked pointer arguments of the GroupNorm forward entry points:
    x, W, b_lin, b_add, gamma, beta, out, then the workspace if one is given
    as (workspace, workspace_bytes)."""
    specs = [(x, dt, _n(M, K)), (W, dt, _n(N, K)), (b_lin, "f32", _n(N)), (b_add, "f32", _n(N)),
             (gamma, "f32", _n(N)), (beta, "f32", _n(N)), (out, "f32", _n(M, N))]
    if workspace:
        specs.append((workspace[0], None, workspace[1]))
    return _ptrs(*specs)


def lgn_forward_f32(x, W, b_lin, b_add, gamma, beta, M, K, N, G, eps, out, stream=None) -> int:
    px, pW, pbl, pba, pg, pb, po = _fwd("f32", x, W, b_lin, b_add, gamma, beta, M, K, N, out)
    return _lib.lgn_forward_f32(px, pW, pbl, pba, pg, pb, M, K, N, G, eps, po, _stream(stream))


def lgn_forward_bf16(x, W, b_lin, b_add, gamma, beta, M, K, N, G, eps, out, stream=None) -> int:
    px, pW, pbl, pba, pg, pb, po = _fwd("bf16", x, W, b_lin, b_add, gamma, beta, M, K, N, out)
    return _lib.lgn_forward_bf16(px, pW, pbl, pba, pg, pb, M, K, N, G, eps, po, _stream(stream))


def lgn_fused_supported(dtype: int, M: int, K: int, N: int, G: int) -> int:
    return _lib.lgn_fused_supported(dtype, M, K, N, G)


def _fwd_ws(cfn, dt, x, W, b_lin, b_add, gamma, beta, M, K, N, G, eps, out, workspace,
            workspace_bytes, stream) -> int:
    px, pW, pbl, pba, pg, pb, po, pws = _fwd(dt, x, W, b_lin, b_add, gamma, beta, M, K, N, out,
                                             workspace, workspace_bytes)
    return cfn(px, pW, pbl, pba, pg, pb, M, K, N, G, eps, po, pws, workspace_bytes,
               _stream(stream))


def lgn_twopass_workspace_bytes(M: int, N: int) -> int:
    return _lib.lgn_twopass_workspace_bytes(M, N)


def lgn_forward_twopass_f32(x, W, b_lin, b_add, gamma, beta, M, K, N, G, eps, out, workspace,
                            workspace_bytes, stream=None) -> int:
    return _fwd_ws(_lib.lgn_forward_twopass_f32, "f32", x, W, b_lin, b_add, gamma, beta, M, K, N,
                   G, eps, out, workspace, workspace_bytes, stream)


def lgn_forward_twopass_bf16(x, W, b_lin, b_add, gamma, beta, M, K, N, G, eps, out, workspace,
                             workspace_bytes, stream=None) -> int:
    return _fwd_ws(_lib.lgn_forward_twopass_bf16, "bf16", x, W, b_lin, b_add, gamma, beta, M, K,
                   N, G, eps, out, workspace, workspace_bytes, stream)


def lgn_wide_workspace_bytes(M: int, N: int) -> int:
    return _lib.lgn_wide_workspace_bytes(M, N)


def lgn_forward_wide_f32(x, W, b_lin, b_add, gamma, beta, M, K, N, G, eps, out, workspace,
                         workspace_bytes, stream=None) -> int:
    return _fwd_ws(_lib.lgn_forward_wide_f32, "f32", x, W, b_lin, b_add, gamma, beta, M, K, N,
                   G, eps, out, workspace, workspace_bytes, stream)


def lgn_forward_wide_bf16(x, W, b_lin, b_add, gamma, beta, M, K, N, G, eps, out, workspace,
                          workspace_bytes, stream=None) -> int:
    return _fwd_ws(_lib.lgn_forward_wide_bf16, "bf16", x, W, b_lin, b_add, gamma, beta, M, K, N,
                   G, eps, out, workspace, workspace_bytes, stream)


def lgn_forward_wide_f32_noalloc(x, W, b_lin, b_add, gamma, beta, M, K, N, G, eps, out,
                                 stream=None) -> int:
    px, pW, pbl, pba, pg, pb, po = _fwd("f32", x, W, b_lin, b_add, gamma, beta, M, K, N, out)
    return _lib.lgn_forward_wide_f32_noalloc(px, pW, pbl, pba, pg, pb, M, K, N, G, eps, po,
                                             _stream(stream))


def lgn_lse_workspace_bytes(M: int, N: int) -> int:
    return _lib.lgn_lse_workspace_bytes(M, N)


def _lse(cfn, dt, x, W, b, M, K, N, out, workspace, workspace_bytes, stream) -> int:
    px, pW, pb, po, pws = _ptrs((x, dt, _n(M, K)), (W, dt, _n(N, K)), (b, "f32", _n(N)),
                                (out, "f32", _n(M)), (workspace, None, workspace_bytes))
    return cfn(px, pW, pb, M, K, N, po, pws, workspace_bytes, _stream(stream))


def lgn_linear_lse_f32(x, W, b, M, K, N, out, workspace, workspace_bytes, stream=None) -> int:
    return _lse(_lib.lgn_linear_lse_f32, "f32", x, W, b, M, K, N, out, workspace,
                workspace_bytes, stream)


def lgn_linear_lse_bf16(x, W, b, M, K, N, out, workspace, workspace_bytes, stream=None) -> int:
    return _lse(_lib.lgn_linear_lse_bf16, "bf16", x, W, b, M, K, N, out, workspace,
                workspace_bytes, stream)


def lgn_sgh_workspace_bytes(Nb: int, C: int, S: int, G: int) -> int:
    return _lib.lgn_sgh_workspace_bytes(Nb, C, S, G)


def lgn_swish_gn_hardswish_f32(y, gamma, beta, Nb, C, S, G, eps, out, workspace,
                               workspace_bytes, stream=None) -> int:
    py, pg, pb, po, pws = _ptrs((y, "f32", _n(Nb, C, S)), (gamma, "f32", _n(C)),
                                (beta, "f32", _n(C)), (out, "f32", _n(Nb, C, S)),
                                (workspace, None, workspace_bytes))
    return _lib.lgn_swish_gn_hardswish_f32(py, pg, pb, Nb, C, S, G, eps, po, pws, workspace_bytes,
                                           _stream(stream))


def lgn_lnconv_workspace_bytes(B: int, C: int, L: int) -> int:
    return _lib.lgn_lnconv_workspace_bytes(B, C, L)


def lgn_ln_gelu_conv1d_f32(x, ln_w, ln_b, conv_w, conv_b, B, C, L, dilation, eps, gelu_tanh, out,
                           workspace, workspace_bytes, stream=None) -> int:
    px, plw, plb, pcw, pcb, po, pws = _ptrs(
        (x, "f32", _n(B, C, L)), (ln_w, "f32", _n(C, L)), (ln_b, "f32", _n(C, L)),
        (conv_w, "f32", _n(C, C, 3)), (conv_b, "f32", _n(C)), (out, "f32", _n(B, C, L)),
        (workspace, None, workspace_bytes))
    return _lib.lgn_ln_gelu_conv1d_f32(px, plw, plb, pcw, pcb, B, C, L, dilation, eps,
                                       int(bool(gelu_tanh)), po, pws, workspace_bytes,
                                       _stream(stream))


def lgn_status_string(status: int) -> str:
    return _lib.lgn_status_string(status).decode()


def lgn_version() -> str:
    return _lib.lgn_version().decode()


def lgn_last_hip_error_string() -> str:
    return _lib.lgn_last_hip_error_string().decode()


def lgn_testing_set_arch(arch: Optional[str]) -> None:
    """Failure-path hook: compare this architecture name instead of the device's (None: undo)."""
    _lib.lgn_testing_set_arch(None if arch is None else arch.encode())


def lgn_testing_fail_launches(hip_error: int, count: int) -> None:
    """Failure-path hook: the next `count` launches return `hip_error` instead of launching."""
    _lib.lgn_testing_fail_launches(hip_error, count)


def lgn_testing_set_sgh_spin_limit(polls: int) -> None:
    """Failure-path hook: polls of the single-pass spatial GroupNorm's bounded wait
    before it forms the group's statistics itself (negative: the default)."""
    _lib.lgn_testing_set_sgh_spin_limit(polls)


def check(status: int) -> None:
    if status != LGN_OK:
        raise LgnError(status)
