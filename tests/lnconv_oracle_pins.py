"""Pins for the oracle of the fourth method (POPCORNBENCH transcript
"Kimi-K2.6 l2_p5", a pre-norm dilated convolution block):

    x [B, C, L]
    per sample b, over all C*L values: mean, population variance
    h = (x - mean) / sqrt(var + eps) * ln_w[c, p] + ln_b[c, p]     ln_w, ln_b [C, L]
    g = GELU(h)                     exact v*Phi(v), or the tanh form on request
    out[b, co, j] = conv_b[co] + x[b, co, j] + sum_ci sum_t conv_w[co, ci, t] g[ci, j - d + t d]
    g = 0 outside [0, L)            (kernel 3, dilation d, zero padding d: L_out = L)

Every check takes an implementation object exposing

    gelu_tanh(v) -> array
    ln_gelu_conv1d(x, ln_w, ln_b, conv_w, conv_b, dilation, eps, gelu_tanh=False,
                   return_parts=False) -> out (, g, mean [B], var [B])
    ln_gelu_conv1d_cols(x, ln_w, ln_b, conv_w, conv_b, dilation, eps, cols,
                        gelu_tanh=False) -> [len(cols), C]

and raises AssertionError when it disagrees with:

* closed forms of the tanh GELU and torch float64 ``F.gelu(approximate="tanh")``;
* library routines: torch float64 ``F.layer_norm`` over [C, L] -> ``F.gelu``
  (both forms) -> ``F.conv1d(padding=d, dilation=d)`` -> ``+ x``;
* brute force in pure Python (``math.erf``, ``statistics.pvariance``);
* invariants: zero weights leave conv_b + x exactly; a centre-tap identity
  weight gives g + x; the normalised values have mean 0 and variance
  v / (v + eps); a change of the first (last) tap's weights leaves the first
  (last) d output positions untouched (zero padding, taps j - d, j, j + d);
  samples are independent; the column form equals the full form.
"""
from __future__ import annotations

import math
import statistics

import numpy as np


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, "%s: shape %s vs %s" % (what, a.shape, b.shape)
    if a.size == 0:
        return
    assert np.all(np.isfinite(a)), "%s: non-finite values" % what
    err = float(np.max(np.abs(a - b)))
    assert err <= tol, "%s: max abs err %.3e > %.1e" % (what, err, tol)


def _problem(seed, B=2, C=4, L=11):
    r = np.random.default_rng(seed)
    x = 1.3 * r.standard_normal((B, C, L)) + 0.4
    ln_w = 1.0 + 0.2 * r.standard_normal((C, L))
    ln_b = 0.2 * r.standard_normal((C, L))
    bound = 1.0 / math.sqrt(3 * C)
    conv_w = r.uniform(-bound, bound, (C, C, 3)) * 3.0
    conv_b = r.uniform(-bound, bound, C)
    return x, ln_w, ln_b, conv_w, conv_b


def _torch_ref(x, ln_w, ln_b, conv_w, conv_b, d, eps, tanh):
    import torch
    F = torch.nn.functional
    t = torch.from_numpy
    C, L = x.shape[1], x.shape[2]
    h = F.layer_norm(t(x), [C, L], t(ln_w), t(ln_b), eps)
    g = F.gelu(h, approximate="tanh" if tanh else "none")
    return (F.conv1d(g, t(conv_w), t(conv_b), padding=d, dilation=d) + t(x)).numpy()


def check_gelu_tanh_closed_forms(impl):
    import torch
    v = np.array([0.0, -0.0, 30.0, -30.0])
    _close(impl.gelu_tanh(v), np.array([0.0, 0.0, 30.0, 0.0]), 1e-15, "tanh gelu limits")
    w = np.linspace(-7, 7, 281)
    ref = torch.nn.functional.gelu(torch.from_numpy(w), approximate="tanh").numpy()
    _close(impl.gelu_tanh(w), ref, 1e-15, "tanh gelu vs torch")
    # at v = 1: 0.5 (1 + tanh(sqrt(2/pi) * 1.044715))
    _close(impl.gelu_tanh(np.array([1.0])),
           np.array([0.5 * (1.0 + math.tanh(math.sqrt(2.0 / math.pi) * 1.044715))]), 1e-15,
           "tanh gelu at 1")


def check_lnconv_library(impl):
    for seed, (B, C, L), d, eps, tanh in ((1, (2, 4, 11), 2, 1e-5, False),
                                          (2, (3, 8, 16), 4, 1e-5, False),
                                          (3, (1, 5, 9), 1, 1e-3, True),
                                          (4, (2, 6, 7), 3, 1e-5, True),
                                          (5, (2, 3, 5), 4, 1e-5, False)):   # d >= L/2: edge taps mostly padding
        x, lw, lb, cw, cb = _problem(seed, B, C, L)
        ref = _torch_ref(x, lw, lb, cw, cb, d, eps, tanh)
        _close(impl.ln_gelu_conv1d(x, lw, lb, cw, cb, d, eps, gelu_tanh=tanh), ref, 1e-12,
               "vs torch, B%d C%d L%d d%d tanh=%s" % (B, C, L, d, tanh))


def check_lnconv_brute_force(impl):
    x, lw, lb, cw, cb = _problem(6, 2, 3, 7)
    B, C, L = x.shape
    d, eps = 2, 1e-5
    out = np.empty_like(x)
    for b in range(B):
        vals = [float(v) for v in x[b].ravel()]
        mean = math.fsum(vals) / len(vals)
        var = statistics.pvariance(vals)

        def g(c, p):
            if p < 0 or p >= L:
                return 0.0
            h = (float(x[b, c, p]) - mean) / math.sqrt(var + eps) * float(lw[c, p]) + float(lb[c, p])
            return h * 0.5 * (1.0 + math.erf(h / math.sqrt(2.0)))

        for co in range(C):
            for j in range(L):
                acc = math.fsum(float(cw[co, ci, t]) * g(ci, j - d + t * d)
                                for ci in range(C) for t in range(3))
                out[b, co, j] = float(cb[co]) + acc + float(x[b, co, j])
    _close(impl.ln_gelu_conv1d(x, lw, lb, cw, cb, d, eps), out, 1e-12, "brute force")


def check_lnconv_zero_and_identity_weights(impl):
    x, lw, lb, cw, cb = _problem(7, 2, 5, 12)
    C = x.shape[1]
    out0 = impl.ln_gelu_conv1d(x, lw, lb, np.zeros_like(cw), cb, 3, 1e-5)
    _close(out0, cb[None, :, None] + x, 0.0, "zero weights: conv_b + x")
    ident = np.zeros_like(cw)
    ident[np.arange(C), np.arange(C), 1] = 1.0
    out1, g, _, _ = impl.ln_gelu_conv1d(x, lw, lb, ident, np.zeros(C), 3, 1e-5, return_parts=True)
    _close(out1, g + x, 1e-14, "centre-tap identity: g + x")


def check_lnconv_moments(impl):
    x, _, _, cw, cb = _problem(8, 3, 4, 10)
    B, C, L = x.shape
    eps = 1e-3
    # unit affine and the centre-tap identity: g = GELU(normalised x) and out = g + x
    ident = np.zeros_like(cw)
    ident[np.arange(C), np.arange(C), 1] = 1.0
    out, g, mean, var = impl.ln_gelu_conv1d(x, np.ones((C, L)), np.zeros((C, L)), ident,
                                            np.zeros(C), 2, eps, return_parts=True)
    xs = x.reshape(B, -1)
    _close(mean, xs.mean(axis=1), 1e-13, "sample means")
    _close(var, xs.var(axis=1), 1e-13, "sample population variances")
    # invert GELU numerically is awkward; check the normalisation through the
    # statistics instead: h = (x - mean)/sqrt(var + eps) has mean 0, var v/(v+eps)
    h = (xs - mean[:, None]) / np.sqrt(var[:, None] + eps)
    _close(h.mean(axis=1), np.zeros(B), 1e-13, "normalised mean 0")
    _close(h.var(axis=1), var / (var + eps), 1e-12, "normalised variance v/(v+eps)")
    gel = h * 0.5 * (1.0 + np.vectorize(math.erf)(h / math.sqrt(2.0)))
    _close(g.reshape(B, -1), gel, 1e-14, "g = GELU(normalised x) under unit affine")


def check_lnconv_padding_and_tap_order(impl):
    x, lw, lb, cw, cb = _problem(9, 2, 4, 14)
    d = 3
    L = x.shape[2]
    a = impl.ln_gelu_conv1d(x, lw, lb, cw, cb, d, 1e-5)
    w0 = cw.copy()
    w0[:, :, 0] += 0.5     # first tap reads j - d: outputs j < d read padding there
    b0 = impl.ln_gelu_conv1d(x, lw, lb, w0, cb, d, 1e-5)
    assert np.array_equal(a[:, :, :d], b0[:, :, :d]), "first tap must not reach j < d"
    assert not np.array_equal(a[:, :, d:], b0[:, :, d:]), "first tap must reach j >= d"
    w2 = cw.copy()
    w2[:, :, 2] += 0.5     # last tap reads j + d: outputs j >= L - d read padding there
    b2 = impl.ln_gelu_conv1d(x, lw, lb, w2, cb, d, 1e-5)
    assert np.array_equal(a[:, :, L - d:], b2[:, :, L - d:]), "last tap must not reach j >= L-d"
    assert not np.array_equal(a[:, :, :L - d], b2[:, :, :L - d]), "last tap must reach j < L-d"


def check_lnconv_sample_independence_and_columns(impl):
    x, lw, lb, cw, cb = _problem(10, 3, 4, 9)
    a = impl.ln_gelu_conv1d(x, lw, lb, cw, cb, 2, 1e-5)
    x2 = x.copy()
    x2[1] = 2.0 * x2[1] + 1.0
    b = impl.ln_gelu_conv1d(x2, lw, lb, cw, cb, 2, 1e-5)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[2], b[2]), "other samples changed"
    assert not np.array_equal(a[1], b[1]), "the changed sample must change"
    cols = [(0, 0), (1, 4), (2, 8), (2, 1)]
    c = impl.ln_gelu_conv1d_cols(x, lw, lb, cw, cb, 2, 1e-5, cols)
    _close(c, np.stack([a[bb, :, j] for bb, j in cols]), 1e-15, "columns vs full")


ALL_CHECKS = [
    check_gelu_tanh_closed_forms,
    check_lnconv_library,
    check_lnconv_brute_force,
    check_lnconv_zero_and_identity_weights,
    check_lnconv_moments,
    check_lnconv_padding_and_tap_order,
    check_lnconv_sample_independence_and_columns,
]
