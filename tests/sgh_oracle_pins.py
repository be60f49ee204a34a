"""Pins for the oracle of the third method (POPCORNBENCH transcript
"Kimi-K2.6 l2_p60", the tail after its 3-D transposed convolution):

    s   = sigmoid(y) * y                                   y [Nb, C, *spatial]
    per sample n and group g of C/G contiguous channels, over those channels
    and every spatial position: mean and population variance of s
    out = hardswish((s - mean) / sqrt(var + eps) * gamma[c] + beta[c])
    hardswish(v) = v * clamp(v + 3, 0, 6) / 6

Every check takes an implementation object exposing

    hardswish(v) -> array
    swish_gn_hardswish(y, gamma, beta, G, eps, return_parts=False)
        -> out (, norm, mean [Nb, G], var [Nb, G])

and raises AssertionError when it disagrees with:

* closed forms of HardSwish on both sides of -3, 0 and 3;
* library routines: torch float64 ``F.hardswish`` and the composition
  ``F.silu`` -> ``F.group_norm`` -> ``F.hardswish``; a brute-force pass in
  pure Python with ``statistics.pvariance`` (exact rational arithmetic);
* invariants: per group the normalised values have mean 0 and variance
  v / (v + eps); a joint permutation of the spatial positions permutes the
  output; groups are independent; a constant group normalises to 0 exactly.

``tests/test_sgh_oracle_pins.py`` plants one plausible mistake at a time in a
numpy re-implementation and shows that each one fails at least one check.
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


def _problem(seed, shape=(2, 8, 3, 4, 5), scale=1.5):
    r = np.random.default_rng(seed)
    C = shape[1]
    y = scale * r.standard_normal(shape)
    gamma = 1.0 + 0.3 * r.standard_normal(C)
    beta = 0.4 * r.standard_normal(C)
    return y, gamma, beta


def check_hardswish_closed_forms(impl):
    v = np.array([-10.0, -3.0, -1.5, -1.0, 0.0, 1.0, 2.5, 3.0, 7.25])
    ref = np.array([0.0, 0.0, -0.375, -1.0 / 3.0, 0.0, 2.0 / 3.0, 2.5 * 5.5 / 6.0, 3.0, 7.25])
    _close(impl.hardswish(v), ref, 1e-15, "hardswish closed forms")
    import torch
    w = np.linspace(-6, 6, 241)
    _close(impl.hardswish(w), torch.nn.functional.hardswish(torch.from_numpy(w)).numpy(), 1e-15,
           "hardswish vs torch")


def check_sgh_library(impl):
    import torch
    F = torch.nn.functional
    for seed, shape, G, eps in ((1, (2, 8, 3, 4, 5), 4, 1e-5), (2, (3, 6, 7, 2), 3, 1e-3),
                                (3, (1, 16, 9), 1, 1e-5), (4, (2, 4, 5, 5), 4, 1e-5)):
        y, gamma, beta = _problem(seed, shape)
        ref = F.hardswish(F.group_norm(F.silu(torch.from_numpy(y)), G, torch.from_numpy(gamma),
                                       torch.from_numpy(beta), eps)).numpy()
        _close(impl.swish_gn_hardswish(y, gamma, beta, G, eps), ref, 1e-12,
               "vs torch, shape %s G=%d" % (shape, G))


def check_sgh_brute_force(impl):
    y, gamma, beta = _problem(5, (2, 4, 3))
    Nb, C, S = y.shape
    G, eps = 2, 1e-5
    Cg = C // G
    out = np.empty_like(y)
    for n in range(Nb):
        for g in range(G):
            s = [float(v) * (1.0 / (1.0 + math.exp(-float(v))))
                 for c in range(g * Cg, (g + 1) * Cg) for v in y[n, c]]
            mean = math.fsum(s) / len(s)
            var = statistics.pvariance(s)
            k = 0
            for c in range(g * Cg, (g + 1) * Cg):
                for j in range(S):
                    t = (s[k] - mean) / math.sqrt(var + eps) * gamma[c] + beta[c]
                    out[n, c, j] = t * min(max(t + 3.0, 0.0), 6.0) / 6.0
                    k += 1
    _close(impl.swish_gn_hardswish(y, gamma, beta, G, eps), out, 1e-12, "brute force")


def check_sgh_moments(impl):
    y, gamma, beta = _problem(6, (3, 8, 4, 6))
    G, eps = 4, 1e-3
    out, norm, mean, var = impl.swish_gn_hardswish(y, gamma, beta, G, eps, return_parts=True)
    s = y / (1.0 + np.exp(-y))
    sg = s.reshape(3, G, -1)
    _close(mean, sg.mean(axis=2), 1e-13, "group means")
    _close(var, sg.var(axis=2), 1e-13, "group population variances")
    ng = norm.reshape(3, G, -1)
    _close(ng.mean(axis=2), np.zeros((3, G)), 1e-13, "normalised mean 0")
    _close(ng.var(axis=2), var / (var + eps), 1e-12, "normalised variance v/(v+eps)")


def check_sgh_spatial_permutation(impl):
    y, gamma, beta = _problem(7, (2, 6, 10))
    perm = np.random.default_rng(8).permutation(10)
    a = impl.swish_gn_hardswish(y, gamma, beta, 3, 1e-5)
    b = impl.swish_gn_hardswish(y[:, :, perm], gamma, beta, 3, 1e-5)
    _close(b, a[:, :, perm], 1e-13, "spatial permutation")


def check_sgh_group_independence(impl):
    y, gamma, beta = _problem(9, (2, 8, 12))
    a = impl.swish_gn_hardswish(y, gamma, beta, 4, 1e-5)
    y2 = y.copy()
    y2[1, 0:2] *= 3.0   # group 0 of sample 1 only
    b = impl.swish_gn_hardswish(y2, gamma, beta, 4, 1e-5)
    assert np.array_equal(np.delete(a.reshape(2, 4, -1), 0, axis=1)[1],
                          np.delete(b.reshape(2, 4, -1), 0, axis=1)[1]), "other groups changed"
    assert np.array_equal(a[0], b[0]), "other sample changed"
    assert not np.array_equal(a[1, 0:2], b[1, 0:2]), "the changed group must change"


def check_sgh_constant_group(impl):
    y, gamma, beta = _problem(10, (1, 4, 6))
    y[0, 2:4] = 0.7   # group 1 constant: normalised value 0, output hardswish(beta)
    out = impl.swish_gn_hardswish(y, gamma, beta, 2, 1e-5)
    ref = np.repeat(impl.hardswish(beta[2:4])[:, None], 6, axis=1)
    _close(out[0, 2:4], ref, 0.0, "constant group")


ALL_CHECKS = [
    check_hardswish_closed_forms,
    check_sgh_library,
    check_sgh_brute_force,
    check_sgh_moments,
    check_sgh_spatial_permutation,
    check_sgh_group_independence,
    check_sgh_constant_group,
]
