"""Pins for the fp64 oracle: checks against facts fixed outside the oracle.

Every check takes an implementation object exposing

    swish(z) -> array            linear(x, W, b_lin) -> z
    groupnorm(u, gamma, beta, G, eps, return_stats=False) -> y [, mean, var]
    lgn_forward(x, W, b_lin, b_add, gamma, beta, G, eps) -> y

and raises AssertionError when the implementation disagrees with:

* closed forms of Swish: sigmoid(ln 3) = 3/4 and sigmoid(-ln 3) = 1/4, the
  global minimum -W(1/e) at z = -1 - W(1/e) (W = Lambert W), z - swish(z) in
  (0, z e^-z] for large z, and swish(-z) = swish(z) - z;
* library routines: torch float64 ``F.linear``, ``F.group_norm``,
  ``F.layer_norm``; Python's ``statistics.pvariance`` (exact rational
  arithmetic) and ``math.fsum`` in a brute-force pass over a tiny input;
* special cases with exact answers: x = identity picks out W^T + b_lin;
  one channel per group gives beta exactly; W = 0 makes every row identical;
* invariants of the method: unit affine gives per-group mean 0 and variance
  v / (v + eps); a per-group constant added to b_add changes nothing;
  permuting channels inside a group permutes the output; rows are independent;
* a hand-derived two-channel-group example whose output has a closed form.

``tests/test_oracle_mutants.py`` plants one plausible mistake at a time in a
numpy re-implementation and shows that each one fails at least one check.
"""
from __future__ import annotations

import math
import statistics

import numpy as np

LN3 = math.log(3.0)


def _rng(seed):
    return np.random.default_rng(seed)


def _rand_problem(seed, M=5, K=7, N=12, G=3):
    r = _rng(seed)
    x = r.standard_normal((M, K))
    W = r.uniform(-1, 1, (N, K))
    b_lin = r.uniform(-0.5, 0.5, N)
    b_add = 0.3 * r.standard_normal(N)
    gamma = 1 + 0.2 * r.standard_normal(N)
    beta = 0.2 * r.standard_normal(N)
    return x, W, b_lin, b_add, gamma, beta, G


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, "%s: shape %s vs %s" % (what, a.shape, b.shape)
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol, "%s: max abs err %.3e > %.1e" % (what, err, tol)


# ---------------------------------------------------------------- Swish ----

def check_swish_closed_forms(impl):
    s = impl.swish(np.array([0.0, LN3, -LN3, math.log(2.0), -2 * LN3]))
    assert s[0] == 0.0, "swish(0) must be exactly 0"
    _close(s[1], 0.75 * LN3, 1e-15, "swish(ln 3) = (3/4) ln 3")
    _close(s[2], -0.25 * LN3, 1e-15, "swish(-ln 3) = -(1/4) ln 3")
    _close(s[3], (2.0 / 3.0) * math.log(2.0), 1e-15, "swish(ln 2) = (2/3) ln 2")
    _close(s[4], -2 * LN3 / 10.0, 1e-15, "swish(-2 ln 3) = -2 ln 3 / 10")


def check_swish_minimum(impl):
    from scipy.special import lambertw
    w = float(np.real(lambertw(1.0 / math.e)))      # 0.27846454276107...
    z = np.linspace(-3.0, 0.0, 30001)
    s = impl.swish(z)
    i = int(np.argmin(s))
    _close(s[i], -w, 1e-8, "min swish = -W(1/e)")
    _close(z[i], -1.0 - w, 2e-4, "argmin swish = -1 - W(1/e)")


def check_swish_tails_and_reflection(impl):
    for zz in (20.0, 30.0, 40.0):
        gap = zz - float(impl.swish(np.array([zz]))[0])
        # exact gap z / (1 + e^z) lies in (0, z e^-z]; allow a few ulps of z
        assert 0.0 <= gap <= zz * math.exp(-zz) + 4 * math.ulp(zz), "swish(z) -> z from below"
        neg = float(impl.swish(np.array([-zz]))[0])
        assert -zz * math.exp(-zz) * (1 + 1e-12) <= neg <= 0.0, "swish(-z) -> 0 from below"
    z = np.linspace(-12.0, 12.0, 241)
    _close(impl.swish(-z), impl.swish(z) - z, 1e-13, "swish(-z) = swish(z) - z")


# --------------------------------------------------------------- Linear ----

def check_linear_library(impl):
    import torch
    import torch.nn.functional as F
    x, W, b, *_ = _rand_problem(1, M=9, K=13, N=11)
    ref = F.linear(torch.from_numpy(x), torch.from_numpy(W), torch.from_numpy(b)).numpy()
    _close(impl.linear(x, W, b), ref, 1e-13, "linear vs torch float64 F.linear")


def check_linear_identity(impl):
    r = _rng(2)
    K, N = 6, 10
    W = r.uniform(-1, 1, (N, K))
    b = r.uniform(-1, 1, N)
    z = impl.linear(np.eye(K), W, b)
    # row k of x = e_k picks out column k of W: z[k, n] = W[n, k] + b[n], exactly
    assert np.array_equal(z, W.T + b[None, :]), "x = I must give W^T + b_lin exactly"
    x = r.standard_normal((4, N))
    assert np.array_equal(impl.linear(x, np.eye(N), np.zeros(N)), x), "W = I, b = 0 gives x"


# ------------------------------------------------------------ GroupNorm ----

def check_groupnorm_library(impl):
    import torch
    import torch.nn.functional as F
    r = _rng(3)
    M, N = 6, 24
    u = 2.0 * r.standard_normal((M, N)) + 0.5
    gamma = 1 + 0.3 * r.standard_normal(N)
    beta = 0.3 * r.standard_normal(N)
    for G in (1, 2, 3, 4, 6, 8, 12, 24):
        for eps in (1e-5, 0.5):
            ref = F.group_norm(torch.from_numpy(u), G, torch.from_numpy(gamma),
                               torch.from_numpy(beta), eps).numpy()
            _close(impl.groupnorm(u, gamma, beta, G, eps), ref, 1e-12,
                   "groupnorm vs torch F.group_norm (G=%d, eps=%g)" % (G, eps))


def check_groupnorm_layernorm(impl):
    import torch
    import torch.nn.functional as F
    r = _rng(4)
    M, N = 5, 16
    u = r.standard_normal((M, N))
    gamma = 1 + 0.3 * r.standard_normal(N)
    beta = 0.3 * r.standard_normal(N)
    ref = F.layer_norm(torch.from_numpy(u), (N,), torch.from_numpy(gamma),
                       torch.from_numpy(beta), 1e-3).numpy()
    _close(impl.groupnorm(u, gamma, beta, 1, 1e-3), ref, 1e-12, "G = 1 is LayerNorm over N")


def check_groupnorm_one_channel(impl):
    r = _rng(5)
    M, N = 4, 8
    u = r.standard_normal((M, N))
    gamma = r.standard_normal(N)
    beta = r.standard_normal(N)
    y = impl.groupnorm(u, gamma, beta, N, 1e-5)
    assert np.array_equal(y, np.broadcast_to(beta, (M, N))), "one channel per group: y = beta"


def check_groupnorm_moments(impl):
    r = _rng(6)
    M, N, G = 7, 32, 4
    C = N // G
    u = 0.3 * r.standard_normal((M, N)) + r.standard_normal((M, 1))
    for eps in (1e-5, 0.1):
        y, mean, var = impl.groupnorm(u, np.ones(N), np.zeros(N), G, eps, return_stats=True)
        ug = u.reshape(M, G, C)
        v = np.var(ug, axis=2)                       # numpy population variance
        _close(mean, np.mean(ug, axis=2), 1e-13, "returned group mean")
        _close(var, v, 1e-13, "returned group variance (population)")
        yg = y.reshape(M, G, C)
        _close(np.mean(yg, axis=2), np.zeros((M, G)), 1e-12, "normalised group mean 0")
        _close(np.var(yg, axis=2), v / (v + eps), 1e-12, "normalised group var v/(v+eps)")


# ------------------------------------------------------ whole pipeline ----

def check_forward_brute_force(impl):
    """Pure Python on a tiny input: math.fsum dot products, math.exp sigmoid,
    statistics.fmean / statistics.pvariance (exact rationals) per group."""
    x, W, b_lin, b_add, gamma, beta, G = _rand_problem(7, M=3, K=4, N=6, G=3)
    eps = 1e-2
    M, K = x.shape
    N = W.shape[0]
    C = N // G
    y = impl.lgn_forward(x, W, b_lin, b_add, gamma, beta, G, eps)
    for m in range(M):
        u = []
        for n in range(N):
            z = math.fsum(float(x[m, k]) * float(W[n, k]) for k in range(K)) + float(b_lin[n])
            u.append(z / (1.0 + math.exp(-z)) + float(b_add[n]))
        for g in range(G):
            grp = u[g * C:(g + 1) * C]
            mu = statistics.fmean(grp)
            var = statistics.pvariance(grp)
            for c in range(C):
                n = g * C + c
                ref = (grp[c] - mu) / math.sqrt(var + eps) * gamma[n] + beta[n]
                assert abs(y[m, n] - ref) <= 1e-12, "brute force (m=%d, n=%d)" % (m, n)


def check_forward_shift_invariance(impl):
    x, W, b_lin, b_add, gamma, beta, G = _rand_problem(8)
    N = W.shape[0]
    C = N // G
    y0 = impl.lgn_forward(x, W, b_lin, b_add, gamma, beta, G, 1e-5)
    shift = np.repeat(np.array([3.0, -1.5, 0.25]), C)
    y1 = impl.lgn_forward(x, W, b_lin, b_add + shift, gamma, beta, G, 1e-5)
    _close(y1, y0, 1e-10, "per-group constant added to b_add leaves y unchanged")


def check_forward_group_permutation(impl):
    x, W, b_lin, b_add, gamma, beta, G = _rand_problem(9)
    N = W.shape[0]
    C = N // G
    r = _rng(10)
    perm = np.concatenate([g * C + r.permutation(C) for g in range(G)])
    y0 = impl.lgn_forward(x, W, b_lin, b_add, gamma, beta, G, 1e-5)
    y1 = impl.lgn_forward(x, W[perm], b_lin[perm], b_add[perm], gamma[perm], beta[perm], G, 1e-5)
    _close(y1, y0[:, perm], 1e-12, "channel permutation within groups permutes y")


def check_forward_row_independence(impl):
    x, W, b_lin, b_add, gamma, beta, G = _rand_problem(11, M=9)
    perm = _rng(12).permutation(x.shape[0])
    y0 = impl.lgn_forward(x, W, b_lin, b_add, gamma, beta, G, 1e-5)
    y1 = impl.lgn_forward(x[perm], W, b_lin, b_add, gamma, beta, G, 1e-5)
    assert np.array_equal(y1, y0[perm]), "row shuffle of x shuffles rows of y"
    y2 = impl.lgn_forward(x[:1], W, b_lin, b_add, gamma, beta, G, 1e-5)
    assert np.array_equal(y2, y0[:1]), "a row alone gives the same row"


def check_forward_zero_weight(impl):
    import torch
    import torch.nn.functional as F
    x, W, b_lin, b_add, gamma, beta, G = _rand_problem(13)
    N = W.shape[0]
    y = impl.lgn_forward(x, np.zeros_like(W), np.zeros(N), b_add, gamma, beta, G, 1e-5)
    ref = F.group_norm(torch.from_numpy(b_add[None, :]), G, torch.from_numpy(gamma),
                       torch.from_numpy(beta), 1e-5).numpy()
    _close(y, np.broadcast_to(ref, y.shape), 1e-12, "W = 0: each row is GroupNorm(b_add)")


def check_forward_hand_example(impl):
    """Two rows, four channels in two groups of two, values chosen so every
    intermediate has a closed form (L = ln 3, sigmoid(L) = 3/4,
    sigmoid(-L) = 1/4, sigmoid(2L) = 9/10).  For a two-channel group (a, b)
    the mean is (a+b)/2 and the variance d^2 with d = (a-b)/2, so
        y_a = +d / sqrt(d^2 + eps) * gamma_a + beta_a,
        y_b = -d / sqrt(d^2 + eps) * gamma_b + beta_b."""
    L = LN3
    x = np.array([[1.0, 0.0], [0.0, 1.0]])
    W = np.array([[L, -L], [0.0, 0.0], [L, L], [-L, 0.0]])
    b_lin = np.array([0.0, L, L, 0.0])
    b_add = np.array([0.5, -0.25, 0.125, 1.0])
    gamma = np.array([1.5, 0.5, 2.0, -1.0])
    beta = np.array([0.1, -0.2, 0.3, 0.0])
    eps = 0.25
    # z = x W^T + b_lin: row 0 -> [L, L, 2L, -L]; row 1 -> [-L, L, 2L, 0]
    # swish(z) + b_add:
    u = np.array([[0.75 * L + 0.5, 0.75 * L - 0.25, 1.8 * L + 0.125, -0.25 * L + 1.0],
                  [-0.25 * L + 0.5, 0.75 * L - 0.25, 1.8 * L + 0.125, 0.0 + 1.0]])
    ref = np.empty_like(u)
    for m in range(2):
        for g in range(2):
            a, b = u[m, 2 * g], u[m, 2 * g + 1]
            d = (a - b) / 2.0
            t = d / math.sqrt(d * d + eps)
            ref[m, 2 * g] = t * gamma[2 * g] + beta[2 * g]
            ref[m, 2 * g + 1] = -t * gamma[2 * g + 1] + beta[2 * g + 1]
    y = impl.lgn_forward(x, W, b_lin, b_add, gamma, beta, 2, eps)
    _close(y, ref, 1e-14, "hand-derived two-channel-group example")


def check_forward_composes_steps(impl):
    x, W, b_lin, b_add, gamma, beta, G = _rand_problem(14)
    y = impl.lgn_forward(x, W, b_lin, b_add, gamma, beta, G, 1e-5)
    u = impl.swish(impl.linear(x, W, b_lin)) + b_add[None, :]
    _close(y, impl.groupnorm(u, gamma, beta, G, 1e-5), 1e-14, "forward = steps in order")


ALL_CHECKS = [
    check_swish_closed_forms,
    check_swish_minimum,
    check_swish_tails_and_reflection,
    check_linear_library,
    check_linear_identity,
    check_groupnorm_library,
    check_groupnorm_layernorm,
    check_groupnorm_one_channel,
    check_groupnorm_moments,
    check_forward_brute_force,
    check_forward_shift_invariance,
    check_forward_group_permutation,
    check_forward_row_independence,
    check_forward_zero_weight,
    check_forward_hand_example,
    check_forward_composes_steps,
]
