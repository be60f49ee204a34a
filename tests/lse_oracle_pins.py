"""Pins for the oracle of the second method (POPCORNBENCH transcript
"Kimi-K2.6 l2_p64", problem statement): one scalar per row,

    out[m] = gelu(gelu(leaky(leaky(logsumexp_n(x[m] . W^T + b)))))

with LeakyReLU of negative slope 0.01 and the exact GELU v * Phi(v).

Every check takes an implementation object exposing

    linear(x, W, b) -> z [M, N]        logsumexp_rows(z) -> [M]
    leaky_relu(v) -> array             gelu(v) -> array
    linear_lse_forward(x, W, b, return_lse=False) -> out [M] (, lse [M])

and raises AssertionError when it disagrees with:

* closed forms: a row of N equal values c has logsumexp c + ln N (also for
  |c| = 1000, where an unshifted exp overflows or underflows); two values
  a >= b give a + log1p(e^(b-a)); Phi(1) and Phi(-1) from the normal table;
  gelu(-v) = gelu(v) - v; leaky on both sides of 0;
* library routines: scipy ``special.logsumexp``, torch float64
  ``F.gelu(approximate="none")`` and ``F.leaky_relu(0.01)``, and a brute-force
  pass in pure Python (``math.fsum``, ``math.exp``, ``math.log``, ``math.erf``);
* invariants: logsumexp(z + c) = logsumexp(z) + c, max <= logsumexp <= max +
  ln N, order inside a row does not matter, rows are independent; a negative
  logsumexp passes through both LeakyReLUs as 1e-4 times itself.

``tests/test_lse_oracle_pins.py`` also plants one plausible mistake at a time
in a numpy re-implementation and shows that each one fails at least one check.
"""
from __future__ import annotations

import math

import numpy as np

PHI_1 = 0.8413447460685429    # standard normal CDF at 1 (normal table)
PHI_M1 = 0.15865525393145707  # ... at -1


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, "%s: shape %s vs %s" % (what, a.shape, b.shape)
    if a.size == 0:
        return
    assert np.all(np.isfinite(a)), "%s: non-finite values" % what
    err = float(np.max(np.abs(a - b)))
    assert err <= tol, "%s: max abs err %.3e > %.1e" % (what, err, tol)


def _problem(seed, M=4, K=6, N=9, bias_shift=0.0):
    r = np.random.default_rng(seed)
    x = r.standard_normal((M, K))
    W = r.uniform(-1, 1, (N, K))
    b = r.uniform(-0.5, 0.5, N) + bias_shift
    return x, W, b


# ------------------------------------------------------------ logsumexp ----

def check_lse_closed_forms(impl):
    for N in (1, 2, 7, 64):
        for c in (0.0, 1.5, -3.25, 1000.0, -1000.0):
            z = np.full((2, N), c)
            _close(impl.logsumexp_rows(z), np.full(2, c + math.log(N)),
                   1e-12 * max(1.0, abs(c)), "lse of %d equal values %g" % (N, c))
    z = np.array([[2.0, -1.0], [-1.0, 2.0], [0.5, 0.5]])
    ref = np.array([2.0 + math.log1p(math.exp(-3.0))] * 2 + [0.5 + math.log(2.0)])
    _close(impl.logsumexp_rows(z), ref, 1e-15, "lse of two values")


def check_lse_library(impl):
    from scipy.special import logsumexp
    r = np.random.default_rng(11)
    for N in (1, 3, 50, 257):
        z = 3.0 * r.standard_normal((5, N)) + r.uniform(-10, 10, (5, 1))
        _close(impl.logsumexp_rows(z), logsumexp(z, axis=1), 1e-12, "lse vs scipy, N=%d" % N)


def check_lse_invariants(impl):
    r = np.random.default_rng(12)
    z = r.standard_normal((6, 33))
    l0 = impl.logsumexp_rows(z)
    _close(impl.logsumexp_rows(z + 7.5), l0 + 7.5, 1e-12, "lse shift")
    perm = r.permutation(33)
    _close(impl.logsumexp_rows(z[:, perm]), l0, 1e-12, "lse order inside a row")
    mx = z.max(axis=1)
    assert np.all(l0 >= mx) and np.all(l0 <= mx + math.log(33) + 1e-12), "lse bounds"


# ---------------------------------------------------------- activations ----

def check_leaky(impl):
    v = np.array([2.0, -2.0, 0.0, 1e-300, -1e-300, 37.5, -37.5])
    _close(impl.leaky_relu(v), np.array([2.0, -0.02, 0.0, 1e-300, -1e-302, 37.5, -0.375]),
           1e-15, "leaky closed forms")
    import torch
    w = np.linspace(-5, 5, 101)
    ref = torch.nn.functional.leaky_relu(torch.from_numpy(w), 0.01).numpy()
    _close(impl.leaky_relu(w), ref, 1e-15, "leaky vs torch")


def check_gelu_closed_forms(impl):
    _close(impl.gelu(np.array([0.0, 1.0, -1.0])), np.array([0.0, PHI_1, -PHI_M1]), 1e-15,
           "gelu(0), gelu(+-1)")
    v = np.linspace(0.0, 6.0, 61)
    _close(impl.gelu(-v), impl.gelu(v) - v, 1e-14, "gelu reflection")
    big = np.array([10.0, 20.0, 40.0])
    _close(impl.gelu(big), big, 1e-13, "gelu tail")


def check_gelu_library(impl):
    import torch
    v = np.linspace(-8, 8, 321)
    ref = torch.nn.functional.gelu(torch.from_numpy(v), approximate="none").numpy()
    _close(impl.gelu(v), ref, 1e-14, "gelu vs torch (exact)")


# -------------------------------------------------------- whole forward ----

def _brute(x, W, b):
    out, lse = [], []
    N = W.shape[0]
    for row in x:
        z = [math.fsum(float(row[k]) * float(W[n, k]) for k in range(len(row))) + float(b[n])
             for n in range(N)]
        mx = max(z)
        l = mx + math.log(math.fsum(math.exp(v - mx) for v in z))
        v = l if l > 0 else 0.01 * l
        v = v if v > 0 else 0.01 * v
        for _ in range(2):
            v = v * 0.5 * (1.0 + math.erf(v / math.sqrt(2.0)))
        out.append(v)
        lse.append(l)
    return np.array(out), np.array(lse)


def check_lse_forward_brute_force(impl):
    for shift in (0.0, -6.0):
        x, W, b = _problem(21, bias_shift=shift)
        out, lse = impl.linear_lse_forward(x, W, b, return_lse=True)
        ref_out, ref_lse = _brute(x, W, b)
        _close(lse, ref_lse, 1e-12, "lse vs brute force, shift %g" % shift)
        _close(out, ref_out, 1e-12, "forward vs brute force, shift %g" % shift)


def check_lse_forward_composes_steps(impl):
    x, W, b = _problem(22, M=5, K=8, N=13)
    out = impl.linear_lse_forward(x, W, b)
    v = impl.logsumexp_rows(impl.linear(x, W, b))
    v = impl.gelu(impl.gelu(impl.leaky_relu(impl.leaky_relu(v))))
    _close(out, v, 1e-13, "forward = its steps")


def check_lse_forward_negative_branch(impl):
    # b far below 0 makes every row's logsumexp negative: both LeakyReLUs then
    # scale it by 0.01, and the GELUs act on a small negative number
    x, W, b = _problem(23, M=3, K=4, N=5, bias_shift=-12.0)
    out, lse = impl.linear_lse_forward(x, W, b, return_lse=True)
    assert np.all(lse < 0), "the case must exercise the negative branch"
    _close(out, impl.gelu(impl.gelu(1e-4 * lse)), 1e-15, "negative branch")


def check_lse_forward_uniform_rows(impl):
    # W = 0, b = c: z = c everywhere, so logsumexp = c + ln N in every row
    M, K, N, c = 3, 5, 16, 0.75
    out, lse = impl.linear_lse_forward(np.ones((M, K)), np.zeros((N, K)), np.full(N, c),
                                       return_lse=True)
    l = c + math.log(N)
    g = l * 0.5 * (1 + math.erf(l / math.sqrt(2)))
    g = g * 0.5 * (1 + math.erf(g / math.sqrt(2)))
    _close(lse, np.full(M, l), 1e-14, "uniform lse")
    _close(out, np.full(M, g), 1e-14, "uniform forward")


def check_lse_forward_row_independence(impl):
    x, W, b = _problem(24, M=6)
    full = impl.linear_lse_forward(x, W, b)
    part = impl.linear_lse_forward(x[2:4], W, b)
    assert np.array_equal(full[2:4], part), "rows must be independent"


ALL_CHECKS = [
    check_lse_closed_forms,
    check_lse_library,
    check_lse_invariants,
    check_leaky,
    check_gelu_closed_forms,
    check_gelu_library,
    check_lse_forward_brute_force,
    check_lse_forward_composes_steps,
    check_lse_forward_negative_branch,
    check_lse_forward_uniform_rows,
    check_lse_forward_row_independence,
]
