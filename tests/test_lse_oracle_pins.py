"""The fp64 oracle of the second method (Linear -> logsumexp -> LeakyReLU x2 ->
GELU x2) against its pins, and each planted mistake in a numpy model against
the same pins.  CPU only."""
import math
import types

import numpy as np
import pytest

import lse_oracle_pins as pins
import oracle

ORACLE = types.SimpleNamespace(
    linear=oracle.linear,
    logsumexp_rows=oracle.logsumexp_rows,
    leaky_relu=oracle.leaky_relu,
    gelu=oracle.gelu,
    linear_lse_forward=oracle.linear_lse_forward,
)


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_lse_oracle_pin(check):
    check(ORACLE)


def test_lse_oracle_empty_batch_and_zero_k():
    out = oracle.linear_lse_forward(np.zeros((0, 3)), np.ones((4, 3)), np.zeros(4))
    assert out.shape == (0,)
    b = np.array([0.0, 1.0, -2.0])
    out, lse = oracle.linear_lse_forward(np.zeros((2, 0)), np.zeros((3, 0)), b, return_lse=True)
    ref = math.log(1.0 + math.e + math.exp(-2.0))
    assert np.allclose(lse, ref, rtol=0, atol=1e-15)


# ---- planted mistakes (numpy model; the oracle itself is never modified) ----

def _model(bug=None):
    def linear(x, W, b):
        x, W, b = (np.asarray(a, np.float64) for a in (x, W, b))
        z = np.stack([W @ x[m] for m in range(x.shape[0])]) if x.shape[0] else \
            np.zeros((0, W.shape[0]))
        return z if bug == "drop_bias" else z + b

    def logsumexp_rows(z):
        z = np.asarray(z, np.float64)
        if bug == "max_only":
            return z.max(axis=1)
        if bug == "no_shift":
            with np.errstate(over="ignore", divide="ignore"):
                return np.log(np.exp(z).sum(axis=1))
        if bug == "over_rows":
            mx = z.max(axis=0, keepdims=True)
            l = (mx + np.log(np.exp(z - mx).sum(axis=0, keepdims=True)))[0]
            return np.resize(l, z.shape[0])
        mx = z.max(axis=1, keepdims=True)
        s = np.exp(z - mx).sum(axis=1, keepdims=True)
        if bug == "mean":
            s = s / z.shape[1]
        return (mx + np.log(s))[:, 0]

    def leaky_relu(v):
        v = np.asarray(v, np.float64)
        slope = {"slope_0.1": 0.1, "relu": 0.0}.get(bug, 0.01)
        return np.where(v > 0, v, slope * v)

    def gelu(v):
        v = np.asarray(v, np.float64)
        if bug == "tanh_gelu":
            return 0.5 * v * (1 + np.tanh(math.sqrt(2 / math.pi) * (v + 0.044715 * v ** 3)))
        if bug == "sigmoid_gelu":
            return v / (1 + np.exp(-1.702 * v))
        from scipy.special import erf
        return v * 0.5 * (1 + erf(v / math.sqrt(2)))

    def linear_lse_forward(x, W, b, return_lse=False):
        l = logsumexp_rows(linear(x, W, b))
        v = leaky_relu(l) if bug == "one_leaky" else leaky_relu(leaky_relu(l))
        if bug == "one_gelu":
            out = gelu(v)
        elif bug == "gelu_first":
            out = leaky_relu(leaky_relu(gelu(gelu(l))))
        else:
            out = gelu(gelu(v))
        return (out, l) if return_lse else out

    return types.SimpleNamespace(linear=linear, logsumexp_rows=logsumexp_rows,
                                 leaky_relu=leaky_relu, gelu=gelu,
                                 linear_lse_forward=linear_lse_forward)


BUGS = ["drop_bias", "max_only", "no_shift", "over_rows", "mean", "slope_0.1", "relu",
        "tanh_gelu", "sigmoid_gelu", "one_leaky", "one_gelu", "gelu_first"]


def test_clean_model_passes_every_pin():
    m = _model()
    for check in pins.ALL_CHECKS:
        check(m)


@pytest.mark.parametrize("bug", BUGS)
def test_each_planted_mistake_fails_a_pin(bug):
    m = _model(bug)
    failed = []
    for check in pins.ALL_CHECKS:
        try:
            check(m)
        except AssertionError:
            failed.append(check.__name__)
    assert failed, "planted mistake %r passed every pin" % bug
