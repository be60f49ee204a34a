"""Each plausible mistake, planted in a numpy re-implementation of the forward
(on the CPU, never in the HIP path), must fail at least one oracle pin, and
the same numpy implementation without a mistake must pass every pin.  This
shows the pins are strong enough to catch the mistakes they are meant for."""
import types

import numpy as np
import pytest

import oracle_pins


def _make(linear_bug=None, swish_bug=None, gn_bug=None, order_bug=None):
    def linear(x, W, b):
        x, W, b = (np.asarray(a, np.float64) for a in (x, W, b))
        # one matrix-vector product per row keeps rows bitwise independent
        if linear_bug == "layout_kn":          # reads W as [K, N]
            Wt = W.reshape(x.shape[1], -1).T.copy()
        else:
            Wt = W
        z = np.stack([Wt @ x[m] for m in range(x.shape[0])]) if x.shape[0] else \
            np.zeros((0, Wt.shape[0]))
        if linear_bug == "drop_bias":
            return z
        if linear_bug == "first_row_only":
            return np.repeat(z[:1], x.shape[0], 0) + b
        return z + b

    def swish(z):
        z = np.asarray(z, np.float64)
        if swish_bug == "sign":
            return z / (1.0 + np.exp(z))
        if swish_bug == "sigmoid_only":
            return 1.0 / (1.0 + np.exp(-z))
        if swish_bug == "missing_one":
            return z / np.exp(-z)
        return z * (1.0 / (1.0 + np.exp(-z)))

    def groupnorm(u, gamma, beta, G, eps, return_stats=False):
        u = np.asarray(u, np.float64)
        M, N = u.shape
        C = N // G
        if gn_bug == "interleaved":
            ug = u.reshape(M, C, G).transpose(0, 2, 1)
        else:
            ug = u.reshape(M, G, C)
        mean = ug.mean(axis=2)
        var = ug.var(axis=2, ddof=1 if (gn_bug == "unbiased" and C > 1) else 0)
        d = ug - mean[..., None]
        if gn_bug == "eps_outside":
            n = d / (np.sqrt(var)[..., None] + eps)
        elif gn_bug == "no_center":
            n = ug / np.sqrt(var + eps)[..., None]
        else:
            n = d / np.sqrt(var + eps)[..., None]
        if gn_bug == "interleaved":
            n = n.transpose(0, 2, 1).reshape(M, N)
        else:
            n = n.reshape(M, N)
        ga, be = np.asarray(gamma, np.float64), np.asarray(beta, np.float64)
        if gn_bug == "affine_per_group":
            ga = np.repeat(ga[::C][:G], C)
            be = np.repeat(be[::C][:G], C)
        if gn_bug == "affine_swapped":
            ga, be = be, ga
        y = n * ga + be
        return (y, mean, var) if return_stats else y

    def lgn_forward(x, W, b_lin, b_add, gamma, beta, G, eps):
        b_add = np.asarray(b_add, np.float64)
        if order_bug == "b_lin_after_swish":
            u = swish(linear(x, W, np.zeros_like(b_add))) + np.asarray(b_lin) + b_add
        elif order_bug == "b_add_before_swish":
            u = swish(linear(x, W, b_lin) + b_add)
        else:
            u = swish(linear(x, W, b_lin)) + b_add
        return groupnorm(u, gamma, beta, G, eps)

    return types.SimpleNamespace(swish=swish, linear=linear, groupnorm=groupnorm,
                                 lgn_forward=lgn_forward)


MUTANTS = {
    "weight_read_as_KxN": dict(linear_bug="layout_kn"),
    "linear_bias_dropped": dict(linear_bug="drop_bias"),
    "rows_mixed_up": dict(linear_bug="first_row_only"),
    "sigmoid_sign_flipped": dict(swish_bug="sign"),
    "swish_missing_factor_z": dict(swish_bug="sigmoid_only"),
    "sigmoid_missing_one": dict(swish_bug="missing_one"),
    "groups_interleaved": dict(gn_bug="interleaved"),
    "unbiased_variance": dict(gn_bug="unbiased"),
    "eps_outside_sqrt": dict(gn_bug="eps_outside"),
    "mean_not_subtracted": dict(gn_bug="no_center"),
    "affine_per_group": dict(gn_bug="affine_per_group"),
    "gamma_beta_swapped": dict(gn_bug="affine_swapped"),
    "linear_bias_after_swish": dict(order_bug="b_lin_after_swish"),
    "add_bias_before_swish": dict(order_bug="b_add_before_swish"),
}


def _failures(impl):
    failed = []
    for check in oracle_pins.ALL_CHECKS:
        try:
            check(impl)
        except Exception:  # noqa: BLE001 -- any failure counts
            failed.append(check.__name__)
    return failed


def test_clean_numpy_model_passes_every_pin():
    assert _failures(_make()) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    failed = _failures(_make(**MUTANTS[name]))
    assert failed, "mutant %s passed every pin" % name
