"""The fp64 CPU oracle against its pins (closed forms, library routines,
special cases, invariants, a hand-derived example).  CPU only."""
import types

import numpy as np
import pytest

import oracle
import oracle_pins


ORACLE = types.SimpleNamespace(
    swish=oracle.swish,
    linear=oracle.linear,
    groupnorm=oracle.groupnorm,
    lgn_forward=oracle.lgn_forward,
)


@pytest.mark.parametrize("check", oracle_pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(check):
    check(ORACLE)


def test_oracle_swish_scalar_matches_array():
    z = np.linspace(-50, 50, 1001)
    assert np.array_equal(oracle.swish(z), np.array([oracle.swish_scalar(v) for v in z]))


def test_oracle_empty_and_degenerate_shapes():
    # M = 0: nothing to compute
    y = oracle.lgn_forward(np.zeros((0, 4)), np.ones((8, 4)), np.zeros(8), np.zeros(8),
                           np.ones(8), np.zeros(8), 2, 1e-5)
    assert y.shape == (0, 8)
    # K = 0: the linear layer is just its bias
    b_lin = np.linspace(-1, 1, 8)
    y0 = oracle.lgn_forward(np.zeros((3, 0)), np.zeros((8, 0)), b_lin, np.zeros(8),
                            np.ones(8), np.zeros(8), 2, 1e-5)
    u = oracle.swish(b_lin)[None, :]
    assert np.array_equal(y0, np.repeat(oracle.groupnorm(u, np.ones(8), np.zeros(8), 2, 1e-5), 3, 0))


def test_oracle_rejects_bad_group_count():
    with pytest.raises(ValueError):
        oracle.lgn_forward(np.zeros((2, 4)), np.ones((6, 4)), np.zeros(6), np.zeros(6),
                           np.ones(6), np.zeros(6), 4, 1e-5)
