"""The fp64 oracle of the third method (Swish -> spatial GroupNorm ->
HardSwish) against its pins, and each planted mistake in a numpy model
against the same pins.  CPU only."""
import types

import numpy as np
import pytest

import oracle
import sgh_oracle_pins as pins

ORACLE = types.SimpleNamespace(hardswish=oracle.hardswish,
                               swish_gn_hardswish=oracle.swish_gn_hardswish)


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_sgh_oracle_pin(check):
    check(ORACLE)


def test_sgh_oracle_rejects_bad_groups_and_takes_empty_batch():
    with pytest.raises(ValueError):
        oracle.swish_gn_hardswish(np.zeros((1, 6, 2)), np.ones(6), np.zeros(6), 4, 1e-5)
    out = oracle.swish_gn_hardswish(np.zeros((0, 4, 3)), np.ones(4), np.zeros(4), 2, 1e-5)
    assert out.shape == (0, 4, 3)


# ---- planted mistakes (numpy model; the oracle itself is never modified) ----

def _model(bug=None):
    def hardswish(v):
        v = np.asarray(v, np.float64)
        if bug == "no_x":
            return np.clip(v + 3, 0, 6) / 6
        if bug == "clamp3":
            return v * np.clip(v + 3, 0, 3) / 6
        if bug == "relu6":
            return np.clip(v, 0, 6)
        return v * np.clip(v + 3, 0, 6) / 6

    def swish_gn_hardswish(y, gamma, beta, G, eps, return_parts=False):
        y = np.asarray(y, np.float64)
        Nb, C = y.shape[:2]
        s = y if bug == "no_swish" else y / (1.0 + np.exp(-y))
        if bug == "hardswish_first":
            s = hardswish(s)
        if bug == "instance":
            grp = s.reshape(Nb, C, -1)
        elif bug == "layer":
            grp = s.reshape(Nb, 1, -1)
        elif bug == "interleaved":
            grp = s.reshape(Nb, C // G, G, -1).transpose(0, 2, 1, 3).reshape(Nb, G, -1)
        else:
            grp = s.reshape(Nb, G, -1)
        mean = grp.mean(axis=2, keepdims=True)
        var = grp.var(axis=2, keepdims=True, ddof=1 if bug == "unbiased" else 0)
        if bug == "eps_outside":
            n = (grp - mean) / (np.sqrt(var) + eps)
        else:
            n = (grp - mean) / np.sqrt(var + eps)
        if bug == "interleaved":
            n = n.reshape(Nb, G, C // G, -1).transpose(0, 2, 1, 3)
        n = n.reshape(y.shape)
        bshape = (1, C) + (1,) * (y.ndim - 2)
        a = n * np.asarray(gamma).reshape(bshape) + np.asarray(beta).reshape(bshape)
        out = a if bug == "hardswish_first" else hardswish(a)
        if return_parts:
            flat = s.reshape(Nb, G, -1)
            return out, n, flat.mean(axis=2), flat.var(axis=2)
        return out

    return types.SimpleNamespace(hardswish=hardswish, swish_gn_hardswish=swish_gn_hardswish)


BUGS = ["no_x", "clamp3", "relu6", "no_swish", "hardswish_first", "instance", "layer",
        "interleaved", "unbiased", "eps_outside"]


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
