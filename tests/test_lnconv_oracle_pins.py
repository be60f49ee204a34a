"""The fp64 oracle of the fourth method (LayerNorm -> GELU -> dilated Conv1d
-> + input) against its pins, and each planted mistake in a numpy model
against the same pins.  CPU only."""
import math
import types

import numpy as np
import pytest

import oracle
import lnconv_oracle_pins as pins

ORACLE = types.SimpleNamespace(gelu_tanh=oracle.gelu_tanh, ln_gelu_conv1d=oracle.ln_gelu_conv1d,
                               ln_gelu_conv1d_cols=oracle.ln_gelu_conv1d_cols)


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_lnconv_oracle_pin(check):
    check(ORACLE)


def test_lnconv_oracle_rejects_bad_arguments_and_takes_empty_batch():
    z = np.zeros
    with pytest.raises(ValueError):
        oracle.ln_gelu_conv1d(z((1, 2, 4)), z((2, 4)), z((2, 4)), z((2, 2, 3)), z(2), 0, 1e-5)
    with pytest.raises(ValueError):
        oracle.ln_gelu_conv1d_cols(z((1, 2, 4)), z((2, 4)), z((2, 4)), z((2, 2, 3)), z(2), 1,
                                   1e-5, [(0, 4)])
    out = oracle.ln_gelu_conv1d(z((0, 2, 4)), z((2, 4)), z((2, 4)), z((2, 2, 3)), z(2), 1, 1e-5)
    assert out.shape == (0, 2, 4)


# ---- planted mistakes (numpy model; the oracle itself is never modified) ----

_erf = np.vectorize(math.erf)


def _model(bug=None):
    def gelu_tanh(v):
        v = np.asarray(v, np.float64)
        k = math.sqrt(2.0 / math.pi)
        return 0.5 * v * (1.0 + np.tanh(k * (v + 0.044715 * v ** 3)))

    def gelu_exact(v):
        return v * 0.5 * (1.0 + _erf(np.asarray(v, np.float64) / math.sqrt(2.0)))

    def forward(x, ln_w, ln_b, conv_w, conv_b, dilation, eps, gelu_tanh_form=False):
        x = np.asarray(x, np.float64)
        B, C, L = x.shape
        d = 1 if bug == "dilation1" else int(dilation)
        if bug == "ln_per_channel":
            mean = x.mean(axis=2, keepdims=True)
            var = x.var(axis=2, keepdims=True)
        else:
            mean = x.reshape(B, -1).mean(axis=1)[:, None, None]
            var = x.reshape(B, -1).var(axis=1, ddof=1 if bug == "ln_unbiased" else 0)[:, None, None]
        if bug == "eps_outside":
            n = (x - mean) / (np.sqrt(var) + eps)
        else:
            n = (x - mean) / np.sqrt(var + eps)
        use_tanh = (not gelu_tanh_form) if bug == "gelu_swapped" else gelu_tanh_form
        act = gelu_tanh if use_tanh else gelu_exact
        if bug == "affine_after_gelu":
            g = act(n) * ln_w + ln_b
        else:
            g = act(n * ln_w + ln_b)
        # padded g: positions outside [0, L) are 0, or, planted, the activation of a raw 0
        pad_val = np.zeros((B, C, 1))
        if bug == "pad_raw_x":
            pad_val = act((0.0 - mean) / np.sqrt(var + eps)) * np.ones((B, C, 1))
        gp = np.concatenate([np.repeat(pad_val, 2 * d, axis=2), g, np.repeat(pad_val, 2 * d, axis=2)], axis=2)
        offs = [-d, 0, d]
        if bug == "flipped_taps":
            offs = offs[::-1]
        if bug == "causal":
            offs = [-2 * d, -d, 0]
        out = np.zeros_like(x)
        for t in range(3):
            sl = gp[:, :, 2 * d + offs[t]: 2 * d + offs[t] + L]
            out += np.einsum("oc,bcl->bol", conv_w[:, :, t], sl)
        if bug != "no_conv_bias":
            out += np.asarray(conv_b)[None, :, None]
        if bug == "residual_g":
            out += g
        elif bug != "no_residual":
            out += x
        return out, g, mean.reshape(B, -1)[:, 0] if bug != "ln_per_channel" else mean[:, 0, 0], \
            var.reshape(B, -1)[:, 0] if bug != "ln_per_channel" else var[:, 0, 0]

    def ln_gelu_conv1d(x, ln_w, ln_b, conv_w, conv_b, dilation, eps, gelu_tanh=False,
                       return_parts=False):
        out, g, mean, var = forward(x, ln_w, ln_b, conv_w, conv_b, dilation, eps, gelu_tanh)
        return (out, g, mean, var) if return_parts else out

    def ln_gelu_conv1d_cols(x, ln_w, ln_b, conv_w, conv_b, dilation, eps, cols, gelu_tanh=False):
        out = forward(x, ln_w, ln_b, conv_w, conv_b, dilation, eps, gelu_tanh)[0]
        return np.stack([out[b, :, j] for b, j in cols])

    return types.SimpleNamespace(gelu_tanh=gelu_tanh, ln_gelu_conv1d=ln_gelu_conv1d,
                                 ln_gelu_conv1d_cols=ln_gelu_conv1d_cols)


BUGS = ["dilation1", "ln_per_channel", "ln_unbiased", "eps_outside", "gelu_swapped",
        "affine_after_gelu", "pad_raw_x", "flipped_taps", "causal", "no_conv_bias", "residual_g",
        "no_residual"]


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
