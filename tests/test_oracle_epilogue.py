"""Pins of the oracle's output step, the gated RMS norm (CPU only).

burn-gdn2 README (docs.rs), "Architecture" diagram: the core's output goes
through a "Gated RMS Norm" fed by a "SiLU Gate"; "Configuration" gives
norm_eps = 1e-5.  Reading: y = o / sqrt(mean over d_v of o^2 + eps) * weight
* g * sigmoid(g), per (token, head), one weight of length d_v for all heads.
The pins fix it by closed forms and invariants; planted slips show each pin
is needed.
"""
import math

import numpy as np
import pytest

from oracle.reference import NORM_EPS, gated_rmsnorm


def _inputs(rng, shape=(2, 5, 3, 16)):
    o = rng.standard_normal(shape) * 2.0
    g = rng.standard_normal(shape)
    wt = rng.standard_normal(shape[-1]) + 1.0
    return o, g, wt


def check_constant_row(f=gated_rmsnorm):
    """o = c (all channels), weight = 1, g = ln 3 (silu = 0.75 ln 3): y = c / sqrt(c^2 + eps) * 0.75 ln 3."""
    c = 2.5
    o = np.full((1, 1, 1, 8), c)
    g = np.full_like(o, math.log(3.0))
    y = f(o, g, np.ones(8))
    np.testing.assert_allclose(y, c / math.sqrt(c * c + NORM_EPS) * 0.75 * math.log(3.0), rtol=1e-14, atol=0)


def check_rms_of_output(f=gated_rmsnorm):
    """With weight = 1 and silu(g) = 1 replaced by dividing it out, each row has RMS ~ 1."""
    rng = np.random.default_rng(2)
    o, g, _ = _inputs(rng)
    y = f(o, g, np.ones(o.shape[-1]))
    z = y / (g / (1 + np.exp(-g)))
    np.testing.assert_allclose(np.sqrt(np.mean(z * z, axis=-1)), 1.0, rtol=0, atol=1e-5)


def check_zero_gate_silences(f=gated_rmsnorm):
    rng = np.random.default_rng(3)
    o, g, wt = _inputs(rng)
    np.testing.assert_array_equal(f(o, np.zeros_like(g), wt), 0.0)


def check_silu_negative_side(f=gated_rmsnorm):
    """silu(-ln 3) = -0.25 ln 3: the gate is x * sigmoid(x), not sigmoid(x) or x."""
    o = np.ones((1, 1, 1, 4))
    y = f(o, np.full_like(o, -math.log(3.0)), np.ones(4))
    np.testing.assert_allclose(y, 1 / math.sqrt(1 + NORM_EPS) * (-0.25 * math.log(3.0)), rtol=1e-14, atol=0)


def check_scale_invariance_in_o(f=gated_rmsnorm):
    rng = np.random.default_rng(4)
    o, g, wt = _inputs(rng)
    np.testing.assert_allclose(f(7.0 * o, g, wt), f(o, g, wt), rtol=1e-5, atol=0)


def check_channelwise_weight(f=gated_rmsnorm):
    """Weight scales channel j of every row by weight[j]; rows of other heads unchanged."""
    rng = np.random.default_rng(5)
    o, g, wt = _inputs(rng)
    wt2 = wt.copy()
    wt2[3] *= 5.0
    y1, y2 = f(o, g, wt), f(o, g, wt2)
    np.testing.assert_allclose(y2[..., 3], 5.0 * y1[..., 3], rtol=1e-14, atol=0)
    np.testing.assert_array_equal(np.delete(y2, 3, axis=-1), np.delete(y1, 3, axis=-1))


def check_rows_independent(f=gated_rmsnorm):
    """The mean runs over d_v of one (token, head): changing another row leaves y unchanged."""
    rng = np.random.default_rng(6)
    o, g, wt = _inputs(rng)
    o2 = o.copy()
    o2[0, 1, 2] *= 9.0
    y1, y2 = f(o, g, wt), f(o2, g, wt)
    mask = np.ones(o.shape[:-1], bool)
    mask[0, 1, 2] = False
    np.testing.assert_array_equal(y1[mask], y2[mask])


CHECKS = [check_constant_row, check_rms_of_output, check_zero_gate_silences, check_silu_negative_side,
          check_scale_invariance_in_o, check_channelwise_weight, check_rows_independent]


@pytest.mark.parametrize("chk", CHECKS, ids=lambda c: c.__name__)
def test_epilogue_pin(chk):
    chk()


def _mutant(kind):
    def f(o, g, weight, eps=NORM_EPS):
        o, g, weight = (np.asarray(x, dtype=np.float64) for x in (o, g, weight))
        axis = -2 if kind == "mean_over_heads" else -1
        ms = np.sum(o * o, axis=axis, keepdims=True) if kind == "sum_not_mean" else np.mean(o * o, axis=axis,
                                                                                              keepdims=True)
        rms = (ms + eps) if kind == "no_sqrt" else np.sqrt(ms + eps)
        sig = 1 / (1 + np.exp(-g))
        gate = {"sigmoid_gate": sig, "plain_gate": g}.get(kind, g * sig)
        w = 1.0 if kind == "no_weight" else weight
        return o / rms * w * gate
    return f


@pytest.mark.parametrize("kind", ["mean_over_heads", "sum_not_mean", "no_sqrt", "sigmoid_gate", "plain_gate",
                                  "no_weight"])
def test_epilogue_mutant_is_rejected(kind):
    bad = _mutant(kind)
    failed = []
    for chk in CHECKS:
        try:
            chk(f=bad)
        except AssertionError:
            failed.append(chk.__name__)
    assert failed, f"epilogue mutant {kind} passed every pin"


def test_correct_epilogue_passes_the_mutant_harness():
    for chk in CHECKS:
        chk(f=_mutant("none"))
