"""Pins of the oracle's prologue options (CPU only).

burn-gdn2 README (docs.rs), "Architecture" diagram: the gate projections and
L2-Norm of q and k come right before the recurrence; "Configuration" lists
allow_neg_eigval ("b x 2").  The README does not name the gate activation;
the logistic sigmoid is the reading taken (the synthetic workloads draw their
gates as sigmoids of normal logits).  The pins below fix the prologue by
closed forms and invariants, and a set of planted slips shows that each of
them is needed.
"""
import math

import numpy as np
import pytest

from oracle import c_oracle
from oracle.reference import (FLAG_GATE_LOGITS, FLAG_NEG_EIGVAL, FLAG_QK_L2NORM, prologue, recurrent,
                              rel_l2)

ALL = FLAG_GATE_LOGITS | FLAG_NEG_EIGVAL | FLAG_QK_L2NORM


def _inputs(rng, shape=(2, 5, 3, 8), dv=6):
    B, T, H, dk = shape
    q = rng.standard_normal(shape) * 3.0
    k = rng.standard_normal(shape) * 0.5
    a = rng.standard_normal(shape) + 2.0
    b = rng.standard_normal(shape)
    w = rng.standard_normal((B, T, H, dv))
    return q, k, a, b, w


def check_logistic_closed_forms(prologue=prologue):
    """sigmoid(0) = 1/2, sigmoid(ln 3) = 3/4, sigmoid(-ln 3) = 1/4 on every gate."""
    x = np.array([0.0, math.log(3.0), -math.log(3.0)]).reshape(1, 1, 1, 3)
    q = np.ones_like(x)
    _, _, a, b, w = prologue(q, q, x, x, x, FLAG_GATE_LOGITS)
    for g in (a, b, w):
        np.testing.assert_allclose(g.ravel(), [0.5, 0.75, 0.25], rtol=0, atol=1e-15)


def check_logistic_symmetry(prologue=prologue):
    """sigmoid(x) + sigmoid(-x) = 1 and sigmoid is increasing, with limits 0 and 1."""
    x = np.linspace(-30, 30, 61).reshape(1, 1, 1, 61)
    q = np.ones_like(x)
    _, _, a, _, _ = prologue(q, q, x, x, x, FLAG_GATE_LOGITS)
    _, _, am, _, _ = prologue(q, q, -x, -x, -x, FLAG_GATE_LOGITS)
    np.testing.assert_allclose(a + am, 1.0, rtol=0, atol=1e-15)
    assert np.all(np.diff(a.ravel()) > 0)
    assert a.ravel()[0] < 1e-12 and a.ravel()[-1] > 1 - 1e-12


def check_neg_eigval_doubles_b_only(prologue=prologue):
    """b x 2 (README "Configuration"): b = 2 sigmoid(x), alpha and w unchanged."""
    rng = np.random.default_rng(3)
    q, k, a, b, w = _inputs(rng)
    _, _, a1, b1, w1 = prologue(q, k, a, b, w, FLAG_GATE_LOGITS)
    _, _, a2, b2, w2 = prologue(q, k, a, b, w, FLAG_GATE_LOGITS | FLAG_NEG_EIGVAL)
    np.testing.assert_array_equal(a1, a2)
    np.testing.assert_array_equal(w1, w2)
    np.testing.assert_allclose(b2, 2.0 * b1, rtol=0, atol=0)
    assert np.all((b2 > 0) & (b2 < 2))


def check_l2norm_unit_rows(prologue=prologue):
    """L2-Norm: every (token, head) row of q and k has unit length along d_k and keeps
    its direction; a row (3, 4) becomes (3/5, 4/5) up to the 1e-6 epsilon."""
    rng = np.random.default_rng(5)
    q, k, a, b, w = _inputs(rng)
    qn, kn, an, bn, wn = prologue(q, k, a, b, w, FLAG_QK_L2NORM)
    for x, xn in ((q, qn), (k, kn)):
        n = np.linalg.norm(xn, axis=-1)
        np.testing.assert_allclose(n, 1.0, rtol=0, atol=1e-5)
        cos = np.sum(x * xn, axis=-1) / np.linalg.norm(x, axis=-1)
        np.testing.assert_allclose(cos, 1.0, rtol=0, atol=1e-5)
    # gates untouched without GATE_LOGITS
    np.testing.assert_array_equal(an, a)
    np.testing.assert_array_equal(bn, b)
    np.testing.assert_array_equal(wn, w)
    r = np.array([3.0, 4.0]).reshape(1, 1, 1, 2)
    rn, _, _, _, _ = prologue(r, r, r, r, r, FLAG_QK_L2NORM)
    np.testing.assert_allclose(rn.ravel(), [0.6, 0.8], rtol=0, atol=1e-7)


def check_l2norm_scale_invariant(prologue=prologue):
    """Normalised rows do not depend on the rows' scale (for norms far above the epsilon)."""
    rng = np.random.default_rng(7)
    q, k, a, b, w = _inputs(rng)
    q1, k1, _, _, _ = prologue(q, k, a, b, w, FLAG_QK_L2NORM)
    q2, k2, _, _, _ = prologue(5.0 * q, 4.0 * k, a, b, w, FLAG_QK_L2NORM)
    np.testing.assert_allclose(q1, q2, rtol=0, atol=1e-6)
    np.testing.assert_allclose(k1, k2, rtol=0, atol=1e-5)


def check_no_flags_is_identity(prologue=prologue):
    rng = np.random.default_rng(11)
    x = _inputs(rng)
    out = prologue(*x, 0)
    for u, v in zip(x, out):
        np.testing.assert_array_equal(u, v)


CHECKS = [check_logistic_closed_forms, check_logistic_symmetry, check_neg_eigval_doubles_b_only,
          check_l2norm_unit_rows, check_l2norm_scale_invariant, check_no_flags_is_identity]


@pytest.mark.parametrize("chk", CHECKS, ids=lambda c: c.__name__)
def test_prologue_pin(chk):
    chk()


def test_neg_eigval_requires_logits():
    rng = np.random.default_rng(1)
    with pytest.raises(ValueError):
        prologue(*_inputs(rng), FLAG_NEG_EIGVAL)


@pytest.mark.parametrize("flags", [0, FLAG_GATE_LOGITS, FLAG_GATE_LOGITS | FLAG_NEG_EIGVAL, FLAG_QK_L2NORM, ALL])
def test_c_oracle_prologue_matches_numpy(flags):
    """The C oracle applies the same prologue in double before each token's step."""
    rng = np.random.default_rng(17)
    B, T, H, dk, dv = 2, 9, 3, 16, 12
    q, k, a, b, w = _inputs(rng, (B, T, H, dk), dv)
    v = rng.standard_normal((B, T, H, dv))
    S0 = rng.standard_normal((B, H, dk, dv)) * 0.1
    f32 = lambda x: x.astype(np.float32).astype(np.float64)
    q, k, v, a, b, w, S0 = map(f32, (q, k, v, a, b, w, S0))
    if not flags & FLAG_GATE_LOGITS:          # activated gates must be in range
        a, b, w = 1 / (1 + np.exp(-a)), 1 / (1 + np.exp(-b)), 1 / (1 + np.exp(-w))
        a, b, w = map(f32, (a, b, w))
    pq, pk, pa, pb, pw = prologue(q, k, a, b, w, flags)
    o_ref, S_ref = recurrent(pq, pk, v, pa, pb, pw, S0)
    o, S = c_oracle.recurrent(q, k, v, a, b, w, S0, flags=flags, col_block=5)
    assert rel_l2(o, o_ref) < 1e-13 and rel_l2(S, S_ref) < 1e-13


# ---- planted slips: each must fail at least one pin --------------------------
def _mutant(kind):
    def mutated(q, k, alpha, b, w, flags=0):
        q, k, alpha, b, w = (np.asarray(x, dtype=np.float64) for x in (q, k, alpha, b, w))
        sig = (lambda x: 1 / (1 + np.exp(x))) if kind == "sigmoid_sign" else (lambda x: 1 / (1 + np.exp(-x)))
        if flags & FLAG_GATE_LOGITS:
            alpha = sig(alpha) * (2.0 if (kind == "double_alpha" and flags & FLAG_NEG_EIGVAL) else 1.0)
            b = sig(b) * (2.0 if (flags & FLAG_NEG_EIGVAL and kind != "double_alpha") else 1.0)
            w = w if kind == "w_not_activated" else sig(w)
        if flags & FLAG_QK_L2NORM:
            axis = 1 if kind == "norm_over_tokens" else -1
            p = 1.0 if kind == "norm_no_sqrt" else 0.5
            q = q / (np.sum(q * q, axis=axis, keepdims=True) + 1e-6) ** p
            k = k if kind == "k_not_normalised" else k / (np.sum(k * k, axis=axis, keepdims=True) + 1e-6) ** p
        return q, k, alpha, b, w
    return mutated


@pytest.mark.parametrize("kind", ["sigmoid_sign", "double_alpha", "w_not_activated", "norm_over_tokens",
                                  "norm_no_sqrt", "k_not_normalised"])
def test_prologue_mutant_is_rejected(kind):
    bad = _mutant(kind)
    failed = []
    for chk in CHECKS:
        try:
            chk(prologue=bad)
        except AssertionError:
            failed.append(chk.__name__)
    assert failed, f"prologue mutant {kind} passed every pin"


def test_correct_prologue_passes_the_mutant_harness():
    good = _mutant("none")
    for chk in CHECKS:
        chk(prologue=good)
