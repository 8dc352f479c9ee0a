"""The oracle's pins must reject plausible mistakes (CPU only).

Each mutant below is a copy of the sequential recurrence with one planted
slip.  For every mutant at least one pin (hand-worked example, special case
or invariant from ``test_oracle_pins``) must fail, which shows the pins
constrain every term of the burn-gdn2 README's per-token formula
("Architecture" section) rather than restating it.
"""
import numpy as np
import pytest

import test_oracle_pins as pins


def _make(step):
    """Build a recurrence from a per-head step(S, q, k, v, alpha, b, w) -> (o_t, S_t)."""
    def rec(q, k, v, alpha, b, w, S0=None):
        q, k, v, alpha, b, w = (np.asarray(x, dtype=np.float64) for x in (q, k, v, alpha, b, w))
        B, T, H, dk = q.shape
        dv = v.shape[-1]
        S = np.zeros((B, H, dk, dv)) if S0 is None else np.array(S0, dtype=np.float64)
        o = np.zeros((B, T, H, dv))
        for t in range(T):
            for bi in range(B):
                for hi in range(H):
                    o[bi, t, hi], S[bi, hi] = step(S[bi, hi], q[bi, t, hi], k[bi, t, hi], v[bi, t, hi],
                                                   alpha[bi, t, hi], b[bi, t, hi], w[bi, t, hi])
        return o, S
    return rec


def _correct(S, q, k, v, a, b, w):
    X = (np.eye(len(k)) - np.outer(k, b * k)) @ (a[:, None] * S) + np.outer(k, w * v)
    return q @ X, X


MUTANTS = {
    "b_on_other_side": lambda S, q, k, v, a, b, w: (lambda X: (q @ X, X))(
        (np.eye(len(k)) - np.outer(b * k, k)) @ (a[:, None] * S) + np.outer(k, w * v)),
    "erase_before_decay": lambda S, q, k, v, a, b, w: (lambda X: (q @ X, X))(
        a[:, None] * ((np.eye(len(k)) - np.outer(k, b * k)) @ S) + np.outer(k, w * v)),
    "decay_after_write": lambda S, q, k, v, a, b, w: (lambda X: (q @ X, X))(
        a[:, None] * ((np.eye(len(k)) - np.outer(k, b * k)) @ S + np.outer(k, w * v))),
    "read_before_update": lambda S, q, k, v, a, b, w: (q @ S, _correct(S, q, k, v, a, b, w)[1]),
    "no_write_gate": lambda S, q, k, v, a, b, w: _correct(S, q, k, v, a, b, np.ones_like(w)),
    "no_erase": lambda S, q, k, v, a, b, w: (lambda X: (q @ X, X))(a[:, None] * S + np.outer(k, w * v)),
    "no_decay": lambda S, q, k, v, a, b, w: _correct(S, q, k, v, np.ones_like(a), b, w),
    "erase_sign": lambda S, q, k, v, a, b, w: (lambda X: (q @ X, X))(
        (np.eye(len(k)) + np.outer(k, b * k)) @ (a[:, None] * S) + np.outer(k, w * v)),
    "no_erase_gate": lambda S, q, k, v, a, b, w: _correct(S, q, k, v, a, np.ones_like(b), w),
    "write_gate_on_key": lambda S, q, k, v, a, b, w: (lambda X: (q @ X, X))(
        (np.eye(len(k)) - np.outer(k, b * k)) @ (a[:, None] * S) + np.outer(k * w.mean(), v)),
    "decay_squared": lambda S, q, k, v, a, b, w: _correct(S, q, k, v, a * a, b, w),
    "erase_reads_undecayed": lambda S, q, k, v, a, b, w: (lambda X: (q @ X, X))(
        a[:, None] * S - np.outer(k, (b * k) @ S) + np.outer(k, w * v)),
}

CHECKS = [getattr(pins, n) for n in dir(pins) if n.startswith("check_")]


def _golden_check(rec):
    for case in pins._golden_cases():
        _, a, S0, o_ref, S_ref = case
        o, S = rec(a["q"], a["k"], a["v"], a["alpha"], a["b"], a["w"], S0)
        np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
        np.testing.assert_allclose(S, S_ref, rtol=0, atol=1e-12)


def test_correct_step_passes_all_pins():
    rec = _make(_correct)
    _golden_check(rec)
    for chk in CHECKS:
        chk(recurrent=rec)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_rejected(name):
    rec = _make(MUTANTS[name])
    failed = []
    for chk in CHECKS + [lambda recurrent: _golden_check(recurrent)]:
        try:
            chk(recurrent=rec)
        except Exception:          # an assertion, or a shape error for a transposed operand
            failed.append(getattr(chk, "__name__", "golden"))
    assert failed, f"mutant {name} passed every pin"
