"""Pins of the oracle's packed variable-length batches (CPU only).

The recurrence of the burn-gdn2 README ("Architecture") runs per sequence from
that sequence's own initial state (empty when none is given, README "Quick
start").  A packed batch puts N sequences back to back on the token axis,
sequence i holding tokens cu_seqlens[i] .. cu_seqlens[i+1]-1.  The pins fix
that by reductions to the unpacked recurrence (one sequence; equal lengths =
an ordinary batch), by isolation (no sequence sees another's tokens or state),
by the empty sequence, and by a closed form for one-token sequences; planted
slips show that each is needed.
"""
import numpy as np
import pytest

from oracle import c_oracle
from oracle.reference import chunked_wy, recurrent, rel_l2, varlen


def _draw(rng, T, H=2, dk=8, dv=6, N=None, s0=True):
    k = rng.standard_normal((1, T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    q = rng.standard_normal((1, T, H, dk))
    v = rng.standard_normal((1, T, H, dv))
    a = 1 / (1 + np.exp(-rng.standard_normal((1, T, H, dk)) - 2))
    b = 2 / (1 + np.exp(-rng.standard_normal((1, T, H, dk))))
    w = 1 / (1 + np.exp(-rng.standard_normal((1, T, H, dv))))
    S0 = rng.standard_normal((N, H, dk, dv)) * 0.3 if (s0 and N) else None
    return q, k, v, a, b, w, S0


def check_one_sequence_is_plain(fn=varlen):
    rng = np.random.default_rng(1)
    x = _draw(rng, 11, N=1)
    o, S = fn([0, 11], *x)
    o1, S1 = recurrent(*x)
    np.testing.assert_allclose(o, o1, rtol=0, atol=1e-13)
    np.testing.assert_allclose(S, S1, rtol=0, atol=1e-13)


def check_equal_lengths_are_a_batch(fn=varlen):
    """Three sequences of 5 tokens packed = an ordinary batch of three."""
    rng = np.random.default_rng(2)
    N, L = 3, 5
    q, k, v, a, b, w, S0 = _draw(rng, N * L, N=N)
    o, S = fn([0, 5, 10, 15], q, k, v, a, b, w, S0)
    unpack = lambda x: x.reshape(N, L, *x.shape[2:])
    ob, Sb = recurrent(*(unpack(x) for x in (q, k, v, a, b, w)), S0)
    np.testing.assert_allclose(o.reshape(N, L, *o.shape[2:]), ob, rtol=0, atol=1e-13)
    np.testing.assert_allclose(S, Sb, rtol=0, atol=1e-13)


def check_sequences_are_isolated(fn=varlen):
    """Changing one sequence's tokens or initial state changes nothing in the others."""
    rng = np.random.default_rng(3)
    cu = [0, 4, 9, 9, 16]
    x = list(_draw(rng, 16, N=4))
    o, S = fn(cu, *x)
    y = [t.copy() for t in x]
    for t in y[:6]:
        t[:, 4:9] = rng.standard_normal(t[:, 4:9].shape) * 0.5 + 0.5    # sequence 1's tokens
    y[6][1] += 1.0                                                      # and its S0
    o2, S2 = fn(cu, *y)
    for i in (0, 2, 3):
        np.testing.assert_array_equal(S2[i], S[i])
        np.testing.assert_array_equal(o2[:, cu[i]:cu[i + 1]], o[:, cu[i]:cu[i + 1]])
    assert not np.allclose(S2[1], S[1])


def check_empty_sequence_keeps_its_state(fn=varlen):
    rng = np.random.default_rng(4)
    x = _draw(rng, 7, N=3)
    _, S = fn([0, 3, 3, 7], *x)
    np.testing.assert_array_equal(S[1], x[6][1])
    _, Sz = fn([0, 3, 3, 7], *x[:6], None)
    np.testing.assert_array_equal(Sz[1], 0.0)


def check_one_token_sequences_closed_form(fn=varlen):
    """From an empty state one token gives S = k (w*v)^T and o = (q.k) (w*v): packing
    one-token sequences must reproduce that for every token."""
    rng = np.random.default_rng(5)
    T = 6
    q, k, v, a, b, w, _ = _draw(rng, T, N=None)
    o, S = fn(list(range(T + 1)), q, k, v, a, b, w, None)
    u = w * v
    np.testing.assert_allclose(o[0], np.sum(q * k, -1)[0][..., None] * u[0], rtol=0, atol=1e-13)
    np.testing.assert_allclose(S, np.einsum("thc,thj->thcj", k[0], u[0]), rtol=0, atol=1e-13)


CHECKS = [check_one_sequence_is_plain, check_equal_lengths_are_a_batch, check_sequences_are_isolated,
          check_empty_sequence_keeps_its_state, check_one_token_sequences_closed_form]


@pytest.mark.parametrize("chk", CHECKS, ids=lambda c: c.__name__)
def test_varlen_pin(chk):
    chk()


@pytest.mark.parametrize("cu", [[1, 5], [0, 4], [0, 3, 2, 5], [0, 6, 5]])
def test_bad_offsets(cu):
    x = _draw(np.random.default_rng(6), 5, N=len(cu) - 1)
    with pytest.raises(ValueError):
        varlen(cu, *x)


def test_varlen_forms_agree():
    """Chunked and C forms per sequence agree with the literal recurrence (lengths across
    the 64-token chunk boundary)."""
    rng = np.random.default_rng(7)
    cu = [0, 1, 64, 64, 130, 200]
    x = [t.astype(np.float32).astype(np.float64) if t is not None else None
         for t in _draw(rng, 200, H=2, dk=16, dv=8, N=5)]
    o, S = varlen(cu, *x)
    oc, Sc = varlen(cu, *x, form=lambda *a: chunked_wy(*a, chunk=64))
    ox, Sx = varlen(cu, *x, form=c_oracle.recurrent)
    assert rel_l2(oc, o) < 1e-12 and rel_l2(Sc, S) < 1e-12
    assert rel_l2(ox, o) < 1e-13 and rel_l2(Sx, S) < 1e-13


# ---- planted slips: each must fail at least one pin --------------------------
def _mutant(kind):
    def mutated(cu, q, k, v, alpha, b, w, S0=None):
        T, H, dk, dv = v.shape[1], v.shape[2], alpha.shape[3], v.shape[3]
        N = len(cu) - 1
        o = np.zeros((1, T, H, dv))
        S = np.zeros((N, H, dk, dv))
        carry = None
        for i in range(N):
            s, e = cu[i], cu[i + 1]
            if kind == "shift" and i > 0:
                s = min(s + 1, e)
            s0 = None if S0 is None else S0[i:i + 1]
            if kind == "s0_first" and S0 is not None:
                s0 = S0[0:1]
            if kind == "carry" and carry is not None:
                s0 = carry
            sl = lambda x: x[:, s:e]
            if e == s:
                S[i] = 0.0 if s0 is None else s0[0]
                carry = S[i:i + 1]
                continue
            oi, Si = recurrent(sl(q), sl(k), sl(v), sl(alpha), sl(b), sl(w), s0)
            o[:, s:e] = oi
            S[i] = Si[0]
            carry = Si
        return o, S
    return mutated


@pytest.mark.parametrize("kind", ["carry", "shift", "s0_first"])
def test_varlen_mutant_is_rejected(kind):
    bad = _mutant(kind)
    failed = []
    for chk in CHECKS:
        try:
            chk(fn=bad)
        except AssertionError:
            failed.append(chk.__name__)
    assert failed, f"varlen mutant {kind} passed every pin"


def test_correct_varlen_passes_the_mutant_harness():
    good = _mutant("none")
    for chk in CHECKS:
        chk(fn=good)
