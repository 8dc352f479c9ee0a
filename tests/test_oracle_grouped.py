"""Pins of the oracle's grouped value heads (CPU only).

burn-gdn2 README (docs.rs), "Configuration": num_v_heads sets the value
heads, by default as many as the query/key heads.  With more value heads than
query/key heads, each value head keeps its own state, gates and values and
reads the q and k of one query/key head; the README does not say which, and
the reading taken is that consecutive groups of Hv / H value heads share one
(value head hv reads head hv // (Hv / H)).  ``share_qk_heads`` widens q and k
to the value heads before the per-head recurrence.  The pins fix what the
README and the mathematics fix (no grouping is the identity; a single
query/key head is read by all value heads; every head is read equally often)
and pin the grouping reading with a run whose groups carry identical values,
then show that planted slips fail them.
"""
import numpy as np
import pytest

from oracle import c_oracle
from oracle.reference import chunked_wy, recurrent, rel_l2, share_qk_heads


def _qk(rng, B=2, T=7, H=3, dk=8):
    return rng.standard_normal((B, T, H, dk)), rng.standard_normal((B, T, H, dk))


def check_no_grouping_is_identity(share=share_qk_heads):
    q, k = _qk(np.random.default_rng(1))
    q2, k2 = share(q, k, q.shape[2])
    np.testing.assert_array_equal(q2, q)
    np.testing.assert_array_equal(k2, k)


def check_single_head_is_read_by_all(share=share_qk_heads):
    """One query/key head: every value head reads it, whatever the grouping."""
    q, k = _qk(np.random.default_rng(2), H=1)
    q2, k2 = share(q, k, 5)
    assert q2.shape == (2, 7, 5, 8) and k2.shape == (2, 7, 5, 8)
    for hv in range(5):
        np.testing.assert_array_equal(q2[:, :, hv], q[:, :, 0])
        np.testing.assert_array_equal(k2[:, :, hv], k[:, :, 0])


def check_each_head_read_equally(share=share_qk_heads):
    """Each of the H heads is read, unchanged and in the same (q, k) pair, by Hv / H value heads."""
    q, k = _qk(np.random.default_rng(3), H=3)
    q2, k2 = share(q, k, 12)
    assert q2.shape[2] == 12
    counts = np.zeros(3, int)
    for hv in range(12):
        hit = [h for h in range(3) if np.array_equal(q2[:, :, hv], q[:, :, h])]
        assert len(hit) == 1 and np.array_equal(k2[:, :, hv], k[:, :, hit[0]])
        counts[hit[0]] += 1
    assert list(counts) == [4, 4, 4]


def check_groups_are_consecutive(share=share_qk_heads):
    """The grouping reading: with the values of each group of 4 consecutive value heads
    identical, their outputs and states agree and equal the ungrouped run of that group's
    query/key head."""
    rng = np.random.default_rng(4)
    B, T, H, G, dk, dv = 1, 9, 2, 4, 8, 6
    q, k = _qk(rng, B, T, H, dk)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, dv))
    a = 1 / (1 + np.exp(-rng.standard_normal((B, T, H, dk)) - 2))
    b = 1 / (1 + np.exp(-rng.standard_normal((B, T, H, dk))))
    w = 1 / (1 + np.exp(-rng.standard_normal((B, T, H, dv))))
    rep = lambda x: np.repeat(x, G, axis=2)          # value head hv carries group hv // G's values
    qg, kg = share(q, k, H * G)
    og, Sg = recurrent(qg, kg, rep(v), rep(a), rep(b), rep(w))
    o1, S1 = recurrent(q, k, v, a, b, w)
    for hv in range(H * G):
        np.testing.assert_allclose(og[:, :, hv], o1[:, :, hv // G], rtol=0, atol=1e-13)
        np.testing.assert_allclose(Sg[:, hv], S1[:, hv // G], rtol=0, atol=1e-13)


CHECKS = [check_no_grouping_is_identity, check_single_head_is_read_by_all, check_each_head_read_equally,
          check_groups_are_consecutive]


@pytest.mark.parametrize("chk", CHECKS, ids=lambda c: c.__name__)
def test_grouped_pin(chk):
    chk()


@pytest.mark.parametrize("Hv", [0, 4, 2, -3])
def test_bad_value_head_counts(Hv):
    q, k = _qk(np.random.default_rng(5), H=3)
    with pytest.raises(ValueError):
        share_qk_heads(q, k, Hv)


def test_grouped_chunked_matches_recurrent_and_c_oracle():
    """The widened q/k feed both oracle forms and the C oracle alike (T spans two chunks)."""
    rng = np.random.default_rng(6)
    B, T, H, Hv, dk, dv = 1, 70, 2, 6, 16, 8
    f32 = lambda x: x.astype(np.float32).astype(np.float64)
    q, k = _qk(rng, B, T, H, dk)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    q, k = f32(q), f32(k)
    v = f32(rng.standard_normal((B, T, Hv, dv)))
    a = f32(1 / (1 + np.exp(-rng.standard_normal((B, T, Hv, dk)) - 3)))
    b = f32(1 / (1 + np.exp(-rng.standard_normal((B, T, Hv, dk)))))
    w = f32(1 / (1 + np.exp(-rng.standard_normal((B, T, Hv, dv)))))
    qg, kg = share_qk_heads(q, k, Hv)
    o_r, S_r = recurrent(qg, kg, v, a, b, w)
    o_c, S_c = chunked_wy(qg, kg, v, a, b, w, chunk=64)
    o_x, S_x = c_oracle.recurrent(np.ascontiguousarray(qg), np.ascontiguousarray(kg), v, a, b, w, None)
    assert rel_l2(o_c, o_r) < 1e-12 and rel_l2(S_c, S_r) < 1e-12
    assert rel_l2(o_x, o_r) < 1e-13 and rel_l2(S_x, S_r) < 1e-13


# ---- planted slips: each must fail at least one pin --------------------------
def _mutant(kind):
    def mutated(q, k, Hv):
        q, k = np.asarray(q, np.float64), np.asarray(k, np.float64)
        H = q.shape[2]
        G = Hv // H
        if kind == "modulo":                  # value head hv reads head hv % H
            src = np.arange(Hv) % H
        elif kind == "first_head":            # every value head reads head 0
            src = np.zeros(Hv, int)
        elif kind == "swap_qk":               # q and k of different heads
            src = np.arange(Hv) // G
            return q[:, :, src], k[:, :, (src + 1) % H]
        elif kind == "no_widen":
            return q, k
        else:
            src = np.arange(Hv) // G
        return q[:, :, src], k[:, :, src]
    return mutated


@pytest.mark.parametrize("kind", ["modulo", "first_head", "swap_qk", "no_widen"])
def test_grouped_mutant_is_rejected(kind):
    bad = _mutant(kind)
    failed = []
    for chk in CHECKS:
        try:
            chk(share=bad)
        except (AssertionError, ValueError, IndexError):
            failed.append(chk.__name__)
    assert failed, f"grouping mutant {kind} passed every pin"


def test_correct_grouping_passes_the_mutant_harness():
    good = _mutant("none")
    for chk in CHECKS:
        chk(share=good)
