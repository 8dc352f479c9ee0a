"""Pins of the comparison every parity test decides with (CPU only).

rel_l2(x, ref) = ||x - ref||_2 / ||ref||_2 over the whole tensor, in fp64, with the
largest absolute difference taken instead when ref is all zeros; rel_l2_chains
gives the same figure per (batch, head) chain.  Each value below is worked by
hand.  The planted slips at the end (the norm of x in the denominator, a mean
instead of a norm, the squared ratio, per-row figures, a broadcast of
mismatched shapes, fp32 accumulation, the max-abs branch dropped or taken on
the wrong side) must each fail at least one pin.
"""
import math

import numpy as np
import pytest

from oracle.reference import rel_l2, rel_l2_chains


def check_three_four_five(rel):
    ref = np.array([3.0, 4.0])                        # ||ref|| = 5
    assert rel(ref, ref) == 0.0
    assert rel(np.array([4.0, 4.0]), ref) == pytest.approx(0.2, abs=0, rel=1e-15)     # ||(1, 0)|| / 5
    assert rel(np.array([3.0, 1.0]), ref) == pytest.approx(0.6, abs=0, rel=1e-15)     # ||(0, -3)|| / 5
    assert rel(np.zeros(2), ref) == 1.0                                               # ||ref|| / ||ref||
    assert rel(np.array([6.0, 8.0]), ref) == 1.0


def check_whole_tensor(rel):
    ref = np.array([[1.0, 2.0], [2.0, 4.0]])          # ||ref|| = 5
    x = ref + np.array([[0.0, 0.0], [0.0, -1.0]])     # ||d|| = 1
    assert rel(x, ref) == pytest.approx(0.2, abs=0, rel=1e-15)
    # per row it would be 0 and 1/sqrt(20)
    assert rel(x[1], ref[1]) == pytest.approx(1.0 / math.sqrt(20.0), rel=1e-15)


def check_zero_reference(rel):
    assert rel(np.array([0.5, -2.0, 1.0]), np.zeros(3)) == 2.0
    assert rel(np.zeros(3), np.zeros(3)) == 0.0
    assert rel(np.zeros((0, 4)), np.zeros((0, 4))) == 0.0


def check_fp64_accumulation(rel):
    # 10^6 elements of 1 against 1 + 1e-9: the fp64 ratio is 1e-9 to 1e-6 relative
    # (in fp32 the difference rounds to 0)
    ref = np.ones(10 ** 6, dtype=np.float32)
    x = np.ones(10 ** 6, dtype=np.float64) * (1.0 + 1e-9)
    assert rel(x, ref) == pytest.approx(1e-9, rel=1e-6)


def check_shapes_must_match(rel):
    with pytest.raises(ValueError):
        rel(np.ones((1, 3)), np.ones(3))
    with pytest.raises(ValueError):
        rel(np.ones((3, 1)), np.ones((1, 3)))


CHECKS = [check_three_four_five, check_whole_tensor, check_zero_reference, check_fp64_accumulation,
          check_shapes_must_match]


@pytest.mark.parametrize("chk", CHECKS, ids=lambda c: c.__name__)
def test_rel_l2_pins(chk):
    chk(rel_l2)


def test_per_chain_figures():
    # o-like [B=2, T=1, H=2, dv=2]: chain (b, h) holds o[b, :, h]
    ref = np.zeros((2, 1, 2, 2))
    ref[0, 0, 0] = [3.0, 4.0]
    ref[0, 0, 1] = [1.0, 0.0]
    ref[1, 0, 0] = [0.0, 2.0]
    ref[1, 0, 1] = [6.0, 8.0]
    x = ref.copy()
    x[0, 0, 0] = [4.0, 4.0]      # 1 / 5
    x[1, 0, 0] = [0.0, 1.0]      # 1 / 2
    x[1, 0, 1] = [6.0, 18.0]     # 10 / 10
    e = rel_l2_chains(x, ref, (0, 2))
    assert e.shape == (2, 2)
    np.testing.assert_allclose(e, [[0.2, 0.0], [0.5, 1.0]], rtol=1e-15, atol=0)
    # the whole-tensor figure: sqrt(1 + 1 + 100) / sqrt(25 + 1 + 4 + 100)
    assert rel_l2(x, ref) == pytest.approx(math.sqrt(102.0) / math.sqrt(130.0), rel=1e-15)
    # S-like [B=2, H=2, dk=1, dv=2]: chain axes (0, 1) give the same numbers
    Sref = np.transpose(ref, (0, 2, 1, 3))
    Sx = np.transpose(x, (0, 2, 1, 3))
    np.testing.assert_allclose(rel_l2_chains(Sx, Sref, (0, 1)), e, rtol=1e-15, atol=0)


# ---- planted slips -------------------------------------------------------------
def _strict(f):
    def g(x, ref):
        x, ref = np.asarray(x), np.asarray(ref)
        if x.shape != ref.shape:
            raise ValueError("shape")
        return f(x.astype(np.float64), ref.astype(np.float64))
    return g


def _maxabs_or(f):
    return lambda x, ref: (float(np.max(np.abs(x - ref))) if x.size else 0.0) if not np.any(ref) else f(x, ref)


MUTANTS = {
    "norm_of_x": _strict(_maxabs_or(lambda x, r: float(np.linalg.norm(x - r) / np.linalg.norm(x)))),
    "mean_abs": _strict(_maxabs_or(lambda x, r: float(np.mean(np.abs(x - r)) / np.mean(np.abs(r))))),
    "squared": _strict(_maxabs_or(lambda x, r: float(np.sum((x - r) ** 2) / np.sum(r ** 2)))),
    "max_row": _strict(_maxabs_or(lambda x, r: float(max(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)
                                                         for a, b in zip(np.atleast_2d(x), np.atleast_2d(r)))))),
    "broadcast": lambda x, r: float(np.linalg.norm(np.asarray(x, np.float64) - np.asarray(r, np.float64))
                                    / max(np.linalg.norm(np.asarray(r, np.float64)), 1e-300)),
    "fp32": lambda x, r: _strict(_maxabs_or(lambda a, b: float(np.linalg.norm((a.astype(np.float32)
                                                                               - b.astype(np.float32)))
                                                                / np.linalg.norm(b))))(x, r),
    "no_zero_branch": _strict(lambda x, r: float(np.linalg.norm(x - r) / np.linalg.norm(r))
                              if x.size else 0.0),
    "abs_not_max": _strict(lambda x, r: (float(np.sum(np.abs(x - r))) if x.size else 0.0) if not np.any(r)
                           else float(np.linalg.norm(x - r) / np.linalg.norm(r))),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_rel_l2_mutant_is_rejected(name):
    failed = []
    with np.errstate(all="ignore"):
        for chk in CHECKS:
            try:
                chk(MUTANTS[name])
            except (Exception, pytest.fail.Exception):   # pytest.raises reports through the latter
                failed.append(chk.__name__)
    assert failed, f"rel_l2 mutant {name} passed every pin"
