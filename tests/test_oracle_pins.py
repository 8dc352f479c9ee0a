"""Pins of the fp64 oracle to facts fixed by the pages and by mathematics (CPU only).

Each test names the passage it follows.  The checks are chosen so that a
plausible slip in the oracle -- a dropped decay/erase/write term, a sign
flip, the output read before the update, b placed on the other side of the
erase product, the decay applied after the erase, a transposed state --
fails at least one of them.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import c_oracle
from oracle.reference import chunked_wy, recurrent, rel_l2

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


def _rng_inputs(rng, B, T, H, dk, dv, unit_k=True, b_scale=1.0, s0=True, alpha_lo=0.5):
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    if unit_k:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, dv))
    alpha = rng.uniform(alpha_lo, 1.0, (B, T, H, dk))
    b = b_scale * rng.uniform(0.0, 1.0, (B, T, H, dk))
    w = rng.uniform(0.0, 1.0, (B, T, H, dv))
    S0 = rng.standard_normal((B, H, dk, dv)) * 0.3 if s0 else None
    return q, k, v, alpha, b, w, S0


def _frac(x):
    return np.array([[float(Fraction(s)) for s in row] for row in x]) if isinstance(x[0], list) \
        else np.array([float(Fraction(s)) for s in x])


# ---------------------------------------------------------------------------
# Hand-worked examples (exact rationals; README "Architecture" formula)
# ---------------------------------------------------------------------------
def _golden_cases():
    with open(GOLDEN) as f:
        data = json.load(f)
    out = []
    for ex in data["examples"]:
        dk, dv = ex["dk"], ex["dv"]
        toks = ex["tokens"]
        T = len(toks)
        arr = {key: np.zeros((1, T, 1, dk if key in ("q", "k", "alpha", "b") else dv))
               for key in ("q", "k", "alpha", "b", "v", "w")}
        for t, tok in enumerate(toks):
            for key in arr:
                arr[key][0, t, 0] = _frac(tok[key])
        S0 = None if ex["S0"] is None else _frac(ex["S0"])[None, None]
        o = _frac(ex["o"])[None, :, None, :]
        S = _frac(ex["S_T"])[None, None]
        out.append((ex["name"], arr, S0, o, S))
    return out


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c[0])
def test_golden_worked_examples(case):
    """burn-gdn2 README, "Architecture": the per-token recurrence, by hand."""
    _, a, S0, o_ref, S_ref = case
    args = (a["q"], a["k"], a["v"], a["alpha"], a["b"], a["w"])
    for fn in (recurrent, c_oracle.recurrent,
               lambda *x, S0=None: chunked_wy(*x, S0=S0, chunk=1),
               lambda *x, S0=None: chunked_wy(*x, S0=S0, chunk=64)):
        o, S = fn(*args, S0=S0)
        np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-14)
        np.testing.assert_allclose(S, S_ref, rtol=0, atol=1e-14)


# ---------------------------------------------------------------------------
# Special cases named on the pages
# ---------------------------------------------------------------------------
def check_kda_special_case(recurrent=recurrent):
    """Gated DeltaNet-2 explainer (asapai.co.kr), section on splitting the gate
    into two knobs and its GDN/KDA/GDN-2 table: with both gates collapsed to
    one scalar per token the rule becomes KDA (channel-wise decay, one scalar
    delta gate).  KDA is written here in its delta-rule (prediction-error)
    form: decay, predict v from the key, move the state toward v by beta."""
    rng = np.random.default_rng(1)
    B, T, H, dk, dv = 2, 37, 3, 8, 5
    q, k, v, alpha, _, _, S0 = _rng_inputs(rng, B, T, H, dk, dv, unit_k=False)
    beta = rng.uniform(0.0, 1.0, (B, T, H, 1))
    o, S = recurrent(q, k, v, alpha, np.broadcast_to(beta, (B, T, H, dk)),
                     np.broadcast_to(beta, (B, T, H, dv)), S0)
    St = S0.copy()
    o_ref = np.zeros_like(o)
    for t in range(T):
        for bi in range(B):
            for hi in range(H):
                X = alpha[bi, t, hi][:, None] * St[bi, hi]
                pred = X.T @ k[bi, t, hi]                     # what the decayed memory returns for k
                St[bi, hi] = X + beta[bi, t, hi, 0] * np.outer(k[bi, t, hi], v[bi, t, hi] - pred)
                o_ref[bi, t, hi] = St[bi, hi].T @ q[bi, t, hi]
    assert rel_l2(o, o_ref) < 1e-13 and rel_l2(S, St) < 1e-13


def check_gated_deltanet_special_case(recurrent=recurrent):
    """Same explainer and table: when the decay also collapses to a scalar the
    rule becomes Gated DeltaNet, S_t = a_t (I - beta_t k k^T) S + beta_t k v^T
    (the scalar decay is applied after the erase matrix here; it commutes)."""
    rng = np.random.default_rng(2)
    B, T, H, dk, dv = 1, 41, 2, 6, 7
    q, k, v, _, _, _, S0 = _rng_inputs(rng, B, T, H, dk, dv)
    a = rng.uniform(0.3, 1.0, (B, T, H, 1))
    beta = rng.uniform(0.0, 1.0, (B, T, H, 1))
    o, S = recurrent(q, k, v, np.broadcast_to(a, (B, T, H, dk)),
                     np.broadcast_to(beta, (B, T, H, dk)), np.broadcast_to(beta, (B, T, H, dv)), S0)
    St = S0.copy()
    o_ref = np.zeros_like(o)
    I = np.eye(dk)
    for t in range(T):
        for hi in range(H):
            kt = k[0, t, hi]
            bt = beta[0, t, hi, 0]
            St[0, hi] = a[0, t, hi, 0] * ((I - bt * np.outer(kt, kt)) @ St[0, hi]) + bt * np.outer(kt, v[0, t, hi])
            o_ref[0, t, hi] = q[0, t, hi] @ St[0, hi]
    assert rel_l2(o, o_ref) < 1e-13 and rel_l2(S, St) < 1e-13


def check_linear_attention_special_case(recurrent=recurrent):
    """b = 0, alpha = 1, w = 1 leaves a purely additive state (the explainer
    contrasts linear attention's fixed-size additive memory): by brute force
    o_t = sum_{i<=t} (q_t . k_i) v_i + q_t^T S0 -- the sum includes i = t."""
    rng = np.random.default_rng(3)
    B, T, H, dk, dv = 2, 29, 2, 5, 4
    q, k, v, _, _, _, S0 = _rng_inputs(rng, B, T, H, dk, dv, unit_k=False)
    ones_k = np.ones((B, T, H, dk))
    o, S = recurrent(q, k, v, ones_k, np.zeros((B, T, H, dk)), np.ones((B, T, H, dv)), S0)
    o_ref = np.zeros_like(o)
    for bi in range(B):
        for hi in range(H):
            for t in range(T):
                acc = q[bi, t, hi] @ S0[bi, hi]
                for i in range(t + 1):
                    acc = acc + (q[bi, t, hi] @ k[bi, i, hi]) * v[bi, i, hi]
                o_ref[bi, t, hi] = acc
    S_ref = S0 + np.einsum("bthc,bthj->bhcj", k, v)
    assert rel_l2(o, o_ref) < 1e-13 and rel_l2(S, S_ref) < 1e-13


# ---------------------------------------------------------------------------
# Invariants of the formula
# ---------------------------------------------------------------------------
def check_exact_recall_after_write(recurrent=recurrent):
    """With a unit-norm key, b = 1 and reading with q = k right after the
    write, k^T S_t = k^T D S - (k^T k) k^T D S + (k^T k) (w*v)^T = (w*v)^T:
    the read returns exactly the written value, for any decay, write gate and
    prior state.  (With w = 1 it returns v.)  Fails if the decay is applied
    after the erase or the output reads the state before the update."""
    rng = np.random.default_rng(4)
    B, T, H, dk, dv = 2, 23, 2, 8, 6
    q, k, v, alpha, _, w, S0 = _rng_inputs(rng, B, T, H, dk, dv)
    o, _ = recurrent(k, k, v, alpha, np.ones_like(alpha), w, S0)
    np.testing.assert_allclose(o, w * v, rtol=0, atol=1e-12)
    o1, _ = recurrent(k, k, v, alpha, np.ones_like(alpha), np.ones_like(w), S0)
    np.testing.assert_allclose(o1, v, rtol=0, atol=1e-12)


def check_decay_only(recurrent=recurrent):
    """b = 0 and w = 0 leave only the decay: S_T = diag(prod_t alpha_t) S0 and
    o_t = q_t^T diag(prod_{j<=t} alpha_j) S0."""
    rng = np.random.default_rng(5)
    B, T, H, dk, dv = 1, 17, 3, 7, 5
    q, k, v, alpha, _, _, S0 = _rng_inputs(rng, B, T, H, dk, dv)
    o, S = recurrent(q, k, v, alpha, np.zeros_like(alpha), np.zeros((B, T, H, dv)), S0)
    cum = np.cumprod(alpha, axis=1)                     # [B,T,H,dk]
    o_ref = np.einsum("bthc,bthc,bhcj->bthj", q, cum, S0)
    S_ref = cum[:, -1][..., None] * S0
    assert rel_l2(o, o_ref) < 1e-13 and rel_l2(S, S_ref) < 1e-13


def check_erase_eigen_direction(recurrent=recurrent):
    """burn-gdn2 README, "Configuration", allow_neg_eigval ("b x 2"): for a
    unit key the erase matrix I - k (b*k)^T maps k to (1 - sum_c b_c k_c^2) k,
    negative when b is large enough.  One step with alpha = 1, w = 0 on
    S0 = k x^T must give (1 - sum_c b_c k_c^2) k x^T, for non-uniform b."""
    rng = np.random.default_rng(6)
    dk, dv = 9, 4
    k = rng.standard_normal(dk)
    k /= np.linalg.norm(k)
    b = rng.uniform(0.0, 2.0, dk)
    x = rng.standard_normal(dv)
    S0 = np.outer(k, x)[None, None]
    lam = 1.0 - np.sum(b * k * k)
    o, S = recurrent(np.zeros((1, 1, 1, dk)), k[None, None, None], np.zeros((1, 1, 1, dv)),
                     np.ones((1, 1, 1, dk)), b[None, None, None], np.zeros((1, 1, 1, dv)), S0)
    np.testing.assert_allclose(S[0, 0], lam * np.outer(k, x), rtol=0, atol=1e-14)


def check_erase_moves_state_along_k_only(recurrent=recurrent):
    """The erase subtracts k (b*k)^T X: every column of the change is parallel
    to k, so z^T S is unchanged for z orthogonal to k; and a state whose
    columns are orthogonal to b*k is left untouched.  Placing b on the other
    side of the product fails the first check."""
    rng = np.random.default_rng(7)
    dk, dv = 6, 5
    k = rng.standard_normal(dk)
    b = rng.uniform(0.1, 1.0, dk)
    S0 = rng.standard_normal((dk, dv))
    args = lambda S: (np.zeros((1, 1, 1, dk)), k[None, None, None], np.zeros((1, 1, 1, dv)),
                      np.ones((1, 1, 1, dk)), b[None, None, None], np.zeros((1, 1, 1, dv)), S[None, None])
    _, S1 = recurrent(*args(S0))
    z = rng.standard_normal(dk)
    z -= (z @ k) / (k @ k) * k
    np.testing.assert_allclose(z @ S1[0, 0], z @ S0, rtol=0, atol=1e-13)
    e = b * k
    S_perp = S0 - np.outer(e, e @ S0) / (e @ e)        # columns orthogonal to b*k
    _, S2 = recurrent(*args(S_perp))
    np.testing.assert_allclose(S2[0, 0], S_perp, rtol=0, atol=1e-13)


def check_householder_preserves_norm(recurrent=recurrent):
    """alpha = 1, b = 2 (the README's "b x 2"), w = 0 and unit keys make every
    step a Householder reflection I - 2kk^T: each state column keeps its norm."""
    rng = np.random.default_rng(8)
    B, T, H, dk, dv = 1, 50, 2, 8, 6
    q, k, v, _, _, _, S0 = _rng_inputs(rng, B, T, H, dk, dv)
    _, S = recurrent(q, k, v, np.ones((B, T, H, dk)), 2 * np.ones((B, T, H, dk)),
                     np.zeros((B, T, H, dv)), S0)
    np.testing.assert_allclose(np.linalg.norm(S, axis=2), np.linalg.norm(S0, axis=2), rtol=1e-12)


def check_superposition(recurrent=recurrent):
    """For fixed q, k, alpha, b, w the map (S0, v) -> (o, S_T) is linear, and o is
    linear in q (every term of the recurrence is linear in S and in v)."""
    rng = np.random.default_rng(9)
    B, T, H, dk, dv = 1, 20, 2, 6, 4
    q, k, v1, alpha, b, w, S1 = _rng_inputs(rng, B, T, H, dk, dv, b_scale=2.0)
    v2 = rng.standard_normal(v1.shape)
    S2 = rng.standard_normal(S1.shape)
    c = -1.7
    oa, Sa = recurrent(q, k, v1, alpha, b, w, S1)
    ob, Sb = recurrent(q, k, v2, alpha, b, w, S2)
    oc, Sc = recurrent(q, k, v1 + c * v2, alpha, b, w, S1 + c * S2)
    assert rel_l2(oc, oa + c * ob) < 1e-12 and rel_l2(Sc, Sa + c * Sb) < 1e-12
    q2 = rng.standard_normal(q.shape)
    od, _ = recurrent(q + c * q2, k, v1, alpha, b, w, S1)
    oe, _ = recurrent(q2, k, v1, alpha, b, w, S1)
    assert rel_l2(od, oa + c * oe) < 1e-12


def check_value_columns_independent(recurrent=recurrent):
    """Gates act on the key axis or on the written row w*v, so permuting the
    value channels of v, w and S0 permutes o and S_T the same way."""
    rng = np.random.default_rng(10)
    B, T, H, dk, dv = 1, 15, 2, 5, 7
    q, k, v, alpha, b, w, S0 = _rng_inputs(rng, B, T, H, dk, dv)
    perm = rng.permutation(dv)
    o, S = recurrent(q, k, v, alpha, b, w, S0)
    op, Sp = recurrent(q, k, v[..., perm], alpha, b, w[..., perm], S0[..., perm])
    np.testing.assert_allclose(op, o[..., perm], rtol=0, atol=1e-13)
    np.testing.assert_allclose(Sp, S[..., perm], rtol=0, atol=1e-13)


def check_split_resume(recurrent=recurrent):
    """burn-gdn2 README, "Quick start": inference carries a persistent state
    between calls.  Running tokens [0, t0) and then [t0, T) from the state
    returned equals one run over [0, T)."""
    rng = np.random.default_rng(11)
    B, T, H, dk, dv = 2, 33, 2, 6, 5
    q, k, v, alpha, b, w, S0 = _rng_inputs(rng, B, T, H, dk, dv, b_scale=2.0)
    o, S = recurrent(q, k, v, alpha, b, w, S0)
    for t0 in (0, 1, 16, 32, 33):
        o1, S1 = recurrent(q[:, :t0], k[:, :t0], v[:, :t0], alpha[:, :t0], b[:, :t0], w[:, :t0], S0)
        o2, S2 = recurrent(q[:, t0:], k[:, t0:], v[:, t0:], alpha[:, t0:], b[:, t0:], w[:, t0:], S1)
        np.testing.assert_allclose(np.concatenate([o1, o2], axis=1), o, rtol=0, atol=1e-12)
        np.testing.assert_allclose(S2, S, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# The chunked form and the C oracle against the sequential definition
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("chunk", [16, 32, 64])
@pytest.mark.parametrize("T", [1, 63, 64, 65, 200])
def test_chunked_matches_sequential(chunk, T):
    """burn-gdn2 README (intro, "Architecture"): the chunked WY forward and the
    token-by-token forward compute the same layer.  Includes b in (0,2),
    S0 != 0 and partial tail chunks."""
    rng = np.random.default_rng(100 + T + chunk)
    B, H, dk, dv = 1, 2, 8, 6
    q, k, v, alpha, b, w, S0 = _rng_inputs(rng, B, T, H, dk, dv, b_scale=2.0, alpha_lo=0.7)
    o, S = recurrent(q, k, v, alpha, b, w, S0)
    oc, Sc = chunked_wy(q, k, v, alpha, b, w, S0, chunk=chunk)
    assert rel_l2(oc, o) < 1e-11 and rel_l2(Sc, S) < 1e-11


def test_chunked_zero_state_default():
    """A missing initial state is the zero state (README "Quick start": the
    inference state starts as None)."""
    rng = np.random.default_rng(12)
    q, k, v, alpha, b, w, _ = _rng_inputs(rng, 1, 70, 2, 8, 8, s0=False)
    o0, S0_ = chunked_wy(q, k, v, alpha, b, w, None)
    o1, S1_ = chunked_wy(q, k, v, alpha, b, w, np.zeros((1, 2, 8, 8)))
    assert rel_l2(o0, o1) == 0.0 and rel_l2(S0_, S1_) == 0.0


@pytest.mark.parametrize("shape", [(2, 40, 3, 16, 16), (1, 9, 2, 128, 128), (3, 5, 1, 32, 48)])
def test_c_oracle_matches_numpy(shape):
    """The C oracle (decay, erase via (I - k e^T) X = X - k (e^T X), write,
    read) equals the literal numpy form with the erase matrix formed."""
    rng = np.random.default_rng(13)
    B, T, H, dk, dv = shape
    q, k, v, alpha, b, w, S0 = _rng_inputs(rng, B, T, H, dk, dv, b_scale=2.0)
    f32 = lambda x: x.astype(np.float32).astype(np.float64)
    args = [f32(x) for x in (q, k, v, alpha, b, w)]
    S0 = f32(S0)
    o, S = recurrent(*args, S0)
    for cb in (16, 5, dv):
        oc, Sc = c_oracle.recurrent(*args, S0, col_block=cb)
        assert rel_l2(oc, o) < 1e-13 and rel_l2(Sc, S) < 1e-13
    oz, Sz = c_oracle.recurrent(*args, None)
    on, Sn = recurrent(*args, None)
    assert rel_l2(oz, on) < 1e-13 and rel_l2(Sz, Sn) < 1e-13


def test_kda_special_case():
    check_kda_special_case()


def test_gated_deltanet_special_case():
    check_gated_deltanet_special_case()


def test_linear_attention_special_case():
    check_linear_attention_special_case()


def test_exact_recall_after_write():
    check_exact_recall_after_write()


def test_decay_only():
    check_decay_only()


def test_erase_eigen_direction():
    check_erase_eigen_direction()


def test_erase_moves_state_along_k_only():
    check_erase_moves_state_along_k_only()


def test_householder_preserves_norm():
    check_householder_preserves_norm()


def test_superposition():
    check_superposition()


def test_value_columns_independent():
    check_value_columns_independent()


def test_split_resume():
    check_split_resume()
