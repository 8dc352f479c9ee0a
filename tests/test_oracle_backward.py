"""Pins of the backward oracle (CPU only).

The gradient of the forward recurrence (burn-gdn2 README, "Architecture") is
fixed by the forward alone.  Both backward routines are checked against
central finite differences of the pinned forward (``oracle.reference.recurrent``)
for every input element, on shapes that span several chunks with a ragged
tail, then against each other on larger shapes; a reverse loop with planted
slips shows that the finite-difference pin rejects each of them.
"""
import numpy as np
import pytest

from oracle.backward import chunked_bwd, loss, recurrent_bwd
from oracle.reference import recurrent, rel_l2

NAMES = ("q", "k", "v", "alpha", "b", "w", "S0")


def _draw(rng, B=1, T=6, H=1, dk=3, dv=2):
    k = rng.standard_normal((B, T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    return dict(q=rng.standard_normal((B, T, H, dk)), k=k, v=rng.standard_normal((B, T, H, dv)),
                alpha=rng.uniform(0.5, 1.0, (B, T, H, dk)), b=rng.uniform(0.0, 2.0, (B, T, H, dk)),
                w=rng.uniform(0.0, 1.0, (B, T, H, dv)), S0=rng.standard_normal((B, H, dk, dv)) * 0.5), \
        rng.standard_normal((B, T, H, dv)), rng.standard_normal((B, H, dk, dv))


def _fd(x, dO, dS, h=1e-6):
    """Central differences of loss(recurrent(x)) for every element of every input."""
    out = {}
    for n in NAMES:
        g = np.zeros_like(x[n])
        for idx in np.ndindex(*x[n].shape):
            vals = []
            for s in (h, -h):
                y = {m: a.copy() for m, a in x.items()}
                y[n][idx] += s
                o, S = recurrent(*(y[m] for m in NAMES[:6]), y["S0"])
                vals.append(loss(o, S, dO, dS))
            g[idx] = (vals[0] - vals[1]) / (2 * h)
        out["d" + n] = g
    return out


def _check_fd(bwd, x, dO, dS, tol=1e-7):
    fd = _fd(x, dO, dS)
    g = bwd(*(x[m] for m in NAMES), dO, dS)
    for n in fd:
        err = np.max(np.abs(g[n] - fd[n])) / max(1.0, np.max(np.abs(fd[n])))
        assert err < tol, f"{n}: max error {err:.2e} against finite differences"


@pytest.mark.parametrize("T", [1, 6])
def test_recurrent_bwd_matches_finite_differences(T):
    x, dO, dS = _draw(np.random.default_rng(T), T=T)
    _check_fd(recurrent_bwd, x, dO, dS)


@pytest.mark.parametrize("T,chunk", [(6, 4), (9, 4), (8, 4), (3, 16)])
def test_chunked_bwd_matches_finite_differences(T, chunk):
    x, dO, dS = _draw(np.random.default_rng(10 + T), B=1, T=T, H=2, dk=3, dv=2)
    _check_fd(lambda *a: chunked_bwd(*a, chunk=chunk), x, dO, dS)


@pytest.mark.parametrize("T,chunk", [(1, 16), (16, 16), (17, 16), (40, 16), (130, 64)])
def test_chunked_equals_recurrent(T, chunk):
    x, dO, dS = _draw(np.random.default_rng(20 + T), B=2, T=T, H=2, dk=8, dv=5)
    g1 = recurrent_bwd(*(x[m] for m in NAMES), dO, dS)
    g2 = chunked_bwd(*(x[m] for m in NAMES), dO, dS, chunk=chunk)
    for n in g1:
        assert rel_l2(g2[n], g1[n]) < 1e-11, n


def test_missing_state_and_state_gradient():
    """S0 = None is the zero state, dS_T = None no gradient on the final state."""
    x, dO, _ = _draw(np.random.default_rng(3), T=5, dk=4, dv=3)
    g1 = recurrent_bwd(*(x[m] for m in NAMES[:6]), None, dO, None)
    g2 = recurrent_bwd(*(x[m] for m in NAMES[:6]), np.zeros_like(x["S0"]), dO, np.zeros_like(x["S0"]))
    for n in g1:
        np.testing.assert_array_equal(g1[n], g2[n])
    g3 = chunked_bwd(*(x[m] for m in NAMES[:6]), None, dO, None, chunk=2)
    for n in g1:
        assert rel_l2(g3[n], g1[n]) < 1e-12


# ---- planted slips: each must fail the finite-difference pin ------------------
def _reverse_with_slip(slip):
    def bwd(q, k, v, alpha, b, w, S0, dO, dS_T=None):
        B, T, H, dk = q.shape
        dv = v.shape[-1]
        S = [S0.copy()]
        for t in range(T):
            z = alpha[:, t] * b[:, t] * k[:, t]
            delta = w[:, t] * v[:, t] - np.einsum("bhcj,bhc->bhj", S[-1], z)
            S.append(alpha[:, t][..., None] * S[-1] + k[:, t][..., :, None] * delta[..., None, :])
        G = dS_T.copy()
        g = {n: np.zeros_like(a) for n, a in (("dq", q), ("dk", k), ("dv", v), ("dalpha", alpha), ("db", b),
                                              ("dw", w))}
        for t in range(T - 1, -1, -1):
            St, Sp = S[t + 1], S[t]
            if slip != "no_output_grad":
                G = G + q[:, t][..., :, None] * dO[:, t][..., None, :]
            g["dq"][:, t] = np.einsum("bhcj,bhj->bhc", Sp if slip == "dq_old_state" else St, dO[:, t])
            z = alpha[:, t] * b[:, t] * k[:, t]
            delta = w[:, t] * v[:, t] - np.einsum("bhcj,bhc->bhj", Sp, z)
            dd = np.einsum("bhcj,bhc->bhj", G, k[:, t])
            dz = -np.einsum("bhcj,bhj->bhc", Sp, dd)
            g["dk"][:, t] = np.einsum("bhcj,bhj->bhc", G, delta) + (0 if slip == "no_dz_in_dk" else
                                                                    dz * alpha[:, t] * b[:, t])
            g["dw"][:, t] = dd * v[:, t]
            g["dv"][:, t] = dd * w[:, t]
            g["db"][:, t] = dz * alpha[:, t] * k[:, t]
            g["dalpha"][:, t] = (0 if slip == "no_decay_grad" else np.sum(G * Sp, axis=-1)) + dz * b[:, t] * k[:, t]
            sign = 1.0 if slip == "erase_sign" else -1.0
            G = alpha[:, t][..., None] * G + sign * z[..., :, None] * dd[..., None, :]
        g["dS0"] = G
        return g
    return bwd


SLIPS = ["no_output_grad", "dq_old_state", "no_dz_in_dk", "no_decay_grad", "erase_sign"]


@pytest.mark.parametrize("slip", SLIPS)
def test_backward_slip_is_rejected(slip):
    x, dO, dS = _draw(np.random.default_rng(5), T=4)
    with pytest.raises(AssertionError):
        _check_fd(_reverse_with_slip(slip), x, dO, dS)


def test_correct_reverse_passes_the_slip_harness():
    x, dO, dS = _draw(np.random.default_rng(5), T=4)
    _check_fd(_reverse_with_slip(None), x, dO, dS)


# ---- prologue options and grouped value heads ------------------------------------
def _fd_full(x, dO, dS, flags, h=1e-6):
    """Central differences of loss(prologue -> shared heads -> recurrence) for every input."""
    from oracle.reference import prologue, share_qk_heads
    Hv = x["v"].shape[2]

    def fwd(y):
        pq, pk, pa, pb, pw = prologue(y["q"], y["k"], y["alpha"], y["b"], y["w"], flags)
        if Hv != pq.shape[2]:
            pq, pk = share_qk_heads(pq, pk, Hv)
        o, S = recurrent(pq, pk, y["v"], pa, pb, pw, y["S0"])
        return loss(o, S, dO, dS)
    out = {}
    for n in NAMES:
        g = np.zeros_like(x[n])
        for idx in np.ndindex(*x[n].shape):
            vals = []
            for s in (h, -h):
                y = {m: a.copy() for m, a in x.items()}
                y[n][idx] += s
                vals.append(fwd(y))
            g[idx] = (vals[0] - vals[1]) / (2 * h)
        out["d" + n] = g
    return out


@pytest.mark.parametrize("flags,G", [(0, 2), (1, 1), (3, 1), (4, 1), (7, 2), (5, 3)])
def test_full_bwd_matches_finite_differences(flags, G):
    from oracle.backward import full_bwd
    rng = np.random.default_rng(40 + flags + G)
    B, T, H, dk, dv = 1, 5, 1, 3, 2
    Hv = H * G
    x = dict(q=rng.standard_normal((B, T, H, dk)) * 2, k=rng.standard_normal((B, T, H, dk)),
             v=rng.standard_normal((B, T, Hv, dv)),
             alpha=(rng.standard_normal((B, T, Hv, dk)) + 2) if flags & 1 else rng.uniform(0.5, 1, (B, T, Hv, dk)),
             b=rng.standard_normal((B, T, Hv, dk)) if flags & 1 else rng.uniform(0, 2, (B, T, Hv, dk)),
             w=rng.standard_normal((B, T, Hv, dv)) if flags & 1 else rng.uniform(0, 1, (B, T, Hv, dv)),
             S0=rng.standard_normal((B, Hv, dk, dv)) * 0.5)
    if not flags & 4:
        x["k"] /= np.linalg.norm(x["k"], axis=-1, keepdims=True)
    dO = rng.standard_normal((B, T, Hv, dv))
    dS = rng.standard_normal((B, Hv, dk, dv))
    fd = _fd_full(x, dO, dS, flags)
    g = full_bwd(*(x[m] for m in NAMES), dO, dS, flags=flags)
    for n in fd:
        err = np.max(np.abs(g[n] - fd[n])) / max(1.0, np.max(np.abs(fd[n])))
        assert err < 1e-7, f"{n}: {err:.2e}"


def test_full_bwd_without_options_is_recurrent_bwd():
    from oracle.backward import full_bwd
    x, dO, dS = _draw(np.random.default_rng(9), T=7, dk=4, dv=3)
    g1 = recurrent_bwd(*(x[m] for m in NAMES), dO, dS)
    g2 = full_bwd(*(x[m] for m in NAMES), dO, dS, flags=0)
    for n in g1:
        np.testing.assert_array_equal(g1[n], g2[n])


# ---- the C backward oracle (gdn2_oracle_bwd_f64) ------------------------------------
def _fp32_exact(x):
    """Round every input to float32 (the C routine takes float32 and widens it exactly),
    so that both sides differentiate at the same point."""
    return {n: (None if a is None else a.astype(np.float32).astype(np.float64)) for n, a in x.items()}


def _fd_subset(x, dO, dS, flags, picks, h=1e-6):
    """Central differences of loss(prologue -> recurrence) at the listed (input, index) pairs."""
    from oracle.reference import prologue

    def fwd(y):
        pq, pk, pa, pb, pw = prologue(y["q"], y["k"], y["alpha"], y["b"], y["w"], flags)
        o, S = recurrent(pq, pk, y["v"], pa, pb, pw, y["S0"])
        return loss(o, S, dO, dS)
    out = []
    for n, idx in picks:
        vals = []
        for s in (h, -h):
            y = {m: a.copy() for m, a in x.items()}
            y[n][idx] += s
            vals.append(fwd(y))
        out.append((vals[0] - vals[1]) / (2 * h))
    return np.array(out)


@pytest.mark.parametrize("T,flags", [(1, 0), (6, 0), (6, 1), (5, 3), (6, 4), (7, 7)])
def test_c_bwd_matches_finite_differences(T, flags):
    """Every element of every input, short sequences, each prologue option."""
    from oracle import c_oracle
    rng = np.random.default_rng(60 + T + flags)
    x, dO, dS = _draw(rng, T=T, dk=3, dv=2)
    if flags & 1:
        x["alpha"] = rng.standard_normal(x["alpha"].shape) + 2
        x["b"] = rng.standard_normal(x["b"].shape)
        x["w"] = rng.standard_normal(x["w"].shape)
    if flags & 4:
        x["q"] = x["q"] * 2
        x["k"] = rng.standard_normal(x["k"].shape)
    x = _fp32_exact(x)
    dO, dS = dO.astype(np.float32).astype(np.float64), dS.astype(np.float32).astype(np.float64)
    g = c_oracle.recurrent_bwd(*(x[m] for m in NAMES), dO, dS, flags=flags)
    picks = [(n, idx) for n in NAMES for idx in np.ndindex(*x[n].shape)]
    fd = _fd_subset(x, dO, dS, flags, picks)
    got = np.array([g["d" + n][idx] for n, idx in picks])
    err = np.max(np.abs(got - fd)) / max(1.0, np.max(np.abs(fd)))
    assert err < 1e-7, f"max error {err:.2e} against finite differences"


def test_c_bwd_across_checkpoint_spans():
    """A 140-token sequence (three 64-token replay spans, the last one ragged): the
    elements at and around the span edges and a random sample elsewhere."""
    from oracle import c_oracle
    rng = np.random.default_rng(71)
    x, dO, dS = _draw(rng, B=1, T=140, H=2, dk=3, dv=2)
    x = _fp32_exact(x)
    dO, dS = dO.astype(np.float32).astype(np.float64), dS.astype(np.float32).astype(np.float64)
    g = c_oracle.recurrent_bwd(*(x[m] for m in NAMES), dO, dS)
    picks = [("S0", (0, 1, 2, 1)), ("S0", (0, 0, 0, 0))]
    for t in (0, 62, 63, 64, 65, 127, 128, 129, 139):
        for n in ("q", "k", "alpha", "b"):
            picks.append((n, (0, t, 1, t % 3)))
        for n in ("v", "w"):
            picks.append((n, (0, t, 0, t % 2)))
    for _ in range(30):
        n = NAMES[rng.integers(0, 6)]
        picks.append((n, tuple(int(rng.integers(0, s)) for s in x[n].shape)))
    fd = _fd_subset(x, dO, dS, 0, picks)
    got = np.array([g["d" + n][idx] for n, idx in picks])
    err = np.max(np.abs(got - fd)) / max(1.0, np.max(np.abs(fd)))
    assert err < 1e-7, f"max error {err:.2e} against finite differences"


@pytest.mark.parametrize("flags", [0, 1, 3, 4, 7])
def test_c_bwd_equals_numpy_bwd(flags):
    """The C routine and ``full_bwd`` on a larger shape (several chains, 150 tokens)."""
    from oracle import c_oracle
    from oracle.backward import full_bwd
    rng = np.random.default_rng(80 + flags)
    x, dO, dS = _draw(rng, B=2, T=150, H=3, dk=8, dv=5)
    if flags & 1:
        x["alpha"] = rng.standard_normal(x["alpha"].shape) + 3
        x["b"] = rng.standard_normal(x["b"].shape)
        x["w"] = rng.standard_normal(x["w"].shape)
    x = _fp32_exact(x)
    dO, dS = dO.astype(np.float32).astype(np.float64), dS.astype(np.float32).astype(np.float64)
    g1 = c_oracle.recurrent_bwd(*(x[m] for m in NAMES), dO, dS, flags=flags)
    g2 = full_bwd(*(x[m] for m in NAMES), dO, dS, flags=flags)
    for n in g1:
        assert rel_l2(g1[n], g2[n]) < 1e-12, n
    # no initial state, no state gradient
    g3 = c_oracle.recurrent_bwd(*(x[m] for m in NAMES[:6]), None, dO, None, flags=flags)
    g4 = full_bwd(*(x[m] for m in NAMES[:6]), None, dO, None, flags=flags)
    for n in g3:
        assert rel_l2(g3[n], g4[n]) < 1e-12, n
