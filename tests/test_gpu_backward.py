"""GPU parity of the chunked backward against the fp64 oracle (needs an MI355X).

``gdn2_chunk_bwd`` returns the gradients of sum(dO * o) + sum(dS_T * S_T)
with respect to q, k, v, alpha, b, w and S0; the oracle
(``oracle.backward.recurrent_bwd``, pinned by finite differences of the
forward) computes them in fp64 from the same inputs (bf16 widened exactly).
Relative L2 error per gradient tensor: <= 1e-4 with fp32 I/O, <= 2e-2 with
bf16 I/O (the forward's operands are bf16 there).  The full-size cases compare
every (batch, head) chain against the fp64 C backward oracle
(``oracle.c_oracle.recurrent_bwd``, pinned by finite differences too) and hold
the worst chain to the same bar.  The bf16 cases with dk in
{32, 64, 128} and dv in {32, 64, 128} run the matrix-core gradient kernels,
the others the vector-ALU ones.
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_19_amd as g
from gated_delta_rule_19_amd import inputs
from oracle.backward import recurrent_bwd
from oracle.reference import rel_l2, rel_l2_chains

pytestmark = pytest.mark.gpu

F32, BF16 = torch.float32, torch.bfloat16
TOL = {F32: 1e-4, BF16: 2e-2}
NAMES = ("dq", "dk", "dv", "dalpha", "db", "dw", "dS0")


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    g.lib()
    return torch.device("cuda:0")


def _np(x):
    return None if x is None else x.detach().to("cpu", torch.float64).numpy()


def run(dev, B, T, H, dk, dv, io, gate, s0, dS, seed, b_scale=1.0):
    inp = inputs.make_raw(B, T, H, dk, dv, io, seed, dev, s0_std=s0, gate_dtype=gate, b_scale=b_scale)
    dO, dS_T = inputs.make_out_grads(B, T, H, dk, dv, io, seed + 1, dev, state_grad=dS)
    got = g.chunk_bwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["b"], inp["w"], dO, inp["S0"], dS_T)
    torch.cuda.synchronize()
    return inp, dO, dS_T, got


def ref(inp, dO, dS_T, chains=None):
    h = {n: _np(x) for n, x in inp.items()}
    dOn, dSn = _np(dO), _np(dS_T)
    if chains is None:
        return recurrent_bwd(h["q"], h["k"], h["v"], h["alpha"], h["b"], h["w"], h["S0"], dOn, dSn)
    out = {n: [] for n in NAMES}
    for bi, hi in chains:
        sl = lambda x: None if x is None else x[bi:bi + 1, :, hi:hi + 1]
        st = lambda x: None if x is None else x[bi:bi + 1, hi:hi + 1]
        r = recurrent_bwd(sl(h["q"]), sl(h["k"]), sl(h["v"]), sl(h["alpha"]), sl(h["b"]), sl(h["w"]), st(h["S0"]),
                          sl(dOn), st(dSn))
        for n in NAMES:
            out[n].append(r[n][0, :, 0] if n != "dS0" else r[n][0, 0])
    return {n: np.stack(v) for n, v in out.items()}


def check(what, got, want, tol, chains=False):
    """rel-L2 per gradient tensor; with chains=True also the worst (batch, head) chain of each
    ([B,T,H,*] tensors on axes 0, 2; dS0 [B,H,dk,dv] on axes 0, 1), held to the same bar."""
    errs = {n: rel_l2(got[n], want[n]) for n in NAMES}
    if chains:
        for n in NAMES:
            ax = (0, 1) if n == "dS0" else (0, 2)
            errs[n + "_worst_chain"] = float(np.max(rel_l2_chains(got[n], want[n], ax)))
    print(f"[parity] {what}: " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()) + f" (tol {tol:g})",
          flush=True)
    bad = {n: e for n, e in errs.items() if not e <= tol}
    assert not bad, f"{what}: {bad}"


CASES = [
    # B, T, H, dk, dv, io, gate dtype, S0 std, dS_T, b_scale
    (1, 64, 1, 16, 16, F32, F32, None, False, 1.0),
    (2, 100, 2, 64, 32, F32, F32, 0.05, True, 1.0),
    (2, 65, 3, 64, 64, F32, F32, 0.05, True, 2.0),
    (1, 130, 2, 128, 128, BF16, F32, 0.05, True, 1.0),
    (1, 47, 2, 32, 48, BF16, BF16, None, True, 1.0),
    (1, 200, 1, 128, 256, BF16, F32, 0.05, False, 2.0),
    (1, 1, 2, 128, 128, BF16, F32, 0.05, True, 1.0),
    (2, 150, 2, 64, 64, BF16, BF16, 0.05, True, 2.0),
    (1, 97, 3, 32, 96, BF16, F32, None, True, 1.0),
    (1, 64, 2, 128, 32, BF16, BF16, 0.05, False, 1.0),
    (2, 80, 2, 32, 64, BF16, F32, 0.05, True, 2.0),
    # the remaining matrix-core shapes: dk 32 with dv 128, dk 64 with dv 32 (last chunk 1 token)
    (1, 70, 2, 32, 128, BF16, F32, 0.05, True, 1.0),
    (2, 129, 1, 64, 32, BF16, BF16, None, True, 2.0),
]


def _id(c):
    B, T, H, dk, dv, io, gt, s0, ds, bs = c
    n = lambda d: "bf16" if d == BF16 else "f32"
    return f"B{B}T{T}H{H}dk{dk}dv{dv}io{n(io)}g{n(gt)}{'S0' if s0 else ''}{'dS' if ds else ''}b{bs:g}"


@pytest.mark.parametrize("case", CASES, ids=_id)
def test_backward_small(dev, case):
    B, T, H, dk, dv, io, gt, s0, ds, bs = case
    inp, dO, dS_T, got = run(dev, B, T, H, dk, dv, io, gt, s0, ds, seed=T + dk + dv, b_scale=bs)
    want = ref(inp, dO, dS_T)
    gn = {n: _np(got[n]) for n in NAMES}
    if inp["S0"] is None:                       # dS0 is still returned: the zero state's gradient
        pass
    check(_id(case), gn, want, TOL[io])


def test_backward_full_size_all_chains(dev):
    """B4 H16 T2048 d128 bf16 (the chunked workload): every (batch, head) chain against the
    fp64 C backward oracle, the worst chain's error held to the same bar."""
    from oracle import c_oracle
    B, T, H, dk, dv = 4, 2048, 16, 128, 128
    inp, dO, dS_T, got = run(dev, B, T, H, dk, dv, BF16, F32, None, True, seed=77)
    h = {n: _np(x) for n, x in inp.items()}
    want = c_oracle.recurrent_bwd(h["q"], h["k"], h["v"], h["alpha"], h["b"], h["w"], None, _np(dO), _np(dS_T))
    check("B4H16T2048 all chains", {n: _np(got[n]) for n in NAMES}, want, 2e-2, chains=True)


FAST_CASES = [
    # B, T, H, dk, dv, io, alpha_mu, b scale
    (1, 260, 2, 128, 128, BF16, 0.0, 2.0),
    (2, 200, 2, 64, 64, BF16, -2.0, 1.0),
    (1, 190, 2, 32, 32, BF16, -2.0, 2.0),
    (1, 210, 2, 32, 48, F32, -2.0, 2.0),      # fp32 I/O: every gradient within 1e-4
]


# The chunked backward forms dlog(alpha) as a reverse cumulative sum over the chunk of
# per-token terms whose pairs inside [t, 64) cancel exactly in real arithmetic.  Both
# sides of every pair are formed from the same bf16 factors (one matrix product per pair
# of 16-token blocks, the decay between the blocks applied to the fp32 sums), so they
# cancel down to fp32 rounding and dalpha keeps the other gradients' accuracy however
# fast the decay: before this, with each side ~2^-9 off, dalpha reached 3.3e-2 (mu 0),
# 0.25 (mu -2) and 3.7e-2 (alpha 0.02 on some channels).
@pytest.mark.parametrize("case", FAST_CASES,
                         ids=lambda c: f"B{c[0]}T{c[1]}H{c[2]}dk{c[3]}dv{c[4]}"
                         f"{'bf16' if c[5] == BF16 else 'f32'}mu{c[6]:g}b{c[7]:g}")
def test_backward_fast_decay(dev, case):
    """alpha = sigmoid(N(mu, 1)) with mu = 0 or -2 (the workloads use 3), S0 and dS_T given."""
    from oracle import c_oracle
    B, T, H, dk, dv, io, mu, bs = case
    inp = inputs.make_raw(B, T, H, dk, dv, io, T + dk, dev, s0_std=0.05, alpha_mu=mu, b_scale=bs)
    dO, dS_T = inputs.make_out_grads(B, T, H, dk, dv, io, T + dk + 1, dev)
    got = g.chunk_bwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["b"], inp["w"], dO, inp["S0"], dS_T)
    torch.cuda.synchronize()
    h = {n: _np(x) for n, x in inp.items()}
    want = c_oracle.recurrent_bwd(h["q"], h["k"], h["v"], h["alpha"], h["b"], h["w"], h["S0"], _np(dO), _np(dS_T))
    check(f"fast decay mu {mu}", {n: _np(got[n]) for n in NAMES}, want, TOL[io], chains=True)


def test_backward_decay_002_on_some_channels(dev):
    """alpha = 0.02 on every fifth key channel (0.02^16 = 6.6e-28 over a 16-token block)."""
    from oracle import c_oracle
    B, T, H, dk, dv = 1, 230, 2, 128, 64
    inp = inputs.make_raw(B, T, H, dk, dv, BF16, 43, dev, s0_std=0.05, b_scale=2.0)
    inp["alpha"][..., ::5] = 0.02
    dO, dS_T = inputs.make_out_grads(B, T, H, dk, dv, BF16, 44, dev)
    got = g.chunk_bwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["b"], inp["w"], dO, inp["S0"], dS_T)
    torch.cuda.synchronize()
    h = {n: _np(x) for n, x in inp.items()}
    want = c_oracle.recurrent_bwd(h["q"], h["k"], h["v"], h["alpha"], h["b"], h["w"], h["S0"], _np(dO), _np(dS_T))
    check("alpha 0.02 on some channels", {n: _np(got[n]) for n in NAMES}, want, 2e-2, chains=True)


LOG, NEG, L2 = g.FLAG_GATE_LOGITS, g.FLAG_NEG_EIGVAL, g.FLAG_QK_L2NORM

# Decay inside the forward's domain (4-token products above ~1e-30) but far past a
# 16-token one: both backward paths refer their decay ratios to 8-token halves
# (products of at most 4 decays or their inverses), as the forward does.
DOMAIN_CASES = [
    # B, T, H, Hv, dk, dv, io, gate dtype, flags, alpha_mu
    (1, 200, 2, 2, 128, 128, BF16, F32, 0, -6.0),
    (2, 150, 2, 2, 64, 64, BF16, BF16, LOG | NEG | L2, -6.0),
    (1, 130, 1, 2, 32, 32, BF16, F32, LOG, -8.0),
    (1, 170, 2, 2, 16, 48, F32, F32, 0, -6.0),            # vector-ALU path
    (2, 90, 1, 2, 64, 32, F32, F32, LOG | L2, -8.0),
    (1, 120, 2, 2, 32, 48, BF16, F32, 0, -6.0),           # bf16 on the vector-ALU path (dv 48)
]


@pytest.mark.parametrize("case", DOMAIN_CASES,
                         ids=lambda c: f"B{c[0]}T{c[1]}H{c[2]}Hv{c[3]}dk{c[4]}dv{c[5]}"
                         f"{'bf16' if c[6] == BF16 else 'f32'}fl{c[8]}mu{c[9]:g}")
def test_backward_fast_decay_domain(dev, case):
    """alpha = sigmoid(N(mu, 1)) with mu = -6 or -8: 16-token products far below 1e-30, 4-token
    products above it; every gradient at the usual bar against full_bwd (prologue and grouped
    heads included)."""
    from oracle.backward import full_bwd
    B, T, H, Hv, dk, dv, io, gt, flags, mu = case
    inp = inputs.make_raw(B, T, H, dk, dv, io, 3 * T + dk, dev, s0_std=0.05, alpha_mu=mu, Hv=Hv,
                          gate_dtype=gt, gate_logits=bool(flags & LOG), unit_qk=not flags & L2)
    dO, dS_T = inputs.make_out_grads(B, T, Hv, dk, dv, io, 3 * T + dk + 1, dev)
    got = g.chunk_bwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["b"], inp["w"], dO, inp["S0"], dS_T,
                      flags=flags)
    torch.cuda.synchronize()
    h = {n: _np(x) for n, x in inp.items()}
    want = full_bwd(h["q"], h["k"], h["v"], h["alpha"], h["b"], h["w"], h["S0"], _np(dO), _np(dS_T), flags=flags)
    check(f"backward, mu {mu}", {n: _np(got[n]) for n in NAMES}, want, TOL[io], chains=True)


@pytest.mark.parametrize("io,dk,dv", [(BF16, 128, 64), (F32, 64, 48)])
def test_backward_alpha_1e3_on_some_channels(dev, io, dk, dv):
    """alpha = 1e-3 on every third key channel (1e-3^16 = 1e-48 over 16 tokens)."""
    from oracle import c_oracle
    B, T, H = 1, 200, 2
    inp = inputs.make_raw(B, T, H, dk, dv, io, 53, dev, s0_std=0.05, b_scale=2.0)
    inp["alpha"][..., ::3] = 1e-3
    dO, dS_T = inputs.make_out_grads(B, T, H, dk, dv, io, 54, dev)
    got = g.chunk_bwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["b"], inp["w"], dO, inp["S0"], dS_T)
    torch.cuda.synchronize()
    h = {n: _np(x) for n, x in inp.items()}
    want = c_oracle.recurrent_bwd(h["q"], h["k"], h["v"], h["alpha"], h["b"], h["w"], h["S0"], _np(dO), _np(dS_T))
    check("alpha 1e-3 on some channels", {n: _np(got[n]) for n in NAMES}, want, TOL[io], chains=True)


def test_backward_deterministic(dev):
    inp, dO, dS_T, g1 = run(dev, 1, 150, 2, 64, 64, BF16, F32, 0.05, True, seed=5)
    g2 = g.chunk_bwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["b"], inp["w"], dO, inp["S0"], dS_T)
    torch.cuda.synchronize()
    for n in NAMES:
        assert torch.equal(g1[n], g2[n]), n


# ---- prologue options and grouped value heads -------------------------------------

FULL_CASES = [
    # B, T, H, Hv, dk, dv, io, gate dtype, flags, S0 std
    (2, 100, 2, 4, 64, 64, F32, F32, 0, 0.05),
    (2, 65, 1, 3, 16, 32, F32, F32, L2, None),
    (1, 70, 2, 2, 64, 32, F32, F32, LOG | NEG, 0.05),
    (1, 130, 1, 2, 128, 128, BF16, F32, LOG | NEG | L2, 0.05),
    (1, 97, 2, 2, 32, 48, BF16, BF16, LOG, None),
    (1, 150, 2, 4, 64, 64, BF16, BF16, LOG | NEG | L2, 0.05),
    (1, 64, 1, 1, 128, 64, BF16, F32, L2, 0.05),
    (2, 33, 2, 4, 128, 128, BF16, F32, 0, None),
    # matrix-core shapes with one value head per query/key head: options applied in-kernel
    (2, 100, 2, 2, 64, 64, BF16, BF16, LOG | NEG, 0.05),
    (1, 130, 2, 2, 128, 128, BF16, F32, LOG | L2, None),
    (1, 65, 3, 3, 32, 32, BF16, BF16, LOG | NEG | L2, 0.05),
    (1, 200, 1, 1, 128, 128, BF16, F32, L2, 0.05),
    (1, 47, 2, 2, 64, 128, BF16, F32, LOG, None),
]


def _fid(c):
    B, T, H, Hv, dk, dv, io, gt, fl, s0 = c
    n = lambda d: "bf16" if d == BF16 else "f32"
    return f"B{B}T{T}H{H}Hv{Hv}dk{dk}dv{dv}io{n(io)}g{n(gt)}fl{fl}{'S0' if s0 else ''}"


@pytest.mark.parametrize("case", FULL_CASES, ids=_fid)
def test_backward_prologue_and_grouped_heads(dev, case):
    """Gradients of the logits, of the raw q/k and of shared query/key heads against
    ``oracle.backward.full_bwd`` (pinned by finite differences of the whole forward)."""
    from oracle.backward import full_bwd
    B, T, H, Hv, dk, dv, io, gt, fl, s0 = case
    seed = 3 * T + dk + fl
    inp = inputs.make_raw(B, T, H, dk, dv, io, seed, dev, s0_std=s0, gate_dtype=gt, Hv=Hv,
                          gate_logits=bool(fl & LOG), unit_qk=not fl & L2)
    dO, dS_T = inputs.make_out_grads(B, T, Hv, dk, dv, io, seed + 1, dev)
    got = g.chunk_bwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["b"], inp["w"], dO, inp["S0"], dS_T,
                      flags=fl)
    torch.cuda.synchronize()
    for n, x in (("dq", inp["q"]), ("dk", inp["k"]), ("dv", inp["v"]), ("dalpha", inp["alpha"]),
                 ("db", inp["b"]), ("dw", inp["w"])):
        assert got[n].shape == x.shape and got[n].dtype == x.dtype, n
    h = {n: _np(x) for n, x in inp.items()}
    want = full_bwd(h["q"], h["k"], h["v"], h["alpha"], h["b"], h["w"], h["S0"], _np(dO), _np(dS_T), flags=fl)
    check(_fid(case), {n: _np(got[n]) for n in NAMES}, want, TOL[io])


def test_backward_grouped_heads_equal_widened_call(dev):
    """G value heads sharing a query/key head = the call on q/k copied to every value
    head, with dq/dk summed over the group (same kernels: equal up to the sum's rounding)."""
    B, T, H, Hv, dk, dv = 1, 140, 2, 4, 64, 64
    inp = inputs.make_raw(B, T, H, dk, dv, BF16, 8, dev, s0_std=0.05, Hv=Hv)
    dO, dS_T = inputs.make_out_grads(B, T, Hv, dk, dv, BF16, 9, dev)
    a = (inp["v"], inp["alpha"], inp["b"], inp["w"], dO, inp["S0"], dS_T)
    g1 = g.chunk_bwd(inp["q"], inp["k"], *a)
    wide = lambda x: x.repeat_interleave(Hv // H, dim=2).contiguous()
    g2 = g.chunk_bwd(wide(inp["q"]), wide(inp["k"]), *a)
    torch.cuda.synchronize()
    for n in ("dv", "dalpha", "db", "dw", "dS0"):
        assert torch.equal(g1[n], g2[n]), n
    for n in ("dq", "dk"):
        s = g2[n].float().reshape(B, T, H, Hv // H, dk).sum(3)
        assert rel_l2(_np(g1[n]), _np(s)) < 1e-2, n


def test_backward_full_size_with_options_all_chains(dev):
    """B4 H16 T2048 d128 bf16 with gate logits in bf16, negative eigenvalues and the
    q/k norm: every (batch, head) chain against the fp64 C backward oracle with the same
    options."""
    from oracle import c_oracle
    B, T, H, dk, dv = 4, 2048, 16, 128, 128
    fl = LOG | NEG | L2
    inp = inputs.make_raw(B, T, H, dk, dv, BF16, 78, dev, gate_dtype=BF16, gate_logits=True, unit_qk=False)
    dO, dS_T = inputs.make_out_grads(B, T, H, dk, dv, BF16, 79, dev)
    got = g.chunk_bwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["b"], inp["w"], dO, None, dS_T, flags=fl)
    torch.cuda.synchronize()
    h = {n: _np(x) for n, x in inp.items()}
    want = c_oracle.recurrent_bwd(h["q"], h["k"], h["v"], h["alpha"], h["b"], h["w"], None, _np(dO), _np(dS_T),
                                  flags=fl)
    check(f"B4H16T2048 flags {fl} all chains", {n: _np(got[n]) for n in NAMES}, want, 2e-2, chains=True)


@pytest.mark.parametrize("flags", [0, LOG | NEG | L2])
@pytest.mark.parametrize("io", [F32, BF16])
def test_backward_without_tokens(dev, io, flags):
    """T = 0: the state passes through unchanged, so dS0 = dS_T (and no token gradient);
    B = 0: nothing at all."""
    B, H, dk, dv = 2, 3, 64, 64
    for T in (0,):
        inp = inputs.make_raw(B, T, H, dk, dv, io, 5, dev, s0_std=0.05, gate_logits=bool(flags & LOG),
                              unit_qk=not flags & L2)
        dO, dS_T = inputs.make_out_grads(B, T, H, dk, dv, io, 6, dev)
        got = g.chunk_bwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["b"], inp["w"], dO, inp["S0"], dS_T,
                          flags=flags)
        torch.cuda.synchronize()
        assert torch.equal(got["dS0"], dS_T)
        assert got["dq"].numel() == 0 and got["dw"].numel() == 0
    inp = inputs.make_raw(0, 10, H, dk, dv, io, 5, dev)
    dO, _ = inputs.make_out_grads(0, 10, H, dk, dv, io, 6, dev)
    got = g.chunk_bwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["b"], inp["w"], dO, flags=flags)
    torch.cuda.synchronize()
    assert got["dS0"].numel() == 0
