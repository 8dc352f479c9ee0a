"""Decay at or near zero in the chunked mode (needs an MI355X).

A decay alpha = 0 erases a key channel of the state; with gate logits a very
negative logit does the same after the sigmoid.  The recurrent mode takes it as
it is.  The chunked mode divides by products of up to 4 consecutive decays, so it
raises any alpha below 2^-20 to 2^-20 (include/gdn2.h, "Domain"): the state then
keeps at most a 2^-20 share of what it should have erased, far below either bar.

Forward: a tenth of the (token, channel) decays are set to 0, 1e-30, 1e-12 or
2^-21 (or the logits to -100 / -1e4), the rest drawn as usual, over several
chunks and a ragged tail; both modes are compared with the fp64 C oracle on the
unraised inputs at the usual bars (rel-L2 <= 1e-4 fp32 I/O, <= 2e-2 bf16, whole
tensor and worst chain).  Backward: the chunked backward is the gradient of the
forward it computes, so its seven gradients are compared with the fp64 reverse
oracle (oracle.backward.full_bwd) on the raised decays, with dalpha 0 where a
decay was raised (the forward does not depend on it there), and every gradient
must be finite.
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_19_amd as g
from gated_delta_rule_19_amd import inputs
from oracle import c_oracle
from oracle.reference import rel_l2, rel_l2_chains

pytestmark = pytest.mark.gpu
F32, BF16 = torch.float32, torch.bfloat16
TOL = {F32: 1e-4, BF16: 2e-2}
FLOOR = 2.0 ** -20
NAMES = ("dq", "dk", "dv", "dalpha", "db", "dw", "dS0")


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    g.lib()
    return torch.device("cuda:0")


def _np(x):
    return None if x is None else x.detach().to("cpu", torch.float32).numpy()


def _check(what, got, ref, tol, chain_axes):
    assert np.all(np.isfinite(got)), f"{what}: not finite"
    e = rel_l2(got, ref)
    w = float(np.max(rel_l2_chains(got, ref, chain_axes))) if got.size else 0.0
    print(f"  {what}: relL2 {e:.2e}, worst chain {w:.2e} (tol {tol:g})", flush=True)
    assert e <= tol and w <= tol, what


def zero_some(alpha, seed, logits):
    """A tenth of the decays (or logits) replaced by values at or below the floor."""
    gen = torch.Generator().manual_seed(seed)
    pick = torch.rand(alpha.shape, generator=gen) < 0.1
    if logits:
        low = torch.tensor([-100.0, -1e4])
    else:
        low = torch.tensor([0.0, 1e-30, 1e-12, 2.0 ** -21])
    which = torch.randint(0, low.numel(), alpha.shape, generator=gen)
    a = alpha.to("cpu", torch.float32).clone()
    a[pick] = low[which[pick]]
    return a.to(alpha.dtype).to(alpha.device)


@pytest.mark.parametrize("io,logits,dk,T", [(F32, False, 64, 200), (BF16, False, 128, 200),
                                            (F32, True, 32, 131), (BF16, True, 128, 300)])
def test_forward_decay_at_zero(dev, io, logits, dk, T):
    B, H, dv, seed = 2, 2, 64, 4100 + dk + T
    print(f"decay floor forward: io {io} logits {logits} B{B} T{T} H{H} dk{dk} dv{dv}", flush=True)
    inp = inputs.make_raw(B, T, H, dk, dv, io, seed, dev, s0_std=0.05, gate_logits=logits)
    inp["alpha"] = zero_some(inp["alpha"], seed, logits)
    flags = g.FLAG_GATE_LOGITS if logits else 0
    args = [inp[n] for n in ("q", "k", "v", "alpha", "b", "w")]
    o, S = g.chunk_fwd(*args, inp["S0"], flags=flags)
    o_r, S_r = g.recurrent_step(*args, inp["S0"], flags=flags)
    torch.cuda.synchronize()
    h = {n: _np(inp[n]) for n in ("q", "k", "v", "alpha", "b", "w", "S0")}
    ro, rS = c_oracle.recurrent(h["q"], h["k"], h["v"], h["alpha"], h["b"], h["w"], h["S0"], flags=flags)
    for mode, (oo, SS) in (("chunked", (o, S)), ("recurrent", (o_r, S_r))):
        _check(f"{mode} o", _np(oo), ro, TOL[io], (0, 2))
        _check(f"{mode} S", _np(SS), rS, TOL[io], (0, 1))


@pytest.mark.parametrize("io,logits", [(F32, False), (BF16, False), (F32, True), (BF16, True)])
def test_backward_decay_at_zero(dev, io, logits):
    from oracle.backward import full_bwd
    B, T, H, dk, dv, seed = 1, 150, 2, 64, 32, 4300
    print(f"decay floor backward: io {io} logits {logits} B{B} T{T} H{H} dk{dk} dv{dv}", flush=True)
    inp = inputs.make_raw(B, T, H, dk, dv, io, seed, dev, s0_std=0.05, gate_logits=logits)
    inp["alpha"] = zero_some(inp["alpha"], seed, logits)
    flags = g.FLAG_GATE_LOGITS if logits else 0
    dO, dS = inputs.make_out_grads(B, T, H, dk, dv, io, seed + 1, dev)
    args = [inp[n] for n in ("q", "k", "v", "alpha", "b", "w")]
    got = g.chunk_bwd(*args, dO, inp["S0"], dS, flags=flags)
    torch.cuda.synchronize()
    h = {n: _np(inp[n]) for n in ("q", "k", "v", "alpha", "b", "w", "S0")}
    a = h["alpha"].astype(np.float64)
    if logits:   # the logit whose sigmoid is the floor, where the sigmoid falls below it
        with np.errstate(over="ignore"):
            low = 1.0 / (1.0 + np.exp(-a)) < FLOOR
        raised = np.where(low, np.log(FLOOR / (1.0 - FLOOR)), a)
    else:
        low = a < FLOOR
        raised = np.maximum(a, FLOOR)
    ref = full_bwd(h["q"], h["k"], h["v"], raised, h["b"], h["w"], h["S0"], _np(dO), _np(dS), flags=flags)
    ref["dalpha"] = np.where(low, 0.0, ref["dalpha"])
    for n in NAMES:
        _check(n, _np(got[n]), ref[n], TOL[io], (0, 1) if n == "dS0" else (0, 2))
