"""Seeded random sweep over the whole option space (needs an MI355X).

The other GPU tests take the options one or two at a time; here every case
draws all of them at once from a seeded generator: batch, length (1..300,
ragged), query/key heads and the value heads grouped over them, dk, dv, the
I/O and gate dtypes, every prologue flag combination, an initial state or
none, and the decay level.  Both forward modes are compared with the fp64 C
oracle on the same inputs (q/k shared by the value heads of a group as
``oracle.reference.share_qk_heads`` states), and the chunked backward with
``oracle.backward.full_bwd``, at the usual bars: rel-L2 <= 1e-4 with fp32 I/O,
<= 2e-2 with bf16, whole tensor and worst (batch, head) chain.
Decay levels stay inside the chunked mode's documented domain (include/gdn2.h;
products over 4 consecutive tokens above ~1e-30): down to alpha ~
sigma(N(-6, 1)) in the forward and the backward alike.
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_19_amd as g
from gated_delta_rule_19_amd import inputs
from oracle import c_oracle
from oracle.reference import rel_l2, rel_l2_chains, share_qk_heads

pytestmark = pytest.mark.gpu
F32, BF16 = torch.float32, torch.bfloat16
TOL = {F32: 1e-4, BF16: 2e-2}
LOG, NEG, L2 = g.FLAG_GATE_LOGITS, g.FLAG_NEG_EIGVAL, g.FLAG_QK_L2NORM
NAMES = ("dq", "dk", "dv", "dalpha", "db", "dw", "dS0")


def case(i, small=False):
    """Case i of the sweep: a dict of every option, drawn from a generator seeded with i."""
    r = np.random.default_rng(7000 + i + (500 if small else 0))
    io = BF16 if r.random() < 0.6 else F32
    flags = int(r.choice([0, LOG, LOG | NEG, L2, LOG | L2, LOG | NEG | L2]))
    H = int(r.integers(1, 3))
    G = int(r.choice([1, 1, 2]))
    return dict(
        B=int(r.integers(1, 3 if small else 4)),
        T=int(r.integers(1, 201 if small else 301)),
        H=H, Hv=H * G,
        dk=int(r.choice([16, 32, 64, 128])),
        dv=int(r.choice([16, 32, 48, 64, 128] if small else [16, 32, 48, 64, 128, 256])),
        io=io,
        gate=BF16 if io == BF16 and r.random() < 0.4 else F32,
        flags=flags,
        s0=0.05 if r.random() < 0.5 else None,
        alpha_mu=float(r.choice([3.0, 3.0, 0.0, -2.0, -6.0])),
        b_scale=2.0 if (flags & LOG) == 0 and r.random() < 0.3 else 1.0,
        seed=int(r.integers(1, 1 << 30)),
    )


def make(dev, c):
    return inputs.make_raw(c["B"], c["T"], c["H"], c["dk"], c["dv"], c["io"], c["seed"], dev,
                           alpha_mu=c["alpha_mu"], b_scale=c["b_scale"], s0_std=c["s0"],
                           gate_logits=bool(c["flags"] & LOG), unit_qk=not c["flags"] & L2,
                           gate_dtype=c["gate"], Hv=c["Hv"])


def _np(x):
    return None if x is None else x.detach().to("cpu", torch.float32).numpy()


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    g.lib()
    return torch.device("cuda:0")


def _check(what, got, ref, tol, chain_axes):
    e = rel_l2(got, ref)
    w = float(np.max(rel_l2_chains(got, ref, chain_axes))) if got.size else 0.0
    print(f"  {what}: relL2 {e:.2e}, worst chain {w:.2e} (tol {tol:g})", flush=True)
    assert e <= tol and w <= tol, what


@pytest.mark.parametrize("i", range(24))
def test_sweep_forward_modes(dev, i):
    c = case(i)
    print(f"sweep forward {i}: {c}", flush=True)
    inp = make(dev, c)
    args = [inp[n] for n in ("q", "k", "v", "alpha", "b", "w")]
    o, S = g.chunk_fwd(*args, inp["S0"], flags=c["flags"])
    o_r, S_r = g.recurrent_step(*args, inp["S0"], flags=c["flags"])
    torch.cuda.synchronize()
    h = {n: _np(inp[n]) for n in ("q", "k", "v", "alpha", "b", "w", "S0")}
    qq, kk = h["q"], h["k"]
    if c["Hv"] != c["H"]:
        qq, kk = (np.ascontiguousarray(x, dtype=np.float32) for x in share_qk_heads(qq, kk, c["Hv"]))
    ro, rS = c_oracle.recurrent(qq, kk, h["v"], h["alpha"], h["b"], h["w"], h["S0"], flags=c["flags"])
    tol = TOL[c["io"]]
    for mode, (oo, SS) in (("chunked", (o, S)), ("recurrent", (o_r, S_r))):
        _check(f"{mode} o", _np(oo), ro, tol, (0, 2))
        _check(f"{mode} S", _np(SS), rS, tol, (0, 1))


@pytest.mark.parametrize("i", range(12))
def test_sweep_backward(dev, i):
    from oracle.backward import full_bwd
    c = case(i, small=True)
    print(f"sweep backward {i}: {c}", flush=True)
    inp = make(dev, c)
    dO, dS = inputs.make_out_grads(c["B"], c["T"], c["Hv"], c["dk"], c["dv"], c["io"], c["seed"] + 1, dev)
    args = [inp[n] for n in ("q", "k", "v", "alpha", "b", "w")]
    got = g.chunk_bwd(*args, dO, inp["S0"], dS, flags=c["flags"])
    torch.cuda.synchronize()
    h = {n: _np(inp[n]) for n in ("q", "k", "v", "alpha", "b", "w", "S0")}
    ref = full_bwd(h["q"], h["k"], h["v"], h["alpha"], h["b"], h["w"], h["S0"], _np(dO), _np(dS), flags=c["flags"])
    tol = TOL[c["io"]]
    for n in NAMES:
        gn = _np(got[n])
        assert gn.shape == ref[n].shape, n
        _check(n, gn, ref[n], tol, (0, 1) if n == "dS0" else (0, 2))


def conv_case(i):
    """Case i of the fused-convolution sweep (equal-length batches, K <= 4)."""
    r = np.random.default_rng(9000 + i)
    io = BF16 if r.random() < 0.6 else F32
    H = int(r.integers(1, 3))
    # q/k are convolved before the recurrence: without the L2 option their rows
    # leave the unit sphere, so the weights stay small there
    flags = int(r.choice([L2, LOG | L2, LOG | NEG | L2, 0, LOG]))
    return dict(B=int(r.integers(1, 3)), T=int(r.integers(1, 260)), H=H, Hv=H * int(r.choice([1, 2])),
                dk=int(r.choice([32, 64, 128])), dv=int(r.choice([32, 64, 128])), io=io,
                gate=BF16 if io == BF16 and r.random() < 0.4 else F32, flags=flags,
                K=int(r.integers(1, 5)), silu=bool(r.random() < 0.5),
                wscale=0.5 if flags & L2 else 0.25, alpha_mu=float(r.choice([3.0, 0.0, -4.0])),
                mode=str(r.choice(["chunk", "recurrent"])), seed=int(r.integers(1, 1 << 30)))


@pytest.mark.parametrize("i", range(16))
def test_sweep_fused_conv(dev, i):
    """Both forward modes with the short convolution fused in, against the oracle chain
    short_conv -> split -> shared q/k heads -> recurrence (tests/test_gpu_conv_fused.py)."""
    from test_gpu_conv_fused import check as conv_check, oracle_chain, run as conv_run
    c = conv_case(i)
    print(f"sweep fused conv {i}: {c}", flush=True)
    inp = inputs.make_raw(c["B"], c["T"], c["H"], c["dk"], c["dv"], c["io"], c["seed"], dev, s0_std=0.05,
                          alpha_mu=c["alpha_mu"], gate_logits=bool(c["flags"] & LOG), unit_qk=True,
                          gate_dtype=c["gate"], Hv=c["Hv"])
    C = 2 * c["H"] * c["dk"] + c["Hv"] * c["dv"]
    gen = torch.Generator().manual_seed(c["seed"] + 7)
    weight = (torch.randn(C, c["K"], generator=gen) * c["wscale"]).to(dev)
    state = (torch.randn(c["B"], c["K"] - 1, C, generator=gen) * 0.5).to(c["io"]).to(dev) if c["K"] > 1 else None
    o, S, win = conv_run(c["mode"], inp, weight, state, c["silu"], c["flags"])
    torch.cuda.synchronize()
    ro, rS, rwin = oracle_chain(inp, weight, state, c["silu"], c["flags"])
    conv_check(f"sweep conv {i}", c["io"], o, S, win, ro, rS, rwin)
