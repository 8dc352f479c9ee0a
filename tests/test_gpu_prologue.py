"""GPU parity of the in-kernel prologue options against the fp64 oracle (needs an MI355X).

The kernels can take the gates as pre-activation logits (sigmoid in-kernel,
b x 2 in negative-eigenvalue mode), bf16 gates, and unnormalised q/k that
they L2-normalise themselves.  Both sides get the same seeded inputs (bf16
widened exactly) and the oracle applies the same prologue in double
(``oracle.reference.prologue`` / the C oracle's flags).  Tolerances as for
the plain path: rel-L2 <= 1e-4 with fp32 I/O, <= 2e-2 with bf16 I/O.
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_19_amd as g
from gated_delta_rule_19_amd import inputs
from oracle import c_oracle
from oracle.reference import rel_l2

pytestmark = pytest.mark.gpu

LOG, NEG, L2 = g.FLAG_GATE_LOGITS, g.FLAG_NEG_EIGVAL, g.FLAG_QK_L2NORM
TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}
F32, BF16 = torch.float32, torch.bfloat16


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    g.lib()
    return torch.device("cuda:0")


def _np(x):
    return None if x is None else x.detach().to("cpu", torch.float32).numpy()


def make(dev, B, T, H, dk, dv, io, gate, flags, seed, s0=None, alpha_mu=3.0):
    return inputs.make_raw(B, T, H, dk, dv, io, seed, dev, alpha_mu=alpha_mu, s0_std=s0,
                           gate_logits=bool(flags & LOG), unit_qk=not (flags & L2), gate_dtype=gate)


def args(inp):
    return inp["q"], inp["k"], inp["v"], inp["alpha"], inp["b"], inp["w"]


def oracle(inp, flags, chains=None, S0=None):
    h = {k_: _np(v_) for k_, v_ in inp.items()}
    s0 = h["S0"] if S0 is None else _np(S0)
    if chains is None:
        return c_oracle.recurrent(h["q"], h["k"], h["v"], h["alpha"], h["b"], h["w"], s0, flags=flags)
    outs, states = [], []
    for bi, hi in chains:
        sl = lambda x: np.ascontiguousarray(x[bi:bi + 1, :, hi:hi + 1])
        ss = None if s0 is None else np.ascontiguousarray(s0[bi:bi + 1, hi:hi + 1])
        o, S = c_oracle.recurrent(sl(h["q"]), sl(h["k"]), sl(h["v"]), sl(h["alpha"]), sl(h["b"]), sl(h["w"]),
                                  ss, flags=flags)
        outs.append(o[0, :, 0])
        states.append(S[0, 0])
    return np.stack(outs), np.stack(states)


def check(what, o, S, ro, rS, tol):
    eo, eS = rel_l2(o, ro), rel_l2(S, rS)
    print(f"[parity] {what}: relL2 o={eo:.3e} S={eS:.3e} (tol {tol:g})", flush=True)
    assert eo <= tol and eS <= tol, f"{what}: o {eo:.3e} S {eS:.3e} > {tol}"


CASES = [
    # B, T, H, dk, dv, io, gate dtype, flags, S0 std
    (2, 100, 3, 128, 128, BF16, BF16, LOG, 0.05),
    (1, 130, 2, 64, 48, BF16, F32, LOG | NEG, None),
    (1, 90, 2, 128, 256, BF16, BF16, LOG | NEG | L2, 0.05),
    (2, 70, 2, 32, 64, F32, F32, LOG | NEG | L2, 0.05),
    (1, 65, 2, 16, 16, F32, F32, L2, None),
    (1, 200, 2, 128, 128, BF16, F32, L2, 0.05),
    (1, 64, 2, 16, 32, BF16, BF16, 0, None),
    (2, 47, 2, 128, 128, BF16, BF16, LOG | L2, None),
]


def _id(c):
    B, T, H, dk, dv, io, gt, fl, s0 = c
    n = lambda d: "bf16" if d == BF16 else "f32"
    return f"B{B}T{T}H{H}dk{dk}dv{dv}io{n(io)}g{n(gt)}fl{fl}{'S0' if s0 else ''}"


@pytest.mark.parametrize("mode", ["chunk", "recurrent"])
@pytest.mark.parametrize("case", CASES, ids=_id)
def test_prologue_small(dev, case, mode):
    B, T, H, dk, dv, io, gt, fl, s0 = case
    inp = make(dev, B, T, H, dk, dv, io, gt, fl, seed=T * 5 + dk + fl, s0=s0)
    fn = g.chunk_fwd if mode == "chunk" else g.recurrent_step
    o, S = fn(*args(inp), inp["S0"], flags=fl)
    torch.cuda.synchronize()
    ro, rS = oracle(inp, fl)
    check(f"{mode} {_id(case)}", _np(o), _np(S), ro, rS, TOL[io])


def test_prologue_flags_are_honoured(dev):
    """Logits with the flag match the same gates activated on the host (bf16-rounded), and
    b x 2 changes the result."""
    inp = make(dev, 1, 64, 2, 64, 64, BF16, BF16, LOG, seed=1)
    a = args(inp)
    o_log, _ = g.chunk_fwd(*a, flags=LOG)
    r_log, _ = g.recurrent_step(*a, flags=LOG)
    act = [torch.sigmoid(x.float()).to(BF16) for x in (inp["alpha"], inp["b"], inp["w"])]
    o_act, _ = g.chunk_fwd(inp["q"], inp["k"], inp["v"], *act, flags=0)
    o_neg, _ = g.chunk_fwd(*a, flags=LOG | NEG)
    torch.cuda.synchronize()
    assert rel_l2(_np(o_log), _np(r_log)) < 2e-2
    assert rel_l2(_np(o_log), _np(o_act)) < 2e-2
    assert rel_l2(_np(o_log), _np(o_neg)) > 0.05


def test_prologue_full_size_chunk_sampled(dev):
    """B4 H16 T2048 d128 with bf16 gate logits, b x 2 and q/k L2 norm in-kernel (the bench's
    prologue workload), sampled chains against the oracle."""
    B, T, H, dk, dv = 4, 2048, 16, 128, 128
    fl = LOG | NEG | L2
    inp = make(dev, B, T, H, dk, dv, BF16, BF16, fl, seed=101)
    o, S = g.chunk_fwd(*args(inp), flags=fl)
    torch.cuda.synchronize()
    chains = [(0, 0), (1, 7), (3, 15)]
    ro, rS = oracle(inp, fl, chains)
    on, Sn = _np(o), _np(S)
    check("chunk B4H16T2048 prologue", np.stack([on[b, :, h] for b, h in chains]),
          np.stack([Sn[b, h] for b, h in chains]), ro, rS, 2e-2)


def test_prologue_decode_in_place_sampled(dev):
    B, H, dk, dv = 256, 16, 128, 128
    fl = LOG | L2
    inp = make(dev, B, 1, H, dk, dv, BF16, BF16, fl, seed=202, s0=0.05)
    S = inp["S0"].clone()
    chains = [(0, 0), (100, 5), (255, 15)]
    ro, rS = oracle(inp, fl, chains, S0=S)
    o, _ = g.recurrent_step(*args(inp), S, inplace=True, flags=fl)
    torch.cuda.synchronize()
    on, Sn = _np(o), _np(S)
    check("decode B256H16 prologue", np.stack([on[b, :, h] for b, h in chains]),
          np.stack([Sn[b, h] for b, h in chains]), ro, rS, 2e-2)
