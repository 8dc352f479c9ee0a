"""GPU parity of grouped value heads against the fp64 oracle (needs an MI355X).

Hv value heads over H query/key heads (burn-gdn2 README, "Configuration":
num_v_heads): each value head has its own state, gates and values and reads
the q and k of head hv // (Hv / H).  The kernels index q and k by that head;
the oracle widens q and k to the value heads (``share_qk_heads``) and runs
the per-head recurrence in double.  Tolerances as for the plain path: rel-L2
<= 1e-4 with fp32 I/O, <= 2e-2 with bf16 I/O.
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_19_amd as g
from gated_delta_rule_19_amd import inputs
from oracle import c_oracle
from oracle.reference import rel_l2, share_qk_heads

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


def make(dev, B, T, H, Hv, dk, dv, io, gate, flags, seed, s0=None):
    return inputs.make_raw(B, T, H, dk, dv, io, seed, dev, s0_std=s0, gate_logits=bool(flags & LOG),
                           unit_qk=not (flags & L2), gate_dtype=gate, Hv=Hv)


def args(inp):
    return inp["q"], inp["k"], inp["v"], inp["alpha"], inp["b"], inp["w"]


def oracle(inp, flags, chains=None, S0=None):
    """Oracle outputs; with ``chains`` = [(batch, value head)], only those chains."""
    h = {k_: _np(v_) for k_, v_ in inp.items()}
    s0 = h["S0"] if S0 is None else _np(S0)
    Hv = h["v"].shape[2]
    qg, kg = (np.ascontiguousarray(x, dtype=np.float32) for x in share_qk_heads(h["q"], h["k"], Hv))
    if chains is None:
        return c_oracle.recurrent(qg, kg, h["v"], h["alpha"], h["b"], h["w"], s0, flags=flags)
    outs, states = [], []
    for bi, hi in chains:
        sl = lambda x: np.ascontiguousarray(x[bi:bi + 1, :, hi:hi + 1])
        ss = None if s0 is None else np.ascontiguousarray(s0[bi:bi + 1, hi:hi + 1])
        o, S = c_oracle.recurrent(sl(qg), sl(kg), sl(h["v"]), sl(h["alpha"]), sl(h["b"]), sl(h["w"]), ss,
                                  flags=flags)
        outs.append(o[0, :, 0])
        states.append(S[0, 0])
    return np.stack(outs), np.stack(states)


def check(what, o, S, ro, rS, tol):
    eo, eS = rel_l2(o, ro), rel_l2(S, rS)
    print(f"[parity] {what}: relL2 o={eo:.3e} S={eS:.3e} (tol {tol:g})", flush=True)
    assert eo <= tol and eS <= tol, f"{what}: o {eo:.3e} S {eS:.3e} > {tol}"


CASES = [
    # B, T, H, Hv, dk, dv, io, gate dtype, flags, S0 std
    (2, 100, 2, 4, 128, 128, BF16, F32, 0, 0.05),
    (1, 130, 1, 4, 64, 64, F32, F32, 0, None),
    (1, 70, 3, 6, 32, 48, BF16, BF16, LOG | NEG | L2, 0.05),
    (2, 65, 2, 8, 16, 32, F32, F32, L2, None),
    (1, 90, 2, 4, 128, 256, BF16, BF16, LOG, None),
    (1, 64, 4, 4, 64, 32, BF16, F32, 0, 0.05),
]


def _id(c):
    B, T, H, Hv, dk, dv, io, gt, fl, s0 = c
    n = lambda d: "bf16" if d == BF16 else "f32"
    return f"B{B}T{T}H{H}Hv{Hv}dk{dk}dv{dv}io{n(io)}g{n(gt)}fl{fl}{'S0' if s0 else ''}"


@pytest.mark.parametrize("mode", ["chunk", "recurrent"])
@pytest.mark.parametrize("case", CASES, ids=_id)
def test_grouped_small(dev, case, mode):
    B, T, H, Hv, dk, dv, io, gt, fl, s0 = case
    inp = make(dev, B, T, H, Hv, dk, dv, io, gt, fl, seed=T * 7 + Hv + dk, s0=s0)
    fn = g.chunk_fwd if mode == "chunk" else g.recurrent_step
    o, S = fn(*args(inp), inp["S0"], flags=fl)
    torch.cuda.synchronize()
    assert tuple(o.shape) == (B, T, Hv, dv) and tuple(S.shape) == (B, Hv, dk, dv)
    ro, rS = oracle(inp, fl)
    check(f"{mode} {_id(case)}", _np(o), _np(S), ro, rS, TOL[io])


def test_grouped_equals_repeated_heads(dev):
    """A grouped call equals the ungrouped call on q, k repeated per value head (bf16
    inputs; the two calls run the same kernels on the same values, so they agree exactly)."""
    B, T, H, Hv, dk, dv = 2, 150, 2, 8, 128, 64
    inp = make(dev, B, T, H, Hv, dk, dv, BF16, BF16, LOG | L2, seed=9, s0=0.05)
    G = Hv // H
    qr, kr = (x.repeat_interleave(G, dim=2).contiguous() for x in (inp["q"], inp["k"]))
    for fn in (g.chunk_fwd, g.recurrent_step):
        o1, S1 = fn(*args(inp), inp["S0"], flags=LOG | L2)
        o2, S2 = fn(qr, kr, inp["v"], inp["alpha"], inp["b"], inp["w"], inp["S0"], flags=LOG | L2)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(S1, S2)


def test_grouped_full_size_chunk_sampled(dev):
    """B4 T2048, 4 query/key heads shared by 16 value heads, d128, bf16: sampled chains."""
    B, T, H, Hv, dk, dv = 4, 2048, 4, 16, 128, 128
    inp = make(dev, B, T, H, Hv, dk, dv, BF16, F32, 0, seed=303)
    o, S = g.chunk_fwd(*args(inp))
    torch.cuda.synchronize()
    chains = [(0, 0), (1, 7), (3, 15), (2, 4)]
    ro, rS = oracle(inp, 0, chains)
    on, Sn = _np(o), _np(S)
    check("chunk B4T2048 H4 Hv16", np.stack([on[b, :, h] for b, h in chains]),
          np.stack([Sn[b, h] for b, h in chains]), ro, rS, 2e-2)


def test_grouped_decode_in_place_sampled(dev):
    B, H, Hv, dk, dv = 256, 4, 16, 128, 128
    inp = make(dev, B, 1, H, Hv, dk, dv, BF16, BF16, LOG | L2, seed=404, s0=0.05)
    S = inp["S0"].clone()
    chains = [(0, 0), (100, 5), (255, 15), (17, 3)]
    ro, rS = oracle(inp, LOG | L2, chains, S0=S)
    o, _ = g.recurrent_step(*args(inp), S, inplace=True, flags=LOG | L2)
    torch.cuda.synchronize()
    on, Sn = _np(o), _np(S)
    check("decode B256 H4 Hv16", np.stack([on[b, :, h] for b, h in chains]),
          np.stack([Sn[b, h] for b, h in chains]), ro, rS, 2e-2)
