"""GPU parity of packed variable-length batches against the fp64 oracle (needs an MI355X).

N sequences of different lengths packed back to back on the token axis; each
runs the recurrence from its own state.  The oracle (``oracle.reference.varlen``)
runs the C oracle on each sequence alone; grouped value heads are widened
with ``share_qk_heads`` first.  Tolerances as for the plain path: rel-L2
<= 1e-4 with fp32 I/O, <= 2e-2 with bf16 I/O.
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_19_amd as g
from gated_delta_rule_19_amd import inputs
from oracle import c_oracle
from oracle.reference import rel_l2, share_qk_heads, varlen

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


def make(dev, lengths, H, Hv, dk, dv, io, gate, flags, seed, s0=None):
    return inputs.make_packed(lengths, H, dk, dv, io, seed, dev, s0_std=s0, gate_logits=bool(flags & LOG),
                              unit_qk=not (flags & L2), gate_dtype=gate, Hv=Hv)


def args(inp):
    return inp["q"], inp["k"], inp["v"], inp["alpha"], inp["b"], inp["w"]


def oracle(inp, flags, cu=None, seqs=None, S0=None):
    """Oracle o and S; with ``seqs``, only those sequences (o rows of the others are 0)."""
    h = {k_: _np(v_) for k_, v_ in inp.items() if k_ != "cu"}
    cu = inp["cu"].cpu().tolist() if cu is None else cu
    s0 = h["S0"] if S0 is None else _np(S0)
    Hv = h["v"].shape[2]
    qg, kg = (np.ascontiguousarray(x, dtype=np.float32) for x in share_qk_heads(h["q"], h["k"], Hv))
    form = lambda *a: c_oracle.recurrent(*a, flags=flags)
    if seqs is None:
        return varlen(cu, qg, kg, h["v"], h["alpha"], h["b"], h["w"], s0, form=form)
    outs, states = [], []
    for i in seqs:
        s, e = cu[i], cu[i + 1]
        sl = lambda x: np.ascontiguousarray(x[:, s:e])
        ss = None if s0 is None else s0[i:i + 1]
        o, S = varlen([0, e - s], sl(qg), sl(kg), sl(h["v"]), sl(h["alpha"]), sl(h["b"]), sl(h["w"]), ss, form=form)
        outs.append(o[0])
        states.append(S[0])
    return outs, states


def check(what, o, S, ro, rS, tol):
    eo, eS = rel_l2(o, ro), rel_l2(S, rS)
    print(f"[parity] {what}: relL2 o={eo:.3e} S={eS:.3e} (tol {tol:g})", flush=True)
    assert eo <= tol and eS <= tol, f"{what}: o {eo:.3e} S {eS:.3e} > {tol}"


CASES = [
    # lengths, H, Hv, dk, dv, io, gate dtype, flags, S0 std
    ([100], 2, 2, 64, 64, F32, F32, 0, 0.05),
    ([1, 63, 64, 65, 130, 0, 7], 2, 2, 128, 128, BF16, F32, 0, 0.05),
    ([0, 0, 5, 0], 1, 2, 32, 48, F32, F32, L2, 0.05),
    ([200, 3, 64, 1], 2, 4, 128, 64, BF16, BF16, LOG | NEG | L2, None),
    ([17, 129, 40], 3, 3, 16, 16, F32, F32, LOG, None),
    ([64, 64, 64, 1, 127], 2, 2, 128, 256, BF16, F32, 0, 0.05),
]


def _id(c):
    lens, H, Hv, dk, dv, io, gt, fl, s0 = c
    n = lambda d: "bf16" if d == BF16 else "f32"
    return (f"N{len(lens)}T{sum(lens)}H{H}Hv{Hv}dk{dk}dv{dv}io{n(io)}g{n(gt)}fl{fl}{'S0' if s0 else ''}")


@pytest.mark.parametrize("mode", ["chunk", "recurrent"])
@pytest.mark.parametrize("case", CASES, ids=_id)
def test_varlen_small(dev, case, mode):
    lens, H, Hv, dk, dv, io, gt, fl, s0 = case
    inp = make(dev, lens, H, Hv, dk, dv, io, gt, fl, seed=sum(lens) + 3 * len(lens) + dk, s0=s0)
    fn = g.chunk_fwd_varlen if mode == "chunk" else g.recurrent_varlen
    o, S = fn(*args(inp), inp["cu"], inp["S0"], flags=fl)
    torch.cuda.synchronize()
    assert tuple(o.shape) == (1, sum(lens), Hv, dv) and tuple(S.shape) == (len(lens), Hv, dk, dv)
    ro, rS = oracle(inp, fl)
    check(f"{mode} {_id(case)}", _np(o), _np(S), ro, rS, TOL[io])


def test_varlen_equal_lengths_match_the_batched_call(dev):
    """Equal lengths packed = the ordinary batched call: same chunks, same kernels, same bits."""
    N, L, H, dk, dv = 4, 300, 2, 128, 128
    inp = make(dev, [L] * N, H, H, dk, dv, BF16, F32, 0, seed=11, s0=0.05)
    unpack = lambda x: x.reshape(N, L, *x.shape[2:]).contiguous()
    for fv, fb in ((g.chunk_fwd_varlen, g.chunk_fwd), (g.recurrent_varlen, g.recurrent_step)):
        o1, S1 = fv(*args(inp), inp["cu"], inp["S0"])
        o2, S2 = fb(*(unpack(x) for x in args(inp)), inp["S0"])
        torch.cuda.synchronize()
        assert torch.equal(unpack(o1), o2) and torch.equal(S1, S2), fv.__name__


def test_varlen_one_token_sequences_are_decode_steps(dev):
    """256 one-token sequences updated in place = one batched decode step, up to the order
    of the fp32 sums (the batched step runs the decode kernel, the packed batch the general
    recurrent kernel): the states agree to fp32 rounding, the bf16 outputs to one rounding."""
    N, H, dk, dv = 256, 16, 128, 128
    inp = make(dev, [1] * N, H, H, dk, dv, BF16, BF16, LOG | L2, seed=12, s0=0.05)
    S1 = inp["S0"].clone()
    S2 = inp["S0"].clone()
    o1, _ = g.recurrent_varlen(*args(inp), inp["cu"], S1, inplace=True, flags=LOG | L2)
    unpack = lambda x: x.reshape(N, 1, *x.shape[2:]).contiguous()
    o2, _ = g.recurrent_step(*(unpack(x) for x in args(inp)), S2, inplace=True, flags=LOG | L2)
    torch.cuda.synchronize()
    eS = rel_l2(_np(S1), _np(S2))
    eo = rel_l2(_np(unpack(o1)), _np(o2))
    print(f"[parity] varlen one-token vs batched decode: S {eS:.2e}, o {eo:.2e}", flush=True)
    assert eS <= 1e-6 and eo <= 4e-3


def test_varlen_full_size_sampled(dev):
    """8192 packed tokens in a seeded log-uniform length mix, H16 d128 bf16: sampled sequences."""
    lens = inputs.length_mix(8192, seed=1)
    H, dk, dv = 16, 128, 128
    inp = make(dev, lens, H, H, dk, dv, BF16, F32, 0, seed=21)
    o, S = g.chunk_fwd_varlen(*args(inp), inp["cu"])
    torch.cuda.synchronize()
    cu = inp["cu"].cpu().tolist()
    seqs = [0, int(np.argmax(lens)), len(lens) - 1]
    ro, rS = oracle(inp, 0, seqs=seqs)
    on, Sn = _np(o), _np(S)
    for i, r_o, r_S in zip(seqs, ro, rS):
        check(f"chunk varlen seq {i} (len {lens[i]})", on[0, cu[i]:cu[i + 1]], Sn[i], r_o, r_S, 2e-2)


def test_varlen_offsets_are_clamped(dev):
    """Offsets that break the rules (decreasing, negative, past T) are clamped into [0, T]
    and raised to the running maximum in the chunked mode; the result then equals the
    oracle on the clamped offsets.  The recurrent mode clamps each offset into [0, T]:
    it must run and give finite states."""
    lens = [50, 30, 120]
    H, dk, dv = 2, 64, 64
    inp = make(dev, lens, H, H, dk, dv, F32, F32, 0, seed=31, s0=0.05)
    T = sum(lens)
    raw = [-5, 40, 20, T + 90]       # N = 3
    cu = torch.tensor(raw, dtype=torch.int32, device=dev)
    clamped = [0, 40, 40, T]
    S0 = inp["S0"]
    o = torch.zeros_like(inp["v"])
    _, S = g.chunk_fwd_varlen(*args(inp), cu, S0, o=o)
    _, S_r = g.recurrent_varlen(*args(inp), cu, S0)
    torch.cuda.synchronize()
    ro, rS = oracle(inp, 0, cu=clamped)
    check("chunk clamped offsets", _np(o), _np(S), ro, rS, 1e-4)
    assert torch.isfinite(S_r).all()
