"""GPU parity of the short convolution fused into the prologue (needs an MI355X).

``gdn2_chunk_fwd_conv`` and ``gdn2_recurrent_step_conv`` are defined as
``gdn2_short_conv`` on the concatenated projection [q | k | v] followed by the
core on its three parts.  The oracle takes that chain in fp64:
``oracle.reference.short_conv`` over the concatenation, the split,
``share_qk_heads`` for grouped value heads, then the C oracle's recurrence
with the same prologue flags.  The fused kernels round the convolution's
output to the I/O dtype, as the standalone call stores it; the oracle keeps
fp64, which the bf16 tolerance (rel-L2 2e-2) covers and which is below 1e-6
relative with fp32 I/O (tolerance 1e-4).  The window after the last token
holds raw inputs and must match exactly.

Covered: both modes; K = 1..4, with and without SiLU; every prologue flag;
grouped value heads; fp32 and bf16; sequences shorter than the window (the
new window then mixes the carried one and the inputs); T = 0 (the window and
the state are only carried over); a sequence split into pieces with the state
and the window carried between calls; the decode step with alternating
window buffers; the chunked call updating the window in place.
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_19_amd as g
from gated_delta_rule_19_amd import inputs
from oracle import c_oracle
from oracle.reference import rel_l2, rel_l2_chains, share_qk_heads, short_conv

pytestmark = pytest.mark.gpu

LOG, NEG, L2 = g.FLAG_GATE_LOGITS, g.FLAG_NEG_EIGVAL, g.FLAG_QK_L2NORM
F32, BF16 = torch.float32, torch.bfloat16
TOL = {F32: 1e-4, BF16: 2e-2}


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    g.lib()
    return torch.device("cuda:0")


def _np(x):
    return None if x is None else x.detach().to("cpu", torch.float64).numpy()


def make(dev, B, T, H, Hv, dk, dv, io, gate, flags, K, seed, wscale):
    inp = inputs.make_raw(B, T, H, dk, dv, io, seed, dev, s0_std=0.05, gate_logits=bool(flags & LOG),
                          unit_qk=True, gate_dtype=gate, Hv=Hv)
    C = 2 * H * dk + Hv * dv
    gen = torch.Generator().manual_seed(seed + 7)
    weight = (torch.randn(C, K, generator=gen) * wscale).to(dev)
    state = (torch.randn(B, K - 1, C, generator=gen) * 0.5).to(io).to(dev) if K > 1 else None
    return inp, weight, state


def oracle_chain(inp, weight, state, silu, flags, S0=None):
    """short_conv on [q | k | v] -> split -> (shared q/k heads) -> recurrence, fp64."""
    q, k, v = _np(inp["q"]), _np(inp["k"]), _np(inp["v"])
    B, T, H, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    x = np.concatenate([q.reshape(B, T, H * dk), k.reshape(B, T, H * dk), v.reshape(B, T, Hv * dv)], axis=-1)
    y, window = short_conv(x, _np(weight), None if state is None else _np(state), silu=silu)
    qc = y[..., :H * dk].reshape(B, T, H, dk)
    kc = y[..., H * dk:2 * H * dk].reshape(B, T, H, dk)
    vc = y[..., 2 * H * dk:].reshape(B, T, Hv, dv)
    if Hv != H:
        qc, kc = share_qk_heads(qc, kc, Hv)
    s0 = _np(inp["S0"]) if S0 is None else _np(S0)
    f32 = lambda a: None if a is None else np.ascontiguousarray(a, dtype=np.float32)
    o, S = c_oracle.recurrent(f32(qc), f32(kc), f32(vc), f32(_np(inp["alpha"])), f32(_np(inp["b"])),
                              f32(_np(inp["w"])), f32(s0), flags=flags)
    return o, S, window


def run(mode, inp, weight, state, silu, flags, S0="inp", state_out=None):
    a = (inp["q"], inp["k"], inp["v"], inp["alpha"], inp["b"], inp["w"], weight, state)
    s0 = inp["S0"] if S0 == "inp" else S0
    if mode == "chunk":
        return g.chunk_fwd_conv(*a, s0, conv_silu=silu, flags=flags, conv_state_out=state_out)
    return g.recurrent_step_conv(*a, s0, conv_silu=silu, flags=flags, conv_state_out=state_out)


def check(what, io, o, S, win, ro, rS, rwin):
    tol = TOL[io]
    eo, eS = rel_l2(_np(o), ro), rel_l2(_np(S), rS)
    wo = float(rel_l2_chains(_np(o), ro, (0, 2)).max())
    print(f"[parity] {what}: relL2 o={eo:.3e} S={eS:.3e}; worst chain o={wo:.3e} (tol {tol:g})", flush=True)
    assert eo <= tol and eS <= tol and wo <= tol, f"{what}: o {eo:.3e} (worst {wo:.3e}) S {eS:.3e} > {tol}"
    if rwin is None or rwin.size == 0:
        return
    assert win is not None
    assert np.array_equal(_np(win), rwin), f"{what}: window differs (max {np.abs(_np(win) - rwin).max():.3e})"


CASES = [
    # B, T, H, Hv, dk, dv, io, gate, flags, K, silu, weight scale
    (2, 200, 2, 2, 64, 64, BF16, BF16, L2, 4, True, 0.5),
    (1, 130, 2, 4, 128, 128, BF16, F32, LOG | NEG | L2, 3, False, 0.5),
    (1, 100, 1, 1, 32, 48, F32, F32, L2, 2, True, 0.5),
    (2, 70, 2, 2, 16, 32, F32, F32, 0, 4, False, 0.3),
    (1, 90, 2, 2, 128, 256, BF16, BF16, LOG | L2, 4, True, 0.5),
    (2, 65, 2, 2, 128, 128, BF16, F32, L2, 1, False, 0.5),
    (1, 1, 2, 2, 128, 128, BF16, F32, L2, 4, True, 0.5),
    (2, 2, 2, 4, 64, 64, F32, F32, L2, 4, False, 0.5),
    (1, 3, 1, 1, 128, 64, BF16, BF16, L2 | LOG, 4, True, 0.5),
]


def _id(c):
    B, T, H, Hv, dk, dv, io, gate, flags, K, silu, _ = c
    return f"B{B}T{T}H{H}Hv{Hv}dk{dk}dv{dv}{'bf16' if io == BF16 else 'f32'}fl{flags}K{K}{'silu' if silu else ''}"


@pytest.mark.parametrize("mode", ["chunk", "recurrent"])
@pytest.mark.parametrize("case", CASES, ids=_id)
def test_fused_conv_against_oracle_chain(dev, mode, case):
    B, T, H, Hv, dk, dv, io, gate, flags, K, silu, ws = case
    inp, weight, state = make(dev, B, T, H, Hv, dk, dv, io, gate, flags, K, seed=31 + T + K, wscale=ws)
    o, S, win = run(mode, inp, weight, state, silu, flags)
    torch.cuda.synchronize()
    ro, rS, rwin = oracle_chain(inp, weight, state, silu, flags)
    check(f"{mode} conv {_id(case)}", io, o, S, win, ro, rS, rwin)


@pytest.mark.parametrize("mode", ["chunk", "recurrent"])
def test_fused_conv_zero_tokens_carries_window_and_state(dev, mode):
    inp, weight, state = make(dev, 2, 0, 2, 2, 64, 64, BF16, F32, L2, 4, seed=5, wscale=0.5)
    o, S, win = run(mode, inp, weight, state, False, L2)
    torch.cuda.synchronize()
    assert torch.equal(win, state)
    assert torch.equal(S, inp["S0"])


@pytest.mark.parametrize("mode", ["chunk", "recurrent"])
def test_fused_conv_pieces_equal_one_call(dev, mode):
    """A sequence in two pieces, state and window carried, against the oracle chain
    on the whole sequence."""
    B, T, H, Hv, dk, dv, io, K = 2, 150, 2, 2, 128, 128, BF16, 4
    inp, weight, state = make(dev, B, T, H, Hv, dk, dv, io, F32, L2, K, seed=77, wscale=0.5)
    T1 = 77
    part = lambda d, a, b_: {n: (x[:, a:b_].contiguous() if n != "S0" else x) for n, x in d.items()}
    p1, p2 = part(inp, 0, T1), part(inp, T1, T)
    o1, S1, w1 = run(mode, p1, weight, state, True, L2)
    o2, S2, w2 = run(mode, p2, weight, w1, True, L2, S0=S1)
    torch.cuda.synchronize()
    ro, rS, rwin = oracle_chain(inp, weight, state, True, L2)
    check(f"{mode} conv in pieces {T1}+{T - T1}", io, torch.cat([o1, o2], 1), S2, w2, ro, rS, rwin)


def test_fused_conv_decode_steps_with_alternating_windows(dev):
    """Five decode steps (T = 1 each) through two window buffers against the oracle
    chain over the five tokens."""
    B, T, H, Hv, dk, dv, io, K = 3, 5, 2, 4, 128, 128, BF16, 4
    inp, weight, state = make(dev, B, T, H, Hv, dk, dv, io, BF16, LOG | L2, K, seed=91, wscale=0.5)
    bufs = [state.clone(), torch.empty_like(state)]
    S = inp["S0"].clone()
    outs = []
    for t in range(T):
        step = {n: (x[:, t:t + 1].contiguous() if n != "S0" else x) for n, x in inp.items()}
        o, S, _ = run("recurrent", step, weight, bufs[t % 2], True, LOG | L2, S0=S, state_out=bufs[(t + 1) % 2])
        outs.append(o)
    torch.cuda.synchronize()
    ro, rS, rwin = oracle_chain(inp, weight, state, True, LOG | L2)
    check("decode x5 with conv window", io, torch.cat(outs, 1), S, bufs[T % 2], ro, rS, rwin)


DECODE_CASES = [
    # B, H, Hv, dk, dv, io, gate, flags, K, silu, carried window, initial state
    (4, 2, 2, 64, 64, F32, F32, L2, 4, True, True, True),
    (3, 2, 4, 128, 256, BF16, BF16, LOG | NEG | L2, 3, False, True, True),
    (2, 4, 4, 128, 128, BF16, F32, 0, 2, True, False, True),
    (5, 1, 2, 64, 128, BF16, F32, LOG | L2, 1, False, True, False),
    (2, 2, 2, 128, 32, F32, F32, L2, 4, True, False, True),
    (7, 2, 2, 128, 128, BF16, BF16, LOG | L2, 4, True, True, True),
    (3, 2, 2, 64, 256, F32, F32, NEG | LOG, 3, True, True, False),
]


def _did(c):
    B, H, Hv, dk, dv, io, gate, flags, K, silu, win, s0 = c
    return (f"B{B}H{H}Hv{Hv}dk{dk}dv{dv}{'bf16' if io == BF16 else 'f32'}g{'bf16' if gate == BF16 else 'f32'}"
            f"fl{flags}K{K}{'silu' if silu else ''}{'win' if win else 'nowin'}{'S0' if s0 else 'zero'}")


@pytest.mark.parametrize("case", DECODE_CASES, ids=_did)
def test_fused_conv_decode_step(dev, case):
    """One token per sequence (the decode kernel's layout, dk >= 64): o, the
    state and the window after the token against the oracle chain."""
    B, H, Hv, dk, dv, io, gate, flags, K, silu, win, s0 = case
    inp, weight, state = make(dev, B, 1, H, Hv, dk, dv, io, gate, flags, K, seed=400 + dk + dv + K, wscale=0.5)
    if not win:
        state = None
    S0 = inp["S0"] if s0 else None
    out = torch.empty(B, K - 1, weight.shape[0], dtype=io, device=dev) if K > 1 else None
    o, S, w = run("recurrent", inp, weight, state, silu, flags, S0=S0, state_out=out)
    torch.cuda.synchronize()
    ro, rS, rwin = oracle_chain(inp, weight, state, silu, flags,
                                S0=None if s0 else torch.zeros_like(inp["S0"]))
    check(f"decode conv {_did(case)}", io, o, S, w, ro, rS, rwin)


def test_fused_conv_chunked_window_in_place(dev):
    B, T, H, Hv, dk, dv, io, K = 2, 140, 2, 2, 64, 128, BF16, 3
    inp, weight, state = make(dev, B, T, H, Hv, dk, dv, io, F32, L2, K, seed=13, wscale=0.5)
    ref_o, ref_S, ref_w = run("chunk", inp, weight, state, False, L2)
    win = state.clone()
    o, S, w = run("chunk", inp, weight, win, False, L2, state_out=win)
    torch.cuda.synchronize()
    assert w.data_ptr() == win.data_ptr()
    assert torch.equal(w, ref_w) and torch.equal(o, ref_o) and torch.equal(S, ref_S)


def test_recurrent_window_in_place_is_refused(dev):
    inp, weight, state = make(dev, 1, 4, 2, 2, 64, 64, BF16, F32, L2, 4, seed=3, wscale=0.5)
    with pytest.raises(g.Gdn2Error) as e:
        run("recurrent", inp, weight, state, False, L2, state_out=state)
    assert e.value.code == 4   # GDN2_ERR_ALIAS
