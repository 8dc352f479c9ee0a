"""GPU parity of the packed-batch backward (``gdn2_chunk_bwd_varlen``) against the fp64
oracle (needs an MI355X).  Sequences of a packed batch are independent (the forward's pins
fix that: isolation of sequences, equal lengths = an ordinary batch), so the expected
gradients are ``oracle.backward.recurrent_bwd`` of each sequence on its own, laid back to
back.  Same bars as the chunked backward: rel-L2 <= 1e-4 (fp32 I/O), <= 2e-2 (bf16).
Lengths include empty sequences, one-token sequences and ragged last chunks; both the
matrix-core (bf16, d 128) and the vector-ALU (fp32) gradient paths run.  With grouped
value heads (Hv = 2H) and the in-kernel prologue (gate logits, b x 2, q/k L2 norm) the
expected gradients are ``oracle.backward.full_bwd`` of each sequence (pinned by finite
differences of the whole forward with its prologue).

The call takes the offsets in device memory, as the packed forward does, and runs the whole
batch from the chunk plan in a fixed number of launches.  A batch of equal lengths must give
the equal-length backward's gradients bit for bit (same per-chunk arithmetic, blocks found
through the plan instead of by position), and a batch of many short sequences of mixed
lengths is compared with the oracle sequence by sequence.
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_19_amd as g
from gated_delta_rule_19_amd import inputs
from oracle.backward import recurrent_bwd
from oracle.reference import rel_l2

pytestmark = pytest.mark.gpu
F32, BF16 = torch.float32, torch.bfloat16
NAMES = ("dq", "dk", "dv", "dalpha", "db", "dw", "dS0")


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    g.lib()
    return torch.device("cuda:0")


def _np(x):
    return None if x is None else x.detach().to("cpu", torch.float64).numpy()


@pytest.mark.parametrize("lengths,H,dk,dv,io,tol", [
    ((70, 0, 129, 1, 64), 2, 128, 128, BF16, 2e-2),
    ((33, 100, 0), 2, 64, 32, F32, 1e-4),
    ((0, 0), 1, 32, 32, BF16, 2e-2),
])
def test_packed_backward_matches_per_sequence_oracle(dev, lengths, H, dk, dv, io, tol):
    print(f"bwd varlen lengths={lengths} H={H} dk={dk} dv={dv} {io}", flush=True)
    N, T = len(lengths), sum(lengths)
    inp = inputs.make_packed(lengths, H, dk, dv, io, 5, dev, s0_std=0.05)
    gen = torch.Generator(device=dev)
    gen.manual_seed(6)
    dO = torch.randn(1, T, H, dv, generator=gen, device=dev).to(io)
    dS_T = torch.randn(N, H, dk, dv, generator=gen, device=dev)
    got = g.chunk_bwd_varlen(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["b"], inp["w"], dO, inp["cu"],
                             inp["S0"], dS_T)
    torch.cuda.synchronize()
    h = {n: _np(inp[n]) for n in ("q", "k", "v", "alpha", "b", "w", "S0")}
    dOn, dSn = _np(dO), _np(dS_T)
    want = {n: [] for n in NAMES}
    cu = [0]
    for n in lengths:
        cu.append(cu[-1] + n)
    for i in range(N):
        a, e = cu[i], cu[i + 1]
        sl = lambda x: x[:, a:e]
        r = recurrent_bwd(sl(h["q"]), sl(h["k"]), sl(h["v"]), sl(h["alpha"]), sl(h["b"]), sl(h["w"]),
                          h["S0"][i:i + 1], sl(dOn), dSn[i:i + 1])
        for n in NAMES:
            want[n].append(r[n] if n == "dS0" else r[n].reshape(1, e - a, *r[n].shape[2:]))
    for n in NAMES:
        ref = np.concatenate(want[n], axis=0 if n == "dS0" else 1)
        got_n = _np(got[n])
        if ref.size == 0:
            assert got_n.size == 0
            continue
        err = rel_l2(got_n, ref)
        print(f"  {n}: {err:.2e}", flush=True)
        assert err <= tol, n


LOG, NEG, L2 = g.FLAG_GATE_LOGITS, g.FLAG_NEG_EIGVAL, g.FLAG_QK_L2NORM


@pytest.mark.parametrize("lengths,H,Hv,dk,dv,io,gate,flags,tol", [
    ((70, 0, 129, 1, 64), 2, 4, 128, 128, BF16, BF16, LOG | NEG | L2, 2e-2),
    ((90, 3, 65), 1, 2, 128, 128, BF16, F32, LOG | L2, 2e-2),
    ((33, 100, 0), 2, 4, 64, 32, F32, F32, LOG | NEG | L2, 1e-4),
])
def test_packed_backward_grouped_heads_and_prologue(dev, lengths, H, Hv, dk, dv, io, gate, flags, tol):
    from oracle.backward import full_bwd
    print(f"bwd varlen lengths={lengths} H={H} Hv={Hv} dk={dk} dv={dv} {io} gates {gate} flags {flags}", flush=True)
    N, T = len(lengths), sum(lengths)
    inp = inputs.make_packed(lengths, H, dk, dv, io, 15, dev, s0_std=0.05, Hv=Hv, gate_dtype=gate,
                             gate_logits=bool(flags & LOG), unit_qk=not flags & L2)
    gen = torch.Generator(device=dev)
    gen.manual_seed(16)
    dO = torch.randn(1, T, Hv, dv, generator=gen, device=dev).to(io)
    dS_T = torch.randn(N, Hv, dk, dv, generator=gen, device=dev)
    got = g.chunk_bwd_varlen(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["b"], inp["w"], dO, inp["cu"],
                             inp["S0"], dS_T, flags=flags)
    torch.cuda.synchronize()
    h = {n: _np(inp[n]) for n in ("q", "k", "v", "alpha", "b", "w", "S0")}
    dOn, dSn = _np(dO), _np(dS_T)
    want = {n: [] for n in NAMES}
    cu = [0]
    for n in lengths:
        cu.append(cu[-1] + n)
    for i in range(N):
        a, e = cu[i], cu[i + 1]
        sl = lambda x: x[:, a:e]
        r = full_bwd(sl(h["q"]), sl(h["k"]), sl(h["v"]), sl(h["alpha"]), sl(h["b"]), sl(h["w"]),
                     h["S0"][i:i + 1], sl(dOn), dSn[i:i + 1], flags=flags)
        for n in NAMES:
            want[n].append(r[n] if n == "dS0" else r[n].reshape(1, e - a, *r[n].shape[2:]))
    for n in NAMES:
        ref = np.concatenate(want[n], axis=0 if n == "dS0" else 1)
        got_n = _np(got[n])
        assert got_n.shape == ref.shape, n
        if ref.size == 0:
            continue
        err = rel_l2(got_n, ref)
        print(f"  {n}: {err:.2e}", flush=True)
        assert err <= tol, n


@pytest.mark.parametrize("N,T,io,flags", [
    (3, 200, BF16, 0),
    (2, 128, BF16, LOG | NEG | L2),
    (3, 70, F32, 0),
])
def test_equal_lengths_equal_the_batched_backward_bitwise(dev, N, T, io, flags):
    print(f"bwd varlen equal lengths N={N} T={T} {io} flags {flags}", flush=True)
    H, dk, dv = 2, 64, 64
    inp = inputs.make_packed([T] * N, H, dk, dv, io, 25, dev, s0_std=0.05, gate_logits=bool(flags & LOG),
                             unit_qk=not flags & L2)
    gen = torch.Generator(device=dev)
    gen.manual_seed(26)
    dO = torch.randn(1, N * T, H, dv, generator=gen, device=dev).to(io)
    dS_T = torch.randn(N, H, dk, dv, generator=gen, device=dev)
    got = g.chunk_bwd_varlen(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["b"], inp["w"], dO, inp["cu"],
                             inp["S0"], dS_T, flags=flags)
    bat = lambda x: x.reshape(N, T, *x.shape[2:])
    ref = g.chunk_bwd(bat(inp["q"]), bat(inp["k"]), bat(inp["v"]), bat(inp["alpha"]), bat(inp["b"]),
                      bat(inp["w"]), bat(dO), inp["S0"], dS_T, flags=flags)
    torch.cuda.synchronize()
    for n in NAMES:
        a, b = got[n], ref[n]
        assert torch.equal(a.reshape(b.shape), b), n


def test_many_short_sequences(dev):
    rng = np.random.default_rng(41)
    lengths = [int(x) for x in rng.integers(0, 90, size=150)]
    lengths[:4] = [0, 1, 64, 65]
    H, dk, dv = 2, 64, 64
    N, T = len(lengths), sum(lengths)
    print(f"bwd varlen {N} sequences, {T} tokens", flush=True)
    inp = inputs.make_packed(lengths, H, dk, dv, BF16, 35, dev, s0_std=0.05)
    gen = torch.Generator(device=dev)
    gen.manual_seed(36)
    dO = torch.randn(1, T, H, dv, generator=gen, device=dev).to(BF16)
    dS_T = torch.randn(N, H, dk, dv, generator=gen, device=dev)
    got = g.chunk_bwd_varlen(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["b"], inp["w"], dO, inp["cu"],
                             inp["S0"], dS_T)
    torch.cuda.synchronize()
    h = {n: _np(inp[n]) for n in ("q", "k", "v", "alpha", "b", "w", "S0")}
    dOn, dSn = _np(dO), _np(dS_T)
    cu = np.concatenate([[0], np.cumsum(lengths)])
    worst = {n: 0.0 for n in NAMES}
    gotn = {n: _np(got[n]) for n in NAMES}
    for i in range(N):
        a, e = int(cu[i]), int(cu[i + 1])
        sl = lambda x: x[:, a:e]
        r = recurrent_bwd(sl(h["q"]), sl(h["k"]), sl(h["v"]), sl(h["alpha"]), sl(h["b"]), sl(h["w"]),
                          h["S0"][i:i + 1], sl(dOn), dSn[i:i + 1])
        for n in NAMES:
            mine = gotn[n][i:i + 1] if n == "dS0" else gotn[n][:, a:e]
            if mine.size == 0:
                continue
            worst[n] = max(worst[n], rel_l2(mine, r[n].reshape(mine.shape)))
    print("  worst per sequence: " + ", ".join(f"{n} {v:.2e}" for n, v in worst.items()), flush=True)
    for n, v in worst.items():
        assert v <= 2e-2, n


@pytest.mark.parametrize("io", [BF16, F32])
def test_offsets_are_clamped_as_in_the_forward(dev, io):
    """Offsets that break the rules (negative, decreasing, past T) go through the forward's
    chunk plan, which clamps them into [0, T] and raises each to the running maximum: the
    gradients equal those for the clamped offsets, bit for bit."""
    lens = [50, 30, 120]
    H, dk, dv = 2, 64, 64
    T = sum(lens)
    print(f"bwd varlen clamped offsets {io}", flush=True)
    inp = inputs.make_packed(lens, H, dk, dv, io, 45, dev, s0_std=0.05)
    gen = torch.Generator(device=dev)
    gen.manual_seed(46)
    dO = torch.randn(1, T, H, dv, generator=gen, device=dev).to(io)
    dS_T = torch.randn(len(lens), H, dk, dv, generator=gen, device=dev)
    raw = torch.tensor([-5, 40, 20, T + 90], dtype=torch.int32, device=dev)
    clamped = torch.tensor([0, 40, 40, T], dtype=torch.int32, device=dev)
    x = (inp["q"], inp["k"], inp["v"], inp["alpha"], inp["b"], inp["w"], dO)
    a = g.chunk_bwd_varlen(*x, raw, inp["S0"], dS_T)
    b = g.chunk_bwd_varlen(*x, clamped, inp["S0"], dS_T)
    torch.cuda.synchronize()
    for n in NAMES:
        assert torch.equal(a[n], b[n]), n
    assert all(torch.isfinite(a[n].float()).all() for n in NAMES)
