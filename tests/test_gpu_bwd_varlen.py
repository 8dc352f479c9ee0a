"""GPU parity of the packed-batch backward (``gdn2_chunk_bwd_varlen``) against the fp64
oracle (needs an MI355X).  Sequences of a packed batch are independent (the forward's pins
fix that: isolation of sequences, equal lengths = an ordinary batch), so the expected
gradients are ``oracle.backward.recurrent_bwd`` of each sequence on its own, laid back to
back.  Same bars as the chunked backward: rel-L2 <= 1e-4 (fp32 I/O), <= 2e-2 (bf16).
Lengths include empty sequences, one-token sequences and ragged last chunks; both the
matrix-core (bf16, d 128) and the vector-ALU (fp32) gradient paths run.
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
