"""GPU parity of the short convolution and its gradient against the fp64 oracle
(needs an MI355X).

Causal depthwise convolution over tokens with K taps, optional SiLU and a carried
state of K-1 positions (burn-gdn2 README "Architecture": ShortConv before the L2
norm; "Configuration": use_short_conv).  Both sides get the same seeded x, dy,
state (bf16 widened exactly) and fp32 weights.  Bars: rel-L2 <= 1e-4 with fp32
I/O, <= 2e-2 for bf16 outputs (rounded once); the fp32 weight gradient <= 1e-4 in
both; the returned state is a copy, compared bit for bit.  Shapes span several
of the kernels' token spans (forward: 32 tokens fp32, 64 bf16, two a workgroup;
backward: 128-token spans of 32-token sub-spans) with ragged tails, channel
counts that leave a wave partly idle, T of 1 and 0, and every K from 1 to 8.
The backward also takes a gradient of the window after the last token
(dstate_out), checked against the oracle and by chaining the backward over the
pieces of a sequence.
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_19_amd as g
from oracle.reference import rel_l2, short_conv, short_conv_bwd

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    g.lib()
    return torch.device("cuda:0")


def _np(x):
    return None if x is None else x.detach().to("cpu", torch.float32).numpy().astype(np.float64)


def _draw(dev, B, T, C, K, dt, seed, state=True):
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    x = torch.randn(B, T, C, generator=gen, device=dev).to(dt)
    w = torch.randn(C, K, generator=gen, device=dev) * (1.0 / K) ** 0.5
    st = torch.randn(B, K - 1, C, generator=gen, device=dev).to(dt) if state else None
    dy = torch.randn(B, T, C, generator=gen, device=dev).to(dt)
    return x, w, st, dy


def _tol(dt):
    return 1e-4 if dt == torch.float32 else 2e-2


def _check(dev, B, T, C, K, dt, silu, state, seed):
    print(f"conv B={B} T={T} C={C} K={K} {dt} silu={silu} state={state} seed={seed}", flush=True)
    x, w, st, dy = _draw(dev, B, T, C, K, dt, seed, state)
    y, so = g.short_conv(x, w, st, silu=silu)
    dx, dw, ds = g.short_conv_bwd(x, w, dy, st, silu=silu)
    torch.cuda.synchronize()
    ry, rso = short_conv(_np(x), _np(w), _np(st), silu)
    rdx, rdw, rds = short_conv_bwd(_np(x), _np(w), _np(dy), _np(st), silu)
    tol = _tol(dt)
    if T > 0:
        assert rel_l2(_np(y), ry) <= tol
        assert rel_l2(_np(dx), rdx) <= tol
    np.testing.assert_array_equal(_np(so), rso)
    if T > 0 and B > 0:
        assert rel_l2(_np(dw), rdw) <= 1e-4
    else:
        assert torch.count_nonzero(dw) == 0
    if K > 1:
        if np.abs(rds).max() > 0:
            assert rel_l2(_np(ds), rds) <= tol
        else:
            assert torch.count_nonzero(ds) == 0


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("silu", [False, True])
@pytest.mark.parametrize("K", [1, 2, 3, 4, 5, 6, 7, 8])
def test_every_width(dev, K, silu, dt):
    _check(dev, 2, 70, 264, K, dt, silu, True, 100 + K)


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("B,T,C", [(1, 1, 8), (3, 5, 40), (2, 63, 1024), (1, 300, 72), (2, 513, 520)])
def test_lengths_and_channels(dev, B, T, C, dt):
    _check(dev, B, T, C, 4, dt, True, True, 7)
    _check(dev, B, T, C, 4, dt, False, False, 8)


@pytest.mark.parametrize("K", [1, 4])
def test_empty_sequences(dev, K):
    """T = 0 carries the state over unchanged and gives zero weight and state gradients."""
    _check(dev, 2, 0, 16, K, torch.float32, True, True, 3)
    x, w, st, dy = _draw(dev, 0, 5, 16, K, torch.bfloat16, 4)
    y, _ = g.short_conv(x, w, st)
    _, dw, _ = g.short_conv_bwd(x, w, dy, st)
    torch.cuda.synchronize()
    assert y.numel() == 0 and torch.count_nonzero(dw) == 0


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16])
def test_streaming_and_in_place_state(dev, dt):
    """Pieces with the state carried (updated in place) equal one call on the whole."""
    B, T, C, K = 2, 90, 48, 4
    x, w, st, _ = _draw(dev, B, T, C, K, dt, 11)
    y_all, s_all = g.short_conv(x, w, st, silu=True)
    state = st.clone()
    parts = []
    for lo, hi in ((0, 1), (1, 3), (3, 40), (40, 41), (41, 90)):
        yp, _ = g.short_conv(x[:, lo:hi].contiguous(), w, state, silu=True, state_out=state)
        parts.append(yp)
    torch.cuda.synchronize()
    assert rel_l2(_np(torch.cat(parts, 1)), _np(y_all)) <= 1e-6
    assert torch.equal(state, s_all)


def test_weight_gradient_is_reproducible(dev):
    x, w, st, dy = _draw(dev, 3, 777, 136, 4, torch.bfloat16, 12)
    a = g.short_conv_bwd(x, w, dy, st, silu=True)[1]
    b = g.short_conv_bwd(x, w, dy, st, silu=True)[1]
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_full_size_sampled_channels(dev):
    """The q/k/v projections of 16 heads of width 128 (C = 6144), 4 x 2048 tokens,
    K = 4, SiLU, bf16: every channel is independent, so the oracle checks a
    sample of channels (tile and wave boundaries included) over all tokens."""
    B, T, C, K = 4, 2048, 6144, 4
    x, w, st, dy = _draw(dev, B, T, C, K, torch.bfloat16, 21)
    y, so = g.short_conv(x, w, st, silu=True)
    dx, dw, ds = g.short_conv_bwd(x, w, dy, st, silu=True)
    torch.cuda.synchronize()
    cols = torch.tensor([0, 1, 3, 4, 255, 256, 1023, 1024, 2047, 3000, 4095, 6000, 6143], device=dev)
    sel = lambda t: t.index_select(-1, cols) if t.dim() == 3 else t.index_select(0, cols)
    ry, rso = short_conv(_np(sel(x)), _np(sel(w)), _np(sel(st)), True)
    rdx, rdw, rds = short_conv_bwd(_np(sel(x)), _np(sel(w)), _np(sel(dy)), _np(sel(st)), True)
    assert rel_l2(_np(sel(y)), ry) <= 2e-2
    assert rel_l2(_np(sel(dx)), rdx) <= 2e-2
    assert rel_l2(_np(sel(ds)), rds) <= 2e-2
    assert rel_l2(_np(sel(dw)), rdw) <= 1e-4
    np.testing.assert_array_equal(_np(sel(so)), rso)


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("K,T", [(4, 70), (4, 2), (3, 0), (8, 5), (2, 129), (5, 300)])
def test_window_gradient(dev, K, T, dt):
    """dstate_out (the gradient of the window after the last token) reaches dx at the
    last K-1 positions and dstate when the sequence is shorter than the window."""
    B, C = 2, 72
    print(f"conv bwd with dstate_out B={B} T={T} C={C} K={K} {dt}", flush=True)
    x, w, st, dy = _draw(dev, B, T, C, K, dt, 40 + K + T)
    gen = torch.Generator(device=dev)
    gen.manual_seed(77 + T)
    dso = torch.randn(B, K - 1, C, generator=gen, device=dev).to(dt)
    dx, dw, ds = g.short_conv_bwd(x, w, dy, st, silu=True, dstate_out=dso)
    torch.cuda.synchronize()
    rdx, rdw, rds = short_conv_bwd(_np(x), _np(w), _np(dy), _np(st), True, dstate_out=_np(dso))
    tol = _tol(dt)
    if T > 0:
        assert rel_l2(_np(dx), rdx) <= tol
        assert rel_l2(_np(dw), rdw) <= 1e-4
    assert rel_l2(_np(ds), rds) <= tol


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16])
def test_backward_over_pieces_equals_whole(dev, dt):
    """A sequence in pieces: forwards with the state carried, then backwards last
    piece first, each piece's dstate handed to the piece before as dstate_out.  The
    pieces' dx, the summed dweight and the first piece's dstate equal one backward
    over the whole sequence."""
    B, T, C, K = 2, 300, 96, 4
    x, w, st, dy = _draw(dev, B, T, C, K, dt, 55)
    dx_all, dw_all, ds_all = g.short_conv_bwd(x, w, dy, st, silu=True)
    cuts = (0, 3, 130, 131, 300)
    states = [st]
    for lo, hi in zip(cuts[:-1], cuts[1:]):
        _, so = g.short_conv(x[:, lo:hi].contiguous(), w, states[-1], silu=True)
        states.append(so)
    dxs, dw_sum, dso = [], torch.zeros_like(dw_all), None
    for i in reversed(range(len(cuts) - 1)):
        lo, hi = cuts[i], cuts[i + 1]
        dxp, dwp, dsp = g.short_conv_bwd(x[:, lo:hi].contiguous(), w, dy[:, lo:hi].contiguous(), states[i],
                                         silu=True, dstate_out=dso)
        dxs.insert(0, dxp)
        dw_sum += dwp
        dso = dsp
    torch.cuda.synchronize()
    tol = 1e-6 if dt == torch.float32 else 2e-2
    assert rel_l2(_np(torch.cat(dxs, 1)), _np(dx_all)) <= tol
    assert rel_l2(_np(dso), _np(ds_all)) <= tol
    assert rel_l2(_np(dw_sum), _np(dw_all)) <= 1e-5
    rdx, rdw, rds = short_conv_bwd(_np(x), _np(w), _np(dy), _np(st), True)
    assert rel_l2(_np(torch.cat(dxs, 1)), rdx) <= _tol(dt)
    assert rel_l2(_np(dso), rds) <= _tol(dt)
