"""Pins of the oracle's short convolution and its gradient (CPU only).

burn-gdn2 README (docs.rs), "Architecture" diagram: the projections pass
through a "ShortConv" before the L2 norm; "Configuration": use_short_conv =
true, "Depthwise conv before recurrence".  The width and the activation are
not on the page.  Reading: a causal depthwise convolution over tokens with K
taps per channel, z[t] = sum_i weight[:, i] x[t - (K-1) + i], y = z or
z * sigmoid(z), earlier positions read from a carried state of the last K-1
inputs.  The pins fix it by special filters, numpy's own convolution, streaming
in pieces, closed forms and central finite differences; planted slips show that
each kind of mistake is caught.
"""
import math

import numpy as np
import pytest

from oracle.reference import short_conv, short_conv_bwd, sigmoid


def _rand(seed, B=2, T=9, C=5, K=4):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, T, C)), rng.standard_normal((C, K)),
            rng.standard_normal((B, K - 1, C)), rng.standard_normal((B, T, C)))


def check_identity_filter(f=short_conv):
    """Only the newest tap set: y = x, whatever the state."""
    x, _, st, _ = _rand(0)
    w = np.zeros((5, 4))
    w[:, 3] = 1.0
    y, _ = f(x, w, st)
    np.testing.assert_allclose(y, x, rtol=0, atol=0)


def check_delay_filter(f=short_conv):
    """Only the oldest tap set: y[t] = x[t - 3], the first three from the state."""
    x, _, st, _ = _rand(1)
    w = np.zeros((5, 4))
    w[:, 0] = 1.0
    y, _ = f(x, w, st)
    np.testing.assert_allclose(y[:, 3:], x[:, :-3], rtol=0, atol=0)
    np.testing.assert_allclose(y[:, :3], st, rtol=0, atol=0)


def check_numpy_convolve(f=short_conv):
    """Each channel equals numpy's 'valid' convolution of [state, x] with the reversed taps."""
    x, w, st, _ = _rand(2)
    y, _ = f(x, w, st)
    for b in range(x.shape[0]):
        for c in range(x.shape[2]):
            xe = np.concatenate([st[b, :, c], x[b, :, c]])
            np.testing.assert_allclose(y[b, :, c], np.convolve(xe, w[c, ::-1], mode="valid"), rtol=1e-13, atol=1e-13)


def check_streaming(f=short_conv):
    """Two pieces with the returned state carried = one call, outputs and final state (pieces
    shorter than the window included)."""
    x, w, st, _ = _rand(3, T=11)
    y, s_end = f(x, w, st, silu=True)
    for cut in (1, 2, 5, 10):
        y1, s1 = f(x[:, :cut], w, st, silu=True)
        y2, s2 = f(x[:, cut:], w, s1, silu=True)
        np.testing.assert_allclose(np.concatenate([y1, y2], axis=1), y, rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(s2, s_end, rtol=0, atol=0)
    np.testing.assert_allclose(s_end, x[:, -3:], rtol=0, atol=0)


def check_zero_state(f=short_conv):
    """No state = a zero state."""
    x, w, _, _ = _rand(4)
    y0, _ = f(x, w, None)
    y1, _ = f(x, w, np.zeros((2, 3, 5)))
    np.testing.assert_allclose(y0, y1, rtol=0, atol=0)


def check_silu_closed_form(f=short_conv):
    """Constant input c with a constant state: z = c * sum of taps; with the SiLU
    option, z = ln 3 gives y = 0.75 ln 3."""
    c = math.log(3.0)
    w = np.full((3, 4), 0.25)
    x = np.full((1, 6, 3), c)
    st = np.full((1, 3, 3), c)
    y, _ = f(x, w, st, silu=True)
    np.testing.assert_allclose(y, 0.75 * math.log(3.0), rtol=1e-14, atol=0)
    y, _ = f(x, 2.0 * w, st, silu=False)
    np.testing.assert_allclose(y, 2.0 * c, rtol=1e-14, atol=0)


PINS = [check_identity_filter, check_delay_filter, check_numpy_convolve, check_streaming, check_zero_state,
        check_silu_closed_form]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_short_conv_pins(pin):
    pin()


@pytest.mark.parametrize("silu", [False, True])
@pytest.mark.parametrize("K", [1, 2, 4])
def test_short_conv_bwd_finite_differences(silu, K):
    """dx, dweight and dstate against central differences of sum(dy * y) for every element."""
    x, w, st, dy = _rand(5, B=2, T=6, C=3, K=K)
    dx, dw, dst = short_conv_bwd(x, w, dy, st, silu)
    loss = lambda x_, w_, s_: float(np.sum(dy * short_conv(x_, w_, s_, silu)[0]))
    h = 1e-6
    for arr, grad in ((x, dx), (w, dw), (st, dst)):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            old = arr[idx]
            arr[idx] = old + h
            lp = loss(x, w, st)
            arr[idx] = old - h
            lm = loss(x, w, st)
            arr[idx] = old
            num[idx] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(grad, num, rtol=1e-6, atol=1e-7)


@pytest.mark.parametrize("silu", [False, True])
@pytest.mark.parametrize("K,T", [(4, 6), (4, 2), (3, 0), (2, 1)])
def test_short_conv_bwd_state_out_finite_differences(silu, K, T):
    """With a gradient on the window after the last token: dx, dweight and dstate
    against central differences of sum(dy * y) + sum(dso * state_out), also for
    sequences shorter than the window (state_out then holds state inputs)."""
    x, w, st, _ = _rand(11 + K + T, B=2, T=T, C=3, K=K)
    rng = np.random.default_rng(100 + K + T)
    dy = rng.standard_normal((2, T, 3))
    dso = rng.standard_normal((2, K - 1, 3))
    dx, dw, dst = short_conv_bwd(x, w, dy, st, silu, dstate_out=dso)

    def loss(x_, w_, s_):
        y, so = short_conv(x_, w_, s_, silu)
        return float(np.sum(dy * y) + np.sum(dso * so))

    h = 1e-6
    for arr, grad in ((x, dx), (w, dw), (st, dst)):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            old = arr[idx]
            arr[idx] = old + h
            lp = loss(x, w, st)
            arr[idx] = old - h
            lm = loss(x, w, st)
            arr[idx] = old
            num[idx] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(grad, num, rtol=1e-6, atol=1e-7)


def check_bwd_pieces(f=short_conv_bwd):
    """The backward over a sequence split in two pieces, the second piece's dstate
    handed to the first as dstate_out, equals the backward over the whole (dweight:
    the sum of the pieces')."""
    x, w, st, dy = _rand(21, B=2, T=11, C=4, K=4)
    for silu in (False, True):
        dx, dw, dst = f(x, w, dy, st, silu)
        T1 = 5
        _, st1 = short_conv(x[:, :T1], w, st, silu)
        dx2, dw2, dst2 = f(x[:, T1:], w, dy[:, T1:], st1, silu)
        dx1, dw1, dst1 = f(x[:, :T1], w, dy[:, :T1], st, silu, dstate_out=dst2)
        np.testing.assert_allclose(np.concatenate([dx1, dx2], axis=1), dx, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(dw1 + dw2, dw, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(dst1, dst, rtol=1e-12, atol=1e-12)


def test_short_conv_bwd_pieces():
    check_bwd_pieces()


def _bslip_state_out_ignored(x, weight, dy, state=None, silu=False, dstate_out=None):
    return short_conv_bwd(x, weight, dy, state, silu)


def _bslip_state_out_shifted(x, weight, dy, state=None, silu=False, dstate_out=None):
    if dstate_out is None:
        return short_conv_bwd(x, weight, dy, state, silu)
    d = np.concatenate([np.asarray(dstate_out)[:, 1:], np.zeros_like(np.asarray(dstate_out)[:, :1])], axis=1)
    return short_conv_bwd(x, weight, dy, state, silu, dstate_out=d)


@pytest.mark.parametrize("slip", [_bslip_state_out_ignored, _bslip_state_out_shifted], ids=lambda f: f.__name__)
def test_short_conv_bwd_slips_rejected(slip):
    with pytest.raises(AssertionError):
        check_bwd_pieces(slip)


# ---- planted slips: each must fail at least one pin --------------------------------------
def _slip_reversed(x, weight, state=None, silu=False):
    return short_conv(x, np.asarray(weight)[:, ::-1], state, silu)


def _slip_no_state(x, weight, state=None, silu=False):
    return short_conv(x, weight, None, silu)


def _slip_off_by_one(x, weight, state=None, silu=False):
    y, s = short_conv(x, weight, state, silu)
    return np.concatenate([y[:, :1], y[:, :-1]], axis=1), s


def _slip_silu_on_input(x, weight, state=None, silu=False):
    x = np.asarray(x, dtype=np.float64)
    if silu:
        x = x * sigmoid(x)
        state = None if state is None else np.asarray(state) * sigmoid(np.asarray(state))
    return short_conv(x, weight, state, False)


def _slip_state_not_carried(x, weight, state=None, silu=False):
    y, s = short_conv(x, weight, state, silu)
    return y, np.zeros_like(s)


@pytest.mark.parametrize("slip", [_slip_reversed, _slip_no_state, _slip_off_by_one, _slip_silu_on_input,
                                  _slip_state_not_carried], ids=lambda f: f.__name__)
def test_short_conv_slips_rejected(slip):
    failed = 0
    for pin in PINS:
        try:
            pin(slip)
        except AssertionError:
            failed += 1
    assert failed >= 1
