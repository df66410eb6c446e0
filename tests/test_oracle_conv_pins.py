"""Pins of the short-convolution oracle (oracle/conv.py) against facts it does
not compute itself: library FIR filters, closed forms, finite differences,
state-carry identities and the index rules the goldens page states.

Planted mistakes in it (bottom of this file) must each fail one of them.
"""
import numpy as np
import pytest
from scipy.signal import lfilter
from scipy.special import expit

from oracle import conv as CV


def rand_conv(rng, lens, C=6, W=4, state=True, bias=True):
    T = sum(lens)
    x = rng.standard_normal((T, C))
    w = rng.standard_normal((C, W)) * 0.5
    b = rng.standard_normal(C) * 0.1 if bias else None
    cu = np.concatenate([[0], np.cumsum(lens)])
    s0 = rng.standard_normal((len(lens), C, W - 1)) if state else None
    return x, w, b, cu, s0


def rel(a, b):
    return np.abs(a - b).max() / max(np.abs(b).max(), 1e-300)


def test_forward_is_a_per_channel_fir_filter():
    """numpy's convolve and scipy's lfilter, each with the taps in filter order."""
    rng = np.random.default_rng(1)
    x, w, b, cu, s0 = rand_conv(rng, [9, 1, 30])
    y, _ = CV.conv_forward(x, w, b, cu, s0, activation=None)
    ys, _ = CV.conv_forward(x, w, b, cu, s0, activation="silu")
    for n in range(3):
        xe = np.concatenate([s0[n].T, x[cu[n]:cu[n + 1]]])
        for c in range(x.shape[1]):
            ref = np.convolve(xe[:, c], w[c, ::-1], mode="valid") + b[c]
            assert rel(y[cu[n]:cu[n + 1], c], ref) < 1e-13
            pre = lfilter(w[c, ::-1], [1.0], xe[:, c])[3:] + b[c]
            assert rel(ys[cu[n]:cu[n + 1], c], pre * expit(pre)) < 1e-13


def test_identity_taps_pass_the_input_and_keep_the_last_inputs():
    rng = np.random.default_rng(2)
    x, _, _, cu, s0 = rand_conv(rng, [5, 2, 7], bias=False)
    w = np.zeros((6, 4))
    w[:, 3] = 1.0
    y, st = CV.conv_forward(x, w, None, cu, s0, activation=None)
    assert np.array_equal(y, x)
    assert np.array_equal(st[0], x[2:5].T)
    assert np.array_equal(st[1][:, 0], s0[1][:, 2]) and np.array_equal(st[1][:, 1:], x[5:7].T)


def test_one_call_equals_two_calls_with_the_state_carried():
    rng = np.random.default_rng(3)
    x, w, b, _, s0 = rand_conv(rng, [40])
    y, st = CV.conv_forward(x, w, b, [0, 40], s0)
    for p in (1, 2, 3, 17):
        ya, sa = CV.conv_forward(x[:p], w, b, [0, p], s0)
        yb, sb = CV.conv_forward(x[p:], w, b, [0, 40 - p], sa)
        assert rel(np.concatenate([ya, yb]), y) < 1e-14 and np.array_equal(sb, st)


def test_silu_and_its_derivative_closed_forms():
    x = np.array([-1000.0, -88.8, -20.0, 0.0, 1.5, 40.0])
    assert np.all(np.isfinite(CV.act_grad(x, "silu")))
    assert CV.act_forward(np.array([0.0]), "silu")[0] == 0.0
    assert CV.act_grad(np.array([0.0]), "silu")[0] == 0.5
    h = 1e-6
    for v in (-3.0, -0.4, 0.7, 5.0):
        fd = (CV.act_forward(np.array([v + h]), "silu") - CV.act_forward(np.array([v - h]), "silu")) / (2 * h)
        assert abs(fd[0] - CV.act_grad(np.array([v]), "silu")[0]) < 1e-8


@pytest.mark.parametrize("activation", ["silu", None])
def test_backward_matches_central_finite_differences(activation):
    rng = np.random.default_rng(4)
    x, w, b, cu, s0 = rand_conv(rng, [5, 2, 4], C=3)
    dy = rng.standard_normal(x.shape)
    dx, dw, db, ds = CV.conv_backward(x, w, b, cu, dy, s0, activation)

    def loss(x_, w_, b_, s_):
        y, _ = CV.conv_forward(x_, w_, b_, cu, s_, activation)
        return float((y * dy).sum())

    h = 1e-6
    for arr, grad, args in ((x, dx, 0), (w, dw, 1), (b, db, 2), (s0, ds, 3)):
        flat = arr.reshape(-1)
        for j in range(0, flat.size, max(1, flat.size // 12)):
            plus = [x.copy(), w.copy(), b.copy(), s0.copy()]
            minus = [x.copy(), w.copy(), b.copy(), s0.copy()]
            plus[args].reshape(-1)[j] += h
            minus[args].reshape(-1)[j] -= h
            fd = (loss(*plus) - loss(*minus)) / (2 * h)
            assert abs(fd - grad.reshape(-1)[j]) < 1e-6 * max(1.0, abs(fd)), (args, j)


def test_update_steps_equal_the_forward():
    rng = np.random.default_rng(5)
    x, w, b, _, s0 = rand_conv(rng, [8])
    y, st = CV.conv_forward(x, w, b, [0, 8], s0)
    pool = np.zeros((4, 6, 3))
    pool[2] = s0[0]
    for t in range(8):
        yt, pool = CV.conv_update(x[t:t + 1], w, b, pool, [2])
        assert rel(yt[0], y[t]) < 1e-14
    assert np.array_equal(pool[2], st[0])


def test_update_index_rules():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((3, 6))
    w = rng.standard_normal((6, 4))
    pool = rng.standard_normal((5, 6, 3))
    y, new = CV.conv_update(x, w, None, pool, [0, 3, 0])
    assert np.array_equal(y[0], np.zeros(6)) and np.array_equal(y[2], np.zeros(6))
    keep = [0, 1, 2, 4]
    assert np.array_equal(new[keep], pool[keep])
    for bad in ([1, -1, 2], [1, 5, 2], [2, 2, 0]):
        with pytest.raises(ValueError):
            CV.conv_update(x, w, None, pool, bad)


def test_paged_prefix_then_continuation_equals_one_pass():
    rng = np.random.default_rng(7)
    lens = [30, 2, 1, 45]
    x, w, b, cu, _ = rand_conv(rng, lens, state=False)
    y, st = CV.conv_forward(x, w, b, cu)
    pool = rng.standard_normal((9, 6, 3))
    idx = np.array([4, 1, 7, 2])
    cut = [10, 1, 0, 44]
    first = np.concatenate([np.arange(cu[n], cu[n] + cut[n]) for n in range(4)])
    second = np.concatenate([np.arange(cu[n] + cut[n], cu[n + 1]) for n in range(4)])
    cu1 = np.concatenate([[0], np.cumsum(cut)])
    cu2 = np.concatenate([[0], np.cumsum([L - c for L, c in zip(lens, cut)])])
    y1, p1 = CV.conv_forward_paged(x[first], w, b, cu1, pool, idx, np.zeros(4))
    y2, p2 = CV.conv_forward_paged(x[second], w, b, cu2, p1, idx, np.ones(4))
    assert rel(y1, y[first]) < 1e-14 and rel(y2, y[second]) < 1e-14
    assert np.array_equal(p2[idx], st)
    others = [s for s in range(9) if s not in idx]
    assert np.array_equal(p2[others], pool[others])
    # the null block: zero start, nothing written
    y0, p0 = CV.conv_forward_paged(x, w, b, cu, pool, [0, 1, 7, 2])
    y_alone, _ = CV.conv_forward(x[:30], w, b, [0, 30])
    assert np.array_equal(y0[:30], y_alone) and np.array_equal(p0[4], pool[4])


# ---------------------------------------------------------------- planted mistakes
_fwd, _grad, _ext = CV.conv_forward, CV.act_grad, CV._extended


def _flipped_taps(x, weight, bias, cu, state_in=None, activation="silu"):
    return _fwd(x, np.asarray(weight)[:, ::-1], bias, cu, state_in, activation)


def _dropped_bias(x, weight, bias, cu, state_in=None, activation="silu"):
    return _fwd(x, weight, None, cu, state_in, activation)


def _sigmoid_as_silu_grad(pre, activation):
    return CV.sigmoid(pre) if activation == "silu" else np.ones_like(pre)


def _history_reversed(x, cu, n, state_in, W):
    xe = _ext(x, cu, n, state_in, W)
    xe[:W - 1] = xe[:W - 1][::-1].copy()
    return xe


MUTATIONS = {
    "taps in reverse order": ("conv_forward", _flipped_taps),
    "bias dropped": ("conv_forward", _dropped_bias),
    "SiLU derivative taken as the sigmoid": ("act_grad", _sigmoid_as_silu_grad),
    "carried inputs in reverse order": ("_extended", _history_reversed),
}

PINS = [
    test_forward_is_a_per_channel_fir_filter,
    test_identity_taps_pass_the_input_and_keep_the_last_inputs,
    test_one_call_equals_two_calls_with_the_state_carried,
    lambda: test_backward_matches_central_finite_differences("silu"),
    test_update_steps_equal_the_forward,
]


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_a_planted_conv_mistake_fails_a_pin(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(CV, attr, fn)
    failed = 0
    for pin in PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            failed += 1
    assert failed >= 1, f"no pin caught: {name}"
