"""Pins of the prologue oracle (oracle/prologue.py) against facts that do
not come from its own code: a one-tap convolution is the identity, a
shifted delta kernel is a delay with zeros at each sequence start,
causality, convolution linearity against numpy's own convolution, unit norms
of q and k, and the gates' ranges and fixed points.  Each is chosen so that
a plausible mistake fails it (taps reversed, padding leaking across
sequences, normalising over the wrong axis, a wrong gate bound)."""
import numpy as np
import pytest

from oracle import prologue as P


def _x(seed, T=23, H=2, D=8):
    return np.random.default_rng(seed).standard_normal((T, H, D))


def test_current_tap_is_identity(f=P.short_conv):
    x = _x(1)
    w = np.zeros((2, 8, P.CONV_TAPS))
    w[:, :, -1] = 1.0                       # the current token's tap
    assert np.array_equal(f(x, w, [0, 23]), x)


def test_delta_tap_delays_with_zero_padding_per_sequence(f=P.short_conv):
    x = _x(2)
    w = np.zeros((2, 8, P.CONV_TAPS))
    w[:, :, 0] = 1.0                        # 3 tokens back
    cu = [0, 10, 10, 23]                    # includes an empty sequence
    y = f(x, w, cu)
    for a, b in ((0, 10), (10, 23)):
        assert np.all(y[a:a + 3] == 0)      # left padding of each sequence
        assert np.array_equal(y[a + 3:b], x[a:b - 3])


def test_causal(f=P.short_conv):
    x = _x(3)
    w = np.random.default_rng(4).standard_normal((2, 8, P.CONV_TAPS))
    y1 = f(x, w, [0, 23])
    x2 = x.copy()
    x2[15:] += 5.0                          # change the future only
    y2 = f(x2, w, [0, 23])
    assert np.array_equal(y1[:15], y2[:15])
    assert not np.allclose(y1[15:], y2[15:])


def test_matches_numpy_convolution(f=P.short_conv):
    """Per channel, the causal convolution is numpy's full convolution with
    the taps reversed, truncated to the sequence length."""
    x = _x(5, T=17)
    w = np.random.default_rng(6).standard_normal((2, 8, P.CONV_TAPS))
    y = f(x, w, [0, 17])
    for h in range(2):
        for c in range(8):
            ref = np.convolve(x[:, h, c], w[h, c, ::-1])[:17]
            assert np.allclose(y[:, h, c], ref, rtol=1e-13, atol=1e-13)


def test_q_k_unit_norm_and_gate_ranges():
    rng = np.random.default_rng(7)
    T, H, D = 19, 3, 16
    xq, xk, xv = (rng.standard_normal((T, H, D)) for _ in range(3))
    w = rng.standard_normal((3, H, D, P.CONV_TAPS))
    a = rng.standard_normal((T, H, D)) * 10
    b = rng.standard_normal((T, H)) * 10
    q, k, v, g, beta = P.prologue(xq, xk, xv, w, a, b, [0, 7, T])
    assert np.allclose(np.linalg.norm(q, axis=-1), 1.0, rtol=1e-13)
    assert np.allclose(np.linalg.norm(k, axis=-1), 1.0, rtol=1e-13)
    assert np.all((g > P.G_MIN) & (g < 0))
    assert np.all((beta > 0) & (beta < 1))
    # fixed points: a = 0 gives g = -5/2, b = 0 gives beta = 1/2
    _, _, _, g0, b0 = P.prologue(xq, xk, xv, w, np.zeros_like(a),
                                 np.zeros_like(b), [0, T])
    assert np.all(g0 == -2.5) and np.all(b0 == 0.5)
    # v is the plain convolution (no normalisation)
    assert np.array_equal(v, P.short_conv(xv, w[2], [0, 7, T]))


def _m_taps_reversed(x, w, cu):
    return P.short_conv(x, np.asarray(w)[..., ::-1], cu)


def _m_no_sequence_restart(x, w, cu):
    return P.short_conv(x, w, [cu[0], cu[-1]])


@pytest.mark.parametrize("mutant", [_m_taps_reversed, _m_no_sequence_restart])
def test_pins_catch_planted_mistakes(mutant):
    caught = 0
    for pin in (test_current_tap_is_identity,
                test_delta_tap_delays_with_zero_padding_per_sequence,
                test_causal, test_matches_numpy_convolution):
        try:
            pin(mutant)
        except AssertionError:
            caught += 1
    assert caught >= 1, mutant.__name__
