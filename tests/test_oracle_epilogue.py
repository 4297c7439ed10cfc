"""Pins of the epilogue oracle (oracle/epilogue.py) against facts that do
not come from its own formula: closed forms, invariants and limits.  Each
pin is chosen so that a plausible mistake fails it: a dropped or misplaced
normalisation, the mean taken over the wrong axis, eps outside the square
root, a missing weight, or the gate applied without its sigmoid."""
import math

import numpy as np
import pytest

import oracle

NG = oracle.norm_gate


def _rng_case(seed, shape=(5, 3, 16)):
    rng = np.random.default_rng(seed)
    o = rng.standard_normal(shape)
    z = rng.standard_normal(shape)
    w = rng.standard_normal(shape[-1])
    return o, z, w


def test_unit_rms_without_weight_gate_eps(f=NG):
    """w = 1, sigmoid(z) -> 1 (z large), eps = 0: every (token, head) row
    has root-mean-square exactly 1 -- over its own channels only."""
    o, _, _ = _rng_case(1)
    o[:, 1] *= 1e3                      # heads of very different scale
    y = f(o, np.full(o.shape, 60.0), np.ones(o.shape[-1]), 0.0)
    rms = np.sqrt(np.mean(y * y, axis=-1))
    assert np.allclose(rms, 1.0, rtol=1e-12, atol=0)


def test_scale_invariance_and_sign(f=NG):
    o, z, w = _rng_case(2)
    y1 = f(o, z, w, 0.0)
    y2 = f(o * 37.5, z, w, 0.0)
    assert np.allclose(y1, y2, rtol=1e-12, atol=0)
    y3 = f(-o, z, w, 0.0)
    assert np.allclose(y3, -y1, rtol=1e-12, atol=0)


def test_constant_row_closed_form_with_eps(f=NG):
    """o = c on every channel: y = c / sqrt(c^2 + eps) * w * sigmoid(z)."""
    c, eps = 0.01, 1e-4
    o = np.full((2, 2, 8), c)
    z = np.zeros_like(o)                # sigmoid(0) = 1/2
    w = np.arange(1, 9, dtype=np.float64)
    y = f(o, z, w, eps)
    expect = c / math.sqrt(c * c + eps) * w * 0.5
    assert np.allclose(y, np.broadcast_to(expect, y.shape), rtol=1e-14, atol=0)


def test_gate_limits_and_symmetry(f=NG):
    o, z, w = _rng_case(3)
    base = f(o, np.full(o.shape, 60.0), w, 1e-6)
    assert np.allclose(f(o, np.zeros_like(z), w, 1e-6),
                       0.5 * base, rtol=1e-12, atol=0)
    assert np.all(np.abs(f(o, np.full(o.shape, -60.0), w,
                                          1e-6)) < 1e-20 * (1 + np.abs(base)))
    # sigmoid(z) + sigmoid(-z) = 1
    s = f(o, z, w, 1e-6) + f(o, -z, w, 1e-6)
    assert np.allclose(s, base, rtol=1e-12, atol=1e-15)


def test_weight_is_per_channel_and_linear(f=NG):
    o, z, w = _rng_case(4)
    y = f(o, z, w, 1e-6)
    y2 = f(o, z, 2.0 * w, 1e-6)
    assert np.allclose(y2, 2.0 * y, rtol=1e-13, atol=0)
    w1 = np.zeros_like(w)
    w1[3] = 1.0
    y1 = f(o, z, w1, 1e-6)
    assert np.all(y1[..., [c for c in range(w.size) if c != 3]] == 0)


PINS = [test_unit_rms_without_weight_gate_eps, test_scale_invariance_and_sign,
        test_constant_row_closed_form_with_eps, test_gate_limits_and_symmetry,
        test_weight_is_per_channel_and_linear]


def _m_no_norm(o, z, w, eps):
    return np.asarray(o, float) * w / (1 + np.exp(-np.asarray(z, float)))


def _m_wrong_axis(o, z, w, eps):          # mean over heads, not channels
    o = np.asarray(o, float)
    ms = np.mean(o * o, axis=-2, keepdims=True)
    return o / np.sqrt(ms + eps) * w / (1 + np.exp(-np.asarray(z, float)))


def _m_eps_outside(o, z, w, eps):
    o = np.asarray(o, float)
    ms = np.mean(o * o, axis=-1, keepdims=True)
    return o / (np.sqrt(ms) + eps) * w / (1 + np.exp(-np.asarray(z, float)))


def _m_no_weight(o, z, w, eps):
    o = np.asarray(o, float)
    ms = np.mean(o * o, axis=-1, keepdims=True)
    return o / np.sqrt(ms + eps) / (1 + np.exp(-np.asarray(z, float)))


def _m_gate_raw(o, z, w, eps):            # z used without its sigmoid
    o = np.asarray(o, float)
    ms = np.mean(o * o, axis=-1, keepdims=True)
    return o / np.sqrt(ms + eps) * w * np.asarray(z, float)


@pytest.mark.parametrize("mutant", [_m_no_norm, _m_wrong_axis, _m_eps_outside,
                                    _m_no_weight, _m_gate_raw])
def test_pins_catch_planted_mistakes(mutant):
    caught = 0
    for pin in PINS:
        try:
            pin(mutant)
        except AssertionError:
            caught += 1
    assert caught >= 1, mutant.__name__
