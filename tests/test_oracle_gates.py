"""Pins of the oracle's gate sigmoids and of its fixed-length batch front end,
against facts that do not come from their own code.

Gates ("Kimi K3: The Manos, The Mythos, The Legendos", section "Kimi
Linear": the decay gate, beta and the output gate come from projections;
"Two Paths: Kimi K3 vs DeepSeek V4 Architecture Divergence", section
"Hardware Adaptation": log-decay bounded below by -5).  The readings are
g = -5 sigmoid(a), beta = sigmoid(b) and an output gate sigmoid(z), with the
logistic function sigmoid(x) = 1 / (1 + e^-x).  What fixes it independently:
  * closed forms at x = +-ln 3: e^-ln3 = 1/3, so sigmoid(ln 3) = 3/4 and
    sigmoid(-ln 3) = 1/4 exactly (g = -3.75 / -1.25, beta = 3/4 / 1/4);
  * the half-angle identity sigmoid(x) = (1 + tanh(x / 2)) / 2, evaluated
    with numpy's tanh, a routine that shares nothing with exp;
  * direction: a larger pre-activation a gives a larger sigmoid, hence a
    more negative g (faster forgetting), and g -> -5 as a -> +inf.
A base-2 logistic 1 / (1 + 2^-x), a rescaled slope sigmoid(2x), or a gate
of the wrong sign each fail at least one of these (checked below).

Fixed-length batches: ``oracle.run_fixed`` packs [B, T] into B sequences of
T tokens.  Pinned by running each batch row alone through the packed entry
(which the brute-force pins fix) at B = 2 and 3 with T != B, so a swapped
batch/time reshape or wrong sequence bounds fail.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import prologue as P

LN3 = math.log(3.0)


# ---------------------------------------------------------------- prologue
def _gate_inputs(a_vals, b_vals, D=8, H=2):
    T = len(a_vals)
    rng = np.random.default_rng(11)
    xq, xk, xv = (rng.standard_normal((T, H, D)) for _ in range(3))
    w = rng.standard_normal((3, H, D, P.CONV_TAPS))
    a = np.broadcast_to(np.asarray(a_vals, np.float64)[:, None, None],
                        (T, H, D)).copy()
    b = np.broadcast_to(np.asarray(b_vals, np.float64)[:, None],
                        (T, H)).copy()
    return xq, xk, xv, w, a, b, [0, T]


def pin_prologue_gates_closed_form(prologue=P.prologue):
    args = _gate_inputs([LN3, -LN3, 0.0], [LN3, -LN3, 0.0])
    _, _, _, g, beta = prologue(*args)
    assert np.allclose(g[0], -3.75, rtol=1e-15, atol=0), g[0, 0, 0]
    assert np.allclose(g[1], -1.25, rtol=1e-15, atol=0), g[1, 0, 0]
    assert np.all(g[2] == -2.5)
    assert np.allclose(beta[0], 0.75, rtol=1e-15, atol=0), beta[0, 0]
    assert np.allclose(beta[1], 0.25, rtol=1e-15, atol=0), beta[1, 0]
    assert np.all(beta[2] == 0.5)
    return True


def pin_prologue_gates_half_angle(prologue=P.prologue):
    x = np.linspace(-12.0, 12.0, 97)
    _, _, _, g, beta = prologue(*_gate_inputs(x, x))
    ref = 0.5 * (1.0 + np.tanh(0.5 * x))
    # 1 + tanh(x / 2) cancels for x << 0: relative accuracy ~1e-11 there
    assert np.allclose(g[:, 0, 0], -5.0 * ref, rtol=1e-10, atol=0)
    assert np.allclose(beta[:, 0], ref, rtol=1e-10, atol=0)
    return True


def pin_prologue_gate_direction(prologue=P.prologue):
    x = np.array([-40.0, -3.0, -0.5, 0.0, 0.5, 3.0, 40.0])
    _, _, _, g, beta = prologue(*_gate_inputs(x, x))
    g0 = g[:, 0, 0]
    assert np.all(np.diff(g0) < 0), g0            # strictly decreasing
    assert abs(g0[-1] + 5.0) < 1e-15 and abs(g0[0]) < 1e-15
    assert np.all(np.diff(beta[:, 0]) > 0)
    return True


PROLOGUE_PINS = [pin_prologue_gates_closed_form, pin_prologue_gates_half_angle,
                 pin_prologue_gate_direction]


@pytest.mark.parametrize("pin", PROLOGUE_PINS,
                         ids=[p.__name__ for p in PROLOGUE_PINS])
def test_prologue_gate_pins(pin):
    assert pin()


def _prologue_with(sig):
    """The prologue with its logistic function replaced by ``sig``."""
    def f(xq, xk, xv, conv_w, a, b, cu):
        q = P.l2norm(P.short_conv(xq, conv_w[0], cu))
        k = P.l2norm(P.short_conv(xk, conv_w[1], cu))
        v = P.short_conv(xv, conv_w[2], cu)
        return q, k, v, P.G_MIN * sig(a), sig(b)
    return f


_SIG_MUTANTS = {
    "base2": lambda x: 1.0 / (1.0 + np.power(2.0, -np.asarray(x, float))),
    "slope2": lambda x: 1.0 / (1.0 + np.exp(-2.0 * np.asarray(x, float))),
    "reversed": lambda x: 1.0 / (1.0 + np.exp(np.asarray(x, float))),
}


def test_unmutated_prologue_copy_passes():
    f = _prologue_with(P.sigmoid)
    for pin in PROLOGUE_PINS:
        assert pin(f)


@pytest.mark.parametrize("name", sorted(_SIG_MUTANTS))
def test_prologue_pins_catch_planted_gate_mistakes(name):
    f = _prologue_with(_SIG_MUTANTS[name])
    caught = 0
    for pin in PROLOGUE_PINS:
        try:
            pin(f)
        except AssertionError:
            caught += 1
    assert caught >= 1, name


# ---------------------------------------------------------------- epilogue
def pin_epilogue_gate(norm_gate=oracle.norm_gate):
    """o constant c on a row, eps = 0, w = 1: y = sign(c) sigmoid(z)."""
    o = np.full((4, 2, 16), -0.37)
    z = np.zeros_like(o)
    z[0], z[1], z[3] = LN3, -LN3, 0.0
    z[2] = np.linspace(-9.0, 9.0, 16)
    y = norm_gate(o, z, np.ones(16), 0.0)
    assert np.allclose(y[0], -0.75, rtol=1e-15, atol=0), y[0, 0, 0]
    assert np.allclose(y[1], -0.25, rtol=1e-15, atol=0), y[1, 0, 0]
    assert np.allclose(y[3], -0.5, rtol=1e-15, atol=0)
    ref = 0.5 * (1.0 + np.tanh(0.5 * z[2]))
    assert np.allclose(y[2], -ref, rtol=1e-10, atol=0)
    return True


def test_epilogue_gate_pin():
    assert pin_epilogue_gate()


def _norm_gate_with(sig):
    def f(o, z, w, eps):
        o = np.asarray(o, np.float64)
        ms = np.mean(o * o, axis=-1, keepdims=True)
        return o / np.sqrt(ms + float(eps)) * np.asarray(w, float) * sig(z)
    return f


def test_unmutated_epilogue_copy_passes():
    assert pin_epilogue_gate(
        _norm_gate_with(lambda x: 1.0 / (1.0 + np.exp(-np.asarray(x, float)))))


@pytest.mark.parametrize("name", sorted(_SIG_MUTANTS))
def test_epilogue_pin_catches_planted_gate_mistakes(name):
    with pytest.raises(AssertionError):
        pin_epilogue_gate(_norm_gate_with(_SIG_MUTANTS[name]))


# ---------------------------------------------------------------- run_fixed
def pin_run_fixed_batches(run_fixed=oracle.run_fixed):
    """Each row of a [B, T] batch equals that sequence run alone."""
    for B, T, seed in ((2, 5, 0), (3, 4, 1)):
        rng = np.random.default_rng(100 + seed)
        H, K, V = 2, 3, 4
        q = rng.standard_normal((B, T, H, K))
        k = rng.standard_normal((B, T, H, K))
        v = rng.standard_normal((B, T, H, V))
        g = -rng.random((B, T, H, K))
        beta = rng.random((B, T, H))
        s0 = rng.standard_normal((B, H, K, V))
        o, s = run_fixed(q, k, v, g, beta, s0, 0.5)
        assert o.shape == (B, T, H, V) and s.shape == (B, H, K, V)
        for b in range(B):
            o1, s1 = oracle.run_varlen(q[b], k[b], v[b], g[b], beta[b],
                                       [0, T], s0[b:b + 1], 0.5)
            assert np.allclose(o[b], o1, rtol=1e-14, atol=1e-14), b
            assert np.allclose(s[b], s1[0], rtol=1e-14, atol=1e-14), b
    return True


def test_run_fixed_pin(oracle_mod):
    assert pin_run_fixed_batches()


def _fixed_swapped(q, k, v, g, beta, s0=None, scale=1.0):
    """Planted mistake: [B, T] packed time-major (axes swapped)."""
    B, T, H, K = np.shape(q)
    V = np.shape(v)[3]
    sw = lambda x: np.swapaxes(np.asarray(x), 0, 1)  # noqa: E731
    cu = np.arange(B + 1, dtype=np.int64) * T
    o, s = oracle.run_varlen(sw(q).reshape(B * T, H, K),
                             sw(k).reshape(B * T, H, K),
                             sw(v).reshape(B * T, H, V),
                             sw(g).reshape(B * T, H, K),
                             sw(beta).reshape(B * T, H), cu, s0, scale)
    return o.reshape(B, T, H, V), s


def _fixed_wrong_bounds(q, k, v, g, beta, s0=None, scale=1.0):
    """Planted mistake: sequence bounds built from B instead of T."""
    B, T, H, K = np.shape(q)
    V = np.shape(v)[3]
    cu = np.minimum(np.arange(B + 1, dtype=np.int64) * B, B * T)
    cu[-1] = B * T
    o, s = oracle.run_varlen(np.reshape(q, (B * T, H, K)),
                             np.reshape(k, (B * T, H, K)),
                             np.reshape(v, (B * T, H, V)),
                             np.reshape(g, (B * T, H, K)),
                             np.reshape(beta, (B * T, H)), cu, s0, scale)
    return o.reshape(B, T, H, V), s


@pytest.mark.parametrize("mutant", [_fixed_swapped, _fixed_wrong_bounds],
                         ids=["swapped_axes", "wrong_bounds"])
def test_run_fixed_pin_catches_planted_mistakes(oracle_mod, mutant):
    with pytest.raises(AssertionError):
        pin_run_fixed_batches(mutant)
