"""Checks that pin the fp64 oracle to things other than itself.

Each ``pin_*`` function runs the oracle (the default build, or a variant
passed as ``lib``) on small inputs and raises AssertionError when the result
disagrees with what the pages and the mathematics fix.  ``test_oracle_pins``
runs them on the real oracle; ``test_oracle_mutations`` runs them on copies of
the oracle with planted mistakes and requires every mistake to be caught.

Sources (page titles and sections):
  [K3vsDSV4/Attention] "Two Paths: Kimi K3 vs DeepSeek V4 Architecture
      Divergence", section "Attention: 69 Layers of Compressed Memory + 24
      Layers of Original Archives": forget -> correct -> write on a fixed-size
      state; 96 x 128^2 x 2 bytes per layer.
  [K3vsDSV4/HW] same page, section "Hardware Adaptation": g_min = -5.
  [SA/KDA] "Kimi K3: The Manos, The Mythos, The Legendos", section "Kimi Delta
      Attention": DeltaNet minimises an L2 retrieval loss (the delta rule);
      Gated DeltaNet adds a scalar forget gate; KDA makes it diagonal.
  [SA/FlashKDA] same page, section "FlashKDA algorithm": D_t = Diag(alpha_t),
      u_t the delta; chunked unrolling with cumulative decay; UT transform.
  [SA/Append] same page, section "Append-Prefill": continue from cached state.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

import brute_force
import chunk_ref
import oracle


def _rel(x, ref):
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    den = max(float(np.max(np.abs(ref))) if ref.size else 0.0, 1e-300)
    return float(np.max(np.abs(x - ref))) / den if ref.size else 0.0


def _rand_problem(rng, T, H, K, V, g_scale=1.0, s0=True, unit_k=False):
    q = rng.standard_normal((T, H, K))
    k = rng.standard_normal((T, H, K))
    if unit_k:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, V))
    g = -g_scale * rng.random((T, H, K))
    beta = rng.random((T, H))
    S0 = rng.standard_normal((1, H, K, V)) * 0.5 if s0 else None
    return q, k, v, g, beta, S0


# --------------------------------------------------------------------------
# P1: exact brute force (transition-matrix product form, rationals)
# --------------------------------------------------------------------------
def pin_brute_force(lib=None, seed=0):
    """Oracle vs exact rational arithmetic on packed sequences (one empty),
    with a non-unit query scale.  [SA/KDA], [SA/FlashKDA]"""
    rng = np.random.default_rng(seed)
    lengths = [3, 0, 4]
    H, K, V = 2, 3, 2
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    Tt = int(cu[-1])

    def dy(shape, den=8, lo=-8, hi=8):     # dyadic rationals, exact in fp64
        return rng.integers(lo, hi + 1, size=shape) / den

    q, k, v = dy((Tt, H, K)), dy((Tt, H, K)), dy((Tt, H, V))
    g = -rng.random((Tt, H, K)) * 2.0
    beta = rng.integers(1, 9, size=(Tt, H)) / 8
    S0 = dy((len(lengths), H, K, V), den=4)
    scale = 0.75
    o, S = oracle.run_varlen(q, k, v, g, beta, cu, S0, scale=scale, lib=lib)

    F = Fraction
    for n in range(len(lengths)):
        for h in range(H):
            ts = range(cu[n], cu[n + 1])
            outs, fin = brute_force.run_sequence(
                [[F(x) for x in q[t, h]] for t in ts],
                [[F(x) for x in k[t, h]] for t in ts],
                [[F(x) for x in v[t, h]] for t in ts],
                [[F(math.exp(x)) for x in g[t, h]] for t in ts],
                [F(beta[t, h]) for t in ts],
                [[F(x) for x in row] for row in S0[n, h]], scale=F(scale))
            ref_o = np.array([[float(x) for x in r] for r in outs]).reshape(
                len(ts), V)
            ref_s = np.array([[float(x) for x in r] for r in fin])
            assert _rel(S[n, h], ref_s) < 1e-13, ("state", n, h)
            if len(ts):
                assert _rel(o[cu[n]:cu[n + 1], h], ref_o) < 1e-13, ("o", n, h)
    return True


# --------------------------------------------------------------------------
# P3 / P4: DeltaNet and Gated DeltaNet as gradient steps on the L2 loss
# --------------------------------------------------------------------------
def _grad_l2(S, k, v):
    """d/dS of 0.5*||S^T k - v||^2, by central finite differences of the
    loss (exact for a quadratic up to rounding).  Independent of any
    closed-form update rule."""
    def loss(M):
        r = M.T @ k - v
        return 0.5 * float(r @ r)
    G = np.zeros_like(S)
    h = 1e-3
    for i in range(S.shape[0]):
        for j in range(S.shape[1]):
            E = np.zeros_like(S)
            E[i, j] = h
            G[i, j] = (loss(S + E) - loss(S - E)) / (2 * h)
    return G


def pin_deltanet_gradient(lib=None, seed=1, scalar_gate=False):
    """g == 0 (DeltaNet) or g equal across channels (Gated DeltaNet): each
    token is one gradient-descent step of step size beta_t on the retrieval
    loss 0.5*||S^T k_t - v_t||^2, taken on the gated state.  [SA/KDA]"""
    rng = np.random.default_rng(seed)
    T, H, K, V = 5, 1, 4, 3
    q, k, v, g, beta, S0 = _rand_problem(rng, T, H, K, V)
    if scalar_gate:
        g = np.repeat(-rng.random((T, H, 1)) * 1.5, K, axis=2)
    else:
        g = np.zeros_like(g)
    o, S = oracle.run_varlen(q, k, v, g, beta, [0, T], S0, lib=lib)
    St = S0[0, 0].copy()
    for t in range(T):
        St = math.exp(g[t, 0, 0]) * St                  # scalar forget gate
        St = St - beta[t, 0] * _grad_l2(St, k[t, 0], v[t, 0])
        assert _rel(o[t, 0], St.T @ q[t, 0]) < 1e-7, t
    assert _rel(S[0, 0], St) < 1e-7
    return True


# --------------------------------------------------------------------------
# P5: delta-rule recall
# --------------------------------------------------------------------------
def pin_recall(lib=None, seed=2):
    """beta = 1 and ||k|| = 1: after the update the state maps k_t exactly to
    v_t, whatever the decay and the earlier state.  With q_t = k_t the output
    is v_t.  Fails if correct used the undecayed state, or if the output
    read the state before the write.  [SA/KDA] (delta rule), [K3vsDSV4/
    Attention] (step order)"""
    rng = np.random.default_rng(seed)
    T, H, K, V = 9, 2, 5, 4
    q, k, v, g, beta, S0 = _rand_problem(rng, T, H, K, V, g_scale=3.0,
                                         unit_k=True)
    beta = np.ones_like(beta)
    o, _ = oracle.run_varlen(k, k, v, g, beta, [0, T], S0, lib=lib)
    assert _rel(o, v) < 1e-12
    return True


# --------------------------------------------------------------------------
# P6: beta = 0 is pure per-channel decay
# --------------------------------------------------------------------------
def pin_pure_decay(lib=None, seed=3):
    """beta = 0: nothing is written, S_t = Diag(exp(g_1 + ... + g_t)) S0, and
    o_t = S_t^T q_t.  Pins which axis the decay scales (the key rows).
    [SA/KDA] (diagonal alpha), [SA/FlashKDA] (cumulative decay)"""
    rng = np.random.default_rng(seed)
    T, H, K, V = 6, 2, 4, 3
    q, k, v, g, beta, S0 = _rand_problem(rng, T, H, K, V, g_scale=2.0)
    beta = np.zeros_like(beta)
    o, S = oracle.run_varlen(q, k, v, g, beta, [0, T], S0, lib=lib)
    a = np.cumsum(g, axis=0)                              # [T, H, K]
    for h in range(H):
        for t in range(T):
            St = np.exp(a[t, h])[:, None] * S0[0, h]
            assert _rel(o[t, h], St.T @ q[t, h]) < 1e-13, (t, h)
        assert _rel(S[0, h], np.exp(a[-1, h])[:, None] * S0[0, h]) < 1e-13
    return True


# --------------------------------------------------------------------------
# P7: linearity in (S0, v) and independence of the value columns
# --------------------------------------------------------------------------
def pin_linearity_columns(lib=None, seed=4):
    """(S0, v) -> (S_T, o) is linear for fixed q, k, g, beta, and each value
    column evolves on its own: running the two halves of d_v separately and
    concatenating equals the whole.  (Follows from the recurrence being
    linear in S and v with coefficients that depend only on q, k, g, beta.)"""
    rng = np.random.default_rng(seed)
    T, H, K, V = 7, 2, 4, 6
    q, k, v, g, beta, S0 = _rand_problem(rng, T, H, K, V)
    _, _, v2, _, _, S02 = _rand_problem(rng, T, H, K, V)
    cu = [0, T]
    o1, s1 = oracle.run_varlen(q, k, v, g, beta, cu, S0, lib=lib)
    o2, s2 = oracle.run_varlen(q, k, v2, g, beta, cu, S02, lib=lib)
    o3, s3 = oracle.run_varlen(q, k, 2 * v - 3 * v2, g, beta, cu,
                               2 * S0 - 3 * S02, lib=lib)
    assert _rel(o3, 2 * o1 - 3 * o2) < 1e-12
    assert _rel(s3, 2 * s1 - 3 * s2) < 1e-12
    oa, sa = oracle.run_varlen(q, k, v[..., :2], g, beta, cu,
                               S0[..., :2], lib=lib)
    ob, sb = oracle.run_varlen(q, k, v[..., 2:], g, beta, cu,
                               S0[..., 2:], lib=lib)
    assert _rel(np.concatenate([oa, ob], -1), o1) < 1e-13
    assert _rel(np.concatenate([sa, sb], -1), s1) < 1e-13
    return True


# --------------------------------------------------------------------------
# P8: split / resume, decode = prefill of one token, varlen = separate calls
# --------------------------------------------------------------------------
def pin_split_resume(lib=None, seed=5):
    """Running T tokens equals running T1 tokens and continuing from the
    returned state ([SA/Append]: append-prefill from a cached state); a
    decode step equals a one-token prefill; packing sequences with
    cu_seqlens equals running them one by one; heads are independent."""
    rng = np.random.default_rng(seed)
    T, H, K, V = 11, 3, 4, 3
    q, k, v, g, beta, S0 = _rand_problem(rng, T, H, K, V)
    o, S = oracle.run_varlen(q, k, v, g, beta, [0, T], S0, lib=lib)
    T1 = 4
    oa, sa = oracle.run_varlen(q[:T1], k[:T1], v[:T1], g[:T1], beta[:T1],
                               [0, T1], S0, lib=lib)
    ob, sb = oracle.run_varlen(q[T1:], k[T1:], v[T1:], g[T1:], beta[T1:],
                               [0, T - T1], sa, lib=lib)
    assert _rel(np.concatenate([oa, ob]), o) < 1e-13
    assert _rel(sb, S) < 1e-13
    # decode step == one-token prefill
    od, sd = oracle.run_decode(q[:1], k[:1], v[:1], g[:1], beta[:1], S0,
                               lib=lib)
    op, sp = oracle.run_varlen(q[:1], k[:1], v[:1], g[:1], beta[:1], [0, 1],
                               S0, lib=lib)
    assert _rel(od, op) == 0.0 and _rel(sd, sp) == 0.0
    # packed sequences == separate calls (lengths 4, 0, 7)
    cu = [0, 4, 4, 11]
    S0s = rng.standard_normal((3, H, K, V))
    opk, spk = oracle.run_varlen(q, k, v, g, beta, cu, S0s, lib=lib)
    for n in range(3):
        a, b = cu[n], cu[n + 1]
        on, sn = oracle.run_varlen(q[a:b], k[a:b], v[a:b], g[a:b], beta[a:b],
                                   [0, b - a], S0s[n:n + 1], lib=lib)
        assert _rel(opk[a:b], on) == 0.0 and _rel(spk[n], sn[0]) == 0.0
    # head independence: permuting heads permutes results
    perm = [2, 0, 1]
    op_, sp_ = oracle.run_varlen(q[:, perm], k[:, perm], v[:, perm],
                                 g[:, perm], beta[:, perm], [0, T],
                                 S0[:, perm], lib=lib)
    assert _rel(op_, o[:, perm]) == 0.0 and _rel(sp_, S[:, perm]) == 0.0
    return True


# --------------------------------------------------------------------------
# P9: chunked UT form == per-token recurrence
# --------------------------------------------------------------------------
def pin_chunked(lib=None, seed=6, cases=None):
    """The chunked form (UT transform, cumulative decay, 16-row sub-tile
    split of the decay) agrees with the oracle in fp64, for chunk sizes
    1, 2, 16, 64, a length that is not a multiple of the chunk, and decay at
    the -5 bound and at 0.  [SA/FlashKDA], [K3vsDSV4/HW]"""
    rng = np.random.default_rng(seed)
    T, K, V = 77, 8, 5
    cases = cases or [(1, "rand"), (2, "rand"), (16, "rand"), (64, "rand"),
                      (64, "min"), (64, "zero"), (16, "min")]
    for C, gk in cases:
        q, k, v, g, beta, S0 = _rand_problem(rng, T, 1, K, V, g_scale=5.0,
                                             unit_k=True)
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        if gk == "min":
            g = np.full_like(g, -5.0)
        elif gk == "zero":
            g = np.zeros_like(g)
        o, S = oracle.run_varlen(q, k, v, g, beta, [0, T], S0, lib=lib)
        for tile in (16, None):
            oc, sc = chunk_ref.run_sequence(q[:, 0], k[:, 0], v[:, 0],
                                            g[:, 0], beta[:, 0], S0[0, 0], C,
                                            tile=tile)
            assert _rel(oc, o[:, 0]) < 1e-11, (C, gk, tile)
            assert _rel(sc, S[0, 0]) < 1e-11, (C, gk, tile)
    return True


# --------------------------------------------------------------------------
# P10: the one-pass decode identity
# --------------------------------------------------------------------------
def pin_decode_identity(lib=None, seed=7):
    """For one token, o = (alpha S)^T q + (q . k) u with
    u = beta (v - (alpha S)^T k): the output can be formed from the decayed
    state before the write, so a decode kernel reads the state once.
    (Algebra of [SA/FlashKDA]'s per-token form.)"""
    rng = np.random.default_rng(seed)
    B, H, K, V = 3, 2, 6, 5
    q = rng.standard_normal((B, H, K))
    k = rng.standard_normal((B, H, K))
    v = rng.standard_normal((B, H, V))
    g = -rng.random((B, H, K)) * 5
    beta = rng.random((B, H))
    S = rng.standard_normal((B, H, K, V))
    o, S1 = oracle.run_decode(q, k, v, g, beta, S, lib=lib)
    for b in range(B):
        for h in range(H):
            aS = np.exp(g[b, h])[:, None] * S[b, h]
            u = beta[b, h] * (v[b, h] - aS.T @ k[b, h])
            ref = aS.T @ q[b, h] + (q[b, h] @ k[b, h]) * u
            assert _rel(o[b, h], ref) < 1e-13
            assert _rel(S1[b, h], aS + np.outer(k[b, h], u)) < 1e-13
    return True


ALL_PINS = [pin_brute_force, pin_deltanet_gradient,
            lambda lib=None: pin_deltanet_gradient(lib, scalar_gate=True),
            pin_recall, pin_pure_decay, pin_linearity_columns,
            pin_split_resume, pin_chunked, pin_decode_identity]
