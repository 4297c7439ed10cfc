"""Exact rational brute force for tiny KDA problems (pins the fp64 oracle).

This is deliberately a *different formulation* from the oracle's four-step
loop.  Every token is one affine map of the state,

    S_t = A_t S_{t-1} + beta_t k_t v_t^T,   A_t = (I - beta_t k_t k_t^T) Diag(alpha_t),

which is what forget (Diag(alpha_t)), correct (the delta rule's removal of the
stale association S^T k_t - v_t) and write compose to ("Kimi K3: The Manos,
The Mythos, The Legendos", section "Kimi Delta Attention": DeltaNet, Gated
DeltaNet and the diagonal gate of KDA).  The whole run is then expanded as
explicit products of the transition matrices,

    S_T = A_T...A_1 S_0 + sum_t A_T...A_{t+1} beta_t k_t v_t^T,

and o_t = scale * S_t^T q_t.  All arithmetic is exact (fractions.Fraction);
alpha is supplied directly as a rational number.
"""
from __future__ import annotations

from fractions import Fraction


def _zeros(r, c):
    return [[Fraction(0)] * c for _ in range(r)]


def _eye(n):
    m = _zeros(n, n)
    for i in range(n):
        m[i][i] = Fraction(1)
    return m


def _matmul(a, b):
    n, k, m = len(a), len(b), len(b[0])
    out = _zeros(n, m)
    for i in range(n):
        for j in range(m):
            s = Fraction(0)
            for p in range(k):
                s += a[i][p] * b[p][j]
            out[i][j] = s
    return out


def _add(a, b):
    return [[x + y for x, y in zip(ra, rb)] for ra, rb in zip(a, b)]


def transition(alpha, k, beta):
    """A_t = (I - beta k k^T) Diag(alpha) as an exact K x K matrix."""
    K = len(k)
    a = _eye(K)
    for i in range(K):
        for j in range(K):
            a[i][j] -= beta * k[i] * k[j]
    d = _zeros(K, K)
    for i in range(K):
        d[i][i] = alpha[i]
    return _matmul(a, d)


def rank_one(beta, k, v):
    return [[beta * kc * vj for vj in v] for kc in k]


def run_sequence(qs, ks, vs, alphas, betas, S0, scale=Fraction(1)):
    """One (sequence, head): lists of exact vectors per token.

    Returns (outputs as a list of V-vectors, final K x V state).  The final
    state is formed from the expanded product sum, the per-token states (for
    the outputs) from the same products truncated at t.
    """
    T = len(qs)
    K = len(S0)
    mats = [transition(alphas[t], ks[t], betas[t]) for t in range(T)]
    outs = []
    for t in range(T):
        # S_t = A_t...A_1 S0 + sum_{s<=t} A_t...A_{s+1} beta_s k_s v_s^T
        prod = _eye(K)
        for s in range(t, -1, -1):
            prod = _matmul(prod, mats[s])
        st = _matmul(prod, S0)
        for s in range(t + 1):
            tail = _eye(K)
            for r in range(t, s, -1):
                tail = _matmul(tail, mats[r])
            st = _add(st, _matmul(tail, rank_one(betas[s], ks[s], vs[s])))
        outs.append([scale * sum(st[c][j] * qs[t][c] for c in range(K))
                     for j in range(len(S0[0]))])
        final = st
    if T == 0:
        final = [row[:] for row in S0]
    return outs, final
