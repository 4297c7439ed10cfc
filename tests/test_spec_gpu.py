"""GPU parity of kda_spec_verify / kda_spec_commit (speculative-decode
verify: T draft tokens from a cached state, then the state advanced by the
accepted prefix only).

By definition the draft outputs are the recurrence's outputs over the T
tokens from the cached state, and the committed state after a accepted
tokens is the recurrence's state after those a tokens: both come from the
fp64 oracle run on the same values.  The state must stay within the fp32
decode tolerance (1e-4); outputs within the decode output tolerance.
Committing all T tokens must also agree with T decode steps of libkda to
rounding."""
import numpy as np
import pytest
import torch

import oracle
from conftest import gpu_available
from linear_recurrent_attention_kda_amd import inputs, kda

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

import gpu_util as U  # noqa: E402


def spec_problem(seed, B, T, H, D, dtype="bf16"):
    """T draft tokens for each of B sequences, from cached states."""
    p = inputs.make("varlen", seed=seed, H=H, K=D, V=D, dtype=dtype,
                    lengths=[T] * B)
    shp = lambda x: x.reshape((B, T) + x.shape[1:])  # noqa: E731
    return p, shp


def oracle_prefix(p, a_per_seq, T):
    """Oracle outputs over all T tokens, and states after a[b] tokens."""
    o_ref, _ = oracle.run_varlen(p.q, p.k, p.v, p.g, p.beta, p.cu_seqlens,
                                 p.initial_state)
    B = len(a_per_seq)
    s_ref = np.array(p.initial_state, dtype=np.float64)
    for b, a in enumerate(a_per_seq):
        if a > 0:
            lo = b * T
            _, s = oracle.run_varlen(p.q[lo:lo + a], p.k[lo:lo + a],
                                     p.v[lo:lo + a], p.g[lo:lo + a],
                                     p.beta[lo:lo + a], np.array([0, a]),
                                     p.initial_state[b:b + 1],
                                     want_output=False)
            s_ref[b] = s[0]
    return o_ref.reshape((B, T) + o_ref.shape[1:]), s_ref


def run_spec(p, shp, accepted):
    q, k, v = (U.to_dev(shp(x), p.dtype) for x in (p.q, p.k, p.v))
    g, beta = U.f32_dev(shp(p.g)), U.f32_dev(shp(p.beta))
    state = U.f32_dev(p.initial_state)
    before = state.clone()
    o, u = kda.kda_spec_verify(q, k, v, g, beta, state)
    torch.cuda.synchronize()
    assert torch.equal(state, before), "verify modified the state"
    acc = torch.tensor(accepted, dtype=torch.int32, device=U.DEV)
    kda.kda_spec_commit(k, g, u, acc, state)
    torch.cuda.synchronize()
    return U.host(o), U.host(state), (q, k, v, g, beta, before)


@pytest.mark.parametrize("D,dtype", [(128, "bf16"), (64, "fp32"),
                                     (32, "bf16"), (16, "fp32")])
def test_spec_verify_commit(D, dtype):
    B, T, H = 6, 5, 3
    p, shp = spec_problem(21 + D, B, T, H, D, dtype)
    accepted = [0, 1, 2, 5, 3, 9]          # 9 is clamped to T
    U.log("spec", "B=%d T=%d H=%d D=%d %s accepted=%s"
          % (B, T, H, D, dtype, accepted))
    o, s, _ = run_spec(p, shp, accepted)
    o_ref, s_ref = oracle_prefix(p, [min(a, T) for a in accepted], T)
    eo = max(U.slice_rel(o[b], o_ref[b], (1,)) for b in range(B))
    es = U.slice_rel(s, s_ref, (0, 1))
    U.log("   o rel err %.3e   committed state rel err %.3e" % (eo, es))
    assert es <= U.DECODE_STATE_TOL
    assert eo <= U.DECODE_O_TOL[dtype]
    # no accepted token: the state is bit-for-bit the cached one
    assert np.array_equal(s[0], p.initial_state[0].astype(np.float64))


def test_spec_commit_all_equals_decode_steps():
    B, T, H, D = 4, 6, 2, 128
    p, shp = spec_problem(31, B, T, H, D)
    o, s, (q, k, v, g, beta, s0) = run_spec(p, shp, [T] * B)
    state = s0.clone()
    outs = []
    for t in range(T):
        outs.append(U.host(kda.kda_decode_step(
            q[:, t].contiguous(), k[:, t].contiguous(), v[:, t].contiguous(),
            g[:, t].contiguous(), beta[:, t].contiguous(), state)))
    torch.cuda.synchronize()
    # the same arithmetic per token; only the order of the cross-lane sums
    # differs (verify runs 4 waves per head, decode 16), so the two agree to
    # fp32 rounding in the state and to bf16 rounding in the outputs
    es = U.slice_rel(U.host(state), s, (0, 1))
    eo = U.slice_rel(np.stack(outs, axis=1), o, (0, 2))
    U.log("   spec vs decode steps: state %.2e, o %.2e" % (es, eo))
    assert es <= 1e-5
    assert eo <= 8e-3


def test_spec_full_decode_batch():
    """The decode workload's shape (64 sequences x 96 heads, d=128) with 4
    draft tokens each and mixed acceptance; sampled sequences vs oracle."""
    B, T, H, D = 64, 4, 96, 128
    p, shp = spec_problem(41, B, T, H, D)
    rng = np.random.default_rng(41)
    accepted = rng.integers(0, T + 1, size=B).tolist()
    o, s, _ = run_spec(p, shp, accepted)
    for b in (0, 17, 63):
        lo = b * T
        sub = inputs.Problem(
            name="seq", kind="varlen", dtype=p.dtype, H=H, K=D, V=D, C=p.C,
            q=p.q[lo:lo + T], k=p.k[lo:lo + T], v=p.v[lo:lo + T],
            g=p.g[lo:lo + T], beta=p.beta[lo:lo + T],
            initial_state=p.initial_state[b:b + 1],
            cu_seqlens=np.array([0, T], np.int32), N=1)
        o_ref, s_ref = oracle_prefix(sub, [accepted[b]], T)
        eo = U.slice_rel(o[b], o_ref[0], (1,))
        es = U.slice_rel(s[b:b + 1], s_ref, (0, 1))
        U.log("   seq %d accepted %d: o %.3e state %.3e"
              % (b, accepted[b], eo, es))
        assert es <= U.DECODE_STATE_TOL and eo <= U.DECODE_O_TOL["bf16"]
