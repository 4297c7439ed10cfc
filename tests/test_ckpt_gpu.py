"""GPU parity of kda_prefill_varlen_ckpt: state checkpoints every
`ckpt_every` tokens inside each sequence ("Kimi K3: The Manos, The Mythos,
The Legendos", section "KDA prefix cache management").

The state after the first p tokens of a sequence is, by definition, the
final state of the recurrence run on that prefix, so each checkpoint is
compared with the fp64 oracle's final state over the prefix (chained segment
by segment, so that one pass of the oracle covers all of a sequence's
checkpoints).  Outputs and final states must equal kda_prefill_varlen's bit
for bit (the same kernels, plus the checkpoint stores)."""
import numpy as np
import pytest
import torch

import oracle
from conftest import gpu_available
from linear_recurrent_attention_kda_amd import inputs, kda

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

import gpu_util as U  # noqa: E402


def ckpt_reference(p, every, heads=None):
    """{(n, tokens done): oracle state [H', K, V]} for every checkpoint."""
    hs = slice(None) if heads is None else heads
    cu = [int(x) for x in p.cu_seqlens]
    ref = {}
    for n in range(len(cu) - 1):
        bos, L = cu[n], cu[n + 1] - cu[n]
        s = None if p.initial_state is None else p.initial_state[n:n + 1][:, hs]
        done = 0
        for pos in range(every, L + 1, every):
            a, b = bos + done, bos + pos
            _, s = oracle.run_varlen(
                p.q[a:b][:, hs], p.k[a:b][:, hs], p.v[a:b][:, hs],
                p.g[a:b][:, hs], p.beta[a:b][:, hs],
                np.array([0, b - a]), s, want_output=False)
            ref[(n, pos)] = s[0]
            done = pos
    return ref


def run_ckpt(p, every, heads=None):
    q, k, v = (U.to_dev(x, p.dtype) for x in (p.q, p.k, p.v))
    g, beta = U.f32_dev(p.g), U.f32_dev(p.beta)
    s0 = U.f32_dev(p.initial_state)
    cu = torch.from_numpy(p.cu_seqlens.astype(np.int32)).to(U.DEV)
    maxlen = int(p.seq_lengths.max(initial=0))
    o, s, ck = kda.kda_prefill_varlen_ckpt(q, k, v, g, beta, cu, maxlen, s0,
                                           ckpt_every=every, chunk_size=p.C)
    o2, s2 = kda.kda_prefill_varlen(q, k, v, g, beta, cu, maxlen, s0,
                                    chunk_size=p.C)
    torch.cuda.synchronize()
    assert torch.equal(o, o2), "outputs differ from kda_prefill_varlen"
    assert torch.equal(s, s2), "final states differ from kda_prefill_varlen"
    return U.host(o), U.host(s), U.host(ck)


def check_ckpt(p, every, heads=None, label=""):
    U.log("ckpt", label, "H=%d D=%d C=%d every=%d lengths=%s"
          % (p.H, p.K, p.C, every, p.seq_lengths.tolist()))
    _, _, ck = run_ckpt(p, every)
    ref = ckpt_reference(p, every, heads)
    slots = kda.kda_ckpt_slots(p.cu_seqlens, every)
    assert len(slots) == len(ref)
    assert ck.shape[0] == int(p.cu_seqlens[-1]) // every
    used = set()
    worst = 0.0
    for n, pos, slot in slots:
        assert slot not in used
        used.add(slot)
        got = ck[slot] if heads is None else ck[slot][heads]
        worst = max(worst, U.slice_rel(got, ref[(n, pos)], (0,)))
    # slots no checkpoint maps to stay as allocated (zeros)
    for slot in range(ck.shape[0]):
        if slot not in used:
            assert not np.any(ck[slot])
    U.log("   %d checkpoints, worst rel err %.3e" % (len(slots), worst))
    assert worst <= U.PREFILL_TOL
    return len(slots)


@pytest.mark.parametrize("every", [64, 96])
def test_ckpt_ragged_varlen(every):
    p = inputs.make("varlen", seed=11, H=3, K=64, V=64, C=32,
                    lengths=[70, 0, 200, 130, 64, 191])
    assert check_ckpt(p, every, label="ragged") > 0


def test_ckpt_every_chunk_no_initial_state():
    p = inputs.make("varlen", seed=12, H=2, K=32, V=32, C=16, s0=False,
                    lengths=[33, 80, 16])
    assert check_ckpt(p, 16, label="every chunk") == 2 + 5 + 1


def test_ckpt_interval_longer_than_sequences():
    """No sequence reaches the interval: nothing written, outputs intact."""
    p = inputs.make("varlen", seed=13, H=2, K=64, V=64, C=64,
                    lengths=[100, 120, 90])
    assert check_ckpt(p, 128, label="none") == 0


def test_ckpt_long_context_sampled_head():
    """H=32, T=131072, d=128, C=64, bf16, nonzero state, decay near -5;
    checkpoints every 32768 tokens (the 32K interval the page mentions)."""
    p = inputs.make("long", seed=0)
    cu = np.array([0, p.T], dtype=np.int64)
    pv = inputs.Problem(
        name="long-as-varlen", kind="varlen", dtype=p.dtype, H=p.H, K=p.K,
        V=p.V, C=p.C, q=p.q[0], k=p.k[0], v=p.v[0], g=p.g[0], beta=p.beta[0],
        initial_state=p.initial_state, cu_seqlens=cu, B=0, T=0, N=1)
    assert check_ckpt(pv, 32768, heads=[17], label="long") == 4
