"""GPU parity of kda_prefill_varlen_ckpt: state checkpoints every
`ckpt_every` tokens inside each sequence ("Kimi K3: The Manos, The Mythos,
The Legendos", section "KDA prefix cache management").

The state after the first p tokens of a sequence is, by definition, the
final state of the recurrence run on that prefix, so each checkpoint is
compared with the fp64 oracle's final state over the prefix (chained segment
by segment, so that one pass of the oracle covers all of a sequence's
checkpoints).  Outputs and final states must equal kda_prefill_varlen's bit
for bit (the same kernels, plus the checkpoint stores).  Both forms are
covered: a fixed interval (kda_prefill_varlen_ckpt) and caller-given
positions (kda_prefill_varlen_ckpt_at)."""
import numpy as np
import pytest
import torch

import oracle
from conftest import gpu_available
from linear_recurrent_attention_kda_amd import inputs, kda

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

import gpu_util as U  # noqa: E402


def ckpt_reference(p, wanted, heads=None):
    """{(n, tokens done): oracle state [H', K, V]} for the (n, p) pairs in
    `wanted`, chained segment by segment along each sequence."""
    hs = slice(None) if heads is None else heads
    cu = [int(x) for x in p.cu_seqlens]
    ref = {}
    for n in range(len(cu) - 1):
        bos = cu[n]
        s = None if p.initial_state is None else p.initial_state[n:n + 1][:, hs]
        done = 0
        for pos in sorted({q for (m, q) in wanted if m == n}):
            a, b = bos + done, bos + pos
            _, s = oracle.run_varlen(
                p.q[a:b][:, hs], p.k[a:b][:, hs], p.v[a:b][:, hs],
                p.g[a:b][:, hs], p.beta[a:b][:, hs],
                np.array([0, b - a]), s, want_output=False)
            ref[(n, pos)] = s[0]
            done = pos
    return ref


def _dev_inputs(p):
    q, k, v = (U.to_dev(x, p.dtype) for x in (p.q, p.k, p.v))
    g, beta = U.f32_dev(p.g), U.f32_dev(p.beta)
    s0 = U.f32_dev(p.initial_state)
    cu = torch.from_numpy(p.cu_seqlens.astype(np.int32)).to(U.DEV)
    return q, k, v, g, beta, s0, cu, int(p.seq_lengths.max(initial=0))


def run_ckpt(p, every):
    q, k, v, g, beta, s0, cu, maxlen = _dev_inputs(p)
    o, s, ck = kda.kda_prefill_varlen_ckpt(q, k, v, g, beta, cu, maxlen, s0,
                                           ckpt_every=every, chunk_size=p.C)
    o2, s2 = kda.kda_prefill_varlen(q, k, v, g, beta, cu, maxlen, s0,
                                    chunk_size=p.C)
    torch.cuda.synchronize()
    assert torch.equal(o, o2), "outputs differ from kda_prefill_varlen"
    assert torch.equal(s, s2), "final states differ from kda_prefill_varlen"
    return ck


def run_ckpt_at(p, positions):
    """positions: one list of token counts per sequence."""
    q, k, v, g, beta, s0, cu, maxlen = _dev_inputs(p)
    flat = [x for lst in positions for x in lst]
    cuc = np.zeros(len(positions) + 1, np.int32)
    cuc[1:] = np.cumsum([len(x) for x in positions])
    pos_d = torch.tensor(flat, dtype=torch.int32, device=U.DEV)
    cuc_d = torch.from_numpy(cuc).to(U.DEV)
    o, s, ck = kda.kda_prefill_varlen_ckpt_at(
        q, k, v, g, beta, cu, maxlen, s0, ckpt_pos=pos_d, cu_ckpt=cuc_d,
        chunk_size=p.C)
    o2, s2 = kda.kda_prefill_varlen(q, k, v, g, beta, cu, maxlen, s0,
                                    chunk_size=p.C)
    torch.cuda.synchronize()
    assert torch.equal(o, o2), "outputs differ from kda_prefill_varlen"
    assert torch.equal(s, s2), "final states differ from kda_prefill_varlen"
    return ck, cuc


def compare_slots(p, ck, slots, head_group=None):
    """slots: list of (n, tokens done, slot).  Every listed slot against the
    oracle's state over the prefix (all heads, in groups); every other slot
    must be untouched (zeros).  Returns the worst relative error."""
    used = set()
    for _, _, slot in slots:
        used.add(slot)
    for slot in range(ck.shape[0]):
        if slot not in used:
            assert not torch.any(ck[slot]), "slot %d was written" % slot
    step = head_group or p.H
    worst = 0.0
    wanted = [(n, pos) for n, pos, _ in slots]
    for h0 in range(0, p.H, step):
        heads = list(range(h0, min(p.H, h0 + step)))
        ref = ckpt_reference(p, wanted, heads)
        for n, pos, slot in slots:
            got = U.host(ck[slot][heads])
            worst = max(worst, U.slice_rel(got, ref[(n, pos)], (0,)))
    return worst


def check_ckpt(p, every, label="", head_group=None):
    U.log("ckpt", label, "H=%d D=%d C=%d every=%d lengths=%s"
          % (p.H, p.K, p.C, every, p.seq_lengths.tolist()))
    ck = run_ckpt(p, every)
    slots = kda.kda_ckpt_slots(p.cu_seqlens, every)
    assert ck.shape[0] == int(p.cu_seqlens[-1]) // every
    assert len({sl for _, _, sl in slots}) == len(slots)
    worst = compare_slots(p, ck, slots, head_group)
    U.log("   %d checkpoints, worst rel err %.3e" % (len(slots), worst))
    assert worst <= U.PREFILL_TOL
    return len(slots)


def check_ckpt_at(p, positions, label="", head_group=None):
    """Checkpoints at listed positions; entries that break the rules (not a
    multiple of C and not the length, out of order, outside 1..length) must
    leave their slots untouched."""
    U.log("ckpt_at", label, "H=%d D=%d C=%d lengths=%s positions=%s"
          % (p.H, p.K, p.C, p.seq_lengths.tolist(), positions))
    ck, cuc = run_ckpt_at(p, positions)
    lengths = p.seq_lengths.tolist()
    slots = []
    for n, lst in enumerate(positions):
        last = 0
        for j, pos in enumerate(lst):
            ok = (0 < pos <= lengths[n] and
                  (pos % p.C == 0 or pos == lengths[n]) and pos >= last)
            if ok:
                slots.append((n, pos, int(cuc[n]) + j))
                last = pos
    worst = compare_slots(p, ck, slots, head_group)
    U.log("   %d of %d positions stored, worst rel err %.3e"
          % (len(slots), int(cuc[-1]), worst))
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


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_ckpt_streamed_slices_96_heads(dtype):
    """96 heads at d = 128, C = 64: the 64-wide streamed recurrence with its
    checkpoint stores (the launch the K3-shaped workloads use)."""
    p = inputs.make("varlen", seed=14, H=96, dtype=dtype,
                    lengths=[300, 0, 64, 513, 129])
    assert check_ckpt(p, 128, label="streamed", head_group=48) == 2 + 4 + 1


def test_ckpt_32_wide_slices():
    """300 heads at d = 32: the 32-wide slices."""
    p = inputs.make("varlen", seed=15, H=300, K=32, V=32, C=32,
                    lengths=[97, 160])
    assert check_ckpt(p, 32, label="32-wide", head_group=100) == 3 + 5


def test_ckpt_long_context():
    """H=32, T=131072, d=128, C=64, bf16, nonzero state, decay near -5;
    checkpoints every 32768 tokens (the 32K interval the page mentions),
    every head."""
    p = inputs.make("long", seed=0)
    cu = np.array([0, p.T], dtype=np.int64)
    pv = inputs.Problem(
        name="long-as-varlen", kind="varlen", dtype=p.dtype, H=p.H, K=p.K,
        V=p.V, C=p.C, q=p.q[0], k=p.k[0], v=p.v[0], g=p.g[0], beta=p.beta[0],
        initial_state=p.initial_state, cu_seqlens=cu, B=0, T=0, N=1)
    assert check_ckpt(pv, 32768, label="long", head_group=8) == 4


# ---- checkpoints at caller-given positions ---------------------------------
@pytest.mark.parametrize("H,D,C", [(3, 64, 32), (96, 128, 64), (4, 128, 64),
                                   (300, 32, 32), (2, 16, 16)])
def test_ckpt_at_ragged_positions(H, D, C):
    """Positions that differ between sequences, including the length of a
    partial last chunk (a prompt boundary), an empty list, duplicates, and
    entries that must be skipped: not a multiple of C, out of order, zero,
    past the end."""
    lengths = [3 * C + 5, 0, 2 * C, 5 * C + 1, C - 3]
    p = inputs.make("varlen", seed=16 + C, H=H, K=D, V=D, C=C,
                    lengths=lengths)
    positions = [[C, 3 * C + 5],                 # chunk edge, then the length
                 [],                             # empty sequence
                 [C, C, 2 * C],                  # a duplicate
                 [2 * C, C + 1, C, 4 * C, 0, 9 * C],  # C+1, C, 0, 9C skipped
                 [C - 3]]                        # shorter than one chunk
    n = check_ckpt_at(p, positions, label="ragged",
                      head_group=48 if H > 48 else None)
    assert n == 2 + 3 + 2 + 1


def test_ckpt_at_none():
    p = inputs.make("varlen", seed=17, H=2, K=64, V=64, C=64,
                    lengths=[100, 64])
    assert check_ckpt_at(p, [[], []], label="none") == 0


def test_ckpt_at_varlen_workload():
    """The 8-sequence, 96-head append-prefill workload with positions that
    differ between sequences: every 4096 tokens, plus two earlier prompt
    ends (multiples of 64) and the sequence's own end; every head."""
    p = inputs.make("varlen", seed=0)
    lengths = p.seq_lengths.tolist()
    rng = np.random.default_rng(18)
    positions = []
    for L in lengths:
        pts = set(range(4096, L + 1, 4096))
        pts |= {int(x) * 64 for x in rng.integers(1, L // 64 + 1, size=2)}
        pts.add(L)
        positions.append(sorted(pts))
    n = check_ckpt_at(p, positions, label="varlen workload", head_group=24)
    assert n == sum(len(x) for x in positions)
