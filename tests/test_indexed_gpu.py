"""GPU tests of the state-pool entry points: kda_decode_step_indexed,
kda_decode_step_gated_indexed, kda_prefill_varlen_indexed and
kda_spec_step_indexed.

Their contract is the plain call on the gathered states followed by a
scatter of the new states, bit for bit (the kernels are the same; only the
state rows they address differ), with padding entries (slot out of range)
running from a zero state and touching no state, and has_initial == 0
starting a sequence from zeros.  The plain calls are checked against the
oracle elsewhere; one case here also goes to the oracle directly."""
import numpy as np
import pytest
import torch

import oracle
from conftest import gpu_available
from linear_recurrent_attention_kda_amd import inputs, kda

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

import gpu_util as U  # noqa: E402


def _pool(rng, slots, H, Dk, Dv):
    return torch.from_numpy(
        (rng.standard_normal((slots, H, Dk, Dv)) * 0.02).astype(np.float32)
    ).to(U.DEV)


@pytest.mark.parametrize("Dk,Dv,dtype", [(128, 128, "bf16"), (64, 128, "fp32"),
                                         (32, 48, "bf16")])
def test_decode_indexed_equals_gather_scatter(Dk, Dv, dtype):
    B, H, slots = 12, 5, 40
    rng = np.random.default_rng(Dk + Dv)
    d = inputs.make("decode", seed=31 + Dk, B=B, H=H, K=Dk, V=Dv, dtype=dtype)
    q, k, v = (U.to_dev(x, d.dtype) for x in (d.q, d.k, d.v))
    g, beta = U.f32_dev(d.g), U.f32_dev(d.beta)
    pool = _pool(rng, slots, H, Dk, Dv)
    idx = [int(x) for x in rng.permutation(slots)[:B]]
    idx[3], idx[7], idx[10] = -1, slots, -7      # padding entries
    U.log("decode indexed Dk=%d Dv=%d %s idx=%s" % (Dk, Dv, dtype, idx))
    sidx = torch.tensor(idx, dtype=torch.int32, device=U.DEV)
    valid = [b for b in range(B) if 0 <= idx[b] < slots]
    # reference: gather (zeros for padding), plain call, scatter
    gathered = torch.zeros((B, H, Dk, Dv), dtype=torch.float32, device=U.DEV)
    for b in valid:
        gathered[b] = pool[idx[b]]
    o_ref = kda.kda_decode_step(q, k, v, g, beta, gathered)
    pool_ref = pool.clone()
    for b in valid:
        pool_ref[idx[b]] = gathered[b]
    pool2 = pool.clone()
    o = kda.kda_decode_step_indexed(q, k, v, g, beta, pool2, sidx)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref), "outputs"
    assert torch.equal(pool2, pool_ref), "pool rows (untouched ones too)"


def test_decode_indexed_at_the_decode_workload():
    """64 sequences x 96 heads scattered over a 256-slot pool."""
    B, H, slots, D = 64, 96, 256, 128
    rng = np.random.default_rng(5)
    d = inputs.make("decode", seed=32, B=B, H=H)
    q, k, v = (U.to_dev(x, d.dtype) for x in (d.q, d.k, d.v))
    g, beta = U.f32_dev(d.g), U.f32_dev(d.beta)
    pool = _pool(rng, slots, H, D, D)
    idx = torch.from_numpy(rng.permutation(slots)[:B].astype(np.int32)).to(
        U.DEV)
    gathered = pool[idx.long()].clone()
    o_ref = kda.kda_decode_step(q, k, v, g, beta, gathered)
    pool_ref = pool.clone()
    pool_ref[idx.long()] = gathered
    o = kda.kda_decode_step_indexed(q, k, v, g, beta, pool, idx)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(pool, pool_ref)


def _prefill_case(seed, lengths, H, Dk, Dv, dtype, C=64):
    p = inputs.make("varlen", seed=seed, H=H, K=Dk, V=Dv, C=C, dtype=dtype,
                    lengths=lengths)
    q, k, v = (U.to_dev(x, p.dtype) for x in (p.q, p.k, p.v))
    g, beta = U.f32_dev(p.g), U.f32_dev(p.beta)
    cu = torch.from_numpy(p.cu_seqlens).to(U.DEV)
    return p, (q, k, v, g, beta, cu, int(p.seq_lengths.max(initial=1)))


@pytest.mark.parametrize("H,Dk,Dv,dtype", [(8, 128, 128, "bf16"),
                                           (70, 128, 128, "bf16"),
                                           (3, 64, 32, "fp32"),
                                           (5, 16, 80, "bf16")])
def test_prefill_indexed_equals_gather_scatter(H, Dk, Dv, dtype):
    """Padding entries, new sequences (has_initial = 0), an empty sequence,
    and 16-, 32- or 64-wide recurrence slices (the streamed kernel at 70
    heads)."""
    lengths = [300, 0, 129, 64, 17, 200]
    N, slots = len(lengths), 16
    rng = np.random.default_rng(H + Dk + Dv)
    p, (q, k, v, g, beta, cu, maxlen) = _prefill_case(
        40 + H, lengths, H, Dk, Dv, dtype)
    pool = _pool(rng, slots, H, Dk, Dv)
    idx = [int(x) for x in rng.permutation(slots)[:N]]
    idx[4] = -1                                  # padding
    has = [1, 1, 0, 1, 1, 0]                     # two new sequences
    U.log("prefill indexed H=%d Dk=%d Dv=%d %s lengths=%s idx=%s has=%s"
          % (H, Dk, Dv, dtype, lengths, idx, has))
    sidx = torch.tensor(idx, dtype=torch.int32, device=U.DEV)
    shas = torch.tensor(has, dtype=torch.int32, device=U.DEV)
    valid = [n for n in range(N) if 0 <= idx[n] < slots]
    s0 = torch.zeros((N, H, Dk, Dv), dtype=torch.float32, device=U.DEV)
    for n in valid:
        if has[n]:
            s0[n] = pool[idx[n]]
    o_ref, fs = kda.kda_prefill_varlen(q, k, v, g, beta, cu, maxlen, s0)
    pool_ref = pool.clone()
    for n in valid:
        pool_ref[idx[n]] = fs[n]
    pool2 = pool.clone()
    o = kda.kda_prefill_varlen_indexed(q, k, v, g, beta, cu, maxlen, pool2,
                                       sidx, shas)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref), "outputs"
    assert torch.equal(pool2, pool_ref), "pool rows (untouched ones too)"
    # without has_initial every sequence continues from its row
    for n in valid:
        s0[n] = pool[idx[n]]
    o_ref2, fs2 = kda.kda_prefill_varlen(q, k, v, g, beta, cu, maxlen, s0)
    pool3 = pool.clone()
    o2 = kda.kda_prefill_varlen_indexed(q, k, v, g, beta, cu, maxlen, pool3,
                                        sidx)
    torch.cuda.synchronize()
    assert torch.equal(o2, o_ref2)
    for n in valid:
        assert torch.equal(pool3[idx[n]], fs2[n])


def test_prefill_then_decode_from_the_pool_against_the_oracle():
    """Append-prefill of three requests from pooled states, then two decode
    steps on the same pool rows: the final pooled states and the decode
    outputs against the oracle run over each request's tokens."""
    H, D, slots = 4, 64, 8
    lengths = [150, 64, 33]
    N = len(lengths)
    rng = np.random.default_rng(77)
    p, (q, k, v, g, beta, cu, maxlen) = _prefill_case(
        78, lengths, H, D, D, "bf16")
    pool = _pool(rng, slots, H, D, D)
    pool_host = pool.double().cpu().numpy()
    idx = [5, 0, 3]
    sidx = torch.tensor(idx, dtype=torch.int32, device=U.DEV)
    kda.kda_prefill_varlen_indexed(q, k, v, g, beta, cu, maxlen, pool, sidx)
    s_ref = np.stack([pool_host[i] for i in idx])
    _, s_ref = oracle.run_varlen(p.q, p.k, p.v, p.g, p.beta, p.cu_seqlens,
                                 s_ref, want_output=False)
    for step in range(2):
        d = inputs.make("decode", seed=90 + step, B=N, H=H, K=D, V=D)
        dq, dk, dv = (U.to_dev(x, d.dtype) for x in (d.q, d.k, d.v))
        o = kda.kda_decode_step_indexed(dq, dk, dv, U.f32_dev(d.g),
                                        U.f32_dev(d.beta), pool, sidx)
        o_ref, s_ref = oracle.run_decode(d.q, d.k, d.v, d.g, d.beta, s_ref)
        torch.cuda.synchronize()
        eo = U.slice_rel(U.host(o), o_ref, (0, 1))
        U.log("   decode step %d: o rel err %.3e" % (step, eo))
        assert eo <= U.DECODE_O_TOL["bf16"]
    got = U.host(pool)[idx]
    es = U.slice_rel(got, s_ref, (0, 1))
    U.log("   pooled states after prefill + 2 decode steps: rel err %.3e"
          % es)
    assert es <= U.PREFILL_TOL
    # rows no request uses are untouched
    for r in set(range(slots)) - set(idx):
        assert np.array_equal(U.host(pool)[r], pool_host[r].astype(np.float32))


def test_gated_decode_indexed_equals_gather_scatter():
    B, H, D, slots = 10, 6, 128, 24
    rng = np.random.default_rng(33)
    d = inputs.make("decode", seed=34, B=B, H=H)
    q, k, v = (U.to_dev(x, d.dtype) for x in (d.q, d.k, d.v))
    g, beta = U.f32_dev(d.g), U.f32_dev(d.beta)
    z = U.to_dev(rng.standard_normal((B, H, D)).astype(np.float32), "bf16")
    w = U.f32_dev((0.5 + rng.random(D)).astype(np.float32))
    pool = _pool(rng, slots, H, D, D)
    idx = [int(x) for x in rng.permutation(slots)[:B]]
    idx[2] = -1
    sidx = torch.tensor(idx, dtype=torch.int32, device=U.DEV)
    valid = [b for b in range(B) if idx[b] >= 0]
    gathered = torch.zeros((B, H, D, D), dtype=torch.float32, device=U.DEV)
    for b in valid:
        gathered[b] = pool[idx[b]]
    y_ref = kda.kda_decode_step_gated(q, k, v, g, beta, gathered, z, w)
    pool_ref = pool.clone()
    for b in valid:
        pool_ref[idx[b]] = gathered[b]
    y = kda.kda_decode_step_gated_indexed(q, k, v, g, beta, pool, sidx, z, w)
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref) and torch.equal(pool, pool_ref)


@pytest.mark.parametrize("Tp,T", [(4, 4), (3, 6), (5, 0), (0, 2)])
def test_spec_step_indexed_equals_gather_scatter(Tp, T):
    """The fused speculative step on pooled states (a padding entry, mixed
    acceptance), against the step on gathered states: commit and verify,
    commit only (T = 0) and verify only (T_prev = 0)."""
    B, H, D, slots = 6, 5, 64, 16
    rng = np.random.default_rng(50 + Tp + 7 * T)

    def draft(seed, n):
        if n == 0:
            z = lambda *s: torch.zeros(s, device=U.DEV)  # noqa: E731
            return (z(B, 0, H, D).to(torch.bfloat16),
                    z(B, 0, H, D).to(torch.bfloat16),
                    z(B, 0, H, D).to(torch.bfloat16), z(B, 0, H, D),
                    z(B, 0, H))
        p = inputs.make("varlen", seed=seed, H=H, K=D, V=D, lengths=[n] * B)
        shp = lambda x: x.reshape((B, n) + x.shape[1:])  # noqa: E731
        q, k, v = (U.to_dev(shp(x), p.dtype) for x in (p.q, p.k, p.v))
        return q, k, v, U.f32_dev(shp(p.g)), U.f32_dev(shp(p.beta))
    new = draft(60 + T, T)
    pool = _pool(rng, slots, H, D, D)
    idx = [int(x) for x in rng.permutation(slots)[:B]]
    idx[4] = slots + 2                            # padding
    sidx = torch.tensor(idx, dtype=torch.int32, device=U.DEV)
    valid = [b for b in range(B) if 0 <= idx[b] < slots]
    gathered = torch.zeros((B, H, D, D), dtype=torch.float32, device=U.DEV)
    for b in valid:
        gathered[b] = pool[idx[b]]
    kw = {}
    if Tp:
        prev = draft(70 + Tp, Tp)
        _, u_prev = kda.kda_spec_verify(*prev, gathered)
        acc = torch.tensor([int(a) for a in rng.integers(0, Tp + 1, B)],
                           dtype=torch.int32, device=U.DEV)
        kw = dict(k_prev=prev[1], g_prev=prev[3], u_prev=u_prev,
                  accepted_prev=acc)
    st_ref = gathered.clone()
    o_ref, u_ref = kda.kda_spec_step(*new, st_ref, **kw)
    pool_ref = pool.clone()
    for b in valid:
        pool_ref[idx[b]] = st_ref[b]
    o, u = kda.kda_spec_step_indexed(*new, pool, sidx, **kw)
    torch.cuda.synchronize()
    assert torch.equal(pool, pool_ref), "pool rows"
    if T:
        assert torch.equal(o, o_ref) and torch.equal(u, u_ref)
