"""Seeded random mixes of the supported sizes against the fp64 oracle.

Each case draws, from its own seed: head dims d_k and d_v (independently,
multiples of 16 up to 128), the chunk size, a head count across the
thresholds that pick 16-, 32- and 64-wide recurrence slices and the streamed
kernel, fixed-length batches or packed sequences (empty, shorter than a
chunk, exact chunk multiples, ragged), the storage dtype, an initial state
or none, the decay's mean (ordinary, or near the g >= -5 bound), and the
output scale.  The prefill and a decode step on the same sizes are compared
with the oracle to the usual bars (per (sequence, head) slices; see
gpu_util).  The cases are fixed by their seeds, so a failure names a case
that reproduces."""
import numpy as np
import pytest

from conftest import gpu_available
from linear_recurrent_attention_kda_amd import inputs

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

import gpu_util as U  # noqa: E402

N_CASES = 48


def draw(seed):
    rng = np.random.default_rng(7000 + seed)
    dims = [16 * i for i in range(1, 9)]
    c = dict(
        K=int(rng.choice(dims)),
        V=int(rng.choice(dims)),
        C=int(rng.choice([16, 32, 64])),
        H=int(rng.choice([1, 2, 3, 7, 33, 64, 70, 130])),
        dtype="bf16" if rng.random() < 0.75 else "fp32",
        s0=bool(rng.random() < 0.7),
        g_mu=float(rng.choice([0.0, 2.0])),
    )
    scale = float(rng.choice([1.0, 0.5, c["K"] ** -0.5]))
    if rng.random() < 0.25:  # fixed-length batch
        c.update(kind="prefill", B=int(rng.integers(1, 4)),
                 T=int(rng.integers(1, 300)))
    else:
        n = int(rng.integers(1, 7))
        lengths = rng.integers(0, 260, size=n)
        for i in range(n):  # some exact chunk multiples and empty sequences
            u = rng.random()
            if u < 0.15:
                lengths[i] = 0
            elif u < 0.3:
                lengths[i] = c["C"] * int(rng.integers(1, 5))
        c.update(kind="varlen", lengths=[int(x) for x in lengths])
    return c, scale


def case_label(c, scale):
    shape = ("B=%d T=%d" % (c["B"], c["T"]) if c["kind"] == "prefill"
             else "lengths=%s" % c["lengths"])
    return "Dk=%d Dv=%d C=%d H=%d %s %s s0=%s g_mu=%.0f scale=%.3f" % (
        c["K"], c["V"], c["C"], c["H"], shape, c["dtype"], c["s0"],
        c["g_mu"], scale)


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_prefill_and_decode(seed):
    c, scale = draw(seed)
    label = "random case %d: %s" % (seed, case_label(c, scale))
    kind = c.pop("kind")
    p = inputs.make(kind, seed=seed, **c)
    U.check_prefill(p, label=label, scale=scale,
                    head_group=48 if p.H > 48 else None)
    d = inputs.make("decode", seed=seed, B=3, H=p.H, K=p.K, V=p.V,
                    dtype=p.dtype)
    U.check_decode(d, scale=scale)


def as_varlen(c):
    """The packed form of a drawn case (fixed-length batches become B
    sequences of T tokens)."""
    c = dict(c)
    if c.pop("kind") == "prefill":
        c["lengths"] = [c.pop("T")] * c.pop("B")
    return c


@pytest.mark.parametrize("seed", range(16))
def test_random_gated_prefill(seed):
    """kda_prefill_varlen_gated on random mixes: the fused kernel where the
    draw gives at least two (sequence, head) pairs per compute unit, the
    two-pass path otherwise (test_prefill_gated_gpu's two measures)."""
    import test_prefill_gated_gpu as G
    c, _ = draw(100 + seed)
    c = as_varlen(c)
    if seed % 4 == 0:  # enough pairs for the fused kernel (130 x 4 >= 512)
        c["H"] = 130
        c["lengths"] = (c["lengths"] + [17, 64, 1, 40])[:max(4, len(c["lengths"]))]
    p = inputs.make("varlen", seed=100 + seed, **c)
    G.check_gated(p, 100 + seed, "random case %d" % seed,
                  head_group=48 if p.H > 48 else None)


@pytest.mark.parametrize("seed", range(16))
def test_random_ckpt_positions(seed):
    """kda_prefill_varlen_ckpt_at with random position lists per sequence
    (chunk edges and the sequence's own length, some lists empty)."""
    import test_ckpt_gpu as CK
    c, _ = draw(200 + seed)
    c = as_varlen(c)
    p = inputs.make("varlen", seed=200 + seed, **c)
    rng = np.random.default_rng(300 + seed)
    C = p.C
    positions = []
    for L in p.seq_lengths.tolist():
        cand = sorted(set(list(range(C, L + 1, C)) + ([L] if L > 0 else [])))
        k = int(rng.integers(0, 4))
        pick = rng.choice(cand, size=min(k, len(cand)), replace=False) \
            if cand else []
        positions.append(sorted(int(x) for x in pick))
    n = CK.check_ckpt_at(p, positions, label="random case %d" % seed,
                         head_group=48 if p.H > 48 else None)
    assert n == sum(len(x) for x in positions)


@pytest.mark.parametrize("seed", range(12))
def test_random_spec_verify_commit(seed):
    """Draft verify of T <= 16 tokens from cached states, then commit of a
    random accepted prefix per sequence (0 .. T, and one count past T, which
    is clamped), on random head dims."""
    import torch
    import oracle
    from linear_recurrent_attention_kda_amd import kda
    rng = np.random.default_rng(400 + seed)
    dims = [16 * i for i in range(1, 9)]
    Dk, Dv = int(rng.choice(dims)), int(rng.choice(dims))
    B, T = int(rng.integers(1, 9)), int(rng.integers(1, 17))
    H = int(rng.choice([1, 2, 5, 33]))
    dtype = "bf16" if rng.random() < 0.75 else "fp32"
    p = inputs.make("varlen", seed=400 + seed, H=H, K=Dk, V=Dv, dtype=dtype,
                    lengths=[T] * B)
    accepted = [int(a) for a in rng.integers(0, T + 1, size=B)]
    accepted[0] = T + 3
    U.log("random spec case %d: B=%d T=%d H=%d Dk=%d Dv=%d %s accepted=%s"
          % (seed, B, T, H, Dk, Dv, dtype, accepted))
    shp = lambda x: x.reshape((B, T) + x.shape[1:])  # noqa: E731
    q, k, v = (U.to_dev(shp(x), p.dtype) for x in (p.q, p.k, p.v))
    g, beta = U.f32_dev(shp(p.g)), U.f32_dev(shp(p.beta))
    state = U.f32_dev(p.initial_state)
    o, u = kda.kda_spec_verify(q, k, v, g, beta, state)
    kda.kda_spec_commit(k, g, u, torch.tensor(accepted, dtype=torch.int32,
                                              device=U.DEV), state)
    torch.cuda.synchronize()
    o_ref, _ = oracle.run_varlen(p.q, p.k, p.v, p.g, p.beta, p.cu_seqlens,
                                 p.initial_state)
    eo = U.slice_rel(U.host(o).reshape(B * T, H, Dv), o_ref, (1,))
    s_ref = np.array(p.initial_state, np.float64)
    for b, a in enumerate(min(a, T) for a in accepted):
        if a:
            lo = b * T
            _, s = oracle.run_varlen(p.q[lo:lo + a], p.k[lo:lo + a],
                                     p.v[lo:lo + a], p.g[lo:lo + a],
                                     p.beta[lo:lo + a], np.array([0, a]),
                                     p.initial_state[b:b + 1],
                                     want_output=False)
            s_ref[b] = s[0]
    es = U.slice_rel(U.host(state), s_ref, (0, 1))
    U.log("   o rel err %.3e   committed state rel err %.3e" % (eo, es))
    assert eo <= U.DECODE_O_TOL[dtype] and es <= U.DECODE_STATE_TOL


@pytest.mark.parametrize("seed", range(12))
def test_random_spec_step(seed):
    """kda_spec_step on random head dims, draft lengths (T_prev and T
    apart) and acceptances, against kda_spec_commit then kda_spec_verify,
    bit for bit."""
    import torch
    from linear_recurrent_attention_kda_amd import kda
    rng = np.random.default_rng(700 + seed)
    dims = [16 * i for i in range(1, 9)]
    Dk, Dv = int(rng.choice(dims)), int(rng.choice(dims))
    B, H = int(rng.integers(1, 9)), int(rng.choice([1, 2, 5, 33]))
    Tp, T = int(rng.integers(1, 17)), int(rng.integers(1, 17))
    dtype = "bf16" if rng.random() < 0.75 else "fp32"
    acc = [int(a) for a in rng.integers(0, Tp + 2, size=B)]
    U.log("random spec step %d: B=%d H=%d Dk=%d Dv=%d %s T_prev=%d T=%d "
          "accepted=%s" % (seed, B, H, Dk, Dv, dtype, Tp, T, acc))

    def draft(s, n):
        p = inputs.make("varlen", seed=s, H=H, K=Dk, V=Dv, dtype=dtype,
                        lengths=[n] * B)
        shp = lambda x: x.reshape((B, n) + x.shape[1:])  # noqa: E731
        q, k, v = (U.to_dev(shp(x), p.dtype) for x in (p.q, p.k, p.v))
        return p, (q, k, v, U.f32_dev(shp(p.g)), U.f32_dev(shp(p.beta)))
    p0, prev = draft(800 + seed, Tp)
    _, new = draft(900 + seed, T)
    s0 = U.f32_dev(p0.initial_state)
    accepted = torch.tensor(acc, dtype=torch.int32, device=U.DEV)
    _, u_prev = kda.kda_spec_verify(*prev, s0)
    st_a = s0.clone()
    kda.kda_spec_commit(prev[1], prev[3], u_prev, accepted, st_a)
    o_a, u_a = kda.kda_spec_verify(*new, st_a)
    st_b = s0.clone()
    o_b, u_b = kda.kda_spec_step(*new, st_b, k_prev=prev[1], g_prev=prev[3],
                                 u_prev=u_prev, accepted_prev=accepted)
    torch.cuda.synchronize()
    assert torch.equal(st_a, st_b) and torch.equal(o_a, o_b) and \
        torch.equal(u_a, u_b)


@pytest.mark.parametrize("seed", range(12))
def test_random_prologue(seed):
    """kda_prefill_varlen_prologue (d_k = d_v) on random sizes and lengths.
    The kernel rounds the prologue's q, k and v to the storage dtype before
    the chunk stages, as stored inputs would be; the reference applies the
    same rounding (the unrounded comparison is logged).  Without it a call
    holding only a 2-token sequence from a zero state (case 4: q . k down to
    0.004) is off by 2.2e-2 from the rounding of its inputs alone."""
    import test_prologue_gpu as PR
    rng = np.random.default_rng(600 + seed)
    D = int(rng.choice([16 * i for i in range(1, 9)]))
    C = int(rng.choice([16, 32, 64]))
    H = int(rng.choice([1, 3, 33, 70]))
    n = int(rng.integers(1, 6))
    lengths = [int(x) for x in rng.integers(0, 200, size=n)]
    lengths[int(rng.integers(0, n))] = int(rng.integers(1, 200))
    dtype = "bf16" if rng.random() < 0.75 else "fp32"
    s0 = bool(rng.random() < 0.7)
    PR.check(PR.make_case(600 + seed, lengths, H, D, C, dtype, s0),
             "random case %d" % seed, rounded_ref=True)


@pytest.mark.parametrize("seed", range(12))
def test_random_state_pools(seed):
    """kda_prefill_varlen_indexed then kda_decode_step_indexed on random
    sizes, pool sizes, slot maps (with padding entries) and new requests,
    against the plain calls on gathered states and a scatter, bit for bit."""
    import torch
    from linear_recurrent_attention_kda_amd import kda
    rng = np.random.default_rng(1000 + seed)
    dims = [16 * i for i in range(1, 9)]
    Dk, Dv = int(rng.choice(dims)), int(rng.choice(dims))
    H = int(rng.choice([1, 3, 8, 70]))
    n = int(rng.integers(1, 7))
    lengths = [int(x) for x in rng.integers(0, 300, size=n)]
    C = int(rng.choice([16, 32, 64]))
    dtype = "bf16" if rng.random() < 0.75 else "fp32"
    slots = n + int(rng.integers(0, 6))
    idx = [int(x) for x in rng.permutation(slots)[:n]]
    for i in range(n):
        if rng.random() < 0.2:
            idx[i] = int(rng.choice([-1, slots, slots + 5]))
    has = [int(rng.random() < 0.7) for _ in range(n)]
    U.log("random pools %d: Dk=%d Dv=%d H=%d C=%d %s lengths=%s slots=%d "
          "idx=%s has=%s" % (seed, Dk, Dv, H, C, dtype, lengths, slots, idx,
                             has))
    p = inputs.make("varlen", seed=1100 + seed, H=H, K=Dk, V=Dv, C=C,
                    dtype=dtype, lengths=lengths)
    q, k, v = (U.to_dev(x, p.dtype) for x in (p.q, p.k, p.v))
    g, beta = U.f32_dev(p.g), U.f32_dev(p.beta)
    cu = torch.from_numpy(p.cu_seqlens).to(U.DEV)
    maxlen = max(1, max(lengths))
    pool = torch.from_numpy((rng.standard_normal((slots, H, Dk, Dv)) * 0.02)
                            .astype(np.float32)).to(U.DEV)
    sidx = torch.tensor(idx, dtype=torch.int32, device=U.DEV)
    valid = [i for i in range(n) if 0 <= idx[i] < slots]
    s0 = torch.zeros((n, H, Dk, Dv), dtype=torch.float32, device=U.DEV)
    for i in valid:
        if has[i]:
            s0[i] = pool[idx[i]]
    o_ref, fs = kda.kda_prefill_varlen(q, k, v, g, beta, cu, maxlen, s0,
                                       chunk_size=C)
    pool_ref = pool.clone()
    for i in valid:
        pool_ref[idx[i]] = fs[i]
    o = kda.kda_prefill_varlen_indexed(
        q, k, v, g, beta, cu, maxlen, pool, sidx,
        torch.tensor(has, dtype=torch.int32, device=U.DEV), chunk_size=C)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(pool, pool_ref)
    # a decode step for the same requests from the pool
    d = inputs.make("decode", seed=1200 + seed, B=n, H=H, K=Dk, V=Dv,
                    dtype=dtype)
    dq, dk, dv = (U.to_dev(x, d.dtype) for x in (d.q, d.k, d.v))
    dg, db = U.f32_dev(d.g), U.f32_dev(d.beta)
    st = torch.zeros((n, H, Dk, Dv), dtype=torch.float32, device=U.DEV)
    for i in valid:
        st[i] = pool[idx[i]]
    od_ref = kda.kda_decode_step(dq, dk, dv, dg, db, st)
    pool_ref = pool.clone()
    for i in valid:
        pool_ref[idx[i]] = st[i]
    od = kda.kda_decode_step_indexed(dq, dk, dv, dg, db, pool, sidx)
    torch.cuda.synchronize()
    assert torch.equal(od, od_ref) and torch.equal(pool, pool_ref)
