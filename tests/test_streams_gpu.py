"""The library keeps no state between calls: calls on two HIP streams that run
at the same time (each with its own workspace, outputs and state) give,
bit for bit, what the same calls give one after another on one stream."""
import pytest
import torch

import gpu_util as U
from conftest import gpu_available
from linear_recurrent_attention_kda_amd import inputs, kda

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def _prefill_dev(p):
    q, k, v = (U.to_dev(x, p.dtype) for x in (p.q, p.k, p.v))
    return q, k, v, U.f32_dev(p.g), U.f32_dev(p.beta), U.f32_dev(
        p.initial_state)


def test_two_streams_equal_one_stream():
    pa = inputs.make("prefill", seed=61, B=2, T=777, H=8, s0=True)
    pb = inputs.make("varlen", seed=62, H=8, lengths=[300, 0, 129, 1000])
    pd = inputs.make("decode", seed=63, B=16, H=8)
    U.log("two streams: prefill %s, varlen %s, decode B=%d"
          % (pa.q.shape, pb.seq_lengths.tolist(), pd.B))
    A = _prefill_dev(pa)
    Bv = _prefill_dev(pb)
    cu = torch.from_numpy(pb.cu_seqlens).to(U.DEV)
    maxlen = int(pb.seq_lengths.max())
    dq, dk, dv = (U.to_dev(x, pd.dtype) for x in (pd.q, pd.k, pd.v))
    dg, dbeta = U.f32_dev(pd.g), U.f32_dev(pd.beta)
    dstate0 = U.f32_dev(pd.initial_state)

    def run_a():
        return kda.kda_prefill_chunked(*A[:5], A[5], chunk_size=64)

    def run_b():
        return kda.kda_prefill_varlen(*Bv[:5], cu, maxlen, Bv[5],
                                      chunk_size=64)

    def run_d(state):
        return kda.kda_decode_step(dq, dk, dv, dg, dbeta, state)

    # one stream, one call after another
    oa, sa = run_a()
    ob, sb = run_b()
    st = dstate0.clone()
    od = run_d(st)
    torch.cuda.synchronize()

    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for rep in range(3):
        st2 = dstate0.clone()
        main = torch.cuda.current_stream()
        s1.wait_stream(main)
        s2.wait_stream(main)
        with torch.cuda.stream(s1):
            oa2, sa2 = run_a()
            od2 = run_d(st2)
        with torch.cuda.stream(s2):
            ob2, sb2 = run_b()
        torch.cuda.synchronize()
        assert torch.equal(oa, oa2) and torch.equal(sa, sa2), rep
        assert torch.equal(ob, ob2) and torch.equal(sb, sb2), rep
        assert torch.equal(od, od2) and torch.equal(st, st2), rep
    U.log("   3 concurrent repetitions equal the sequential results")


def test_graph_replay_equals_eager():
    """A prefill and a decode step captured in one HIP graph: every replay,
    with eager work and synchronisations between replays, gives the eager
    results bit for bit (the library issues kernel launches only, no
    memset or allocation, so it can be captured)."""
    pa = inputs.make("prefill", seed=64, B=1, T=1000, H=8, s0=True)
    pd = inputs.make("decode", seed=65, B=16, H=8)
    q, k, v, g, beta, s0 = _prefill_dev(pa)
    dq, dk, dv = (U.to_dev(x, pd.dtype) for x in (pd.q, pd.k, pd.v))
    dg, dbeta = U.f32_dev(pd.g), U.f32_dev(pd.beta)
    dstate0 = U.f32_dev(pd.initial_state)
    o = torch.empty_like(v)
    fs = torch.empty_like(s0)
    ws = kda.workspace_for(1, 1000, 8, 128, 128, 64, U.DEV)
    od = torch.empty_like(dv)
    state = dstate0.clone()

    def step():
        kda.kda_prefill_chunked(q, k, v, g, beta, s0, chunk_size=64, o=o,
                                final_state=fs, workspace=ws)
        kda.kda_decode_step(dq, dk, dv, dg, dbeta, state, o=od)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (o, fs, od, state)]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):       # warm-up on a side stream
        state.copy_(dstate0)
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    state.copy_(dstate0)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        o.zero_(); fs.zero_(); od.zero_()
        state.copy_(dstate0)             # the decode step updates in place
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for got, want in zip((o, fs, od, state), ref):
            assert torch.equal(got, want), rep
    U.log("   4 graph replays equal the eager step")
