"""Every entry point of the library in one captured HIP graph.

The entry points issue kernel launches only (no memset, allocation or
synchronising call), so a caller can capture them.  One graph holds: the
varlen prefill, its two stages as separate calls, checkpoints at an interval
and at listed positions, the gated prefill on both of its paths (fused into
the recurrence, and plain prefill then the epilogue), the prologue-fused
prefill, the standalone epilogue, the gated decode step, speculative verify,
commit and the fused step, the prefill that uses the library's own
scratch array, and the state-pool forms of prefill, decode, gated decode
and the speculative step.
Each replay, with eager resets and synchronisations between replays, must
give the eager calls' results bit for bit."""
import numpy as np
import pytest
import torch

import gpu_util as U
from conftest import gpu_available
from linear_recurrent_attention_kda_amd import inputs, kda

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def _dev_varlen(p):
    q, k, v = (U.to_dev(x, p.dtype) for x in (p.q, p.k, p.v))
    cu = torch.from_numpy(p.cu_seqlens).to(U.DEV)
    return dict(q=q, k=k, v=v, g=U.f32_dev(p.g), beta=U.f32_dev(p.beta),
                s0=U.f32_dev(p.initial_state), cu=cu,
                maxlen=int(p.seq_lengths.max()), N=len(p.seq_lengths),
                T=int(p.cu_seqlens[-1]), H=p.H, K=p.K, V=p.V, C=p.C)


def test_graph_of_every_entry_point():
    C = 64
    pv = inputs.make("varlen", seed=81, H=8, lengths=[300, 0, 129, 64])
    # 130 heads x 4 sequences = 520 pairs: the gated call fuses the epilogue
    pf = inputs.make("varlen", seed=82, H=130, lengths=[17, 64, 1, 40])
    pd = inputs.make("decode", seed=83, B=16, H=8)
    U.log("graph of every entry point: varlen %s, fused-gate H=%d %s, "
          "decode B=%d" % (pv.seq_lengths.tolist(), pf.H,
                           pf.seq_lengths.tolist(), pd.B))
    a, f = _dev_varlen(pv), _dev_varlen(pf)
    rng = np.random.default_rng(84)

    def zw(x):
        z = U.to_dev(rng.standard_normal((x["T"], x["H"], x["V"]))
                     .astype(np.float32), "bf16")
        w = U.f32_dev((0.5 + rng.random(x["V"])).astype(np.float32))
        return z, w
    za, wa = zw(a)
    zf, wf = zw(f)

    def ws(x):
        return kda.workspace_for(x["N"], x["T"], x["H"], x["K"], x["V"], C,
                                 U.DEV)

    def out(x):
        return torch.empty_like(x["v"])

    def fstate(x):
        return torch.empty((x["N"], x["H"], x["K"], x["V"]),
                           dtype=torch.float32, device=U.DEV)

    # outputs and workspaces, allocated once (a graph replays into them)
    bufs = {}
    for name, x in (("varlen", a), ("stages", a), ("ckpt", a),
                    ("ckpt_at", a), ("gated2", a), ("gated1", f),
                    ("noalloc", a)):
        bufs[name] = dict(o=out(x), fs=fstate(x), ws=ws(x))
    every = 2 * C
    bufs["ckpt"]["ck"] = torch.zeros((a["T"] // every, a["H"], a["K"],
                                      a["V"]), dtype=torch.float32,
                                     device=U.DEV)
    # checkpoint positions per sequence: [64, 300], [], [64, 129], [64]
    pos = torch.tensor([64, 300, 64, 129, 64], dtype=torch.int32,
                       device=U.DEV)
    cu_pos = torch.tensor([0, 2, 2, 4, 5], dtype=torch.int32, device=U.DEV)
    bufs["ckpt_at"]["ck"] = torch.zeros((5, a["H"], a["K"], a["V"]),
                                        dtype=torch.float32, device=U.DEV)
    # prologue inputs (d_k = d_v), on the varlen lengths
    D = a["K"]
    xq, xk, xv = (U.to_dev(rng.standard_normal((a["T"], a["H"], D))
                           .astype(np.float32), "bf16") for _ in range(3))
    conv_w = U.f32_dev((rng.standard_normal((3, a["H"], D, 4)) * 0.5)
                       .astype(np.float32))
    ga = U.f32_dev(rng.standard_normal((a["T"], a["H"], D))
                   .astype(np.float32))
    gb = U.f32_dev(rng.standard_normal((a["T"], a["H"])).astype(np.float32))
    bufs["prologue"] = dict(o=out(a), fs=fstate(a), ws=ws(a))
    # standalone epilogue on the varlen prefill's output
    y_epi = torch.empty_like(a["v"])
    # decode (gated) and speculative verify / commit from cached states
    dq, dk, dv = (U.to_dev(x, pd.dtype) for x in (pd.q, pd.k, pd.v))
    dg, dbeta = U.f32_dev(pd.g), U.f32_dev(pd.beta)
    dz = U.to_dev(rng.standard_normal((pd.B, pd.H, pd.V))
                  .astype(np.float32), "bf16")
    dw = U.f32_dev((0.5 + rng.random(pd.V)).astype(np.float32))
    dstate0 = U.f32_dev(pd.initial_state)
    dstate = dstate0.clone()
    y_dec = torch.empty_like(dv)
    Bs, Ts = 4, 6
    ps = inputs.make("varlen", seed=85, H=8, lengths=[Ts] * Bs)
    shp = lambda x: x.reshape((Bs, Ts) + x.shape[1:])  # noqa: E731
    sq, sk, sv = (U.to_dev(shp(x), ps.dtype) for x in (ps.q, ps.k, ps.v))
    sg, sbeta = U.f32_dev(shp(ps.g)), U.f32_dev(shp(ps.beta))
    sstate0 = U.f32_dev(ps.initial_state)
    sstate = sstate0.clone()
    so = torch.empty_like(sv)
    su = torch.empty(sv.shape, dtype=torch.float32, device=U.DEV)
    accepted = torch.tensor([0, 3, 6, 2], dtype=torch.int32, device=U.DEV)
    # the fused step commits that draft to its own copy of the states and
    # verifies the same tokens again
    sstate2 = sstate0.clone()
    so2, su2 = torch.empty_like(so), torch.empty_like(su)
    # state pools: the varlen sequences and the decode batch in pool rows
    pv_pool0 = torch.randn((6, a["H"], a["K"], a["V"]), device=U.DEV) * 0.02
    pv_pool = pv_pool0.clone()
    pv_idx = torch.tensor([4, 0, -1, 2], dtype=torch.int32, device=U.DEV)
    pv_has = torch.tensor([1, 0, 1, 1], dtype=torch.int32, device=U.DEV)
    pv_o = out(a)
    pv_ws = ws(a)
    dpool0 = torch.randn((20,) + tuple(dstate0.shape[1:]),
                         device=U.DEV) * 0.02
    dpool = dpool0.clone()
    didx = torch.tensor([(3 * b + 1) % 20 for b in range(pd.B)],
                        dtype=torch.int32, device=U.DEV)
    od_idx = torch.empty_like(dv)
    yd_idx = torch.empty_like(dv)
    spool0 = torch.randn((9,) + tuple(sstate0.shape[1:]), device=U.DEV) * 0.02
    spool = spool0.clone()
    sidx = torch.tensor([7, -1, 2, 4], dtype=torch.int32, device=U.DEV)
    so3, su3 = torch.empty_like(so), torch.empty_like(su)

    def varlen_args(x):
        return (x["q"], x["k"], x["v"], x["g"], x["beta"], x["cu"],
                x["maxlen"], x["s0"])

    def step():
        b = bufs["varlen"]
        kda.kda_prefill_varlen(*varlen_args(a), chunk_size=C, o=b["o"],
                               final_state=b["fs"], workspace=b["ws"])
        b = bufs["stages"]
        kda.kda_prefill_varlen_prep(a["q"], a["k"], a["v"], a["g"],
                                    a["beta"], a["cu"], a["maxlen"],
                                    chunk_size=C, workspace=b["ws"])
        kda.kda_prefill_varlen_recur(b["ws"], a["cu"], a["maxlen"], a["T"],
                                     a["H"], a["K"], a["V"], a["q"].dtype,
                                     a["s0"], chunk_size=C,
                                     final_state=b["fs"], o=b["o"])
        b = bufs["ckpt"]
        kda.kda_prefill_varlen_ckpt(*varlen_args(a), ckpt_every=every,
                                    chunk_size=C, o=b["o"],
                                    final_state=b["fs"], ckpt_states=b["ck"],
                                    workspace=b["ws"])
        b = bufs["ckpt_at"]
        kda.kda_prefill_varlen_ckpt_at(*varlen_args(a), ckpt_pos=pos,
                                       cu_ckpt=cu_pos, chunk_size=C,
                                       o=b["o"], final_state=b["fs"],
                                       ckpt_states=b["ck"],
                                       workspace=b["ws"])
        b = bufs["gated2"]          # 32 pairs: plain prefill, then epilogue
        kda.kda_prefill_varlen_gated(*varlen_args(a), z=za, w=wa,
                                     chunk_size=C, y=b["o"],
                                     final_state=b["fs"], workspace=b["ws"])
        b = bufs["gated1"]          # 520 pairs: fused into the recurrence
        kda.kda_prefill_varlen_gated(*varlen_args(f), z=zf, w=wf,
                                     chunk_size=C, y=b["o"],
                                     final_state=b["fs"], workspace=b["ws"])
        b = bufs["prologue"]
        kda.kda_prefill_varlen_prologue(xq, xk, xv, conv_w, ga, gb, a["cu"],
                                        a["maxlen"], a["s0"], chunk_size=C,
                                        o=b["o"], final_state=b["fs"],
                                        workspace=b["ws"])
        kda.kda_output_norm_gate(bufs["varlen"]["o"], za, wa, y=y_epi)
        kda.kda_decode_step_gated(dq, dk, dv, dg, dbeta, dstate, dz, dw,
                                  y=y_dec)
        kda.kda_spec_verify(sq, sk, sv, sg, sbeta, sstate, o=so, u=su)
        kda.kda_spec_commit(sk, sg, su, accepted, sstate)
        kda.kda_spec_step(sq, sk, sv, sg, sbeta, sstate2, k_prev=sk,
                          g_prev=sg, u_prev=su, accepted_prev=accepted,
                          o=so2, u=su2)
        b = bufs["noalloc"]
        kda.kda_prefill_varlen_noalloc(*varlen_args(a), chunk_size=C,
                                       o=b["o"], final_state=b["fs"])
        kda.kda_prefill_varlen_indexed(a["q"], a["k"], a["v"], a["g"],
                                       a["beta"], a["cu"], a["maxlen"],
                                       pv_pool, pv_idx, pv_has, chunk_size=C,
                                       o=pv_o, workspace=pv_ws)
        kda.kda_decode_step_indexed(dq, dk, dv, dg, dbeta, dpool, didx,
                                    o=od_idx)
        kda.kda_decode_step_gated_indexed(dq, dk, dv, dg, dbeta, dpool, didx,
                                          dz, dw, y=yd_idx)
        kda.kda_spec_step_indexed(sq, sk, sv, sg, sbeta, spool, sidx,
                                  k_prev=sk, g_prev=sg, u_prev=su,
                                  accepted_prev=accepted, o=so3, u=su3)

    results = [b[key] for b in bufs.values() for key in ("o", "fs", "ck")
               if key in b] + [y_epi, y_dec, dstate, so, su, sstate, so2,
                               su2, sstate2, pv_o, pv_pool, dpool, od_idx,
                               yd_idx, spool, so3, su3]

    def reset():
        for t in results:
            t.zero_()
        dstate.copy_(dstate0)        # updated in place by each step
        sstate.copy_(sstate0)
        sstate2.copy_(sstate0)
        pv_pool.copy_(pv_pool0)
        dpool.copy_(dpool0)
        spool.copy_(spool0)

    reset()
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in results]
    # the stages equal the fused call; the eager step is deterministic
    assert torch.equal(bufs["stages"]["o"], bufs["varlen"]["o"])
    assert torch.equal(bufs["noalloc"]["o"], bufs["varlen"]["o"])
    # the step's commit equals the separate commit
    assert torch.equal(sstate2, sstate)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):    # warm-up on a side stream
        reset()
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    reset()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        reset()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (got, want) in enumerate(zip(results, ref)):
            assert torch.equal(got, want), (rep, i)
    U.log("   4 replays of %d results equal the eager calls" % len(results))
