"""GPU parity of the two prefill stages (kda_prefill_varlen_prep, then
kda_prefill_varlen_recur on the same stream): they must compute what
kda_prefill_varlen computes, bit for bit, and so agree with the fp64 oracle
within the prefill tolerance ("Kimi K3: The Manos, The Mythos, The
Legendos", section "FlashKDA algorithm": the chunk preparation and the
chunk recurrence are separate kernels)."""
import numpy as np
import pytest
import torch

import gpu_util as U
from conftest import gpu_available
from linear_recurrent_attention_kda_amd import inputs, kda

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def _split(q, k, v, g, beta, cu, maxlen, s0, C, scale=1.0):
    total, H, Dk = q.shape
    ws = kda.kda_prefill_varlen_prep(q, k, v, g, beta, cu, maxlen,
                                     chunk_size=C)
    return kda.kda_prefill_varlen_recur(ws, cu, maxlen, total, H, Dk,
                                        v.shape[-1], q.dtype, s0,
                                        chunk_size=C, scale=scale)


@pytest.mark.parametrize("D,C,dt", [(64, 32, "bf16"), (128, 64, "bf16"),
                                    (32, 16, "fp32")])
def test_stages_equal_fused_call(D, C, dt):
    p = inputs.make("varlen", seed=11, H=3, K=D, V=D, C=C, dtype=dt,
                    lengths=[70, 0, 33, 130, 1])
    U.log("stages D=%d C=%d %s lengths %s" % (D, C, dt, p.seq_lengths))
    q, k, v = (U.to_dev(x, p.dtype) for x in (p.q, p.k, p.v))
    g, beta = U.f32_dev(p.g), U.f32_dev(p.beta)
    s0 = U.f32_dev(p.initial_state)
    cu = torch.from_numpy(p.cu_seqlens).to(U.DEV)
    maxlen = int(p.seq_lengths.max())
    o1, s1 = kda.kda_prefill_varlen(q, k, v, g, beta, cu, maxlen, s0,
                                    chunk_size=C, scale=0.5)
    o2, s2 = _split(q, k, v, g, beta, cu, maxlen, s0, C, scale=0.5)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    assert torch.equal(s1, s2)
    # and against the oracle, to the prefill tolerance
    o_ref, s_ref = U.oracle.run_varlen(p.q, p.k, p.v, p.g, p.beta,
                                       p.cu_seqlens, p.initial_state,
                                       scale=0.5)
    eo = U.slice_rel(U.host(o2), o_ref, (1,))
    es = U.slice_rel(U.host(s2), s_ref, (0, 1))
    U.log("  o rel %.2e, state rel %.2e" % (eo, es))
    assert eo < U.PREFILL_TOL and es < U.PREFILL_TOL


def test_stages_at_the_benchmark_shape():
    """The 8192-token, 96-head prefill the benchmark times: the two stages
    (one packed sequence) equal kda_prefill_chunked bit for bit."""
    p = inputs.make("prefill", seed=0)
    U.log("stages at the benchmark shape: T=%d H=%d" % (p.T, p.H))
    q, k, v = (U.to_dev(x, p.dtype) for x in (p.q, p.k, p.v))
    g, beta = U.f32_dev(p.g), U.f32_dev(p.beta)
    o1, s1 = kda.kda_prefill_chunked(q, k, v, g, beta, None,
                                     chunk_size=p.C)
    total = p.B * p.T
    cu = torch.tensor([0, total], dtype=torch.int32, device=U.DEV)
    o2, s2 = _split(q.reshape(total, p.H, -1), k.reshape(total, p.H, -1),
                    v.reshape(total, p.H, -1), g.reshape(total, p.H, -1),
                    beta.reshape(total, p.H), cu, total, None, p.C)
    torch.cuda.synchronize()
    assert torch.equal(o1.reshape(o2.shape), o2)
    assert torch.equal(s1, s2)
    assert np.isfinite(U.host(s2)).all()
