"""GPU test of kda_prefill_varlen_noalloc, the prefill entry point that
allocates nothing (its workspace is the library's fixed device scratch
array): through the C ABI, two calls in a row, the second with a smaller
input, each equal bit for bit to kda_prefill_varlen on the same inputs and
within the prefill tolerance of the fp64 oracle.  Also the clear error for
a problem beyond the scratch array's size."""
import numpy as np
import pytest
import torch

from conftest import gpu_available
from linear_recurrent_attention_kda_amd import inputs, kda

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

import gpu_util as U  # noqa: E402


def _run_both(p):
    q, k, v = (U.to_dev(x, p.dtype) for x in (p.q, p.k, p.v))
    g, beta = U.f32_dev(p.g), U.f32_dev(p.beta)
    s0 = U.f32_dev(p.initial_state)
    cu = torch.from_numpy(p.cu_seqlens.astype(np.int32)).to(U.DEV)
    maxlen = int(p.seq_lengths.max(initial=0))
    o = torch.empty((p.tokens, p.H, p.V), dtype=q.dtype, device=U.DEV)
    fs = torch.empty((p.N, p.H, p.K, p.V), dtype=torch.float32, device=U.DEV)
    kda.kda_prefill_varlen_noalloc(q, k, v, g, beta, cu, maxlen, s0,
                                   chunk_size=p.C, final_state=fs, o=o)
    o2, s2 = kda.kda_prefill_varlen(q, k, v, g, beta, cu, maxlen, s0,
                                    chunk_size=p.C)
    torch.cuda.synchronize()
    return o, fs, o2, s2


def test_noalloc_matches_varlen_twice_shrinking():
    big = inputs.make("varlen", seed=61, H=24, lengths=[700, 0, 1, 333, 640])
    small = inputs.make("varlen", seed=62, H=8, K=64, V=64, C=32,
                        lengths=[45, 100])
    need = kda.kda_prefill_workspace_size(big.N, big.tokens, big.H, big.K,
                                          big.V, big.C)
    assert need <= kda.KDA_NOALLOC_SCRATCH_BYTES
    for p in (big, small):
        U.log("noalloc", "H=%d D=%d C=%d lengths=%s"
              % (p.H, p.K, p.C, p.seq_lengths.tolist()))
        o, fs, o2, s2 = _run_both(p)
        assert torch.equal(o, o2) and torch.equal(fs, s2)
        o_ref, s_ref = U.run_oracle(p)
        eo = max(U.prefill_o_rel(U.host(o), o_ref, p.cu_seqlens, p.C))
        es = U.slice_rel(U.host(fs), s_ref, (0, 1))
        U.log("   o rel err %.3e   final state rel err %.3e" % (eo, es))
        assert eo <= U.PREFILL_TOL and es <= U.PREFILL_TOL


def test_noalloc_rejects_problems_beyond_the_scratch():
    """96 heads x 8192 tokens need 912 MB of workspace: KDA_ERR_SCRATCH."""
    H, T, D = 96, 8192, 128
    need = kda.kda_prefill_workspace_size(1, T, H, D, D, 64)
    assert need > kda.KDA_NOALLOC_SCRATCH_BYTES
    x = torch.zeros((T, H, D), dtype=torch.bfloat16, device=U.DEV)
    g = torch.zeros((T, H, D), dtype=torch.float32, device=U.DEV)
    b = torch.zeros((T, H), dtype=torch.float32, device=U.DEV)
    cu = torch.tensor([0, T], dtype=torch.int32, device=U.DEV)
    o = torch.empty_like(x)
    with pytest.raises(kda.KDAError) as e:
        kda.kda_prefill_varlen_noalloc(x, x, x, g, b, cu, T, o=o)
    assert e.value.status == kda.KDA_ERR_SCRATCH
