"""GPU parity of kda_decode_step against the fp64 oracle (through the C ABI).

The full decode workload (64 sequences x 96 heads, d = 128, fp32 state
~N(0, 0.02^2), bf16 q/k/v) is checked completely, element by element; the
oracle finishes it in about a second."""
import numpy as np
import pytest
import torch

from conftest import gpu_available
from linear_recurrent_attention_kda_amd import inputs, kda

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

import gpu_util as U  # noqa: E402


def test_decode_full_workload():
    U.check_decode(inputs.make("decode", seed=0))


@pytest.mark.parametrize("D", [16, 32, 64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_decode_head_dims(D, dtype):
    U.check_decode(inputs.make("decode", seed=D, B=3, H=5, K=D, V=D,
                               dtype=dtype))


@pytest.mark.parametrize("case", ["g_min", "g_zero", "beta0", "beta1"])
def test_decode_edge_values(case):
    kw = dict(g_min=dict(g_const=-5.0), g_zero=dict(g_const=0.0),
              beta0=dict(beta_const=0.0), beta1=dict(beta_const=1.0))[case]
    U.check_decode(inputs.make("decode", seed=11, B=4, H=6, **kw))


def test_decode_scale_and_single_head():
    U.check_decode(inputs.make("decode", seed=3, B=1, H=1), scale=0.0883883)


def test_decode_repeated_steps_match_prefill_tokens():
    """Ten decode steps from a state equal a ten-token append-prefill from
    the same state (both against the oracle, and to each other)."""
    p = inputs.make("prefill", seed=5, B=2, T=10, H=3, K=64, V=64, s0=True)
    state = U.f32_dev(p.initial_state)
    outs = []
    for t in range(p.T):
        o = kda.kda_decode_step(U.to_dev(p.q[:, t], p.dtype),
                                U.to_dev(p.k[:, t], p.dtype),
                                U.to_dev(p.v[:, t], p.dtype),
                                U.f32_dev(p.g[:, t]), U.f32_dev(p.beta[:, t]),
                                state)
        outs.append(U.host(o))
    torch.cuda.synchronize()
    o_dec = np.stack(outs, axis=1)
    o_ref, s_ref = U.run_oracle(p)
    assert U.slice_rel(o_dec, o_ref, (0, 2)) < 2e-2
    assert U.slice_rel(U.host(state), s_ref, (0, 1)) < 1e-4


def test_decode_deterministic():
    p = inputs.make("decode", seed=9, B=8, H=16)
    res = []
    for _ in range(2):
        st = U.f32_dev(p.initial_state)
        o = kda.kda_decode_step(U.to_dev(p.q, p.dtype), U.to_dev(p.k, p.dtype),
                                U.to_dev(p.v, p.dtype), U.f32_dev(p.g),
                                U.f32_dev(p.beta), st)
        torch.cuda.synchronize()
        res.append((o.cpu(), st.cpu()))
    assert torch.equal(res[0][0], res[1][0])
    assert torch.equal(res[0][1], res[1][1])
