"""GPU parity of the output epilogue (per-head RMS norm and sigmoid output
gate; "Kimi K3: The Manos, The Mythos, The Legendos", section "Kimi
Linear"): the standalone kda_output_norm_gate against the fp64 epilogue
oracle on the same values, and kda_decode_step_gated against the oracle's
decode step followed by the same epilogue."""
import numpy as np
import pytest
import torch

import oracle
from conftest import gpu_available
from linear_recurrent_attention_kda_amd import inputs, kda

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

import gpu_util as U  # noqa: E402

TOL = {"bf16": 2e-2, "fp32": 1e-4}


def _round(x, dtype):
    x = np.asarray(x, np.float32)
    return inputs.bf16_round(x) if dtype == "bf16" else x


@pytest.mark.parametrize("D", [16, 32, 64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_norm_gate(D, dtype):
    rng = np.random.default_rng(D)
    T, H = 77, 5                               # rows not a multiple of a block
    o = _round(rng.standard_normal((T, H, D)) * np.exp(rng.standard_normal(
        (T, H, 1))), dtype)
    z = _round(rng.standard_normal((T, H, D)) * 3, dtype)
    w = rng.standard_normal(D).astype(np.float32)
    eps = 1e-5
    y = kda.kda_output_norm_gate(U.to_dev(o, dtype), U.to_dev(z, dtype),
                                 U.f32_dev(w), eps=eps)
    torch.cuda.synchronize()
    ref = oracle.norm_gate(o, z, w, eps)
    err = U.slice_rel(U.host(y), ref, (0, 1))
    U.log("norm_gate D=%d %s rel err %.3e" % (D, dtype, err))
    assert err <= TOL[dtype]


def test_norm_gate_in_place_and_zero_rows():
    rng = np.random.default_rng(3)
    o = _round(rng.standard_normal((40, 3, 128)), "bf16")
    o[5, 1] = 0.0                              # an all-zero row: y = 0
    z = _round(rng.standard_normal((40, 3, 128)), "bf16")
    w = rng.standard_normal(128).astype(np.float32)
    od = U.to_dev(o, "bf16")
    y = kda.kda_output_norm_gate(od, U.to_dev(z, "bf16"), U.f32_dev(w),
                                 eps=1e-6, y=od)
    torch.cuda.synchronize()
    assert y.data_ptr() == od.data_ptr()
    ref = oracle.norm_gate(o, z, w, 1e-6)
    assert U.slice_rel(U.host(y), ref, (0, 1)) <= TOL["bf16"]
    assert not np.any(U.host(y)[5, 1])


@pytest.mark.parametrize("D,dtype", [(128, "bf16"), (64, "fp32"),
                                     (16, "bf16")])
def test_decode_step_gated(D, dtype):
    p = inputs.make("decode", seed=D + 1, B=6, H=7, K=D, V=D, dtype=dtype)
    rng = np.random.default_rng(D + 2)
    z = _round(rng.standard_normal((p.B, p.H, D)), dtype)
    w = rng.standard_normal(D).astype(np.float32)
    state = U.f32_dev(p.initial_state)
    y = kda.kda_decode_step_gated(
        U.to_dev(p.q, dtype), U.to_dev(p.k, dtype), U.to_dev(p.v, dtype),
        U.f32_dev(p.g), U.f32_dev(p.beta), state, U.to_dev(z, dtype),
        U.f32_dev(w), eps=1e-6)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.run_decode(p.q, p.k, p.v, p.g, p.beta,
                                     p.initial_state)
    y_ref = oracle.norm_gate(o_ref, z, w, 1e-6)
    ey = U.slice_rel(U.host(y), y_ref, (0, 1))
    es = U.slice_rel(U.host(state), s_ref, (0, 1))
    U.log("decode gated D=%d %s: y %.3e state %.3e" % (D, dtype, ey, es))
    assert es <= U.DECODE_STATE_TOL
    assert ey <= TOL[dtype]


def test_decode_gated_full_batch_matches_two_passes():
    """Decode workload shape: the fused epilogue equals decode followed by
    the standalone epilogue (to bf16 rounding), and the state is the same
    bit for bit."""
    p = inputs.make("decode", seed=9)
    rng = np.random.default_rng(9)
    z = U.to_dev(_round(rng.standard_normal((p.B, p.H, p.V)), "bf16"), "bf16")
    w = U.f32_dev(rng.standard_normal(p.V).astype(np.float32))
    q, k, v = (U.to_dev(x, "bf16") for x in (p.q, p.k, p.v))
    g, beta = U.f32_dev(p.g), U.f32_dev(p.beta)
    s1 = U.f32_dev(p.initial_state)
    s2 = s1.clone()
    y1 = kda.kda_decode_step_gated(q, k, v, g, beta, s1, z, w, eps=1e-6)
    o2 = kda.kda_decode_step(q, k, v, g, beta, s2)
    y2 = kda.kda_output_norm_gate(o2, z, w, eps=1e-6)
    torch.cuda.synchronize()
    assert torch.equal(s1, s2)
    # y1 normalises the fp32 output, y2 its bf16 rounding
    assert U.slice_rel(U.host(y1), U.host(y2), (0, 1)) <= 2e-2
