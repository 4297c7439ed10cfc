"""GPU parity at every supported head-dim shape: d_k and d_v any multiples
of 16 up to 128, independently ("Two Paths: Kimi K3 vs DeepSeek V4
Architecture Divergence", section "Attention": a d_k x d_v state per head).

The kernels run on the smallest 16 / 32 / 64 / 128 tile that holds both
dims, with the channels past them zero inside the kernels; every entry point
is compared with the fp64 oracle on such shapes.  The prefill cases include
64-wide d_v slices that the stored d_v only partly covers, and slices past
it (which do no work), on the streamed and register-prefetch recurrences."""
import numpy as np
import pytest
import torch

import oracle
from conftest import gpu_available
from linear_recurrent_attention_kda_amd import inputs, kda

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

import gpu_util as U  # noqa: E402

SHAPES = [(64, 128), (128, 64), (48, 48), (80, 112), (16, 128), (112, 32),
          (96, 96), (128, 80), (96, 48)]


@pytest.mark.parametrize("Dk,Dv", SHAPES)
@pytest.mark.parametrize("H", [3, 100])
def test_prefill_varlen_dims(Dk, Dv, H):
    """3 heads: 16-wide slices.  100 heads: 64-wide slices (streamed at
    C = 64), which at d_v = 80 or 48 are partly or wholly padding."""
    p = inputs.make("varlen", seed=Dk + 3 * Dv + H, H=H, K=Dk, V=Dv,
                    lengths=[150, 0, 1, 64, 129])
    U.check_prefill(p, label="Dk%d Dv%d H%d" % (Dk, Dv, H), head_group=50)


@pytest.mark.parametrize("Dk,Dv,C", [(64, 128, 32), (48, 80, 16),
                                     (112, 16, 64)])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_prefill_chunked_dims(Dk, Dv, C, dtype):
    p = inputs.make("prefill", seed=Dk + Dv + C, B=2, T=203, H=3, K=Dk, V=Dv,
                    C=C, s0=True, dtype=dtype)
    U.check_prefill(p, label="chunked Dk%d Dv%d C%d %s" % (Dk, Dv, C, dtype))


@pytest.mark.parametrize("Dk,Dv,H", [(64, 128, 96), (96, 48, 3)])
def test_ckpt_at_dims(Dk, Dv, H):
    """Checkpoint stores of a d_k x d_v state (streamed kernel at 96 heads)."""
    import test_ckpt_gpu as CK
    p = inputs.make("varlen", seed=90 + H, H=H, K=Dk, V=Dv,
                    lengths=[200, 64, 0, 130])
    n = CK.check_ckpt_at(p, [[64, 128, 200], [64], [], [64, 130]],
                         label="Dk%d Dv%d" % (Dk, Dv), head_group=48)
    assert n == 6


@pytest.mark.parametrize("Dk,Dv,H", [(64, 80, 3), (128, 80, 110),
                                     (48, 112, 110)])
def test_gated_prefill_dims(Dk, Dv, H):
    """The output norm's mean runs over the stored d_v channels: the
    two-pass path (3 heads) and the fused one (5 x 110 pairs)."""
    import test_prefill_gated_gpu as G
    p = inputs.make("varlen", seed=95 + H, H=H, K=Dk, V=Dv,
                    lengths=[70, 0, 1, 192, 145])
    assert G.fused_expected(p) == (H == 110)
    G.check_gated(p, 3, "Dk%d Dv%d" % (Dk, Dv), head_group=55)


@pytest.mark.parametrize("Dk,Dv", SHAPES)
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_decode_dims(Dk, Dv, dtype):
    U.check_decode(inputs.make("decode", seed=Dk + Dv, B=3, H=5, K=Dk, V=Dv,
                               dtype=dtype))


@pytest.mark.parametrize("Dk,Dv", [(64, 128), (48, 80), (128, 32)])
def test_decode_gated_dims(Dk, Dv):
    p = inputs.make("decode", seed=7, B=3, H=4, K=Dk, V=Dv)
    rng = np.random.default_rng(8)
    z = inputs.bf16_round(rng.standard_normal((3, 4, Dv)).astype(np.float32))
    w = (0.5 + rng.random(Dv)).astype(np.float32)
    q, k, v = (U.to_dev(x, p.dtype) for x in (p.q, p.k, p.v))
    state = U.f32_dev(p.initial_state)
    y = kda.kda_decode_step_gated(q, k, v, U.f32_dev(p.g), U.f32_dev(p.beta),
                                  state, U.to_dev(z, "bf16"), U.f32_dev(w),
                                  eps=1e-6)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.run_decode(p.q, p.k, p.v, p.g, p.beta,
                                     p.initial_state)
    y_ref = oracle.norm_gate(o_ref, z, w, 1e-6)
    ey = U.slice_rel(U.host(y), y_ref, (0, 1))
    es = U.slice_rel(U.host(state), s_ref, (0, 1))
    U.log("decode gated Dk%d Dv%d: y %.3e state %.3e" % (Dk, Dv, ey, es))
    assert ey <= 2e-2 and es <= U.DECODE_STATE_TOL


@pytest.mark.parametrize("Dk,Dv", [(64, 128), (96, 48), (16, 112)])
def test_spec_dims(Dk, Dv):
    """Draft verify of T = 5 tokens and commit of 0, 2 and 5 of them."""
    B, T, H = 3, 5, 4
    p = inputs.make("varlen", seed=Dk * Dv, H=H, K=Dk, V=Dv, lengths=[T] * B)
    shp = lambda x: x.reshape((B, T) + x.shape[1:])  # noqa: E731
    q, k, v = (U.to_dev(shp(x), p.dtype) for x in (p.q, p.k, p.v))
    g, beta = U.f32_dev(shp(p.g)), U.f32_dev(shp(p.beta))
    state = U.f32_dev(p.initial_state)
    o, u = kda.kda_spec_verify(q, k, v, g, beta, state)
    accepted = [0, 2, 5]
    kda.kda_spec_commit(k, g, u, torch.tensor(accepted, dtype=torch.int32,
                                              device=U.DEV), state)
    torch.cuda.synchronize()
    o_ref, _ = oracle.run_varlen(p.q, p.k, p.v, p.g, p.beta, p.cu_seqlens,
                                 p.initial_state)
    eo = U.slice_rel(U.host(o).reshape(B * T, H, Dv), o_ref, (1,))
    s_ref = np.array(p.initial_state, np.float64)
    for b, a in enumerate(accepted):
        if a:
            lo = b * T
            _, s = oracle.run_varlen(p.q[lo:lo + a], p.k[lo:lo + a],
                                     p.v[lo:lo + a], p.g[lo:lo + a],
                                     p.beta[lo:lo + a], np.array([0, a]),
                                     p.initial_state[b:b + 1],
                                     want_output=False)
            s_ref[b] = s[0]
    es = U.slice_rel(U.host(state), s_ref, (0, 1))
    U.log("spec Dk%d Dv%d: o %.3e state %.3e" % (Dk, Dv, eo, es))
    assert eo <= U.DECODE_O_TOL["bf16"] and es <= U.DECODE_STATE_TOL


@pytest.mark.parametrize("Dv", [16, 48, 80, 112])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_epilogue_dims(Dv, dtype):
    rng = np.random.default_rng(Dv)
    T, H = 37, 3
    rnd = (inputs.bf16_round if dtype == "bf16" else
           (lambda x: x))
    o = rnd(rng.standard_normal((T, H, Dv)).astype(np.float32))
    z = rnd(rng.standard_normal((T, H, Dv)).astype(np.float32))
    w = rng.standard_normal(Dv).astype(np.float32)
    y = kda.kda_output_norm_gate(U.to_dev(o, dtype), U.to_dev(z, dtype),
                                 U.f32_dev(w), eps=1e-5)
    torch.cuda.synchronize()
    err = U.slice_rel(U.host(y), oracle.norm_gate(o, z, w, 1e-5), (0, 1))
    U.log("norm_gate Dv%d %s: %.3e" % (Dv, dtype, err))
    assert err <= (2e-2 if dtype == "bf16" else 1e-4)


@pytest.mark.parametrize("D,C", [(48, 64), (80, 32), (112, 16)])
def test_prologue_dims(D, C):
    import test_prologue_gpu as PR
    PR.check(PR.make_case(D + C, [1, 2, 70, 0, 130], 3, D, C),
             "D%d" % D)
