"""GPU parity of kda_prefill_varlen_prologue: the input prologue (causal
short convolution, q/k L2 norm, g = -5 sigmoid(a), beta = sigmoid(b);
"Kimi K3: The Manos, The Mythos, The Legendos", section "Kimi Linear")
fused into the chunk-prep kernel, against the fp64 prologue oracle followed
by the fp64 recurrence oracle on the same values."""
import numpy as np
import pytest
import torch

import oracle
from conftest import gpu_available
from linear_recurrent_attention_kda_amd import inputs, kda

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

import gpu_util as U  # noqa: E402


def make_case(seed, lengths, H, D, C, dtype="bf16", s0=True):
    rng = np.random.default_rng(seed)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T = int(cu[-1])
    rnd = lambda x: (inputs.bf16_round(x.astype(np.float32))  # noqa: E731
                     if dtype == "bf16" else x.astype(np.float32))
    xq, xk, xv = (rnd(rng.standard_normal((T, H, D))) for _ in range(3))
    w = (rng.standard_normal((3, H, D, 4)) * 0.5).astype(np.float32)
    a = rng.standard_normal((T, H, D)).astype(np.float32)
    b = rng.standard_normal((T, H)).astype(np.float32)
    S0 = (rng.standard_normal((len(lengths), H, D, D)) * 0.02).astype(
        np.float32) if s0 else None
    return dict(xq=xq, xk=xk, xv=xv, w=w, a=a, b=b, cu=cu, S0=S0, H=H, D=D,
                C=C, dtype=dtype, lengths=list(lengths))


def check(c, label, rounded_ref=False):
    """GPU prologue-fused prefill against the oracle prologue followed by the
    oracle recurrence.  With rounded_ref, the prologue's q, k and v are first
    rounded to the storage dtype, as the kernel rounds them before the chunk
    stages (the reference then differs from the kernel by the kernels'
    arithmetic only; the unrounded comparison is logged beside it)."""
    U.log("prologue", label, "H=%d D=%d C=%d %s lengths=%s"
          % (c["H"], c["D"], c["C"], c["dtype"], c["lengths"]))
    dev = lambda x: U.to_dev(x, c["dtype"])  # noqa: E731
    cu = torch.from_numpy(c["cu"]).to(U.DEV)
    o, s = kda.kda_prefill_varlen_prologue(
        dev(c["xq"]), dev(c["xk"]), dev(c["xv"]), U.f32_dev(c["w"]),
        U.f32_dev(c["a"]), U.f32_dev(c["b"]), cu, max(c["lengths"]),
        U.f32_dev(c["S0"]), chunk_size=c["C"])
    torch.cuda.synchronize()
    q, k, v, g, beta = oracle.prologue.prologue(
        c["xq"], c["xk"], c["xv"], c["w"], c["a"], c["b"], c["cu"])
    o_ref, s_ref = oracle.run_varlen(q, k, v, g, beta, c["cu"], c["S0"])
    eo = max(U.prefill_o_rel(U.host(o), o_ref, c["cu"], c["C"]))
    es = U.slice_rel(U.host(s), s_ref, (0, 1))
    U.log("   o rel err %.3e   final state rel err %.3e" % (eo, es))
    if rounded_ref and c["dtype"] == "bf16":
        rnd = lambda x: inputs.bf16_round(  # noqa: E731
            np.asarray(x, np.float32)).astype(np.float64)
        o_ref, s_ref = oracle.run_varlen(rnd(q), rnd(k), rnd(v), g, beta,
                                         c["cu"], c["S0"])
        eo = max(U.prefill_o_rel(U.host(o), o_ref, c["cu"], c["C"]))
        es = U.slice_rel(U.host(s), s_ref, (0, 1))
        U.log("   against q, k, v rounded to bf16 as stored: o rel err "
              "%.3e   final state rel err %.3e" % (eo, es))
    assert eo <= U.PREFILL_TOL and es <= U.PREFILL_TOL


@pytest.mark.parametrize("D,C", [(128, 64), (64, 32), (32, 16), (16, 16)])
def test_prologue_ragged(D, C):
    check(make_case(D + C, [1, 2, 3, 70, 0, 130, C + 3], 3, D, C),
          "ragged")


def test_prologue_fp32_zero_state():
    check(make_case(5, [64, 100, 17], 2, 64, 64, dtype="fp32", s0=False),
          "fp32")


def test_prologue_equals_unfused_path():
    """The fused path equals kda_prefill_varlen on the prologue's results
    computed on the host (rounded to bf16 as the fused kernel rounds them)."""
    c = make_case(9, [200, 45, 128], 4, 128, 64)
    q, k, v, g, beta = oracle.prologue.prologue(
        c["xq"], c["xk"], c["xv"], c["w"], c["a"], c["b"], c["cu"])
    dev = lambda x: U.to_dev(inputs.bf16_round(  # noqa: E731
        np.asarray(x, np.float32)), "bf16")
    cu = torch.from_numpy(c["cu"]).to(U.DEV)
    o1, s1 = kda.kda_prefill_varlen(
        dev(q), dev(k), dev(v), U.f32_dev(g.astype(np.float32)),
        U.f32_dev(beta.astype(np.float32)), cu, 200, U.f32_dev(c["S0"]))
    o2, s2 = kda.kda_prefill_varlen_prologue(
        U.to_dev(c["xq"], "bf16"), U.to_dev(c["xk"], "bf16"),
        U.to_dev(c["xv"], "bf16"), U.f32_dev(c["w"]), U.f32_dev(c["a"]),
        U.f32_dev(c["b"]), cu, 200, U.f32_dev(c["S0"]))
    torch.cuda.synchronize()
    eo = max(U.prefill_o_rel(U.host(o2), U.host(o1), c["cu"], c["C"]))
    es = U.slice_rel(U.host(s2), U.host(s1), (0, 1))
    U.log("   fused vs unfused: o %.3e state %.3e" % (eo, es))
    assert eo <= 1e-2 and es <= 1e-2
