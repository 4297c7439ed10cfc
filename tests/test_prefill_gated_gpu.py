"""GPU parity of kda_prefill_varlen_gated: the output epilogue (per-head RMS
norm and sigmoid output gate; "Kimi K3: The Manos, The Mythos, The
Legendos", section "Kimi Linear") fused into the chunk-recurrence kernel.

Two measures, because the epilogue rescales every (token, head) row to unit
RMS: a row whose outputs are small (a sequence's first token from a small
state) has its error amplified by the ratio of the slice's largest output to
the row's RMS, which is the inputs' conditioning, not the kernel's.
  (a) the epilogue's arithmetic, row by row: y against the fp64 epilogue
      oracle applied to the GPU's own outputs of the plain prefill (the
      state recurrence is the same kernel family, bit for bit): 1e-2 per row
      in bf16 (the fused kernel normalises the fp32 outputs, the plain path
      rounds them to bf16 first; y itself is rounded to bf16), 1e-4 in fp32;
  (b) end to end against the fp64 oracle: the outputs recovered from y
      through the row's gate and norm, y * rms(o) / (w sigmoid(z)) with the
      row norms of the plain prefill's outputs (themselves within the
      prefill bar of the oracle), measured like a prefill output (per
      (sequence, head) for sequences of at least one chunk, per head for
      shorter ones) against the oracle's outputs and the prefill bar.
"""
import numpy as np
import pytest
import torch

import oracle
from conftest import gpu_available
from linear_recurrent_attention_kda_amd import inputs, kda

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

import gpu_util as U  # noqa: E402

EPS = 1e-6


def gate_inputs(p, seed):
    """Gate pre-activations ~ N(0, 1) in the storage dtype, and weights
    uniform in [0.5, 1.5] (kept away from 0 so that measure (b) can divide
    by them)."""
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((p.tokens, p.H, p.V)).astype(np.float32)
    if p.dtype == "bf16":
        z = inputs.bf16_round(z)
    w = (0.5 + rng.random(p.V)).astype(np.float32)
    return z, w


def row_rel(x, ref):
    """Largest per-row relative error over (token, head) rows."""
    num = np.max(np.abs(x - ref), axis=-1)
    den = np.maximum(np.max(np.abs(ref), axis=-1), 1e-30)
    return float(np.max(num / den)) if num.size else 0.0


def run_gated(p, z, w):
    q, k, v = (U.to_dev(x, p.dtype) for x in (p.q, p.k, p.v))
    g, beta = U.f32_dev(p.g), U.f32_dev(p.beta)
    s0 = U.f32_dev(p.initial_state)
    cu = torch.from_numpy(np.asarray(U.seq_bounds(p), np.int32)).to(U.DEV)
    maxlen = int(p.seq_lengths.max(initial=0))
    flat = lambda x: x.reshape(p.tokens, p.H, -1)  # noqa: E731
    fq, fk, fv, fg = flat(q), flat(k), flat(v), flat(g)
    fb = beta.reshape(p.tokens, p.H)
    y, s = kda.kda_prefill_varlen_gated(
        fq, fk, fv, fg, fb, cu, maxlen, s0, z=U.to_dev(z, p.dtype),
        w=U.f32_dev(w), eps=EPS, chunk_size=p.C)
    o2, s2 = kda.kda_prefill_varlen(fq, fk, fv, fg, fb, cu, maxlen, s0,
                                    chunk_size=p.C)
    torch.cuda.synchronize()
    return y, s, o2, s2


def fused_expected(p):
    """The entry point fuses the epilogue when N * H is at least twice the
    device's compute units (include/kda.h)."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    return len(U.seq_bounds(p)) - 1 >= 1 and \
        (len(U.seq_bounds(p)) - 1) * p.H >= 2 * cus


def check_gated(p, seed, label, head_group=None):
    fused = fused_expected(p)
    U.log("gated prefill", label, "H=%d D=%d C=%d tokens=%d %s, %s path"
          % (p.H, p.K, p.C, p.tokens, p.dtype,
             "fused" if fused else "two-pass"))
    z, w = gate_inputs(p, seed)
    y, s, o2, s2 = run_gated(p, z, w)
    y2 = kda.kda_output_norm_gate(o2, U.to_dev(z, p.dtype), U.f32_dev(w),
                                  eps=EPS)
    torch.cuda.synchronize()
    # which path ran: the two-pass one is plain prefill + epilogue kernel,
    # bit for bit; the fused kernel normalises the fp32 outputs instead
    assert torch.equal(y, y2) != fused, "unexpected path"
    cu = U.seq_bounds(p)
    step = head_group or p.H
    e_epi = e_end = es = 0.0
    for h0 in range(0, p.H, step):
        heads = list(range(h0, min(p.H, h0 + step)))
        yh = U.host(y[:, heads])
        zh = z[:, heads].astype(np.float64)
        # (a) the epilogue on the GPU's own plain-prefill outputs
        o2h = U.host(o2.reshape(p.tokens, p.H, p.V)[:, heads])
        e_epi = max(e_epi, row_rel(yh, oracle.norm_gate(o2h, zh, w, EPS)))
        # (b) end to end: outputs recovered from y, against the oracle
        o_ref, s_ref = U.run_oracle(p, heads)
        o_ref = o_ref.reshape(p.tokens, len(heads), p.V)
        rms = np.sqrt(np.mean(o2h * o2h, axis=-1, keepdims=True) + EPS)
        back = yh * rms / (w * (1.0 / (1.0 + np.exp(-zh))))
        e_end = max(e_end, max(U.prefill_o_rel(back, o_ref, cu, p.C)))
        es = max(es, U.slice_rel(U.host(s[:, heads]), s_ref, (0, 1)))
    same_state = bool(torch.equal(s, s2))
    U.log("   epilogue per row %.3e   end to end %.3e   final state %.3e   "
          "state equal to the plain prefill's: %s"
          % (e_epi, e_end, es, same_state))
    assert e_epi <= (1e-2 if p.dtype == "bf16" else 1e-4)
    assert e_end <= U.PREFILL_TOL and es <= U.PREFILL_TOL
    # the state recurrence is the plain prefill's, column by column
    assert U.slice_rel(U.host(s), U.host(s2), (0, 1)) <= 1e-6


def _ragged(D, C, H, dtype="bf16"):
    return inputs.make("varlen", seed=70 + D + C + H, H=H, K=D, V=D, C=C,
                       dtype=dtype, lengths=[C + 5, 0, 1, 3 * C, 2 * C + 17])


@pytest.mark.parametrize("D", [16, 32, 64, 128])
@pytest.mark.parametrize("C", [16, 32, 64])
def test_gated_prefill_fused_ragged(D, C):
    """5 sequences x 110 heads: 550 pairs, the fused kernel."""
    p = _ragged(D, C, 110)
    assert fused_expected(p)
    check_gated(p, D + C, "ragged, fused", head_group=55)


@pytest.mark.parametrize("D,C", [(16, 16), (32, 32), (64, 64), (128, 64)])
def test_gated_prefill_two_pass_ragged(D, C):
    """5 sequences x 3 heads: the plain recurrence, then the epilogue."""
    p = _ragged(D, C, 3)
    assert not fused_expected(p)
    check_gated(p, D + C, "ragged, two-pass")


@pytest.mark.parametrize("H", [2, 300])
def test_gated_prefill_fp32_zero_state(H):
    p = inputs.make("varlen", seed=71, H=H, K=64, V=64, C=64, dtype="fp32",
                    s0=False, lengths=[150, 64, 33])
    check_gated(p, 5, "fp32", head_group=100)


def test_gated_prefill_varlen_workload():
    """The 8-sequence, 96-head append-prefill workload (768 pairs: the
    fused kernel), every head."""
    p = inputs.make("varlen", seed=0)
    assert fused_expected(p)
    check_gated(p, 9, "varlen workload", head_group=24)


def test_gated_prefill_workload():
    """8192 tokens x 96 heads, d = 128, C = 64 (96 pairs: the two-pass
    path), every head."""
    p = inputs.make("prefill", seed=0)
    assert not fused_expected(p)
    check_gated(p, 9, "8K-token workload", head_group=48)
