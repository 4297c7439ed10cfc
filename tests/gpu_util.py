"""Helpers for the GPU parity tests: move seeded problems to the device, run
libkda through its C ABI, run the fp64 oracle on the same values, compare.

Error measure: max |x - x_ref| / max |x_ref| over a slice, maximum over
slices.  Final states and decode outputs: one slice per (sequence, head).
Prefill outputs: one slice per head, over every token of the call.  The
prefill path multiplies bf16 operands on the matrix cores by design, so its
error in an output is relative to the magnitudes of the summed terms; a
sequence of a token or two that starts from a zero state has the output
(q . k) beta v, and q . k of two unit vectors can nearly vanish, so the
relative error of such a slice measures the inputs' conditioning, not the
kernel.  Every output of a head has the same scale whatever its sequence's
length (the state's size is bounded by the decay), so a wrong or misplaced
sequence still shows as an error of order one.  Tolerances: 2e-2 for
prefill outputs and final states, 1e-4 for the fp32 decode state, 2e-2 for
bf16 decode outputs and 1e-4 for fp32 decode outputs.
"""
from __future__ import annotations

import sys
import time

import numpy as np
import torch

import oracle
from linear_recurrent_attention_kda_amd import inputs, kda

DEV = torch.device("cuda:0")
PREFILL_TOL = 2e-2
DECODE_STATE_TOL = 1e-4
DECODE_O_TOL = {"bf16": 2e-2, "fp32": 1e-4}


def log(*a):
    print("[gpu-test %.1fs]" % (time.time() - _T0), *a, flush=True)
    sys.stdout.flush()


_T0 = time.time()


def to_dev(x, dtype: str):
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)       # exact: values are bf16-representable
    return t.to(DEV)


def f32_dev(x):
    return None if x is None else torch.from_numpy(
        np.ascontiguousarray(x, np.float32)).to(DEV)


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def slice_rel(x, ref, slice_axes):
    """Max over slices (indexed by `slice_axes`) of the per-slice relative
    error."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    other = tuple(i for i in range(x.ndim) if i not in slice_axes)
    num = np.max(np.abs(x - ref), axis=other) if other else np.abs(x - ref)
    den = np.max(np.abs(ref), axis=other) if other else np.abs(ref)
    den = np.maximum(den, 1e-30)
    if not np.all(np.isfinite(x)):
        return float("inf")
    return float(np.max(num / den)) if num.size else 0.0


def prefill_o_rel(o, ref):
    """Per-head relative error of prefill outputs, packed [total, H, V] or
    batched [B, T, H, V] (heads on the second-to-last axis)."""
    return slice_rel(o, ref, (np.ndim(o) - 2,))


def worst_sequence_rel(o, ref, cu):
    """Largest per-(sequence, head) relative error of packed outputs (for
    the log: it reflects the conditioning of the shortest sequences)."""
    worst = 0.0
    for n in range(len(cu) - 1):
        a, b = int(cu[n]), int(cu[n + 1])
        if b > a:
            worst = max(worst, slice_rel(o[a:b], ref[a:b], (1,)))
    return worst


def run_prefill_gpu(p: inputs.Problem, heads=None, alias_state=False,
                    scale=1.0):
    """Run the problem through libkda.  Returns host (o, final_state)."""
    q, k, v = (to_dev(x, p.dtype) for x in (p.q, p.k, p.v))
    g, beta = f32_dev(p.g), f32_dev(p.beta)
    s0 = f32_dev(p.initial_state)
    fs = s0 if (alias_state and s0 is not None) else None
    if p.kind == "varlen":
        cu = torch.from_numpy(p.cu_seqlens.astype(np.int32)).to(DEV)
        o, s = kda.kda_prefill_varlen(q, k, v, g, beta, cu,
                                      int(p.seq_lengths.max(initial=0)), s0,
                                      chunk_size=p.C, scale=scale,
                                      final_state=fs)
    else:
        o, s = kda.kda_prefill_chunked(q, k, v, g, beta, s0, chunk_size=p.C,
                                       scale=scale, final_state=fs)
    torch.cuda.synchronize()
    if heads is not None:
        o = o[..., heads, :]
        s = s[:, heads]
    return host(o), host(s)


def run_oracle(p: inputs.Problem, heads=None, scale=1.0):
    """fp64 oracle on the same values (optionally only some heads)."""
    sel = (lambda x: x) if heads is None else (lambda x: x[..., heads, :])
    selb = (lambda x: x) if heads is None else (lambda x: x[..., heads])
    s0 = p.initial_state
    if s0 is not None and heads is not None:
        s0 = s0[:, heads]
    if p.kind == "varlen":
        return oracle.run_varlen(sel(p.q), sel(p.k), sel(p.v), sel(p.g),
                                 selb(p.beta), p.cu_seqlens, s0, scale)
    return oracle.run_fixed(sel(p.q), sel(p.k), sel(p.v), sel(p.g),
                            selb(p.beta), s0, scale)


def check_prefill(p: inputs.Problem, heads=None, tol=PREFILL_TOL, label="",
                  alias_state=False, scale=1.0):
    log("prefill", label or p.name, "kind=%s H=%d D=%d C=%d tokens=%d dtype=%s"
        % (p.kind, p.H, p.K, p.C, p.tokens, p.dtype))
    o, s = run_prefill_gpu(p, heads, alias_state, scale)
    o_ref, s_ref = run_oracle(p, heads, scale)
    eo = prefill_o_rel(o, o_ref)
    es = slice_rel(s, s_ref, (0, 1))
    extra = ""
    if p.kind == "varlen":
        extra = "   (worst single sequence %.3e)" % worst_sequence_rel(
            o, o_ref, p.cu_seqlens)
    log("   o rel err %.3e   final state rel err %.3e%s" % (eo, es, extra))
    assert eo <= tol, ("output", eo)
    assert es <= tol, ("final state", es)
    return eo, es


def check_decode(p: inputs.Problem, scale=1.0):
    log("decode", p.name, "B=%d H=%d D=%d dtype=%s" % (p.B, p.H, p.K, p.dtype))
    q, k, v = (to_dev(x, p.dtype) for x in (p.q, p.k, p.v))
    g, beta = f32_dev(p.g), f32_dev(p.beta)
    state = f32_dev(p.initial_state)
    o = kda.kda_decode_step(q, k, v, g, beta, state, scale=scale)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.run_decode(p.q, p.k, p.v, p.g, p.beta,
                                     p.initial_state, scale)
    eo = slice_rel(host(o), o_ref, (0, 1))
    es = slice_rel(host(state), s_ref, (0, 1))
    log("   o rel err %.3e   state rel err %.3e" % (eo, es))
    assert es <= DECODE_STATE_TOL, ("state", es)
    assert eo <= DECODE_O_TOL[p.dtype], ("output", eo)
    return eo, es
