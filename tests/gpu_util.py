"""Helpers for the GPU parity tests: move seeded problems to the device, run
libkda through its C ABI, run the fp64 oracle on the same values, compare.

Error measure: max |x - x_ref| / max |x_ref| over a slice, maximum over
slices.  Final states and decode outputs: one slice per (sequence, head).
Prefill outputs: one slice per (sequence, head) for every sequence of at
least one chunk (C tokens).  Sequences shorter than a chunk keep the per-head
measure: their largest error in a head, over the head's largest output in
the whole call.  Why: the prefill path multiplies
bf16 operands on the matrix cores by design, so an output's error is
relative to the magnitudes of the terms it sums.  A sequence of a token or
two that starts from a zero state has the output (q . k) beta v, and q . k
of two unit vectors can nearly vanish; the relative error of such a slice
then measures the inputs' conditioning, not the kernel.  A sequence of a
chunk or more has outputs of the state's full size (the decay bounds it), so
its own slice is well scaled.  Tolerances: 2e-2 for prefill outputs and
final states, 1e-4 for the fp32 decode state, 2e-2 for bf16 decode outputs
and 1e-4 for fp32 decode outputs.
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


def seq_bounds(p: inputs.Problem):
    """Packed token bounds [N+1] of the problem's sequences."""
    if p.kind == "varlen":
        return np.asarray(p.cu_seqlens, np.int64)
    return np.arange(p.B + 1, dtype=np.int64) * p.T


def prefill_o_rel(o, ref, cu, C):
    """Prefill output errors: (worst per-(sequence, head) error over the
    sequences of at least C tokens, worst per-head error of the shorter
    sequences' tokens over the head's largest output in the whole call).
    o / ref: packed [total, H, V] or batched [B, T, H, V]."""
    o = np.asarray(o, np.float64).reshape(-1, *np.shape(o)[-2:])
    ref = np.asarray(ref, np.float64).reshape(-1, *np.shape(ref)[-2:])
    if not np.all(np.isfinite(o)):
        return float("inf"), float("inf")
    long_err = 0.0
    short = np.zeros(o.shape[0], bool)
    for n in range(len(cu) - 1):
        a, b = int(cu[n]), int(cu[n + 1])
        if b - a >= C:
            long_err = max(long_err, slice_rel(o[a:b], ref[a:b], (1,)))
        elif b > a:
            short[a:b] = True
    short_err = 0.0
    if short.any():
        num = np.max(np.abs(o[short] - ref[short]), axis=(0, 2))   # per head
        den = np.maximum(np.max(np.abs(ref), axis=(0, 2)), 1e-30)
        short_err = float(np.max(num / den))
    return long_err, short_err


def worst_sequence_rel(o, ref, cu):
    """Largest per-(sequence, head) relative error of packed outputs, any
    length (logged: for sequences shorter than a chunk it reflects the
    conditioning of q . k)."""
    o = np.asarray(o).reshape(-1, *np.shape(o)[-2:])
    ref = np.asarray(ref).reshape(-1, *np.shape(ref)[-2:])
    worst = 0.0
    for n in range(len(cu) - 1):
        a, b = int(cu[n]), int(cu[n + 1])
        if b > a:
            worst = max(worst, slice_rel(o[a:b], ref[a:b], (1,)))
    return worst


def prefill_gpu(p: inputs.Problem, alias_state=False, scale=1.0,
                workspace=None):
    """Run the problem through libkda.  Returns device (o, final_state)."""
    q, k, v = (to_dev(x, p.dtype) for x in (p.q, p.k, p.v))
    g, beta = f32_dev(p.g), f32_dev(p.beta)
    s0 = f32_dev(p.initial_state)
    fs = s0 if (alias_state and s0 is not None) else None
    if p.kind == "varlen":
        cu = torch.from_numpy(p.cu_seqlens.astype(np.int32)).to(DEV)
        o, s = kda.kda_prefill_varlen(q, k, v, g, beta, cu,
                                      int(p.seq_lengths.max(initial=0)), s0,
                                      chunk_size=p.C, scale=scale,
                                      final_state=fs, workspace=workspace)
    else:
        o, s = kda.kda_prefill_chunked(q, k, v, g, beta, s0, chunk_size=p.C,
                                       scale=scale, final_state=fs,
                                       workspace=workspace)
    torch.cuda.synchronize()
    del q, k, v, g, beta
    return o, s


def run_prefill_gpu(p: inputs.Problem, heads=None, alias_state=False,
                    scale=1.0):
    """Run the problem through libkda.  Returns host (o, final_state)."""
    o, s = prefill_gpu(p, alias_state, scale)
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


def check_prefill(p: inputs.Problem, tol=PREFILL_TOL, label="",
                  alias_state=False, scale=1.0, head_group=None):
    """GPU prefill against the oracle on every head.  The GPU runs the whole
    call once; the oracle and the comparison go over groups of head_group
    heads (all at once when None) to bound the fp64 host memory."""
    log("prefill", label or p.name, "kind=%s H=%d Dk=%d Dv=%d C=%d tokens=%d "
        "dtype=%s" % (p.kind, p.H, p.K, p.V, p.C, p.tokens, p.dtype))
    o_dev, s_dev = prefill_gpu(p, alias_state, scale)
    cu = seq_bounds(p)
    step = head_group or p.H
    eo_long = eo_short = es = worst = 0.0
    for h0 in range(0, p.H, step):
        heads = list(range(h0, min(p.H, h0 + step)))
        o = host(o_dev[..., heads, :])
        s = host(s_dev[:, heads])
        o_ref, s_ref = run_oracle(p, heads, scale)
        el, esh = prefill_o_rel(o, o_ref, cu, p.C)
        eo_long, eo_short = max(eo_long, el), max(eo_short, esh)
        es = max(es, slice_rel(s, s_ref, (0, 1)))
        if p.kind == "varlen":
            worst = max(worst, worst_sequence_rel(o, o_ref, cu))
        del o, s, o_ref, s_ref
    extra = ""
    if p.kind == "varlen":
        extra = "   (any single sequence %.3e)" % worst
    log("   o rel err: per (sequence, head) %.3e, shorter than a chunk "
        "(per head) %.3e   final state rel err %.3e%s"
        % (eo_long, eo_short, es, extra))
    assert eo_long <= tol, ("output, per (sequence, head)", eo_long)
    assert eo_short <= tol, ("output, short sequences per head", eo_short)
    assert es <= tol, ("final state", es)
    return max(eo_long, eo_short), es


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
