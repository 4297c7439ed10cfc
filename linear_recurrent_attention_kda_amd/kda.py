"""Thin ctypes binding of libkda (include/kda.h), with the same entry-point
names.  It only marshals arguments: checks tensor shapes, dtypes and
devices, allocates outputs and the workspace with torch when the caller
does not pass them, and hands raw device pointers and the current HIP stream
to the library.  Every step of the computation runs in libkda's kernels; if
the library is missing this module raises, it never falls back to anything
else.
"""
from __future__ import annotations

import ctypes
import os
import re
import threading
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("KDA_LIB", os.path.join(_PKG, "libkda.so"))
HEADER = os.path.join(os.path.dirname(_PKG), "include", "kda.h")

KDA_OK = 0
KDA_ERR_SCRATCH = -5
KDA_NOALLOC_SCRATCH_BYTES = 256 << 20
KDA_DTYPE_BF16 = 0
KDA_DTYPE_FP32 = 1

_lock = threading.Lock()
_lib = None


class KDAError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__("%s failed: %s (status %d)" %
                         (fn, kda_status_string(status), status))
        self.status = status


def load() -> ctypes.CDLL:
    """Load libkda.so (once).  Raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                "libkda.so not found at %s; build it with "
                "`python -m linear_recurrent_attention_kda_amd.build`" % LIB_PATH)
        lib = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, f32, sz = (ctypes.c_void_p, ctypes.c_int32,
                                 ctypes.c_int64, ctypes.c_float,
                                 ctypes.c_size_t)
        lib.kda_abi_version.restype = i32
        lib.kda_abi_version.argtypes = []
        lib.kda_status_string.restype = ctypes.c_char_p
        lib.kda_status_string.argtypes = [i32]
        lib.kda_prefill_workspace_size.restype = sz
        lib.kda_prefill_workspace_size.argtypes = [i32, i64, i32, i32, i32, i32]
        lib.kda_prefill_chunked.restype = i32
        lib.kda_prefill_chunked.argtypes = [
            vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32,
            i32, vp, sz, vp]
        lib.kda_prefill_varlen.restype = i32
        lib.kda_prefill_varlen.argtypes = [
            vp, vp, vp, vp, vp, vp, i32, i64, i32, vp, vp, vp, i32, i32, i32,
            i32, f32, i32, vp, sz, vp]
        lib.kda_prefill_varlen_gated.restype = i32
        lib.kda_prefill_varlen_gated.argtypes = [
            vp, vp, vp, vp, vp, vp, i32, i64, i32, vp, vp, vp, vp, f32, vp,
            i32, i32, i32, i32, f32, i32, vp, sz, vp]
        lib.kda_prefill_varlen_noalloc.restype = i32
        lib.kda_prefill_varlen_noalloc.argtypes = [
            vp, vp, vp, vp, vp, vp, i32, i64, i32, vp, vp, vp, i32, i32, i32,
            i32, f32, i32, vp]
        lib.kda_prefill_varlen_prep.restype = i32
        lib.kda_prefill_varlen_prep.argtypes = [
            vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32, i32, i32, i32,
            vp, sz, vp]
        lib.kda_prefill_varlen_recur.restype = i32
        lib.kda_prefill_varlen_recur.argtypes = [
            vp, i32, i64, i32, vp, vp, vp, i32, i32, i32, i32, f32, i32, vp,
            sz, vp]
        lib.kda_prefill_varlen_ckpt.restype = i32
        lib.kda_prefill_varlen_ckpt.argtypes = [
            vp, vp, vp, vp, vp, vp, i32, i64, i32, vp, vp, vp, i32, i32, i32,
            i32, f32, i32, i32, vp, sz, vp, sz, vp]
        lib.kda_prefill_varlen_ckpt_at.restype = i32
        lib.kda_prefill_varlen_ckpt_at.argtypes = [
            vp, vp, vp, vp, vp, vp, i32, i64, i32, vp, vp, vp, i32, i32, i32,
            i32, f32, i32, vp, vp, i32, vp, sz, vp, sz, vp]
        lib.kda_spec_verify.restype = i32
        lib.kda_spec_verify.argtypes = [
            vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32,
            vp]
        lib.kda_spec_commit.restype = i32
        lib.kda_spec_commit.argtypes = [
            vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, vp]
        lib.kda_spec_step.restype = i32
        lib.kda_spec_step.argtypes = [
            vp, vp, vp, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32,
            i32, i32, i32, f32, i32, vp]
        lib.kda_spec_step_indexed.restype = i32
        lib.kda_spec_step_indexed.argtypes = [
            vp, vp, vp, vp, i32, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, i32,
            i32, i32, i32, i32, f32, i32, vp]
        lib.kda_decode_step_gated_indexed.restype = i32
        lib.kda_decode_step_gated_indexed.argtypes = [
            vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, f32, vp, i32, i32, i32,
            i32, f32, i32, vp]
        lib.kda_output_norm_gate.restype = i32
        lib.kda_output_norm_gate.argtypes = [vp, vp, vp, f32, vp, i64, i32,
                                             i32, i32, vp]
        lib.kda_decode_step_gated.restype = i32
        lib.kda_decode_step_gated.argtypes = [
            vp, vp, vp, vp, vp, vp, vp, vp, f32, vp, i32, i32, i32, i32, f32,
            i32, vp]
        lib.kda_prefill_varlen_prologue.restype = i32
        lib.kda_prefill_varlen_prologue.argtypes = [
            vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, vp, vp, vp, i32, i32,
            i32, i32, f32, i32, vp, sz, vp]
        lib.kda_decode_step.restype = i32
        lib.kda_decode_step.argtypes = [
            vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, f32, i32, vp]
        lib.kda_decode_step_indexed.restype = i32
        lib.kda_decode_step_indexed.argtypes = [
            vp, vp, vp, vp, vp, vp, vp, i32, vp, i32, i32, i32, i32, f32, i32,
            vp]
        lib.kda_prefill_varlen_indexed.restype = i32
        lib.kda_prefill_varlen_indexed.argtypes = [
            vp, vp, vp, vp, vp, vp, i32, i64, i32, vp, vp, vp, i32, vp, i32,
            i32, i32, i32, f32, i32, vp, sz, vp]
        _lib = lib
        return lib


def declared_functions(header: str = HEADER):
    """Names of the functions include/kda.h declares."""
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_0-9]+)\s*\(", text)))


# ---------------------------------------------------------------------------
def kda_abi_version() -> int:
    return int(load().kda_abi_version())


def kda_status_string(status: int) -> str:
    return load().kda_status_string(int(status)).decode()


def kda_prefill_workspace_size(N: int, total_T: int, H: int, Dk: int,
                               Dv: int, C: int) -> int:
    return int(load().kda_prefill_workspace_size(N, total_T, H, Dk, Dv, C))


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return KDA_DTYPE_BF16
    if t.dtype == torch.float32:
        return KDA_DTYPE_FP32
    raise TypeError("q, k, v must be bfloat16 or float32, got %s" % t.dtype)


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check(t: torch.Tensor, name: str, shape, dtype, device):
    if t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" %
                         (name, tuple(t.shape), tuple(shape)))
    if t.dtype != dtype:
        raise TypeError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def workspace_for(N, total_T, H, Dk, Dv, C, device) -> torch.Tensor:
    n = kda_prefill_workspace_size(N, total_T, H, Dk, Dv, C)
    if n == 0:
        raise ValueError("unsupported prefill sizes")
    return torch.empty(n, dtype=torch.uint8, device=device)


def kda_prefill_chunked(q, k, v, g, beta, initial_state=None, *,
                        chunk_size: int = 64, scale: float = 1.0,
                        output_final_state: bool = True, final_state=None,
                        o=None, workspace=None):
    """Chunked prefill of a fixed-length batch.

    q, k, g: [B, T, H, Dk]; v: [B, T, H, Dv]; beta: [B, T, H] (q, k, v bf16
    or fp32; g, beta fp32); initial_state: [B, H, Dk, Dv] fp32 or None.
    Returns (o [B, T, H, Dv], final_state [B, H, Dk, Dv] fp32 or None).
    final_state may be initial_state itself (updated in place).
    """
    lib = load()
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    dev = q.device
    for t, n, s, dt in ((q, "q", (B, T, H, Dk), q.dtype),
                        (k, "k", (B, T, H, Dk), q.dtype),
                        (v, "v", (B, T, H, Dv), q.dtype),
                        (g, "g", (B, T, H, Dk), torch.float32),
                        (beta, "beta", (B, T, H), torch.float32)):
        _check(t, n, s, dt, dev)
    if initial_state is not None:
        _check(initial_state, "initial_state", (B, H, Dk, Dv), torch.float32,
               dev)
    if final_state is None and output_final_state:
        final_state = torch.empty((B, H, Dk, Dv), dtype=torch.float32,
                                  device=dev)
    if final_state is not None:
        _check(final_state, "final_state", (B, H, Dk, Dv), torch.float32, dev)
    if o is None:
        o = torch.empty((B, T, H, Dv), dtype=q.dtype, device=dev)
    _check(o, "o", (B, T, H, Dv), q.dtype, dev)
    if workspace is None:
        workspace = workspace_for(B, B * T, H, Dk, Dv, chunk_size, dev)
    st = lib.kda_prefill_chunked(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state),
        _ptr(final_state), _ptr(o), B, T, H, Dk, Dv, chunk_size, scale,
        _dtype_code(q), _ptr(workspace), workspace.numel(), _stream(dev))
    if st != KDA_OK:
        raise KDAError("kda_prefill_chunked", st)
    return o, final_state


def kda_prefill_varlen(q, k, v, g, beta, cu_seqlens, max_seqlen: int,
                       initial_state=None, *, chunk_size: int = 64,
                       scale: float = 1.0, output_final_state: bool = True,
                       final_state=None, o=None, workspace=None):
    """Chunked prefill of N packed sequences (append-prefill when an initial
    state is given).

    q, k, g: [total_T, H, Dk]; v: [total_T, H, Dv]; beta: [total_T, H];
    cu_seqlens: int32 [N+1] on the device; max_seqlen: host int >= every
    length; initial_state: [N, H, Dk, Dv] fp32 or None.
    Returns (o [total_T, H, Dv], final_state [N, H, Dk, Dv] or None).
    """
    lib = load()
    total_T, H, Dk = q.shape
    Dv = v.shape[-1]
    dev = q.device
    N = cu_seqlens.numel() - 1
    for t, n, s, dt in ((q, "q", (total_T, H, Dk), q.dtype),
                        (k, "k", (total_T, H, Dk), q.dtype),
                        (v, "v", (total_T, H, Dv), q.dtype),
                        (g, "g", (total_T, H, Dk), torch.float32),
                        (beta, "beta", (total_T, H), torch.float32),
                        (cu_seqlens, "cu_seqlens", (N + 1,), torch.int32)):
        _check(t, n, s, dt, dev)
    if initial_state is not None:
        _check(initial_state, "initial_state", (N, H, Dk, Dv), torch.float32,
               dev)
    if final_state is None and output_final_state:
        final_state = torch.empty((N, H, Dk, Dv), dtype=torch.float32,
                                  device=dev)
    if final_state is not None:
        _check(final_state, "final_state", (N, H, Dk, Dv), torch.float32, dev)
    if o is None:
        o = torch.empty((total_T, H, Dv), dtype=q.dtype, device=dev)
    _check(o, "o", (total_T, H, Dv), q.dtype, dev)
    if workspace is None:
        workspace = workspace_for(N, total_T, H, Dk, Dv, chunk_size, dev)
    st = lib.kda_prefill_varlen(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens), N,
        total_T, int(max_seqlen), _ptr(initial_state), _ptr(final_state),
        _ptr(o), H, Dk, Dv, chunk_size, scale, _dtype_code(q),
        _ptr(workspace), workspace.numel(), _stream(dev))
    if st != KDA_OK:
        raise KDAError("kda_prefill_varlen", st)
    return o, final_state


def kda_prefill_varlen_prep(q, k, v, g, beta, cu_seqlens, max_seqlen: int,
                            *, chunk_size: int = 64, workspace=None):
    """First stage of kda_prefill_varlen: every chunk's tensors, written to
    the workspace (allocated when None).  Returns the workspace, to be passed
    unchanged to kda_prefill_varlen_recur."""
    lib = load()
    total_T, H, Dk = q.shape
    Dv = v.shape[-1]
    dev = q.device
    N = cu_seqlens.numel() - 1
    for t, n, s, dt in ((q, "q", (total_T, H, Dk), q.dtype),
                        (k, "k", (total_T, H, Dk), q.dtype),
                        (v, "v", (total_T, H, Dv), q.dtype),
                        (g, "g", (total_T, H, Dk), torch.float32),
                        (beta, "beta", (total_T, H), torch.float32),
                        (cu_seqlens, "cu_seqlens", (N + 1,), torch.int32)):
        _check(t, n, s, dt, dev)
    if workspace is None:
        workspace = workspace_for(N, total_T, H, Dk, Dv, chunk_size, dev)
    st = lib.kda_prefill_varlen_prep(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens), N,
        total_T, int(max_seqlen), H, Dk, Dv, chunk_size, _dtype_code(q),
        _ptr(workspace), workspace.numel(), _stream(dev))
    if st != KDA_OK:
        raise KDAError("kda_prefill_varlen_prep", st)
    return workspace


def kda_prefill_varlen_recur(workspace, cu_seqlens, max_seqlen: int,
                             total_T: int, H: int, Dk: int, Dv: int,
                             dtype, initial_state=None, *,
                             chunk_size: int = 64, scale: float = 1.0,
                             output_final_state: bool = True,
                             final_state=None, o=None):
    """Second stage of kda_prefill_varlen: the recurrence over the chunks
    that kda_prefill_varlen_prep wrote to `workspace`.  dtype is the torch
    dtype of q, k, v (and of o).  Returns (o, final_state or None)."""
    lib = load()
    dev = workspace.device
    N = cu_seqlens.numel() - 1
    _check(cu_seqlens, "cu_seqlens", (N + 1,), torch.int32, dev)
    if initial_state is not None:
        _check(initial_state, "initial_state", (N, H, Dk, Dv), torch.float32,
               dev)
    if final_state is None and output_final_state:
        final_state = torch.empty((N, H, Dk, Dv), dtype=torch.float32,
                                  device=dev)
    if final_state is not None:
        _check(final_state, "final_state", (N, H, Dk, Dv), torch.float32, dev)
    if o is None:
        o = torch.empty((total_T, H, Dv), dtype=dtype, device=dev)
    _check(o, "o", (total_T, H, Dv), dtype, dev)
    st = lib.kda_prefill_varlen_recur(
        _ptr(cu_seqlens), N, total_T, int(max_seqlen), _ptr(initial_state),
        _ptr(final_state), _ptr(o), H, Dk, Dv, chunk_size, scale,
        _dtype_code(o), _ptr(workspace), workspace.numel(), _stream(dev))
    if st != KDA_OK:
        raise KDAError("kda_prefill_varlen_recur", st)
    return o, final_state


def kda_prefill_varlen_gated(q, k, v, g, beta, cu_seqlens, max_seqlen: int,
                             initial_state=None, *, z, w, eps: float = 1e-6,
                             chunk_size: int = 64, scale: float = 1.0,
                             output_final_state: bool = True,
                             final_state=None, y=None, workspace=None):
    """kda_prefill_varlen with the output epilogue fused into the recurrence:
    returns (y, final_state) with y = o * rsqrt(mean(o^2) + eps) * w *
    sigmoid(z) per (token, head) row.  z: [total_T, H, Dv] (dtype of q);
    w: [Dv] fp32."""
    lib = load()
    total_T, H, Dk = q.shape
    Dv = v.shape[-1]
    dev = q.device
    N = cu_seqlens.numel() - 1
    for t, n, s, dt in ((q, "q", (total_T, H, Dk), q.dtype),
                        (k, "k", (total_T, H, Dk), q.dtype),
                        (v, "v", (total_T, H, Dv), q.dtype),
                        (g, "g", (total_T, H, Dk), torch.float32),
                        (beta, "beta", (total_T, H), torch.float32),
                        (cu_seqlens, "cu_seqlens", (N + 1,), torch.int32),
                        (z, "z", (total_T, H, Dv), q.dtype),
                        (w, "w", (Dv,), torch.float32)):
        _check(t, n, s, dt, dev)
    if initial_state is not None:
        _check(initial_state, "initial_state", (N, H, Dk, Dv), torch.float32,
               dev)
    if final_state is None and output_final_state:
        final_state = torch.empty((N, H, Dk, Dv), dtype=torch.float32,
                                  device=dev)
    if final_state is not None:
        _check(final_state, "final_state", (N, H, Dk, Dv), torch.float32, dev)
    if y is None:
        y = torch.empty((total_T, H, Dv), dtype=q.dtype, device=dev)
    _check(y, "y", (total_T, H, Dv), q.dtype, dev)
    if workspace is None:
        workspace = workspace_for(N, total_T, H, Dk, Dv, chunk_size, dev)
    st = lib.kda_prefill_varlen_gated(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens), N,
        total_T, int(max_seqlen), _ptr(initial_state), _ptr(final_state),
        _ptr(z), _ptr(w), float(eps), _ptr(y), H, Dk, Dv, chunk_size, scale,
        _dtype_code(q), _ptr(workspace), workspace.numel(), _stream(dev))
    if st != KDA_OK:
        raise KDAError("kda_prefill_varlen_gated", st)
    return y, final_state


def kda_prefill_varlen_noalloc(q, k, v, g, beta, cu_seqlens,
                               max_seqlen: int, initial_state=None, *,
                               chunk_size: int = 64, scale: float = 1.0,
                               final_state=None, o=None):
    """kda_prefill_varlen with the workspace in the library's fixed device
    scratch array (no workspace argument; the library call allocates
    nothing).  final_state and o must be passed in (this wrapper allocates
    nothing either).  Calls that overlap on one GPU race on the scratch
    array.  Returns (o, final_state)."""
    lib = load()
    total_T, H, Dk = q.shape
    Dv = v.shape[-1]
    dev = q.device
    N = cu_seqlens.numel() - 1
    for t, n, s, dt in ((q, "q", (total_T, H, Dk), q.dtype),
                        (k, "k", (total_T, H, Dk), q.dtype),
                        (v, "v", (total_T, H, Dv), q.dtype),
                        (g, "g", (total_T, H, Dk), torch.float32),
                        (beta, "beta", (total_T, H), torch.float32),
                        (cu_seqlens, "cu_seqlens", (N + 1,), torch.int32),
                        (o, "o", (total_T, H, Dv), q.dtype)):
        _check(t, n, s, dt, dev)
    if initial_state is not None:
        _check(initial_state, "initial_state", (N, H, Dk, Dv), torch.float32,
               dev)
    if final_state is not None:
        _check(final_state, "final_state", (N, H, Dk, Dv), torch.float32, dev)
    st = lib.kda_prefill_varlen_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens), N,
        total_T, int(max_seqlen), _ptr(initial_state), _ptr(final_state),
        _ptr(o), H, Dk, Dv, chunk_size, scale, _dtype_code(q), _stream(dev))
    if st != KDA_OK:
        raise KDAError("kda_prefill_varlen_noalloc", st)
    return o, final_state


def kda_prefill_varlen_ckpt(q, k, v, g, beta, cu_seqlens, max_seqlen: int,
                            initial_state=None, *, ckpt_every: int,
                            chunk_size: int = 64, scale: float = 1.0,
                            output_final_state: bool = True, final_state=None,
                            o=None, ckpt_states=None, workspace=None):
    """kda_prefill_varlen that also stores the state every `ckpt_every`
    tokens (a multiple of chunk_size) inside each sequence.

    Returns (o, final_state, ckpt_states) with ckpt_states
    [total_T // ckpt_every, H, Dk, Dv] fp32: the state after the first
    j * ckpt_every tokens of sequence n sits in slot
    (cu_seqlens[n] + j * ckpt_every) // ckpt_every - 1 (see
    `kda_ckpt_slots`); other slots are left as allocated.
    """
    lib = load()
    total_T, H, Dk = q.shape
    Dv = v.shape[-1]
    dev = q.device
    N = cu_seqlens.numel() - 1
    for t, n, s, dt in ((q, "q", (total_T, H, Dk), q.dtype),
                        (k, "k", (total_T, H, Dk), q.dtype),
                        (v, "v", (total_T, H, Dv), q.dtype),
                        (g, "g", (total_T, H, Dk), torch.float32),
                        (beta, "beta", (total_T, H), torch.float32),
                        (cu_seqlens, "cu_seqlens", (N + 1,), torch.int32)):
        _check(t, n, s, dt, dev)
    if initial_state is not None:
        _check(initial_state, "initial_state", (N, H, Dk, Dv), torch.float32,
               dev)
    if final_state is None and output_final_state:
        final_state = torch.empty((N, H, Dk, Dv), dtype=torch.float32,
                                  device=dev)
    if final_state is not None:
        _check(final_state, "final_state", (N, H, Dk, Dv), torch.float32, dev)
    if o is None:
        o = torch.empty((total_T, H, Dv), dtype=q.dtype, device=dev)
    _check(o, "o", (total_T, H, Dv), q.dtype, dev)
    if ckpt_every <= 0:
        raise ValueError("ckpt_every must be positive")
    slots = total_T // ckpt_every
    if ckpt_states is None:
        ckpt_states = torch.zeros((slots, H, Dk, Dv), dtype=torch.float32,
                                  device=dev)
    _check(ckpt_states, "ckpt_states", (slots, H, Dk, Dv), torch.float32, dev)
    if workspace is None:
        workspace = workspace_for(N, total_T, H, Dk, Dv, chunk_size, dev)
    st = lib.kda_prefill_varlen_ckpt(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens), N,
        total_T, int(max_seqlen), _ptr(initial_state), _ptr(final_state),
        _ptr(o), H, Dk, Dv, chunk_size, scale, _dtype_code(q),
        int(ckpt_every), _ptr(ckpt_states) if slots > 0 else None,
        ckpt_states.numel() * 4, _ptr(workspace), workspace.numel(),
        _stream(dev))
    if st != KDA_OK:
        raise KDAError("kda_prefill_varlen_ckpt", st)
    return o, final_state, ckpt_states


def kda_prefill_varlen_ckpt_at(q, k, v, g, beta, cu_seqlens,
                               max_seqlen: int, initial_state=None, *,
                               ckpt_pos, cu_ckpt, chunk_size: int = 64,
                               scale: float = 1.0,
                               output_final_state: bool = True,
                               final_state=None, o=None, ckpt_states=None,
                               workspace=None):
    """kda_prefill_varlen that also stores the state at caller-given token
    positions: sequence n's positions are ckpt_pos[cu_ckpt[n]:cu_ckpt[n+1]]
    (device int32, increasing, each a multiple of chunk_size or the
    sequence's length).  Returns (o, final_state, ckpt_states) with
    ckpt_states [len(ckpt_pos), H, Dk, Dv] fp32, slot j holding the state
    after position j; slots of positions that break the rules are left as
    allocated (zeros)."""
    lib = load()
    total_T, H, Dk = q.shape
    Dv = v.shape[-1]
    dev = q.device
    N = cu_seqlens.numel() - 1
    n_ckpt = ckpt_pos.numel()
    for t, n, s, dt in ((q, "q", (total_T, H, Dk), q.dtype),
                        (k, "k", (total_T, H, Dk), q.dtype),
                        (v, "v", (total_T, H, Dv), q.dtype),
                        (g, "g", (total_T, H, Dk), torch.float32),
                        (beta, "beta", (total_T, H), torch.float32),
                        (cu_seqlens, "cu_seqlens", (N + 1,), torch.int32),
                        (ckpt_pos, "ckpt_pos", (n_ckpt,), torch.int32),
                        (cu_ckpt, "cu_ckpt", (N + 1,), torch.int32)):
        _check(t, n, s, dt, dev)
    if initial_state is not None:
        _check(initial_state, "initial_state", (N, H, Dk, Dv), torch.float32,
               dev)
    if final_state is None and output_final_state:
        final_state = torch.empty((N, H, Dk, Dv), dtype=torch.float32,
                                  device=dev)
    if final_state is not None:
        _check(final_state, "final_state", (N, H, Dk, Dv), torch.float32, dev)
    if o is None:
        o = torch.empty((total_T, H, Dv), dtype=q.dtype, device=dev)
    _check(o, "o", (total_T, H, Dv), q.dtype, dev)
    if ckpt_states is None:
        ckpt_states = torch.zeros((n_ckpt, H, Dk, Dv), dtype=torch.float32,
                                  device=dev)
    _check(ckpt_states, "ckpt_states", (n_ckpt, H, Dk, Dv), torch.float32,
           dev)
    if workspace is None:
        workspace = workspace_for(N, total_T, H, Dk, Dv, chunk_size, dev)
    st = lib.kda_prefill_varlen_ckpt_at(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens), N,
        total_T, int(max_seqlen), _ptr(initial_state), _ptr(final_state),
        _ptr(o), H, Dk, Dv, chunk_size, scale, _dtype_code(q),
        _ptr(ckpt_pos) if n_ckpt > 0 else None, _ptr(cu_ckpt), n_ckpt,
        _ptr(ckpt_states) if n_ckpt > 0 else None, ckpt_states.numel() * 4,
        _ptr(workspace), workspace.numel(), _stream(dev))
    if st != KDA_OK:
        raise KDAError("kda_prefill_varlen_ckpt_at", st)
    return o, final_state, ckpt_states


def kda_ckpt_slots(cu_seqlens, ckpt_every: int):
    """Host-side map of the checkpoints kda_prefill_varlen_ckpt writes:
    a list of (sequence n, tokens done p, slot), p = j * ckpt_every."""
    cu = [int(x) for x in cu_seqlens]
    out = []
    for n in range(len(cu) - 1):
        p = ckpt_every
        while p <= cu[n + 1] - cu[n]:
            out.append((n, p, (cu[n] + p) // ckpt_every - 1))
            p += ckpt_every
    return out


def kda_decode_step(q, k, v, g, beta, state, *, scale: float = 1.0, o=None):
    """One decode token per sequence; `state` [B, H, Dk, Dv] fp32 is updated
    in place.  q, k, g: [B, H, Dk]; v: [B, H, Dv]; beta: [B, H].
    Returns o [B, H, Dv]."""
    lib = load()
    B, H, Dk = q.shape
    Dv = v.shape[-1]
    dev = q.device
    for t, n, s, dt in ((q, "q", (B, H, Dk), q.dtype),
                        (k, "k", (B, H, Dk), q.dtype),
                        (v, "v", (B, H, Dv), q.dtype),
                        (g, "g", (B, H, Dk), torch.float32),
                        (beta, "beta", (B, H), torch.float32),
                        (state, "state", (B, H, Dk, Dv), torch.float32)):
        _check(t, n, s, dt, dev)
    if o is None:
        o = torch.empty((B, H, Dv), dtype=q.dtype, device=dev)
    _check(o, "o", (B, H, Dv), q.dtype, dev)
    st = lib.kda_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                             _ptr(state), _ptr(o), B, H, Dk, Dv, scale,
                             _dtype_code(q), _stream(dev))
    if st != KDA_OK:
        raise KDAError("kda_decode_step", st)
    return o


def kda_decode_step_indexed(q, k, v, g, beta, state_pool, state_idx, *,
                            scale: float = 1.0, o=None):
    """kda_decode_step with the states in a pool: sequence b uses row
    state_idx[b] (device int32 [B]) of state_pool [slots, H, Dk, Dv] fp32,
    updated in place; a slot outside [0, slots) is padding (zero state,
    nothing read or written).  Returns o [B, H, Dv]."""
    lib = load()
    B, H, Dk = q.shape
    Dv = v.shape[-1]
    dev = q.device
    slots = state_pool.shape[0]
    for t, n, s, dt in ((q, "q", (B, H, Dk), q.dtype),
                        (k, "k", (B, H, Dk), q.dtype),
                        (v, "v", (B, H, Dv), q.dtype),
                        (g, "g", (B, H, Dk), torch.float32),
                        (beta, "beta", (B, H), torch.float32),
                        (state_pool, "state_pool", (slots, H, Dk, Dv),
                         torch.float32),
                        (state_idx, "state_idx", (B,), torch.int32)):
        _check(t, n, s, dt, dev)
    if o is None:
        o = torch.empty((B, H, Dv), dtype=q.dtype, device=dev)
    _check(o, "o", (B, H, Dv), q.dtype, dev)
    st = lib.kda_decode_step_indexed(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state_pool),
        _ptr(state_idx), slots, _ptr(o), B, H, Dk, Dv, scale, _dtype_code(q),
        _stream(dev))
    if st != KDA_OK:
        raise KDAError("kda_decode_step_indexed", st)
    return o


def kda_prefill_varlen_indexed(q, k, v, g, beta, cu_seqlens, max_seqlen: int,
                               state_pool, state_idx, has_initial=None, *,
                               chunk_size: int = 64, scale: float = 1.0,
                               o=None, workspace=None):
    """kda_prefill_varlen with the states in a pool: sequence n starts from
    row state_idx[n] of state_pool [slots, H, Dk, Dv] fp32 (from zeros where
    has_initial[n] == 0) and its final state is written back to that row.
    A slot outside [0, slots) is padding.  Returns o."""
    lib = load()
    total_T, H, Dk = q.shape
    Dv = v.shape[-1]
    dev = q.device
    N = cu_seqlens.numel() - 1
    slots = state_pool.shape[0]
    for t, n, s, dt in ((q, "q", (total_T, H, Dk), q.dtype),
                        (k, "k", (total_T, H, Dk), q.dtype),
                        (v, "v", (total_T, H, Dv), q.dtype),
                        (g, "g", (total_T, H, Dk), torch.float32),
                        (beta, "beta", (total_T, H), torch.float32),
                        (cu_seqlens, "cu_seqlens", (N + 1,), torch.int32),
                        (state_pool, "state_pool", (slots, H, Dk, Dv),
                         torch.float32),
                        (state_idx, "state_idx", (N,), torch.int32)):
        _check(t, n, s, dt, dev)
    if has_initial is not None:
        _check(has_initial, "has_initial", (N,), torch.int32, dev)
    if o is None:
        o = torch.empty((total_T, H, Dv), dtype=q.dtype, device=dev)
    _check(o, "o", (total_T, H, Dv), q.dtype, dev)
    if workspace is None:
        workspace = workspace_for(N, total_T, H, Dk, Dv, chunk_size, dev)
    st = lib.kda_prefill_varlen_indexed(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens), N,
        total_T, int(max_seqlen), _ptr(state_pool), _ptr(state_idx),
        _ptr(has_initial), slots, _ptr(o), H, Dk, Dv, chunk_size, scale,
        _dtype_code(q), _ptr(workspace), workspace.numel(), _stream(dev))
    if st != KDA_OK:
        raise KDAError("kda_prefill_varlen_indexed", st)
    return o


def kda_spec_verify(q, k, v, g, beta, state, *, scale: float = 1.0, o=None,
                    u=None):
    """Run T draft tokens per sequence from `state` (left unchanged).

    q, k, g: [B, T, H, Dk]; v: [B, T, H, Dv]; beta: [B, T, H];
    state: [B, H, Dk, Dv] fp32.  Returns (o [B, T, H, Dv], u [B, T, H, Dv]
    fp32), u being what kda_spec_commit needs.
    """
    lib = load()
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    dev = q.device
    for t, n, s_, dt in ((q, "q", (B, T, H, Dk), q.dtype),
                         (k, "k", (B, T, H, Dk), q.dtype),
                         (v, "v", (B, T, H, Dv), q.dtype),
                         (g, "g", (B, T, H, Dk), torch.float32),
                         (beta, "beta", (B, T, H), torch.float32),
                         (state, "state", (B, H, Dk, Dv), torch.float32)):
        _check(t, n, s_, dt, dev)
    if o is None:
        o = torch.empty((B, T, H, Dv), dtype=q.dtype, device=dev)
    _check(o, "o", (B, T, H, Dv), q.dtype, dev)
    if u is None:
        u = torch.empty((B, T, H, Dv), dtype=torch.float32, device=dev)
    _check(u, "u", (B, T, H, Dv), torch.float32, dev)
    st = lib.kda_spec_verify(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                             _ptr(state), _ptr(o), _ptr(u), B, T, H, Dk, Dv,
                             scale, _dtype_code(q), _stream(dev))
    if st != KDA_OK:
        raise KDAError("kda_spec_verify", st)
    return o, u


def kda_spec_commit(k, g, u, accepted, state):
    """Advance `state` [B, H, Dk, Dv] in place by accepted[b] (device int32
    [B]) of the draft tokens verified with kda_spec_verify.  Returns state."""
    lib = load()
    B, T, H, Dk = k.shape
    Dv = u.shape[-1]
    dev = k.device
    for t, n, s_, dt in ((k, "k", (B, T, H, Dk), k.dtype),
                         (g, "g", (B, T, H, Dk), torch.float32),
                         (u, "u", (B, T, H, Dv), torch.float32),
                         (accepted, "accepted", (B,), torch.int32),
                         (state, "state", (B, H, Dk, Dv), torch.float32)):
        _check(t, n, s_, dt, dev)
    st = lib.kda_spec_commit(_ptr(k), _ptr(g), _ptr(u), _ptr(accepted),
                             _ptr(state), B, T, H, Dk, Dv, _dtype_code(k),
                             _stream(dev))
    if st != KDA_OK:
        raise KDAError("kda_spec_commit", st)
    return state


def _spec_step(entry, q, k, v, g, beta, state, state_idx, k_prev, g_prev,
               u_prev, accepted_prev, scale, o, u):
    lib = load()
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    dev = q.device
    for t, n, s_, dt in ((q, "q", (B, T, H, Dk), q.dtype),
                         (k, "k", (B, T, H, Dk), q.dtype),
                         (v, "v", (B, T, H, Dv), q.dtype),
                         (g, "g", (B, T, H, Dk), torch.float32),
                         (beta, "beta", (B, T, H), torch.float32)):
        _check(t, n, s_, dt, dev)
    slots = state.shape[0]
    _check(state, "state", (slots if state_idx is not None else B, H, Dk, Dv),
           torch.float32, dev)
    if state_idx is not None:
        _check(state_idx, "state_idx", (B,), torch.int32, dev)
    T_prev = 0
    if k_prev is not None:
        T_prev = k_prev.shape[1]
        for t, n, s_, dt in ((k_prev, "k_prev", (B, T_prev, H, Dk), q.dtype),
                             (g_prev, "g_prev", (B, T_prev, H, Dk),
                              torch.float32),
                             (u_prev, "u_prev", (B, T_prev, H, Dv),
                              torch.float32),
                             (accepted_prev, "accepted_prev", (B,),
                              torch.int32)):
            if t is None:
                raise ValueError("%s is required with k_prev" % n)
            _check(t, n, s_, dt, dev)
    if o is None:
        o = torch.empty((B, T, H, Dv), dtype=q.dtype, device=dev)
    _check(o, "o", (B, T, H, Dv), q.dtype, dev)
    if u is None:
        u = torch.empty((B, T, H, Dv), dtype=torch.float32, device=dev)
    _check(u, "u", (B, T, H, Dv), torch.float32, dev)
    head = (_ptr(k_prev), _ptr(g_prev), _ptr(u_prev), _ptr(accepted_prev),
            T_prev, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta))
    tail = (B, T, H, Dk, Dv, scale, _dtype_code(q), _stream(dev))
    if state_idx is None:
        st = lib.kda_spec_step(*head, _ptr(state), _ptr(o), _ptr(u), *tail)
    else:
        st = lib.kda_spec_step_indexed(*head, _ptr(state), _ptr(state_idx),
                                       slots, _ptr(o), _ptr(u), *tail)
    if st != KDA_OK:
        raise KDAError(entry, st)
    return o, u


def kda_spec_step(q, k, v, g, beta, state, *, k_prev=None, g_prev=None,
                  u_prev=None, accepted_prev=None, scale: float = 1.0,
                  o=None, u=None):
    """Commit the previous draft's accepted prefix to `state` (in place) and
    verify the new draft from the updated state, in one pass over the state:
    kda_spec_commit(k_prev, g_prev, u_prev, accepted_prev, state) followed by
    kda_spec_verify(q, k, v, g, beta, state), bit for bit.  Without k_prev
    (no previous draft) it is kda_spec_verify; with a draft of T = 0 tokens
    (q of shape [B, 0, H, Dk]) it is kda_spec_commit.  u may be u_prev
    itself when both drafts have the same length.  Returns (o, u)."""
    return _spec_step("kda_spec_step", q, k, v, g, beta, state, None, k_prev,
                      g_prev, u_prev, accepted_prev, scale, o, u)


def kda_spec_step_indexed(q, k, v, g, beta, state_pool, state_idx, *,
                          k_prev=None, g_prev=None, u_prev=None,
                          accepted_prev=None, scale: float = 1.0, o=None,
                          u=None):
    """kda_spec_step with the states in a pool: sequence b uses row
    state_idx[b] (device int32 [B]) of state_pool [slots, H, Dk, Dv]; a slot
    outside [0, slots) is padding.  Returns (o, u)."""
    return _spec_step("kda_spec_step_indexed", q, k, v, g, beta, state_pool,
                      state_idx, k_prev, g_prev, u_prev, accepted_prev, scale,
                      o, u)


def kda_output_norm_gate(o, z, w, *, eps: float = 1e-6, y=None):
    """y = o * rsqrt(mean(o^2) + eps) * w * sigmoid(z) per (token, head) row.

    o, z: [..., H, Dv] (bf16 or fp32, same dtype); w: [Dv] fp32.  y may be
    o itself.  Returns y.
    """
    lib = load()
    Dv = o.shape[-1]
    H = o.shape[-2]
    tokens = o.numel() // (H * Dv) if o.numel() else 0
    dev = o.device
    _check(z, "z", tuple(o.shape), o.dtype, dev)
    _check(w, "w", (Dv,), torch.float32, dev)
    if not o.is_contiguous():
        raise ValueError("o must be contiguous")
    if y is None:
        y = torch.empty_like(o)
    _check(y, "y", tuple(o.shape), o.dtype, dev)
    st = lib.kda_output_norm_gate(_ptr(o), _ptr(z), _ptr(w), eps, _ptr(y),
                                  tokens, H, Dv, _dtype_code(o), _stream(dev))
    if st != KDA_OK:
        raise KDAError("kda_output_norm_gate", st)
    return y


def kda_decode_step_gated(q, k, v, g, beta, state, z, w, *,
                          eps: float = 1e-6, scale: float = 1.0, y=None):
    """kda_decode_step with the output epilogue fused: returns
    y = o * rsqrt(mean(o^2) + eps) * w * sigmoid(z) [B, H, Dv]; `state` is
    updated in place."""
    lib = load()
    B, H, Dk = q.shape
    Dv = v.shape[-1]
    dev = q.device
    for t, n, s_, dt in ((q, "q", (B, H, Dk), q.dtype),
                         (k, "k", (B, H, Dk), q.dtype),
                         (v, "v", (B, H, Dv), q.dtype),
                         (g, "g", (B, H, Dk), torch.float32),
                         (beta, "beta", (B, H), torch.float32),
                         (state, "state", (B, H, Dk, Dv), torch.float32),
                         (z, "z", (B, H, Dv), q.dtype),
                         (w, "w", (Dv,), torch.float32)):
        _check(t, n, s_, dt, dev)
    if y is None:
        y = torch.empty((B, H, Dv), dtype=q.dtype, device=dev)
    _check(y, "y", (B, H, Dv), q.dtype, dev)
    st = lib.kda_decode_step_gated(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state), _ptr(z),
        _ptr(w), eps, _ptr(y), B, H, Dk, Dv, scale, _dtype_code(q),
        _stream(dev))
    if st != KDA_OK:
        raise KDAError("kda_decode_step_gated", st)
    return y


def kda_decode_step_gated_indexed(q, k, v, g, beta, state_pool, state_idx, z,
                                  w, *, eps: float = 1e-6, scale: float = 1.0,
                                  y=None):
    """kda_decode_step_gated with the states in a pool (as
    kda_decode_step_indexed).  Returns y [B, H, Dv]."""
    lib = load()
    B, H, Dk = q.shape
    Dv = v.shape[-1]
    dev = q.device
    slots = state_pool.shape[0]
    for t, n, s_, dt in ((q, "q", (B, H, Dk), q.dtype),
                         (k, "k", (B, H, Dk), q.dtype),
                         (v, "v", (B, H, Dv), q.dtype),
                         (g, "g", (B, H, Dk), torch.float32),
                         (beta, "beta", (B, H), torch.float32),
                         (state_pool, "state_pool", (slots, H, Dk, Dv),
                          torch.float32),
                         (state_idx, "state_idx", (B,), torch.int32),
                         (z, "z", (B, H, Dv), q.dtype),
                         (w, "w", (Dv,), torch.float32)):
        _check(t, n, s_, dt, dev)
    if y is None:
        y = torch.empty((B, H, Dv), dtype=q.dtype, device=dev)
    _check(y, "y", (B, H, Dv), q.dtype, dev)
    st = lib.kda_decode_step_gated_indexed(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state_pool),
        _ptr(state_idx), slots, _ptr(z), _ptr(w), eps, _ptr(y), B, H, Dk, Dv,
        scale, _dtype_code(q), _stream(dev))
    if st != KDA_OK:
        raise KDAError("kda_decode_step_gated_indexed", st)
    return y


def kda_prefill_varlen_prologue(xq, xk, xv, conv_w, a, b, cu_seqlens,
                                max_seqlen: int, initial_state=None, *,
                                chunk_size: int = 64, scale: float = 1.0,
                                output_final_state: bool = True,
                                final_state=None, o=None, workspace=None):
    """kda_prefill_varlen with the input prologue fused: xq, xk, xv
    [total_T, H, D] (inputs of the short convolutions), conv_w [3, H, D, 4]
    fp32, a [total_T, H, Dk] fp32 (g = -5 sigmoid(a)), b [total_T, H] fp32
    (beta = sigmoid(b)).  Returns (o, final_state)."""
    lib = load()
    total_T, H, Dk = xq.shape
    Dv = xv.shape[-1]
    dev = xq.device
    N = cu_seqlens.numel() - 1
    for t, n, s_, dt in ((xq, "xq", (total_T, H, Dk), xq.dtype),
                         (xk, "xk", (total_T, H, Dk), xq.dtype),
                         (xv, "xv", (total_T, H, Dv), xq.dtype),
                         (conv_w, "conv_w", (3, H, Dk, 4), torch.float32),
                         (a, "a", (total_T, H, Dk), torch.float32),
                         (b, "b", (total_T, H), torch.float32),
                         (cu_seqlens, "cu_seqlens", (N + 1,), torch.int32)):
        _check(t, n, s_, dt, dev)
    if initial_state is not None:
        _check(initial_state, "initial_state", (N, H, Dk, Dv), torch.float32,
               dev)
    if final_state is None and output_final_state:
        final_state = torch.empty((N, H, Dk, Dv), dtype=torch.float32,
                                  device=dev)
    if final_state is not None:
        _check(final_state, "final_state", (N, H, Dk, Dv), torch.float32, dev)
    if o is None:
        o = torch.empty((total_T, H, Dv), dtype=xq.dtype, device=dev)
    _check(o, "o", (total_T, H, Dv), xq.dtype, dev)
    if workspace is None:
        workspace = workspace_for(N, total_T, H, Dk, Dv, chunk_size, dev)
    st = lib.kda_prefill_varlen_prologue(
        _ptr(xq), _ptr(xk), _ptr(xv), _ptr(conv_w), _ptr(a), _ptr(b),
        _ptr(cu_seqlens), N, total_T, int(max_seqlen), _ptr(initial_state),
        _ptr(final_state), _ptr(o), H, Dk, Dv, chunk_size, scale,
        _dtype_code(xq), _ptr(workspace), workspace.numel(), _stream(dev))
    if st != KDA_OK:
        raise KDAError("kda_prefill_varlen_prologue", st)
    return o, final_state
