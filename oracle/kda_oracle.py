"""Loader and numpy front end for the fp64 KDA oracle (``kda_oracle.c``).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, the smoke check and the CPU
baseline leg of the benchmark may import this module.  The HIP library never
imports, links or calls it, and it never imports the HIP library.

The oracle is the per-token recurrence written out in fp64 (forget, correct,
write, read), following "Two Paths: Kimi K3 vs DeepSeek V4 Architecture
Divergence" (section "Attention: 69 Layers of Compressed Memory ...": the
forget -> correct -> write update of a fixed-size state) and "Kimi K3: The
Manos, The Mythos, The Legendos" (sections "Kimi Delta Attention" and
"FlashKDA algorithm": the delta rule with a diagonal, per-channel forget gate).

Inputs of any float dtype are upcast exactly to float64 before the call, so
the oracle sees exactly the values (bf16 or fp32) that the GPU saw.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
SOURCE = _SRC
_BUILD_DIR = os.path.join(_HERE, "_build")
_LIB_PATH = os.path.join(_BUILD_DIR, "libkda_oracle.so")

# Plain IEEE fp64: no fast-math, no FMA contraction, so the loop is the
# definition evaluated in the written order.
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
          "-fno-fast-math", "-ffp-contract=off"]

_lock = threading.Lock()
_lib = None


def compile_source(src: str, out: str) -> str:
    """gcc one oracle source file into a shared library at ``out``."""
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.check_call(["gcc", *CFLAGS, src, "-o", tmp, "-lm"])
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into ``oracle/_build/libkda_oracle.so``."""
    os.makedirs(_BUILD_DIR, exist_ok=True)
    if force or not os.path.exists(_LIB_PATH) or \
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        compile_source(_SRC, _LIB_PATH)
    return _LIB_PATH


def load_library(path: str):
    """Load an oracle build (the default one, or a test-built variant)."""
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    lib.kda_oracle_run.restype = ctypes.c_int
    lib.kda_oracle_run.argtypes = [
        ctypes.c_int32, ctypes.POINTER(ctypes.c_int64), ctypes.c_int32,
        ctypes.c_int32, ctypes.c_int32, dp, dp, dp, dp, dp, dp,
        ctypes.c_double, dp, dp]
    lib.kda_oracle_threads.restype = ctypes.c_int
    lib.kda_oracle_set_threads.argtypes = [ctypes.c_int]
    lib.kda_oracle_set_threads.restype = None
    return lib


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH) or \
                    os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
                build(force=True)
            _lib = load_library(_LIB_PATH)
    return _lib


def threads() -> int:
    """Number of OpenMP threads the oracle will use."""
    return int(_load().kda_oracle_threads())


def set_threads(n: int) -> None:
    _load().kda_oracle_set_threads(int(n))


def _f64(x):
    return None if x is None else np.ascontiguousarray(x, dtype=np.float64)


def _ptr(x):
    if x is None:
        return ctypes.POINTER(ctypes.c_double)()
    return x.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def run_varlen(q, k, v, g, beta, cu_seqlens, initial_state=None, scale=1.0,
               want_output=True, lib=None):
    """The recurrence over packed sequences.

    q, k, g: [total_T, H, K]; v: [total_T, H, V]; beta: [total_T, H];
    cu_seqlens: [N+1] integers; initial_state: [N, H, K, V] or None (zeros).
    Returns (o [total_T, H, V] float64 or None, S [N, H, K, V] float64).
    """
    q, k, v, g, beta = map(_f64, (q, k, v, g, beta))
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int64)
    total_T, H, K = q.shape
    V = v.shape[2]
    N = cu.shape[0] - 1
    if k.shape != (total_T, H, K) or g.shape != (total_T, H, K):
        raise ValueError("q, k, g must share the shape [total_T, H, K]")
    if v.shape != (total_T, H, V) or beta.shape != (total_T, H):
        raise ValueError("v must be [total_T, H, V] and beta [total_T, H]")
    if cu[0] != 0 or cu[-1] != total_T or np.any(np.diff(cu) < 0):
        raise ValueError("cu_seqlens must start at 0, end at total_T and "
                         "never decrease")
    s0 = _f64(initial_state)
    if s0 is not None and s0.shape != (N, H, K, V):
        raise ValueError("initial_state must be [N, H, K, V]")
    o = np.zeros((total_T, H, V), np.float64) if want_output else None
    s_out = np.zeros((N, H, K, V), np.float64)
    rc = (lib or _load()).kda_oracle_run(
        N, cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), H, K, V,
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(s0),
        float(scale), _ptr(o), _ptr(s_out))
    if rc != 0:
        raise RuntimeError("kda_oracle_run failed with status %d" % rc)
    return o, s_out


def run_fixed(q, k, v, g, beta, initial_state=None, scale=1.0,
              want_output=True, lib=None):
    """Fixed-length batch: q, k, g [B, T, H, K]; v [B, T, H, V]; beta [B, T, H];
    initial_state [B, H, K, V] or None.  Returns (o [B, T, H, V], S [B, H, K, V])."""
    B, T, H, K = np.shape(q)
    V = np.shape(v)[3]
    cu = np.arange(B + 1, dtype=np.int64) * T
    o, s = run_varlen(np.reshape(q, (B * T, H, K)), np.reshape(k, (B * T, H, K)),
                      np.reshape(v, (B * T, H, V)), np.reshape(g, (B * T, H, K)),
                      np.reshape(beta, (B * T, H)), cu, initial_state, scale,
                      want_output, lib)
    return (None if o is None else o.reshape(B, T, H, V)), s


def run_decode(q, k, v, g, beta, state, scale=1.0, lib=None):
    """One token per sequence: q, k, g [B, H, K]; v [B, H, V]; beta [B, H];
    state [B, H, K, V].  Returns (o [B, H, V], new state [B, H, K, V])."""
    B, H, K = np.shape(q)
    V = np.shape(v)[2]
    cu = np.arange(B + 1, dtype=np.int64)
    return run_varlen(q, k, v, g, beta, cu, state, scale, lib=lib)
