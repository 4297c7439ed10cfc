"""fp64 CPU oracle for Kimi Delta Attention -- test infrastructure only.

Only ``tests/``, the smoke check and the benchmark's CPU-baseline leg use
this package; the HIP library and its Python binding never import it.
"""
from .epilogue import norm_gate
from . import prologue
from .kda_oracle import (SOURCE, build, compile_source, load_library,
                         run_decode, run_fixed, run_varlen, set_threads,
                         threads)

__all__ = ["SOURCE", "build", "compile_source", "load_library", "norm_gate",
           "prologue", "run_decode", "run_fixed", "run_varlen", "set_threads",
           "threads"]
