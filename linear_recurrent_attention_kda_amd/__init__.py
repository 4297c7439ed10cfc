"""libkda: Kimi Delta Attention for AMD Instinct MI355X (gfx950).

The compute path is the C-ABI shared library ``libkda.so`` (hand-written HIP
kernels); ``kda`` is a thin ctypes binding with the same entry-point names.
Importing this package loads nothing; the first call into ``kda`` loads the
library and raises if it is missing.
"""
__all__ = ["kda", "inputs", "counts"]
