"""Build tests/c_consumer/kda_from_c, a program that uses libkda through its
C ABI only (hipcc, linked against the in-tree libkda.so by a relative rpath).

    python tests/c_consumer/build_consumer.py
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
PKG = os.path.join(ROOT, "linear_recurrent_attention_kda_amd")
SRC = os.path.join(HERE, "kda_from_c.cpp")
OUT = os.path.join(HERE, "kda_from_c")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build() -> str:
    """Compile and link the consumer; returns its path."""
    if not os.path.exists(os.path.join(PKG, "libkda.so")):
        raise RuntimeError("build libkda.so first")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O2", "-std=c++17",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I" + os.path.join(ROOT, "include"), SRC, "-o", OUT + ".tmp",
           "-L" + PKG, "-lkda",
           "-Wl,-rpath,$ORIGIN/../../linear_recurrent_attention_kda_amd"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(OUT + ".tmp", OUT)
    return OUT


if __name__ == "__main__":
    print(build())
    sys.exit(0)
