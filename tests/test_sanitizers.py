"""CPU sanitizer builds (no GPU): the fp64 oracle built with gcc's
AddressSanitizer and UndefinedBehaviorSanitizer and run through pins, and
libkda's host-side validation layer built with the same sanitizers (host
code only, no device code) and driven through every entry point with
invalid arguments.  Any sanitizer report fails the test."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.dirname(os.path.abspath(__file__))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN_OPTS = dict(ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
                UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _no_reports(r):
    text = r.stdout + r.stderr
    assert "AddressSanitizer" not in text, text[-3000:]
    assert "runtime error" not in text, text[-3000:]
    assert r.returncode == 0, text[-3000:]


def test_oracle_under_asan_ubsan(tmp_path):
    if not shutil.which("gcc"):
        pytest.skip("gcc not available")
    so = str(tmp_path / "liboracle_san.so")
    import oracle
    subprocess.check_call(
        ["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-fopenmp",
         "-fno-fast-math", "-ffp-contract=off", "-fno-omit-frame-pointer",
         "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
         oracle.SOURCE, "-o", so, "-lm"])
    libasan = subprocess.check_output(
        ["gcc", "-print-file-name=libasan.so"], text=True).strip()
    script = (
        "import sys; sys.path[:0] = [%r, %r]\n"
        "import oracle, oracle_pins as P\n"
        "lib = oracle.load_library(%r)\n"
        "for pin in (P.pin_brute_force, P.pin_split_resume,\n"
        "            P.pin_linearity_columns, P.pin_pure_decay):\n"
        "    assert pin(lib=lib), pin.__name__\n"
        "print('oracle pins ok under ASan/UBSan')\n" % (ROOT, HERE, so))
    env = dict(os.environ, LD_PRELOAD=libasan, OMP_NUM_THREADS="2",
               **SAN_OPTS)
    r = subprocess.run([sys.executable, "-c", script], env=env,
                       capture_output=True, text=True, timeout=600)
    _no_reports(r)


def test_validation_layer_under_asan_ubsan(tmp_path):
    """kda_api.hip (the C ABI: argument validation, workspace sizes, the
    no-alloc scratch lookup) with the sanitizers on its host code, linked
    with stand-in launchers (tests/sanitize/launch_stubs.cpp) that no
    validation path reaches, driven by tests/sanitize/abi_validation.cpp."""
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    csrc = os.path.join(ROOT, "linear_recurrent_attention_kda_amd", "csrc")
    exe = str(tmp_path / "abi_validation")
    # the sanitizers apply to the host pass only (-Xarch_host before each)
    cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
           "-fno-omit-frame-pointer",
           "-Xarch_host", "-fsanitize=address",
           "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all",
           "-I" + os.path.join(ROOT, "include"), "-I" + csrc,
           os.path.join(HERE, "sanitize", "abi_validation.cpp"),
           os.path.join(csrc, "kda_api.hip"),
           os.path.join(HERE, "sanitize", "launch_stubs.cpp"),
           "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run([exe], env=dict(os.environ, **SAN_OPTS),
                       capture_output=True, text=True, timeout=300)
    _no_reports(r)
    assert "all statuses as expected" in r.stdout
