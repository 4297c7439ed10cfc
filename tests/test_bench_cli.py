"""Host-side checks of bench.py's command line (no GPU needed).

The benchmark measures one GPU: asked for more it must stop before touching
a device and say why.  Its derived figures use the pages' counts from
linear_recurrent_attention_kda_amd/counts.py, checked here against the
decode workload's byte count ("Kimi K3: The Manos, The Mythos, The
Legendos", section "Complexity analysis": 8 d^2 bytes of fp32 state per head
and token).
"""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"),
                        "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_decode_byte_count_of_the_workload():
    from linear_recurrent_attention_kda_amd import counts
    # 64 sequences x 96 heads, d = 128: the fp32 state read and written once
    assert counts.decode_bytes_per_head(128) * 64 * 96 == 805_306_368
