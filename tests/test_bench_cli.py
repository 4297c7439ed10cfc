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


def _stored(kind, name):
    kv = {}
    for line in open(os.path.join(ROOT, "profiles", "%s_%s.txt" % (kind, name))):
        if "=" in line and not line.startswith("#"):
            key, val = line.split("=", 1)
            kv[key.strip()] = val.strip()
    return kv


def test_stored_mfma_counts_equal_the_kernels_products():
    """The matrix-core FLOPs rocprofv3 counted per launch (512 per MOPS unit)
    equal a count of the products each kernel issues, on the 8192-token,
    96-head prefill (C = 64, d = 128: 128 chunks x 96 heads)."""
    C, D, units = 64, 128, 128 * 96
    # prep: A and M over the 10 sub-tile pairs n <= m (16 x 16 x D each);
    # W and U~ per 16-row tile m over k-extents 32, 32, 64, 64 (16 (m + 1)
    # rounded up to the 32-deep bf16 MFMA step)
    prep = 10 * 2 * (16 * 16 * D * 2) + 2 * (16 * D * 2) * (32 + 32 + 64 + 64)
    # recurrence: W S, Q^ S and K^T U (2 C D^2 each) and M U over the six
    # of M's eight 16 x 32 fragments that are not all zero
    recur = 3 * 2 * C * D * D + 2 * C * C * D * 6 // 8
    assert float(_stored("mfma", "kda_prep")["bf16_mops"]) * 512 == \
        prep * units
    assert float(_stored("mfma", "kda_recur")["bf16_mops"]) * 512 == \
        recur * units
    assert float(_stored("mfma", "kda_decode")["bf16_mops"]) == 0.0


def test_parity_figure_is_the_worst_sequence_head_slice():
    """The oracle leg's parity figure: per (sequence, head) slice, the
    largest absolute error over the slice's largest reference magnitude,
    maximised over slices.  One slice scaled by 1.01 reads 1e-2, whether
    the layout is packed tokens (with sequence bounds) or states."""
    import numpy as np
    sys.path.insert(0, ROOT)
    import bench
    ref = np.random.default_rng(0).standard_normal((100, 3, 8))
    x = ref.copy()
    x[10:20, 1] *= 1.01          # inside sequence 0, head 1
    assert abs(bench._rel_per_slice(x, ref, np.array([0, 50, 100]))
               - 0.01) < 1e-12
    # the same rows measured as their own sequence: the whole slice is off
    # by 1 %, the other sequences not at all
    assert abs(bench._rel_per_slice(x, ref, np.array([0, 10, 20, 100]))
               - 0.01) < 1e-12
    assert bench._rel_per_slice(ref, ref, np.array([0, 0, 100])) == 0.0
    s = ref.reshape(4, 25, 3, 8).transpose(0, 2, 1, 3)   # [seq, head, ...]
    t = s.copy()
    t[2, 0] += 0.5 * np.abs(s[2, 0]).max()
    assert abs(bench._rel_per_slice(t, s) - 0.5) < 1e-12
