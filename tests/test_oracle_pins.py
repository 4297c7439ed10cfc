"""The fp64 oracle against what the pages and the mathematics fix.

CPU only.  See ``oracle_pins.py`` for what each pin checks and the passages
it follows.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle_pins as P

GOLDEN = os.path.join(os.path.dirname(__file__), "golden",
                      "page_constants.json")


@pytest.fixture(scope="module", autouse=True)
def _built(oracle_mod):
    return oracle_mod


def test_brute_force_exact():
    assert P.pin_brute_force()


def test_deltanet_is_gradient_step():
    assert P.pin_deltanet_gradient()


def test_gated_deltanet_scalar_gate():
    assert P.pin_deltanet_gradient(scalar_gate=True)


def test_delta_rule_recall():
    assert P.pin_recall()


def test_beta_zero_pure_decay():
    assert P.pin_pure_decay()


def test_linearity_and_column_independence():
    assert P.pin_linearity_columns()


def test_split_resume_decode_varlen():
    assert P.pin_split_resume()


def test_chunked_form_equals_recurrence():
    assert P.pin_chunked()


def test_decode_one_pass_identity():
    assert P.pin_decode_identity()


def test_state_size_constant_in_T(oracle_mod):
    """The state has the same shape (and bytes) after 64 and 4096 tokens
    ("Two Paths ...", section "Attention ...": the matrix size does not
    depend on the sequence length)."""
    rng = np.random.default_rng(0)
    H, K, V = 2, 4, 4
    shapes = []
    for T in (64, 4096):
        q = rng.standard_normal((T, H, K))
        k = q / np.linalg.norm(q, axis=-1, keepdims=True)
        _, S = oracle_mod.run_varlen(q, k, rng.standard_normal((T, H, V)),
                                     -rng.random((T, H, K)),
                                     rng.random((T, H)), [0, T])
        shapes.append((S.shape, S.nbytes))
        assert np.all(np.isfinite(S))
    assert shapes[0] == shapes[1]


def test_page_constants():
    """Sizes and bounds printed on the pages (tests/golden)."""
    c = json.load(open(GOLDEN))
    s = c["state_bytes_per_layer"]
    assert s["heads"] * s["d_head"] ** 2 * s["bytes_per_element"] == s["value"]
    assert s["value"] == 3145728
    # 69 layers: the printed "207 MB" is MiB
    tot = c["state_bytes_all_kda_layers"]["kda_layers"] * s["value"]
    assert tot == 217055232
    assert round(tot / 2 ** 20) == c["state_bytes_all_kda_layers"][
        "value_mb_as_printed"]
    # our fp32 state: twice the printed 2-byte figure, still T-independent
    assert 96 * 128 * 128 * 4 == 2 * s["value"]
    r = c["retention_lower_bound"]
    assert round(math.exp(r["g_min"]), 4) == r["retention_printed"]
    t = c["tile_log_decay_bound"]
    assert t["tile"] * r["g_min"] == t["value"]


def test_bf16_range_of_tile_factors():
    """The 16-row tile's decay factors e^{+-80} are normal bf16 numbers, and
    the overflow horizon at g = -5 is ln(fp32 max)/5 = 17.7 tokens, which is
    why a 16-token tile is the limit ("Two Paths ...", section "Hardware
    Adaptation")."""
    from linear_recurrent_attention_kda_amd.inputs import bf16_round
    bf16_max = float(np.frombuffer(np.uint32(0x7F7F0000).tobytes(),
                                   np.float32)[0])
    bf16_min_normal = 2.0 ** -126
    assert math.exp(80) < bf16_max
    assert math.exp(-80) > bf16_min_normal
    x = bf16_round(np.array([math.exp(80), math.exp(-80)], np.float32))
    assert np.all(np.isfinite(x)) and np.all(x > 0)
    assert abs(x[0] / math.exp(80) - 1) < 2 ** -8
    horizon = math.log(float(np.finfo(np.float32).max)) / 5
    assert 17 < horizon < 18


def test_algorithmic_counts_match_pages():
    """The benchmark's counts are the pages' formulas, and the pages' byte
    terms add up to their stated total."""
    from linear_recurrent_attention_kda_amd import counts
    C, D = 64, 128
    assert counts.decode_flops_per_head(D) == 7 * D * D == 114688
    assert counts.decode_bytes_per_head(D) == 8 * D * D == 131072
    assert counts.prefill_flops_per_chunk(C, D) == 13631488
    terms = 3 * 2 * C * D + 2 * (3 * 2 * C * D + 2 * 2 * C * C) + 2 * 2 * C * D
    assert terms == 8 * C * C + 22 * C * D == counts.prefill_bytes_per_chunk(
        C, D) == 212992
