"""The pins are sharp enough: every plausible mistake planted in a copy of
the oracle (a dropped term, a wrong sign, a swapped operand or index, a
transposed access, the wrong step order) makes at least one pin fail.

The mistakes are planted only in temporary copies of the oracle source,
compiled with the same flags, on the CPU.
"""
import os

import pytest

import oracle
import oracle_pins as P

# (name, original text, planted text).  Each original must occur exactly once.
MUTATIONS = [
    ("no_decay", "row[j] *= alpha;", "row[j] *= 1.0;"),
    ("decay_wrong_channel", "const double alpha = exp(gt[c]);",
     "const double alpha = exp(gt[K - 1 - c]);"),
    ("delta_sign", "u[j] = bt * (vt[j] - u[j]);",
     "u[j] = bt * (vt[j] + u[j]);"),
    ("no_beta", "u[j] = bt * (vt[j] - u[j]);", "u[j] = (vt[j] - u[j]);"),
    ("write_with_q", "row[j] += kc * u[j];", "row[j] += qt[c] * u[j];"),
    ("read_with_k", "ot[j] += row[j] * qc;", "ot[j] += row[j] * kt[c];"),
    ("no_scale", "ot[j] *= scale;", "ot[j] *= 1.0;"),
    ("transposed_read",
     "const double* row = S + (int64_t)c * V;\n      for (int32_t j = 0; j < V; ++j) u[j] += row[j] * kc;",
     "for (int32_t j = 0; j < V; ++j) u[j] += S[(int64_t)j * V + c % V] * kc;"),
    ("drop_last_token", "run_one(cu_seqlens[n], cu_seqlens[n + 1],",
     "run_one(cu_seqlens[n], cu_seqlens[n + 1] - (cu_seqlens[n + 1] > cu_seqlens[n]),"),
    ("state_by_head", "memcpy(S, S0 + (size_t)p * sz,",
     "memcpy(S, S0 + (size_t)h * sz,"),
    ("value_head_stride", "const double* vt = v + (t * H + h) * (int64_t)V;",
     "const double* vt = v + (t * H + 0) * (int64_t)V;"),
]

# Step order: decay applied after the correction (forget moved behind the
# delta computation) -- planted by swapping two blocks.
_FORGET = """    /* 1. forget: scale row c of S by alpha_t[c] = exp(g_t[c]). */
    for (int32_t c = 0; c < K; ++c) {
      const double alpha = exp(gt[c]);
      double* row = S + (int64_t)c * V;
      for (int32_t j = 0; j < V; ++j) row[j] *= alpha;
    }
"""


def _variant(tmp_path, name, src_text):
    c = tmp_path / ("oracle_%s.c" % name)
    c.write_text(src_text)
    so = str(tmp_path / ("liboracle_%s.so" % name))
    oracle.compile_source(str(c), so)
    return oracle.load_library(so)


def _caught(lib):
    for pin in P.ALL_PINS:
        try:
            pin(lib=lib)
        except (AssertionError, RuntimeError, ValueError):
            return True
    return False


@pytest.mark.parametrize("name,old,new", MUTATIONS,
                         ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(tmp_path, name, old, new):
    src = open(oracle.SOURCE).read()
    assert src.count(old) == 1, name
    lib = _variant(tmp_path, name, src.replace(old, new))
    assert _caught(lib), "pins missed planted mistake %r" % name


def test_forget_after_correct_is_caught(tmp_path):
    src = open(oracle.SOURCE).read()
    assert src.count(_FORGET) == 1
    body = src.replace(_FORGET, "")
    anchor = "    /* 3. write: S <- S + k u^T. */\n"
    assert body.count(anchor) == 1
    body = body.replace(anchor, _FORGET + anchor)
    assert _caught(_variant(tmp_path, "forget_after_correct", body))


def test_read_before_write_is_caught(tmp_path):
    src = open(oracle.SOURCE).read()
    start = src.index("    /* 4. read: o = scale * S^T q. */")
    end = src.index("  }\n}\n", start)
    read_block = src[start:end]
    body = src[:start] + src[end:]
    anchor = "    /* 3. write: S <- S + k u^T. */\n"
    body = body.replace(anchor, read_block + anchor)
    assert _caught(_variant(tmp_path, "read_before_write", body))


def test_unmutated_copy_passes(tmp_path):
    lib = _variant(tmp_path, "identity", open(oracle.SOURCE).read())
    assert not _caught(lib)
