"""Seeded random mixes of the supported sizes against the fp64 oracle.

Each case draws, from its own seed: head dims d_k and d_v (independently,
multiples of 16 up to 128), the chunk size, a head count across the
thresholds that pick 16-, 32- and 64-wide recurrence slices and the streamed
kernel, fixed-length batches or packed sequences (empty, shorter than a
chunk, exact chunk multiples, ragged), the storage dtype, an initial state
or none, the decay's mean (ordinary, or near the g >= -5 bound), and the
output scale.  The prefill and a decode step on the same sizes are compared
with the oracle to the usual bars (per (sequence, head) slices; see
gpu_util).  The cases are fixed by their seeds, so a failure names a case
that reproduces."""
import numpy as np
import pytest

from conftest import gpu_available
from linear_recurrent_attention_kda_amd import inputs

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

import gpu_util as U  # noqa: E402

N_CASES = 48


def draw(seed):
    rng = np.random.default_rng(7000 + seed)
    dims = [16 * i for i in range(1, 9)]
    c = dict(
        K=int(rng.choice(dims)),
        V=int(rng.choice(dims)),
        C=int(rng.choice([16, 32, 64])),
        H=int(rng.choice([1, 2, 3, 7, 33, 64, 70, 130])),
        dtype="bf16" if rng.random() < 0.75 else "fp32",
        s0=bool(rng.random() < 0.7),
        g_mu=float(rng.choice([0.0, 2.0])),
    )
    scale = float(rng.choice([1.0, 0.5, c["K"] ** -0.5]))
    if rng.random() < 0.25:  # fixed-length batch
        c.update(kind="prefill", B=int(rng.integers(1, 4)),
                 T=int(rng.integers(1, 300)))
    else:
        n = int(rng.integers(1, 7))
        lengths = rng.integers(0, 260, size=n)
        for i in range(n):  # some exact chunk multiples and empty sequences
            u = rng.random()
            if u < 0.15:
                lengths[i] = 0
            elif u < 0.3:
                lengths[i] = c["C"] * int(rng.integers(1, 5))
        c.update(kind="varlen", lengths=[int(x) for x in lengths])
    return c, scale


def case_label(c, scale):
    shape = ("B=%d T=%d" % (c["B"], c["T"]) if c["kind"] == "prefill"
             else "lengths=%s" % c["lengths"])
    return "Dk=%d Dv=%d C=%d H=%d %s %s s0=%s g_mu=%.0f scale=%.3f" % (
        c["K"], c["V"], c["C"], c["H"], shape, c["dtype"], c["s0"],
        c["g_mu"], scale)


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_prefill_and_decode(seed):
    c, scale = draw(seed)
    label = "random case %d: %s" % (seed, case_label(c, scale))
    kind = c.pop("kind")
    p = inputs.make(kind, seed=seed, **c)
    U.check_prefill(p, label=label, scale=scale,
                    head_group=48 if p.H > 48 else None)
    d = inputs.make("decode", seed=seed, B=3, H=p.H, K=p.K, V=p.V,
                    dtype=p.dtype)
    U.check_decode(d, scale=scale)
