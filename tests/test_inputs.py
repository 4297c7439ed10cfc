"""Seeded input generators: recipes, determinism, bf16 rounding (CPU)."""
import numpy as np
import torch

from linear_recurrent_attention_kda_amd import inputs


def test_bf16_round_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -0.0, 0.0,
                                  2 ** -130, 3e38], np.float32)])
    ours = inputs.bf16_round(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(ours.view(np.uint32), ref.view(np.uint32))
    bits = inputs.bf16_bits(ours)
    back = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
    assert np.array_equal(back.float().numpy().view(np.uint32),
                          ours.view(np.uint32))


def test_tiny_recipe():
    p = inputs.make("tiny", seed=0)
    assert p.q.shape == (1, 64, 2, 16) and p.v.shape == (1, 64, 2, 16)
    assert p.beta.shape == (1, 64, 2) and p.initial_state is None
    assert np.allclose(np.linalg.norm(p.q, axis=-1), 1, atol=1e-5)
    assert np.all(p.g <= 0) and np.all(p.g >= -5)
    assert np.all((p.beta > 0) & (p.beta < 1))
    p2 = inputs.make("tiny", seed=0)
    assert np.array_equal(p.k, p2.k) and np.array_equal(p.g, p2.g)
    p3 = inputs.make("tiny", seed=1)
    assert not np.array_equal(p.k, p3.k)


def test_bf16_workloads_are_bf16_exact_and_sized():
    p = inputs.make("prefill", T=256, H=4)
    for x in (p.q, p.k, p.v):
        assert np.array_equal(inputs.bf16_round(x), x)
    assert p.q.shape == (1, 256, 4, 128)
    d = inputs.make("decode", B=4, H=3)
    assert d.initial_state.shape == (4, 3, 128, 128)
    assert abs(float(d.initial_state.std()) - 0.02) < 2e-3


def test_varlen_lengths_and_near_bound_decay():
    p = inputs.make("varlen", H=2, K=16, V=16)
    L = p.seq_lengths
    assert len(L) == 8 and L.min() >= 1024 and L.max() <= 16384
    assert p.cu_seqlens[0] == 0 and p.cu_seqlens[-1] == p.q.shape[0]
    lo = inputs.make("long", T=512, H=2, K=16, V=16)
    mid = inputs.make("prefill", T=512, H=2, K=16, V=16)
    assert lo.g.mean() < mid.g.mean() - 1.0       # drawn near the -5 bound
    assert lo.initial_state is not None
