"""Input generators: shapes, seeds, poison, and the latent-cache byte model."""
import math

import torch

import workloads


def test_cache_byte_model_c2():
    # glossary capacity model M = L * B * T * (d_c + d_rope) * s with one layer, bf16 (s = 2)
    c = workloads.CONFIGS[2]
    assert c.b * c.t_max * (512 + 64) * 2 == 301_989_888


def test_scale():
    assert abs(workloads.SCALE - 1.0 / math.sqrt(192.0)) < 1e-15
    assert abs(workloads.SCALE - 0.07216878364870323) < 1e-15


def test_c1_shapes_and_poison():
    w = workloads.make(1)
    assert w.cache.shape == (2, 257, 576) and w.cache.dtype == torch.float32
    assert w.q_nope.shape == (2, 16, 128) and w.q_rope.shape == (2, 16, 64)
    assert w.w_uk.shape == (16, 128, 512) and w.w_uv.shape == (16, 512, 128)
    assert w.seqlens.tolist() == [128, 257]
    assert torch.isnan(w.cache[0, 128:]).all() and torch.isfinite(w.cache[0, :128]).all()
    assert torch.isfinite(w.cache[1]).all()
    # weights scaled by 1/sqrt(fan_in)
    assert abs(float(w.w_uk.float().std()) - 1 / math.sqrt(128)) < 0.01
    assert abs(float(w.w_uv.float().std()) - 1 / math.sqrt(512)) < 0.005


def test_seeded_and_deterministic():
    a = workloads.make_custom(2, 3, [5, 9], seed=5)
    b = workloads.make_custom(2, 3, [5, 9], seed=5)
    assert torch.equal(a.q_prime, b.q_prime)
    assert torch.equal(torch.nan_to_num(a.cache), torch.nan_to_num(b.cache))
    c = workloads.make_custom(2, 3, [5, 9], seed=6)
    assert not torch.equal(a.q_prime, c.q_prime)


def test_ragged_lengths_range():
    # a batch-truncated ragged workload keeps lengths in U[1, 32768] and poisons past them
    w = workloads.make_custom(3, 2, [1, 40, 17], t_max=64, seed=3)
    assert w.cache.shape == (3, 64, 576)
    for i, L in enumerate([1, 40, 17]):
        assert torch.isnan(w.cache[i, L:].float()).all()
        assert torch.isfinite(w.cache[i, :L].float()).all()
