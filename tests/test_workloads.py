"""The seeded input generator: determinism, distribution, rounding."""
import numpy as np
import torch

import workloads as W


def test_generator_is_deterministic_and_keyed():
    a = W.fill_normal((64, 33), 1.0, "f32", 0, 1, 0)
    b = W.fill_normal((64, 33), 1.0, "f32", 0, 1, 0)
    assert torch.equal(a, b)
    for other in [W.fill_normal((64, 33), 1.0, "f32", 1, 1, 0),
                  W.fill_normal((64, 33), 1.0, "f32", 0, 2, 0),
                  W.fill_normal((64, 33), 1.0, "f32", 0, 1, 1)]:
        assert (a != other).float().mean() > 0.99


def test_mixer_is_a_bijection_on_a_window():
    v = torch.arange(1 << 20, dtype=torch.int64)
    h = W.mix32(v)
    assert h.unique().numel() == v.numel()
    assert int(h.max()) < (1 << 32) and int(h.min()) >= 0


def test_moments_close_to_standard_normal():
    a = W.fill_normal((1 << 20,), 1.0, "f32", 0, 5, 0).double()
    assert abs(a.mean().item()) < 5e-3
    assert abs(a.std().item() - 1.0) < 5e-3
    # quantile table is symmetric with exact zero mean
    z = W.quantile_table(1.0, "f32").astype(np.float64)
    assert np.array_equal(z, -z[::-1])


def test_bf16_rounding_matches_torch_round_to_nearest_even():
    x = torch.from_numpy(W.quantile_table(0.37, "f32").copy())
    ours = torch.from_numpy(W.f32_to_bf16_bits(x.numpy()).view(np.int16))
    theirs = x.to(torch.bfloat16).view(torch.int16)
    assert torch.equal(ours, theirs)
    back = W.bf16_bits_to_f32(W.f32_to_bf16_bits(x.numpy()))
    assert np.array_equal(back, x.to(torch.bfloat16).float().numpy())


def test_stacked_equals_per_expert():
    wl = W.custom_workload("s", T=8, d_model=16, n_routed=3, top_k=1, n_shared=1, d_ff=8,
                           dtype="bf16", expert_bias=True)
    w1, b1, w2, b2 = wl.stacked(shared=False)
    for e in range(3):
        r = wl.routed_expert(e)
        assert torch.equal(w1[e], r[0]) and torch.equal(b1[e], r[1])
        assert torch.equal(w2[e], r[2]) and torch.equal(b2[e], r[3])
