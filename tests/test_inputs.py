"""The seeded input generator: deterministic, right shapes, dtypes and laws."""

import numpy as np
import torch

from sample_gradient_clipping_amd.inputs import linear_inputs, sample_scales, theta_init


def test_linear_inputs_deterministic_and_shaped():
    A, G = linear_inputs(3, 16, 8, 12, "bf16", "llama_logu", seed=5)
    A2, G2 = linear_inputs(3, 16, 8, 12, "bf16", "llama_logu", seed=5)
    assert A.dtype == torch.bfloat16 and A.shape == (3, 16, 8) and G.shape == (3, 16, 12)
    assert torch.equal(A, A2) and torch.equal(G, G2)
    A3, _ = linear_inputs(3, 16, 8, 12, "bf16", "llama_logu", seed=6)
    assert not torch.equal(A, A3)


def test_recipe_laws():
    A, G = linear_inputs(4, 256, 64, 64, "f32", "llama_logu", seed=1)
    s = sample_scales(4, "llama_logu", 1)
    assert np.all((s >= 0.1) & (s <= 10))
    g = G.double().numpy()
    for i in range(4):
        assert abs(g[i].std() / (0.01 * s[i]) - 1) < 0.02
    assert abs(A.double().std().item() - 1) < 0.02
    s1 = sample_scales(4, "unit_u0.1_3", 1)
    assert np.all((s1 >= 0.1) & (s1 <= 3))


def test_theta_init():
    assert torch.count_nonzero(theta_init(4, 5, 1, zero=True)) == 0
    t = theta_init(64, 64, 1)
    assert abs(t.std().item() - 0.02) < 0.002


def test_lowrank_recipe_spectrum():
    # rank-8 signal plus 0.05 noise: for T >> 8 the top 8 singular values of
    # each A_i hold almost all of its energy, the 9th drops to the noise floor
    A, G = linear_inputs(2, 512, 96, 80, "f32", "lowrank", seed=3)
    for X in (A, G):
        for i in range(2):
            sv = np.linalg.svd(X[i].double().numpy(), compute_uv=False)
            assert sv[8] < 0.1 * sv[7]
            assert np.sum(sv[:8] ** 2) > 0.97 * np.sum(sv ** 2)
    s = sample_scales(2, "lowrank", 3)
    assert np.all((s >= 0.1) & (s <= 10))


def test_ragged_lengths_recipe():
    from sample_gradient_clipping_amd.inputs import ragged_lengths
    L = ragged_lengths(6, 100, 7, min_len=3)
    assert L[0] == 100 and L[-1] == 3 and all(3 <= x <= 100 for x in L)
    assert L == ragged_lengths(6, 100, 7, min_len=3)
    assert ragged_lengths(1, 10, 1) == [10]
