"""Pins for the oracle's clip, aggregation, noise + update and whole step (CPU).

Fixed by the glossary page's DP-SGD algorithm (section DP-SGDのアルゴリズム):
||c_i g_i|| = min(||g_i||, C) <= C under exact clipping, sigma = 0 reduces
the update to theta - eta S / |B|, and the noise has variance sigma^2 C^2.
Aggregation is checked against brute-force loops and its c = 1 special case
(the plain batch gradient).
"""

import math

import numpy as np
from scipy import stats

import oracle


def _batch(seed, B, T, d, p, scales=None):
    r = np.random.default_rng(seed)
    A = r.standard_normal((B, T, d))
    G = r.standard_normal((B, T, p))
    if scales is not None:
        G *= np.asarray(scales)[:, None, None]
    return A, G


def test_clip_bounds_with_exact_norms():
    A, G = _batch(1, 6, 5, 4, 3, scales=[0.01, 0.1, 0.5, 1, 3, 10])
    n = oracle.norm_est("fgc", A, G)
    C = float(np.median(np.sqrt(n)))  # both branches occur
    c, flag = oracle.clip_factors(n, C)
    assert not flag
    assert np.all(c > 0) and np.all(c <= 1)
    assert np.any(c == 1) and np.any(c < 1)
    for i in range(6):
        g = (A[i].T @ G[i])
        clipped = np.linalg.norm(c[i] * g)
        assert clipped <= C * (1 + 1e-12)
        assert abs(clipped - min(np.linalg.norm(g), C)) <= 1e-12 * max(1, C)


def test_clip_edge_cases():
    c, flag = oracle.clip_factors([0.0, -1e-9, 4.0, 16.0, float("nan"), float("inf")], 2.0)
    assert list(c[:4]) == [1.0, 1.0, 1.0, 0.5]
    assert c[4] == 0.0 and c[5] == 0.0 and flag


def test_planted_clip_mistake_fails_bound():
    n = np.array([25.0, 100.0])
    c_wrong = np.minimum(1.0, 2.0 / n)  # C / n instead of C / sqrt(n)
    assert not np.allclose(c_wrong * np.sqrt(n), np.minimum(np.sqrt(n), 2.0))
    c, _ = oracle.clip_factors(n, 2.0)
    assert np.allclose(c * np.sqrt(n), np.minimum(np.sqrt(n), 2.0))


def test_aggregate_brute_force():
    A, G = _batch(2, 3, 4, 3, 5)
    c = np.array([0.3, 1.0, 0.05])
    S = oracle.aggregate(A, G, c)
    assert S.shape == (5, 3)
    for o in range(5):
        for q in range(3):
            want = 0.0
            for i in range(3):
                for t in range(4):
                    want += c[i] * G[i, t, o] * A[i, t, q]
            assert abs(S[o, q] - want) <= 1e-12 * max(1.0, abs(want))


def test_aggregate_unit_c_is_batch_gradient_and_linear():
    A, G = _batch(3, 4, 6, 5, 7)
    S1 = oracle.aggregate(A, G, np.ones(4))
    # the plain batch gradient of the (p, d) weight: sum over all tokens of g a^T
    flatA = A.reshape(-1, 5)
    flatG = G.reshape(-1, 7)
    want = np.zeros((7, 5))
    for t in range(flatA.shape[0]):
        want += np.outer(flatG[t], flatA[t])
    np.testing.assert_allclose(S1, want, rtol=1e-12, atol=1e-12)
    c1 = np.array([0.1, 0.2, 0.3, 0.4])
    c2 = np.array([1.0, 0.5, 0.0, 0.25])
    np.testing.assert_allclose(oracle.aggregate(A, G, c1 + c2),
                               oracle.aggregate(A, G, c1) + oracle.aggregate(A, G, c2),
                               rtol=1e-12, atol=1e-12)
    rows = [6, 0, 3]
    np.testing.assert_allclose(oracle.aggregate_rows(A, G, c1, rows),
                               oracle.aggregate(A, G, c1)[rows], rtol=1e-12, atol=1e-12)


def test_update_without_noise_is_plain_sgd():
    r = np.random.default_rng(4)
    theta = r.standard_normal((5, 7))
    S = r.standard_normal((5, 7))
    out = oracle.noise_update(theta, S, sigma=0.0, C=1.0, eta=0.1, B=4, seed=1, layer=0)
    np.testing.assert_array_equal(out, theta - (0.1 / 4) * S)


def test_update_noise_variance_is_sigma2_C2():
    p, d = 256, 512
    S = np.zeros((p, d))
    theta = np.zeros((p, d))
    sigma, C, eta, B = 1.3, 0.7, 0.05, 8
    out = oracle.noise_update(theta, S, sigma, C, eta, B, seed=9, layer=4)
    noise = -(B / eta) * (out - theta) - S
    n = noise.size
    assert abs(noise.mean()) < 5 * sigma * C / math.sqrt(n)
    assert abs(noise.var() / (sigma * C) ** 2 - 1) < 5 * math.sqrt(2 / n)
    assert stats.kstest(noise.ravel() / (sigma * C), "norm").pvalue > 1e-4
    # planted mistake: noise std sigma instead of sigma C
    wrong = sigma * oracle.noise_vector(9, 4, n)
    assert abs(wrong.var() / (sigma * C) ** 2 - 1) > 5 * math.sqrt(2 / n)


def test_update_rows_match_full_layer():
    r = np.random.default_rng(5)
    theta = r.standard_normal((6, 9))
    S = r.standard_normal((6, 9))
    full = oracle.noise_update(theta, S, 1.0, 1.0, 0.1, 4, seed=2, layer=3)
    rows = [5, 1]
    part = oracle.noise_update(theta[rows], S[rows], 1.0, 1.0, 0.1, 4, seed=2, layer=3, rows=rows)
    np.testing.assert_array_equal(part, full[rows])


def test_step_flat_clipping_and_resume():
    r = np.random.default_rng(6)
    layers = []
    for lid, (d, p) in enumerate([(4, 6), (6, 3)]):
        A = r.standard_normal((3, 5, d))
        G = r.standard_normal((3, 5, p)) * np.array([0.1, 1.0, 5.0])[:, None, None]
        layers.append((lid, A, G, np.zeros((p, d))))
    n, c, S, th = oracle.dp_step(layers, "fgc", None, C=1.0, sigma=0.0, eta=1.0,
                                 seed_norm=1, seed_noise=2)
    # flat clipping: squared norms add over layers
    n_sep = sum(oracle.norm_est("fgc", A, G) for _, A, G, _ in layers)
    np.testing.assert_allclose(n, n_sep, rtol=1e-12)
    # the clipped whole-model per-sample gradient has norm <= C
    for i in range(3):
        tot = sum(np.sum((c[i] * (layers[l][2][i].T @ layers[l][1][i])) ** 2) for l in range(2))
        assert math.sqrt(tot) <= 1.0 + 1e-12
    # sigma = 0, eta = 1, theta0 = 0: theta' = -S / B
    for S_l, th_l in zip(S, th):
        np.testing.assert_allclose(th_l, -S_l / 3, rtol=1e-12)
    # counter-based streams: a re-run (resume from the same theta and seeds) is identical
    out2 = oracle.dp_step(layers, "hutch", 4, 1.0, 1.0, 0.1, 1, 2)
    out3 = oracle.dp_step(layers, "hutch", 4, 1.0, 1.0, 0.1, 1, 2)
    for a, b in zip(out2[3], out3[3]):
        np.testing.assert_array_equal(a, b)
