"""Pins for the per-sample gradients of RMSNorm gains and embedding tables (CPU).

What fixes them, other than the functions themselves:
  * RMSNorm: v_i is the diagonal of the matrix X^_i^T Delta_i (a matmul route),
    and the gradient in gamma of the linear loss sum_t <gamma * xhat_t, delta_t>
    by central finite differences (exact up to rounding for a linear loss);
    a single token gives the closed form (xhat * delta)^2.
  * Embedding: the table's gradient is the linear-layer gradient with a one-hot
    input, so its squared norm equals the FGC and ghost norms of (one_hot(ids),
    Delta), both pinned elsewhere; all-distinct ids give sum_t ||delta_t||^2 and
    one repeated id gives ||sum_t delta_t||^2; the clipped sum equals the
    linear layers' clipped sum with the one-hot input.
Planted mistakes (summing over d instead of t, squaring before summing the
rows of a repeated id) fail.
"""

import numpy as np
import pytest

import oracle
from oracle.other_layers import (embedding_aggregate, embedding_norm_sq, embedding_rows,
                                 rmsnorm_aggregate, rmsnorm_grad, rmsnorm_norm_sq)


def _rms_inputs(seed, B=3, T=7, d=5):
    r = np.random.default_rng(seed)
    return r.standard_normal((B, T, d)), r.standard_normal((B, T, d))


def test_rmsnorm_grad_is_the_diagonal_of_xhat_t_delta():
    X, D = _rms_inputs(1)
    v = rmsnorm_grad(X, D)
    for i in range(3):
        assert np.allclose(v[i], np.diag(X[i].T @ D[i]), rtol=1e-13, atol=1e-13)
    assert np.allclose(rmsnorm_norm_sq(X, D), np.sum(v * v, axis=1), rtol=1e-14)


def test_rmsnorm_grad_by_finite_differences():
    X, D = _rms_inputs(2, B=1, T=6, d=4)
    gamma = np.random.default_rng(3).standard_normal(4)

    def loss(g):
        return float(np.sum((g[None, :] * X[0]) * D[0]))

    h = 1e-3
    fd = np.array([(loss(gamma + h * e) - loss(gamma - h * e)) / (2 * h) for e in np.eye(4)])
    assert np.allclose(rmsnorm_grad(X, D)[0], fd, rtol=1e-9, atol=1e-9)


def test_rmsnorm_single_token_and_planted_axis():
    X, D = _rms_inputs(4, B=2, T=1, d=6)
    assert np.allclose(rmsnorm_norm_sq(X, D), np.sum((X[:, 0] * D[:, 0]) ** 2, axis=1))
    X, D = _rms_inputs(5)
    wrong = np.einsum("btc,btc->bt", X, D)  # summed over d instead of t
    assert not np.allclose(np.sum(wrong * wrong, axis=1), rmsnorm_norm_sq(X, D))


def test_rmsnorm_aggregate_is_linear_in_c():
    X, D = _rms_inputs(6)
    c = np.array([0.2, 1.0, 0.7])
    assert np.allclose(rmsnorm_aggregate(X, D, c), sum(c[i] * rmsnorm_grad(X, D)[i] for i in range(3)))
    assert np.allclose(rmsnorm_aggregate(X, D, np.ones(3)), np.diag(sum(X[i].T @ D[i] for i in range(3))))


def _one_hot(ids, V):
    out = np.zeros((len(ids), V))
    out[np.arange(len(ids)), ids] = 1.0
    return out


def _emb_inputs(seed, B=3, T=12, d=5, V=9):
    r = np.random.default_rng(seed)
    return r.integers(0, V, size=(B, T)), r.standard_normal((B, T, d)), V


def test_embedding_norm_is_fgc_and_ghost_of_the_one_hot_input():
    ids, D, V = _emb_inputs(7)
    n = embedding_norm_sq(ids, D)
    for i in range(3):
        A = _one_hot(ids[i], V)
        assert np.isclose(n[i], oracle.fgc_norm_sq(A, D[i]), rtol=1e-12)
        assert np.isclose(n[i], oracle.ghost_norm_sq(A, D[i]), rtol=1e-12)


def test_embedding_special_cases_and_planted_mistake():
    r = np.random.default_rng(8)
    D = r.standard_normal((2, 6, 4))
    distinct = np.array([[0, 1, 2, 3, 4, 5], [5, 4, 3, 2, 1, 0]])
    assert np.allclose(embedding_norm_sq(distinct, D), np.sum(D * D, axis=(1, 2)))
    same = np.full((2, 6), 3)
    assert np.allclose(embedding_norm_sq(same, D), np.sum(np.sum(D, axis=1) ** 2, axis=1))
    # squaring each token before summing the rows of a repeated id is wrong
    assert not np.allclose(embedding_norm_sq(same, D), np.sum(D * D, axis=(1, 2)))
    rows = embedding_rows(same[0], D[0])
    assert list(rows) == [3] and np.allclose(rows[3], D[0].sum(axis=0))


def test_embedding_aggregate_is_the_linear_clipped_sum_of_the_one_hot_input():
    ids, D, V = _emb_inputs(9)
    c = np.array([0.5, 0.1, 1.0])
    A = np.stack([_one_hot(ids[i], V) for i in range(3)])
    assert np.allclose(embedding_aggregate(ids, D, c, V), oracle.aggregate(A, D, c).T,
                       rtol=1e-13, atol=1e-13)
