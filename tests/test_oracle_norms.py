"""Pins for the oracle's exact and estimated per-sample norms (CPU only).

What fixes them, other than the oracle itself:
  * the trace identity of the randomized-clipping summary (section
    中核メカニズム) checked against brute-force loops and an explicit O;
  * closed forms (T = 1: ||a||^2 ||g||^2), the textbook laws of Gaussian
    quadratic forms (mean tr(O), variance 2 ||O||_F^2 / k, chi^2_k / k for a
    rank-one O) and Hutch++'s exactness on rank <= s;
  * Householder QR against numpy.linalg.qr (LAPACK) through the projector.
Planted mistakes (a dropped 1/k, a transposed operand, a missing deflation)
are shown to fail these pins.
"""

import math

import numpy as np
import pytest
from scipy import stats

import oracle
from oracle.norms import hutch_core


def _tiny(seed, T, d, p):
    r = np.random.default_rng(seed)
    return r.standard_normal((T, d)), r.standard_normal((T, p))


def _brute_M(A, G):
    T, d = A.shape
    p = G.shape[1]
    M = [[0.0] * p for _ in range(d)]
    for q in range(d):
        for o in range(p):
            s = 0.0
            for t in range(T):
                s += float(A[t, q]) * float(G[t, o])
            M[q][o] = s
    return M


def _explicit_trace_O(A, G):
    O = G.T @ A @ A.T @ G
    return float(np.trace(O)), O


@pytest.mark.parametrize("shape", [(1, 3, 4), (5, 4, 6), (9, 7, 3), (16, 16, 16), (3, 12, 2)])
def test_trace_identity_exact_paths(shape):
    T, d, p = shape
    A, G = _tiny(sum(shape), T, d, p)
    M = _brute_M(A, G)
    brute = sum(v * v for row in M for v in row)
    tr, _ = _explicit_trace_O(A, G)
    fgc = oracle.fgc_norm_sq(A, G)
    ghost = oracle.ghost_norm_sq(A, G)
    for v in (fgc, ghost, tr):
        assert abs(v - brute) <= 1e-12 * max(1.0, abs(brute))


def test_single_token_closed_form():
    A, G = _tiny(3, 1, 6, 5)
    want = float(np.dot(A[0], A[0]) * np.dot(G[0], G[0]))
    for fn in (oracle.fgc_norm_sq, oracle.ghost_norm_sq):
        assert abs(fn(A, G) - want) <= 1e-12 * want


def test_hutch_identity_probe_is_exact():
    # P = I_p (k = p) with no 1/k: the sum over columns is exactly tr(O).
    A, G = _tiny(4, 7, 5, 6)
    exact = oracle.fgc_norm_sq(A, G)
    got = hutch_core(A, G, np.eye(6), 1.0)
    assert abs(got - exact) <= 1e-12 * exact
    # equivalently sqrt(p) I with the 1/k normalisation
    got2 = hutch_core(A, G, math.sqrt(6) * np.eye(6), 1.0 / 6)
    assert abs(got2 - exact) <= 1e-12 * exact


def _hutch_mean_ok(fn, A, G, k, nseeds=3000):
    tr, O = _explicit_trace_O(A, G)
    est = np.array([fn(A, G, k, s) for s in range(nseeds)])
    se = math.sqrt(2 * np.sum(O * O) / (k * nseeds))
    return abs(est.mean() - tr) < 5 * se, est, tr, O


def test_hutch_unbiased_and_variance():
    A, G = _tiny(5, 6, 5, 7)
    k = 4
    ok, est, tr, O = _hutch_mean_ok(
        lambda A, G, k, s: oracle.hutch_norm_sq(A, G, k, seed=s, layer=1, sample=2), A, G, k)
    assert ok
    var_theory = 2 * np.sum(O * O) / k
    assert abs(est.var() / var_theory - 1.0) < 0.2


def test_hutch_rank_one_is_chi2():
    # T = 1: O is rank one, so n_hat / tr(O) ~ chi^2_k / k exactly.
    A, G = _tiny(6, 1, 8, 9)
    k = 8
    tr = oracle.fgc_norm_sq(A, G)
    ratios = np.array([oracle.hutch_norm_sq(A, G, k, seed=s, layer=0, sample=0) / tr
                       for s in range(2000)])
    assert stats.kstest(ratios, stats.chi2(df=k, scale=1.0 / k).cdf).pvalue > 1e-3


def test_planted_hutch_mistakes_fail_pins():
    A, G = _tiny(5, 6, 5, 7)

    def no_inverse_k(A, G, k, s):  # dropped 1/k
        P = oracle.probe_matrix(s, 1, 2, G.shape[1], k)
        return hutch_core(A, G, P, 1.0)

    ok, *_ = _hutch_mean_ok(no_inverse_k, A, G, 4, nseeds=500)
    assert not ok

    # transposed operand: A Y instead of A^T Y (shapes allow it when T = d)
    A2, G2 = _tiny(8, 5, 5, 6)
    exact = oracle.fgc_norm_sq(A2, G2)
    wrong = float(np.sum((A2 @ (G2 @ np.eye(6))) ** 2))
    assert abs(wrong - exact) > 1e-6 * exact


def test_householder_q_matches_lapack_projector():
    r = np.random.default_rng(9)
    for m, n in ((50, 10), (17, 17), (200, 3)):
        X = r.standard_normal((m, n))
        Q = oracle.householder_thin_q(X)
        np.testing.assert_allclose(Q.T @ Q, np.eye(n), atol=1e-12)
        Ql, _ = np.linalg.qr(X)
        np.testing.assert_allclose(Q @ Q.T, Ql @ Ql.T, atol=1e-11)
        R = Q.T @ X
        assert np.abs(np.tril(R, -1)).max() < 1e-10 * np.abs(X).max()
        np.testing.assert_allclose(Q @ R, X, atol=1e-10)


def test_householder_rank_deficient_stays_orthonormal():
    r = np.random.default_rng(10)
    X = r.standard_normal((30, 5))
    X[:, 2] = X[:, 0] + X[:, 1]
    X[:, 4] = 0.0
    Q = oracle.householder_thin_q(X)
    np.testing.assert_allclose(Q.T @ Q, np.eye(5), atol=1e-12)


@pytest.mark.parametrize("k", [3, 6, 7, 32])
def test_hutchpp_exact_on_rank_at_most_s(k):
    s, r = oracle.hutchpp_split(k)
    assert 2 * s + r == k
    T = s  # rank(O) <= T <= s
    A, G = _tiny(11 + k, T, 40, 37)
    exact = oracle.fgc_norm_sq(A, G)
    for seed in range(5):
        est = oracle.hutchpp_norm_sq(A, G, k, seed=seed, layer=0, sample=0)
        assert abs(est - exact) <= 1e-9 * exact


def test_planted_hutchpp_missing_deflation_fails():
    k = 9
    s, r = oracle.hutchpp_split(k)
    A, G = _tiny(12, s, 30, 25)
    exact = oracle.fgc_norm_sq(A, G)
    P = oracle.probe_matrix(0, 0, 0, 25, s + r)
    X = G.T @ (A @ (A.T @ (G @ P[:, :s])))
    Q = oracle.householder_thin_q(X)
    wrong = hutch_core(A, G, Q, 1.0) + hutch_core(A, G, P[:, s:], 1.0 / r)  # tail not deflated
    assert abs(wrong - exact) > 1e-3 * exact


def test_hutchpp_unbiased():
    A, G = _tiny(13, 10, 6, 8)
    k = 6
    ok, *_ = _hutch_mean_ok(
        lambda A, G, k, s: oracle.hutchpp_norm_sq(A, G, k, seed=s, layer=0, sample=0), A, G, k,
        nseeds=3000)
    assert ok


def test_hutchpp_beats_hutch_on_decaying_spectrum():
    # rank-3 signal plus small noise: the QR head captures most of tr(O)
    r = np.random.default_rng(14)
    T, d, p = 40, 30, 30
    A = r.standard_normal((T, 3)) @ r.standard_normal((3, d)) + 0.01 * r.standard_normal((T, d))
    G = r.standard_normal((T, 3)) @ r.standard_normal((3, p)) + 0.01 * r.standard_normal((T, p))
    exact = oracle.fgc_norm_sq(A, G)
    k = 12
    h = np.array([oracle.hutch_norm_sq(A, G, k, s, 0, 0) for s in range(300)])
    hpp = np.array([oracle.hutchpp_norm_sq(A, G, k, s, 0, 0) for s in range(300)])
    assert np.mean((hpp - exact) ** 2) < 0.1 * np.mean((h - exact) ** 2)


def test_norm_est_batch_and_shared_probe():
    r = np.random.default_rng(15)
    A = r.standard_normal((3, 5, 4))
    G = r.standard_normal((3, 5, 6))
    n = oracle.norm_est("hutch", A, G, k=3, seed=1, layer=2)
    for i in range(3):
        assert n[i] == oracle.hutch_norm_sq(A[i], G[i], 3, 1, 2, i)
    ns = oracle.norm_est("hutch", A, G, k=3, seed=1, layer=2, shared=True)
    for i in range(3):
        assert ns[i] == oracle.hutch_norm_sq(A[i], G[i], 3, 1, 2, 0)
    ex = oracle.norm_est("fgc", A, G)
    gh = oracle.norm_est("ghost", A, G)
    np.testing.assert_allclose(ex, gh, rtol=1e-12)
