"""Pins for the oracle's sign (Rademacher) probes, CPU only.

The randomized-clipping summary (section 意義と主張) names {+-1}-valued
sketching matrices as future work for cutting the overhead further.  What fixes
the oracle's version, other than the oracle itself:
  * the counter/lane layout against a scalar loop over the (already pinned)
    Philox words, and fair, independent signs;
  * an exact property of sign probes: when O is diagonal every column gives
    sum_r O_rr P_rj^2 = tr(O), so the estimate is exact for every seed (not so
    for Gaussian probes);
  * the textbook mean tr(O) and variance 2 (||O||_F^2 - sum_r O_rr^2) / k of
    the Hutchinson estimator with sign probes;
  * Hutch++ exactness on rank(O) <= s with sign probes.
Planted mistakes (Gaussian entries, a dropped 1/k, entries of size 2) fail.
"""

import math

import numpy as np
import pytest
from scipy import stats

import oracle
from oracle.norms import hutch_core


def _diag_O_inputs(seed, d, p):
    """A = I_d (T = d tokens), G = U diag(s) with orthonormal U: A^T G = G has
    orthogonal columns, so O = G^T G = diag(s^2)."""
    r = np.random.default_rng(seed)
    U, _ = np.linalg.qr(r.standard_normal((d, p)))
    s = r.uniform(0.5, 3.0, size=p)
    return np.eye(d), U * s[None, :], s * s


def test_layout_matches_scalar_definition():
    seed, layer, sample, p, k = 77, 5, 3, 11, 6
    P = oracle.rademacher_probe_matrix(seed, layer, sample, p, k)
    for r_ in range(p):
        for j in range(k):
            w = oracle.philox4x32_10(np.uint64(r_ // 4), np.uint64(j), sample, layer, seed)
            word = int(np.asarray(w).reshape(-1)[r_ % 4])
            assert P[r_, j] == (1.0 if word < 2**31 else -1.0)


def test_signs_fair_and_independent():
    P = oracle.rademacher_probe_matrix(2024, 0, 0, 4096, 32)
    assert set(np.unique(P)) == {-1.0, 1.0}
    plus = int(np.sum(P > 0))
    assert stats.binomtest(plus, P.size, 0.5).pvalue > 1e-3
    # neighbouring rows (same counter, other lane) and columns are uncorrelated
    c_rows = np.mean(P[0::2] * P[1::2])
    c_cols = np.mean(P[:, :-1] * P[:, 1:])
    assert abs(c_rows) < 5 / math.sqrt(P[0::2].size)
    assert abs(c_cols) < 5 / math.sqrt(P[:, 1:].size)


@pytest.mark.parametrize("k", [1, 4, 32])
def test_exact_when_O_is_diagonal(k):
    A, G, diag = _diag_O_inputs(10 + k, 12, 9)
    tr = float(np.sum(diag))
    assert abs(oracle.fgc_norm_sq(A, G) - tr) <= 1e-12 * tr
    for seed in range(20):
        est = oracle.hutch_norm_sq(A, G, k, seed=seed, layer=1, sample=0, rademacher=True)
        assert abs(est - tr) <= 1e-12 * tr


def test_gaussian_probes_are_not_exact_on_diagonal_O():
    # the property above is specific to sign probes (guards against a path
    # that silently draws Gaussian entries)
    A, G, diag = _diag_O_inputs(3, 12, 9)
    tr = float(np.sum(diag))
    errs = [abs(oracle.hutch_norm_sq(A, G, 4, seed=s, layer=1, sample=0) - tr) / tr
            for s in range(10)]
    assert max(errs) > 1e-3


def test_planted_mistakes_fail_the_diagonal_pin():
    A, G, diag = _diag_O_inputs(4, 12, 9)
    tr = float(np.sum(diag))
    P = oracle.rademacher_probe_matrix(0, 1, 0, 9, 4)
    assert abs(hutch_core(A, G, P, 1.0) - tr) > 0.5 * tr          # dropped 1/k
    assert abs(hutch_core(A, G, 2 * P, 1.0 / 4) - tr) > 0.5 * tr  # entries of size 2


def test_unbiased_with_textbook_variance():
    r = np.random.default_rng(5)
    A, G = r.standard_normal((6, 5)), r.standard_normal((6, 7))
    O = G.T @ A @ A.T @ G
    tr = float(np.trace(O))
    k, nseeds = 4, 3000
    est = np.array([oracle.hutch_norm_sq(A, G, k, seed=s, layer=2, sample=1, rademacher=True)
                    for s in range(nseeds)])
    var_theory = 2 * (np.sum(O * O) - np.sum(np.diag(O) ** 2)) / k
    assert abs(est.mean() - tr) < 5 * math.sqrt(var_theory / nseeds)
    assert abs(est.var() / var_theory - 1.0) < 0.2
    # and below the Gaussian variance 2 ||O||_F^2 / k on this O
    assert var_theory < 2 * np.sum(O * O) / k


@pytest.mark.parametrize("k", [3, 7, 32])
def test_hutchpp_exact_on_rank_at_most_s(k):
    s, _ = oracle.hutchpp_split(k)
    r = np.random.default_rng(30 + k)
    A, G = r.standard_normal((s, 40)), r.standard_normal((s, 37))  # rank(O) <= T = s
    exact = oracle.fgc_norm_sq(A, G)
    for seed in range(5):
        est = oracle.hutchpp_norm_sq(A, G, k, seed=seed, layer=0, sample=0, rademacher=True)
        assert abs(est - exact) <= 1e-9 * exact


def test_norm_est_threads_the_flag():
    r = np.random.default_rng(6)
    A, G = r.standard_normal((3, 5, 4)), r.standard_normal((3, 5, 6))
    n = oracle.norm_est("hutch", A, G, k=3, seed=1, layer=2, rademacher=True)
    for i in range(3):
        assert n[i] == oracle.hutch_norm_sq(A[i], G[i], 3, 1, 2, i, rademacher=True)
    ns = oracle.norm_est("hutchpp", A, G, k=3, seed=1, layer=2, shared=True, rademacher=True)
    for i in range(3):
        assert ns[i] == oracle.hutchpp_norm_sq(A[i], G[i], 3, 1, 2, 0, rademacher=True)
