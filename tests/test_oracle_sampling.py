"""Pins for the oracle's Poisson subsampling and ragged-batch functions (CPU).

[DPSGD] section DP-SGDのアルゴリズム, step 1: each example is in the minibatch
independently with probability q.  What fixes the oracle's sampler, other than
the oracle itself:
  * the counter/lane layout against a scalar loop over the (already pinned)
    Philox words, and the integer threshold floor(q 2^32) at exact values;
  * q = 0 and q = 1, and nesting: the minibatch at q1 <= q2 is a subset of the
    one at q2 (the same words against a higher threshold);
  * the law: |B| ~ Binomial(N, q) (mean and variance over many steps), each
    example in with frequency q, neighbours and consecutive steps independent.
The ragged functions are pinned by invariants of their definitions: a padded
batch whose pad rows of G are zero has the same norms and clipped sum as the
truncated one, full lengths give the dense functions, zero lengths give zero.
Planted mistakes (lanes reversed, counter words swapped, a non-zero pad row of G) fail.
"""

import math

import numpy as np
import pytest

import oracle
from oracle.sampling import POISSON_C3, poisson_threshold, poisson_words


def test_layout_matches_scalar_definition():
    seed, step, N = 99, 7, 23
    w = poisson_words(seed, step, N)
    for n in range(N):
        ref = oracle.philox4x32_10(np.uint64(n // 4), np.uint64(0), step, POISSON_C3, seed)
        assert int(w[n]) == int(np.asarray(ref).reshape(-1)[n % 4])
    q = 0.37
    thr = poisson_threshold(q)
    idx = oracle.poisson_sample(seed, step, N, q)
    assert list(idx) == [n for n in range(N) if int(w[n]) < thr]


def test_high_counter_word_used_beyond_2_32_groups():
    # example n = 4 * 2^32 + 1 lies in group 2^32: counter (0, 1, step, C3)
    seed, step = 5, 3
    n = 4 * (1 << 32) + 1
    direct = oracle.philox4x32_10(np.uint64(0), np.uint64(1), step, POISSON_C3, seed)
    groups = np.array([n // 4], dtype=np.uint64)
    w = oracle.philox4x32_10(groups & np.uint64(0xFFFFFFFF), groups >> np.uint64(32), step,
                             POISSON_C3, seed)
    assert int(np.asarray(w).reshape(-1)[n % 4]) == int(np.asarray(direct).reshape(-1)[1])


def test_threshold_exact():
    assert poisson_threshold(0.0) == 0
    assert poisson_threshold(1.0) == 1 << 32
    assert poisson_threshold(0.5) == 1 << 31
    assert poisson_threshold(3 / 2**32) == 3
    assert poisson_threshold(math.nextafter(3 / 2**32, 0.0)) == 2
    with pytest.raises(ValueError):
        poisson_threshold(1.5)


def test_q_zero_one_and_nesting():
    N = 1000
    assert oracle.poisson_sample(1, 0, N, 0.0).size == 0
    assert np.array_equal(oracle.poisson_sample(1, 0, N, 1.0), np.arange(N))
    prev = set()
    for q in (0.01, 0.05, 0.2, 0.5, 0.9):
        cur = set(oracle.poisson_sample(11, 4, N, q).tolist())
        assert prev <= cur
        prev = cur


def test_binomial_batch_size_and_bernoulli_membership():
    N, q, steps = 64, 0.125, 3000
    seed = 2024
    sizes = np.zeros(steps)
    member = np.zeros((steps, N), dtype=bool)
    for t in range(steps):
        idx = oracle.poisson_sample(seed, t, N, q)
        sizes[t] = idx.size
        member[t, idx] = True
    mean, var = N * q, N * q * (1 - q)
    assert abs(sizes.mean() - mean) < 5 * math.sqrt(var / steps)
    assert abs(sizes.var() / var - 1) < 0.1
    # per-example frequency q; indicators of neighbours and of consecutive steps uncorrelated
    freq = member.mean(axis=0)
    assert np.all(np.abs(freq - q) < 6 * math.sqrt(q * (1 - q) / steps))
    x = member.astype(float) - q
    c_nb = np.mean(x[:, :-1] * x[:, 1:]) / (q * (1 - q))
    c_st = np.mean(x[:-1] * x[1:]) / (q * (1 - q))
    assert abs(c_nb) < 5 / math.sqrt(x[:, 1:].size)
    assert abs(c_st) < 5 / math.sqrt(x[1:].size)


def test_planted_sampler_mistakes_fail_the_pins():
    seed, step, N, q = 99, 7, 64, 0.4
    w = poisson_words(seed, step, N).astype(np.uint64)
    thr = np.uint64(poisson_threshold(q))
    good = oracle.poisson_sample(seed, step, N, q)
    # lanes taken in reverse order within each counter, or the step in the wrong word
    rev = np.nonzero(w.reshape(-1, 4)[:, ::-1].reshape(-1) < thr)[0]
    groups = np.arange(N // 4, dtype=np.uint64)
    swapped = oracle.philox4x32_10(groups, np.uint64(step), np.uint64(0), POISSON_C3, seed)
    swp = np.nonzero(np.asarray(swapped).reshape(-1).astype(np.uint64) < thr)[0]
    assert not np.array_equal(rev, good)
    assert not np.array_equal(swp, good)


def _padded(seed, B, T, d, p, lengths, junk=3.0):
    r = np.random.default_rng(seed)
    A = r.standard_normal((B, T, d))
    G = r.standard_normal((B, T, p))
    for i, Ti in enumerate(lengths):
        A[i, Ti:] = junk * r.standard_normal((T - Ti, d))  # finite junk in the pad
        G[i, Ti:] = 0.0
    return A, G


@pytest.mark.parametrize("method,k", [("fgc", 0), ("ghost", 0), ("hutch", 5), ("hutchpp", 6)])
def test_zero_pad_rows_of_G_leave_norms_unchanged(method, k):
    lengths = [7, 0, 16, 3]
    A, G = _padded(3, 4, 16, 9, 11, lengths)
    padded = oracle.norm_est(method, A, G, k=k, seed=4, layer=2)
    ragged = oracle.norm_est_ragged(method, A, G, lengths, k=k, seed=4, layer=2)
    assert np.allclose(padded, ragged, rtol=1e-12, atol=0)
    assert ragged[1] == 0.0


def test_full_lengths_equal_the_dense_functions():
    A, G = _padded(5, 3, 12, 6, 8, [12, 12, 12])
    for method, k in (("fgc", 0), ("hutch", 4)):
        dense = oracle.norm_est(method, A, G, k=k, seed=1, layer=0)
        rag = oracle.norm_est_ragged(method, A, G, [12] * 3, k=k, seed=1, layer=0)
        assert np.array_equal(dense, rag)
    c = np.array([0.5, 1.0, 0.25])
    assert np.allclose(oracle.aggregate_ragged(A, G, c, [12] * 3), oracle.aggregate(A, G, c),
                       rtol=1e-13, atol=1e-13)


def test_ragged_aggregate_is_the_padded_one_and_planted_mask_fails():
    lengths = [5, 9, 0]
    A, G = _padded(8, 3, 9, 7, 6, lengths)
    c = np.array([0.3, 1.0, 0.8])
    S = oracle.aggregate_ragged(A, G, c, lengths)
    assert np.allclose(S, oracle.aggregate(A, G, c), rtol=1e-12, atol=1e-12)
    # the same batch with the pad rows of G left non-zero differs: the zero rows matter
    Gbad = G.copy()
    Gbad[0, 5:] = 1.0
    assert not np.allclose(oracle.aggregate(A, Gbad, c), S, rtol=1e-6, atol=1e-6)
