"""Poisson subsampling of the minibatch, and batches of ragged sequences.

TEST INFRASTRUCTURE ONLY (see the package docstring).

[DPSGD] section DP-SGDのアルゴリズム: step 1 draws each step's minibatch by
Poisson subsampling -- every example of the training set is in it
independently with probability q, so |B| is random -- and step 5 divides the
noisy clipped sum by |B|.

Readings (the pages give no generator, no index order and no rule for an
empty batch):
  * Example n (0 <= n < N) is in the minibatch of step ``step`` when word
    n mod 4 of Philox4x32-10 at the counter (low word of n // 4, high word of
    n // 4, step, POISSON_C3) is below floor(q 2^32).  The comparison is on
    integers, so membership is decided identically on any device; q = 1
    takes every example (the threshold is 2^32), q = 0 none.  POISSON_C3 sits
    in the counter word that the probe and noise streams fill with a layer id,
    so the streams stay disjoint while layer ids stay below it.
  * The minibatch lists its examples in ascending index order.
  * The update divides by the realized |B| (the page's G/|B|); an empty
    minibatch leaves that quotient undefined and is the caller's choice.

A ragged batch holds sequences of lengths T_i <= T, padded to T tokens.  The
pages' per-sample quantities are defined on the T_i real tokens only; the
functions here compute them on the truncated arrays, by definition.
"""

import math

import numpy as np

from .philox import MASK32, philox4x32_10
from .norms import to_f64, fgc_norm_sq, ghost_norm_sq, hutch_norm_sq, hutchpp_norm_sq
from .step import clip_factors

POISSON_C3 = 0xFFFFFFFE


def poisson_threshold(q):
    """floor(q 2^32) as an int in [0, 2^32]; exact (scaling by 2^32 is exact)."""
    q = float(q)
    if not (0.0 <= q <= 1.0):
        raise ValueError("q must lie in [0, 1]")
    return int(math.floor(q * 4294967296.0))


def poisson_words(seed, step, N):
    """The N membership words of step ``step`` (uint32, example order)."""
    if not (0 <= step <= MASK32):
        raise ValueError("step must fit 32 bits")
    if N == 0:
        return np.zeros(0, dtype=np.uint32)
    groups = np.arange((N + 3) // 4, dtype=np.uint64)
    w = philox4x32_10(groups & np.uint64(MASK32), groups >> np.uint64(32), step, POISSON_C3,
                      seed)  # [N / 4, 4]: word j of group g is example 4 g + j
    return w.reshape(-1)[:N]


def poisson_sample(seed, step, N, q):
    """Ascending indices of the examples in step ``step``'s minibatch."""
    thr = poisson_threshold(q)
    words = poisson_words(seed, step, N).astype(np.uint64)
    return np.nonzero(words < np.uint64(thr))[0].astype(np.int64)


def norm_est_ragged(method, A, G, lengths, k=0, seed=0, layer=0, rademacher=False):
    """Per-sample squared norms of A_i[:T_i]^T G_i[:T_i] (sample index i keeps
    its own probe stream, as in the padded batch)."""
    A = to_f64(A)
    G = to_f64(G)
    out = np.zeros(A.shape[0], dtype=np.float64)
    for i, Ti in enumerate(lengths):
        a, g = A[i, :Ti], G[i, :Ti]
        if method == "fgc":
            out[i] = fgc_norm_sq(a, g)
        elif method == "ghost":
            out[i] = ghost_norm_sq(a, g)
        elif method == "hutch":
            out[i] = hutch_norm_sq(a, g, k, seed, layer, i, rademacher=rademacher)
        elif method == "hutchpp":
            out[i] = hutchpp_norm_sq(a, g, k, seed, layer, i, rademacher=rademacher)
        else:
            raise ValueError(method)
    return out


def aggregate_ragged(A, G, c, lengths):
    """sum_i c_i G_i[:T_i]^T A_i[:T_i] (fp64)."""
    A = to_f64(A)
    G = to_f64(G)
    S = np.zeros((G.shape[2], A.shape[2]), dtype=np.float64)
    for i, Ti in enumerate(lengths):
        S += float(c[i]) * (G[i, :Ti].T @ A[i, :Ti])
    return S


def clip_ragged(n, C):
    """Clip factors of the ragged norms (the same rule as the padded batch)."""
    return clip_factors(n, C)
