"""Clip, weighted aggregation, noise + SGD update, and the whole step.

TEST INFRASTRUCTURE ONLY (see the package docstring).
"""

import math

import numpy as np

from .norms import norm_est, to_f64
from .philox import noise_vector


def clip_factors(n_sq, C):
    """Per-sample clip factors c_i from squared norms n_i.

    [DPSGD] section DP-SGDのアルゴリズム, step 3: g_i <- g_i / max(1, ||g_i|| / C),
    i.e. g_i is scaled by min(1, C / ||g_i||); [RC] section アルゴリズム的フロー,
    step 4 rescales by min(C / n_i, 1) with n_i the *estimated norm*, which is the
    square root of the squared-norm estimate (a reading: the estimator returns the
    squared norm).
    Readings for the cases the pages leave open: n_i <= C^2 (including 0 and a
    negative value from rounding) gives c_i = 1; a non-finite n_i gives c_i = 0
    (the sample is dropped, which keeps its contribution within C) and raises the
    returned flag.
    """
    n_sq = np.asarray(n_sq, dtype=np.float64)
    c = np.empty(n_sq.shape, dtype=np.float64)
    flag = False
    for i, v in enumerate(n_sq):
        if not math.isfinite(v):
            c[i] = 0.0
            flag = True
        elif v <= C * C:
            c[i] = 1.0
        else:
            c[i] = C / math.sqrt(v)
    return c, flag


def aggregate(A, G, c):
    """Clipped sum S = sum_i c_i G_i^T A_i in the (p, d) weight layout.

    [DPSGD] step 4 sums the clipped per-sample gradients; [RC] section
    アルゴリズム的フロー, step 5 gets them by a second backward pass on the loss
    rescaled by c_i.  For a linear layer that pass yields exactly
    sum_i c_i G_i^T A_i (backpropagation is linear in the loss scale), which is
    computed here sample by sample.
    """
    A = to_f64(A)
    G = to_f64(G)
    S = np.zeros((G.shape[2], A.shape[2]), dtype=np.float64)
    for i in range(A.shape[0]):
        S += float(c[i]) * (G[i].T @ A[i])
    return S


def aggregate_rows(A, G, c, rows):
    """Rows ``rows`` of the clipped sum S (for sampled checks at full size)."""
    A = to_f64(A)
    G = to_f64(G)
    rows = np.asarray(rows, dtype=np.int64)
    S = np.zeros((len(rows), A.shape[2]), dtype=np.float64)
    for i in range(A.shape[0]):
        S += float(c[i]) * (G[i][:, rows].T @ A[i])
    return S


def noise_update(theta, S, sigma, C, eta, B, seed, layer, rows=None):
    """theta' = theta - (eta / |B|) (S + sigma C xi), xi ~ N(0, I).

    [DPSGD] section DP-SGDのアルゴリズム, steps 4-5: Gaussian noise of standard
    deviation sigma C is added once to the clipped sum, then the SGD step divides
    by the batch size.  |B| = B (fixed batches; a reading).  ``theta`` and ``S``
    are (p, d) arrays, or only the rows listed in ``rows`` of a (p, d) layer
    whose full width is theta.shape[1].
    """
    theta = np.asarray(theta, dtype=np.float64)
    S = np.asarray(S, dtype=np.float64)
    nrows, d = theta.shape
    if rows is None:
        rows = np.arange(nrows)
    xi = np.empty((len(rows), d), dtype=np.float64)
    for idx, o in enumerate(rows):
        xi[idx] = noise_vector(seed, layer, d, offset=int(o) * d)
    return theta - (eta / B) * (S + sigma * C * xi)


def dp_step(layers, method, k, C, sigma, eta, seed_norm, seed_noise, shared=False,
            rademacher=False):
    """One DP-SGD-RC step over a stack of linear layers.

    ``layers``: list of (layer_id, A [B][T][d], G [B][T][p], theta [p][d]).
    [RC] section アルゴリズム的フロー, steps 3-5: squared norms estimated per
    layer and summed over layers (flat clipping of the whole per-sample gradient,
    a reading), one clip factor per sample, then per layer the clipped sum,
    noise and update.
    Returns (n [B], c [B], [S per layer], [theta' per layer]).
    """
    n = None
    for layer_id, A, G, _theta in layers:
        n_l = norm_est(method, A, G, k=k, seed=seed_norm, layer=layer_id, shared=shared,
                       rademacher=rademacher)
        n = n_l if n is None else n + n_l
    c, _flag = clip_factors(n, C)
    S_out, theta_out = [], []
    for layer_id, A, G, theta in layers:
        S = aggregate(A, G, c)
        B = to_f64(A).shape[0]
        S_out.append(S)
        theta_out.append(noise_update(theta, S, sigma, C, eta, B, seed_noise, layer_id))
    return n, c, S_out, theta_out
