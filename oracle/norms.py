"""Per-sample squared gradient norms of a linear layer: exact and estimated.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Notation of [RC]: sample i has activations A_i (T x d) and output gradients
G_i (T x p) for a linear layer of shape (p, d).  Its per-sample weight
gradient is M_i = A_i^T G_i (d x p, the transpose of the (p, d) weight
layout; the norm is the same) and O_i = G_i^T A_i A_i^T G_i (p x p).
[RC] section 中核メカニズム: ||A_i^T G_i||_F^2 = tr(O_i).
"""

import math

import numpy as np

from .philox import probe_matrix, rademacher_probe_matrix


def to_f64(x):
    """Exact upcast of the bytes the GPU reads (torch fp32/bf16 or numpy) to fp64."""
    if hasattr(x, "detach"):  # torch tensor; bf16 -> fp64 is exact
        import torch
        return x.detach().to("cpu").to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def fgc_norm_sq(A_i, G_i):
    """FGC baseline: materialise M_i = A_i^T G_i (d x p), return sum of its squares.

    [RC] sections 問題定義 and 1. 複雑性の削減: fast gradient clipping forms
    the per-sample gradient of the linear layer, O(T p d) work per sample.
    """
    M = A_i.T @ G_i
    return float(np.sum(M * M))


def ghost_norm_sq(A_i, G_i):
    """Ghost-clipping baseline: <A_i A_i^T, G_i G_i^T>_F from the two T x T Grams.

    [RC] sections 問題定義 and 1. 複雑性の削減 (GC: T x T products, O(T^2 (p+d))
    work).  Equal to tr(G^T A A^T G) by cyclicity of the trace and symmetry of
    the Grams ([RC] section 中核メカニズム, the trace identity).
    """
    gram_a = A_i @ A_i.T
    gram_g = G_i @ G_i.T
    return float(np.sum(gram_a * gram_g))


def hutch_core(A_i, G_i, P, scale):
    """Hutchinson quadratic form through the two thin products.

    [RC] section 中核メカニズム, item 1: sum_j P_j^T O P_j over the columns of
    P, computed as ||A_i^T (G_i P)||_F^2 without forming O or A_i^T G_i:
    Y = G_i P (T x k), Z = A_i^T Y (d x k), result = scale * sum(Z^2).
    """
    Y = G_i @ P
    Z = A_i.T @ Y
    return float(scale * np.sum(Z * Z))


def probes(seed, layer, sample, p, k, rademacher=False):
    """The p x k probe block: Gaussian (default) or Rademacher signs."""
    if rademacher:
        return rademacher_probe_matrix(seed, layer, sample, p, k)
    return probe_matrix(seed, layer, sample, p, k)


def hutch_norm_sq(A_i, G_i, k, seed, layer, sample, rademacher=False):
    """Hutch estimate of ||A_i^T G_i||_F^2 with k Gaussian (or sign) probes.

    Reading (pages print sum_j P_j^T O P_j without a 1/k): with N(0, 1)
    entries that sum has mean k tr(O), so the estimate is divided by k.  Sign
    probes have the same second moment (E[P P^T] = k I), so the same 1/k.
    """
    P = probes(seed, layer, sample, G_i.shape[1], k, rademacher)
    return hutch_core(A_i, G_i, P, 1.0 / k)


def householder_thin_q(X):
    """Thin Q (m x n, orthonormal columns) of X by Householder reflections.

    Textbook Householder QR: for column j, reflect R[j:, j] onto
    alpha e_1 with alpha = -sign(x_0) ||x||, apply the reflector to the
    trailing block, then accumulate Q = H_0 H_1 ... H_{n-1} [I_n; 0].
    A zero column (rank deficiency) skips its reflector; Q stays orthonormal.
    """
    R = np.array(X, dtype=np.float64, copy=True)
    m, n = R.shape
    reflectors = []
    for j in range(n):
        x = R[j:, j]
        normx = math.sqrt(float(np.dot(x, x)))
        alpha = -normx if x[0] >= 0 else normx
        v = x.copy()
        v[0] -= alpha
        vnorm = math.sqrt(float(np.dot(v, v)))
        if vnorm == 0.0:
            reflectors.append(None)
            continue
        v /= vnorm
        R[j:, j:] -= 2.0 * np.outer(v, v @ R[j:, j:])
        reflectors.append(v)
    Q = np.zeros((m, n), dtype=np.float64)
    Q[np.arange(n), np.arange(n)] = 1.0
    for j in reversed(range(n)):
        v = reflectors[j]
        if v is None:
            continue
        Q[j:, :] -= 2.0 * np.outer(v, v @ Q[j:, :])
    return Q


def hutchpp_split(k):
    """Hutch++ budget split (a reading): s = k // 3 sketch columns, s head
    columns (the QR basis) and r = k - 2 s tail columns, k products in all."""
    if k < 3:
        raise ValueError("Hutch++ needs k >= 3")
    s = k // 3
    return s, k - 2 * s


def hutchpp_norm_sq(A_i, G_i, k, seed, layer, sample, rademacher=False):
    """Hutch++ estimate of tr(O_i) = ||A_i^T G_i||_F^2.

    [RC] section 中核メカニズム, item 2: a low-rank (QR) approximation takes
    the head of the spectrum exactly and Hutchinson estimates the tail.  Steps
    in the textbook order (the pages call the estimators off the shelf):
      1. sketch S (p x s) and tail probes W (p x r): columns 0..s-1 and
         s..s+r-1 of the same Gaussian probe stream as Hutch;
      2. X = O S = G^T (A (A^T (G S)));
      3. Q = orthonormal basis of X (Householder);
      4. head = tr(Q^T O Q) = ||A^T (G Q)||_F^2;
      5. W' = (I - Q Q^T) W, tail = ||A^T (G W')||_F^2 / r;
      6. estimate = head + tail.
    """
    s, r = hutchpp_split(k)
    p = G_i.shape[1]
    P = probes(seed, layer, sample, p, s + r, rademacher)
    S = P[:, :s]
    W = P[:, s:s + r]
    X = G_i.T @ (A_i @ (A_i.T @ (G_i @ S)))
    Q = householder_thin_q(X)
    head = hutch_core(A_i, G_i, Q, 1.0)
    W_defl = W - Q @ (Q.T @ W)
    tail = hutch_core(A_i, G_i, W_defl, 1.0 / r)
    return head + tail


def norm_est(method, A, G, k=None, seed=0, layer=0, shared=False, rademacher=False):
    """Squared norms n[B] of one linear layer for the whole batch.

    A: [B][T][d], G: [B][T][p] (any array the caller upcasts with to_f64).
    method: "fgc" | "ghost" | "hutch" | "hutchpp".  ``shared`` uses the
    sample-0 probe for every sample (one P for the batch); ``rademacher``
    draws sign probes instead of Gaussian ones.
    """
    A = to_f64(A)
    G = to_f64(G)
    B = A.shape[0]
    out = np.zeros(B, dtype=np.float64)
    for i in range(B):
        probe_sample = 0 if shared else i
        if method == "fgc":
            out[i] = fgc_norm_sq(A[i], G[i])
        elif method == "ghost":
            out[i] = ghost_norm_sq(A[i], G[i])
        elif method == "hutch":
            out[i] = hutch_norm_sq(A[i], G[i], k, seed, layer, probe_sample, rademacher)
        elif method == "hutchpp":
            out[i] = hutchpp_norm_sq(A[i], G[i], k, seed, layer, probe_sample, rademacher)
        else:
            raise ValueError(method)
    return out
