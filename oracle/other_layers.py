"""Per-sample gradients of the parameters that are not linear layers.

TEST INFRASTRUCTURE ONLY (see the package docstring).

[DPSGD] section DP-SGDのアルゴリズム clips each sample's whole gradient g_i
(steps 2-3); the randomized-clipping summary (section 中核メカニズム) gives the
linear layers' share.  A Llama-shaped model also has RMSNorm gains and an
embedding table, whose per-sample gradients follow from their definitions:

* RMSNorm, y_t = gamma * xhat_t with xhat_t = x_t / rms(x_t): the gradient of
  sample i in gamma is v_i = sum_t xhat_{i,t} * delta_{i,t} (elementwise),
  delta = dl_i / dy.  Its squared norm adds to n_i like any layer's.
* Embedding, h_t = E[id_t]: the gradient of sample i in E has row v equal to
  sum_{t : id_{i,t} = v} delta_{i,t}; the squared norm is the sum over v of
  the squared row norms.

The clipped sums are sum_i c_i (per-sample gradient), as for every parameter.
"""

import numpy as np

from .norms import to_f64


def rmsnorm_grad(Xhat, Delta):
    """Per-sample gain gradients v [B][d] = sum_t Xhat[i,t] * Delta[i,t] (fp64)."""
    X = to_f64(Xhat)
    D = to_f64(Delta)
    return np.einsum("btc,btc->bc", X, D)


def rmsnorm_norm_sq(Xhat, Delta):
    """||v_i||^2 per sample."""
    v = rmsnorm_grad(Xhat, Delta)
    return np.sum(v * v, axis=1)


def rmsnorm_aggregate(Xhat, Delta, c):
    """sum_i c_i v_i [d]."""
    return np.asarray(c, dtype=np.float64) @ rmsnorm_grad(Xhat, Delta)


def embedding_rows(ids_i, Delta_i):
    """Sample i's gradient in the embedding table, as {row v: sum of delta_t over id_t = v}."""
    D = to_f64(Delta_i)
    rows = {}
    for t, v in enumerate(np.asarray(ids_i).tolist()):
        rows[v] = rows[v] + D[t] if v in rows else D[t].copy()
    return rows


def embedding_norm_sq(ids, Delta):
    """Per-sample squared norm of the embedding-table gradient."""
    out = np.zeros(len(ids), dtype=np.float64)
    for i in range(len(ids)):
        rows = embedding_rows(ids[i], Delta[i])
        out[i] = sum(float(r @ r) for r in rows.values())
    return out


def embedding_aggregate(ids, Delta, c, V):
    """sum_i c_i (gradient of sample i in E) as a dense [V][d] array."""
    d = to_f64(Delta).shape[-1]
    S = np.zeros((V, d), dtype=np.float64)
    for i in range(len(ids)):
        for v, r in embedding_rows(ids[i], Delta[i]).items():
            S[v] += float(c[i]) * r
    return S
