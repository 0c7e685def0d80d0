"""Forward pass and backward pass 1 of a Llama attention block, and the block's
whole DP-SGD-RC step.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The attention half of a Llama decoder layer ([RC] アルゴリズム的フロー steps 1-2,
the model of [RC] 実証結果), with its usual definitions (readings listed with
the design notes):

  xhat, y = RMSNorm(x), gamma * xhat
  q = y Wq^T [T][H dh], k = y Wk^T, v = y Wv^T [T][KV dh]     (grouped heads)
  q, k <- RoPE(q), RoPE(k): in each head, the pair (i, i + dh/2) is rotated by
          t * base^(-2 i / dh) at position t
  o_h = softmax(q_h k_g^T / sqrt(dh) + causal mask) v_g,   g = h // (H / KV)
  out = x + o Wo^T

and, from R = dL/d(out), backward pass 1 from the chain rule:

  G_o = R (A_o = o), do = R Wo
  P = softmax(S), dV_g = sum_{h in g} P^T dO_h, dP = dO V^T,
  dS = P * (dP - rowsum(dO * O)), dQ = dS K / sqrt(dh), dK_g = sum_h dS^T Q / sqrt(dh)
  G_q = RoPE^T(dQ), G_k = RoPE^T(dK), G_v = dV (A = y for all three)
  dy = G_q Wq + G_k Wk + G_v Wv, dx = RMSNorm backward + R.
"""

import numpy as np

from .mlp_block import linear_forward, rmsnorm_backward, rmsnorm_forward
from .norms import norm_est, to_f64
from .other_layers import rmsnorm_aggregate, rmsnorm_norm_sq
from .step import aggregate, clip_factors, noise_update


def rope(x, n_heads, head_dim, base, inverse=False):
    """Rotary position embedding of x [..][T][n_heads * head_dim] (position = index
    along T): each head's pair (i, i + head_dim/2) is rotated by t * base^(-2i/dh);
    ``inverse`` rotates by the opposite angle (the transpose, for the backward)."""
    x = to_f64(x)
    T = x.shape[-2]
    half = head_dim // 2
    inv = base ** (-2.0 * np.arange(half) / head_dim)
    ang = np.arange(T)[:, None] * inv[None, :]            # [T][half]
    c, s = np.cos(ang), np.sin(ang)
    if inverse:
        s = -s
    xs = x.reshape(x.shape[:-1] + (n_heads, head_dim))
    x1, x2 = xs[..., :half], xs[..., half:]
    c = c[:, None, :]
    s = s[:, None, :]
    out = np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)
    return out.reshape(x.shape)


def _heads(x, n, dh):
    return to_f64(x).reshape(x.shape[:-1] + (n, dh))


def attention_forward(q, k, v, n_heads, n_kv, head_dim):
    """Causal grouped-query attention of one sample: q [T][H dh], k, v [T][KV dh].
    Returns (o [T][H dh], lse [H][T] = log of each softmax row's normaliser)."""
    T = q.shape[0]
    qh, kh, vh = _heads(q, n_heads, head_dim), _heads(k, n_kv, head_dim), _heads(v, n_kv, head_dim)
    grp = n_heads // n_kv
    scale = 1.0 / np.sqrt(head_dim)
    mask = np.triu(np.ones((T, T), dtype=bool), 1)
    o = np.zeros((T, n_heads, head_dim))
    lse = np.zeros((n_heads, T))
    for h in range(n_heads):
        g = h // grp
        S = (qh[:, h, :] @ kh[:, g, :].T) * scale
        S[mask] = -np.inf
        m = S.max(axis=1, keepdims=True)
        E = np.exp(S - m)
        Z = E.sum(axis=1, keepdims=True)
        o[:, h, :] = (E / Z) @ vh[:, g, :]
        lse[h] = (m + np.log(Z))[:, 0]
    return o.reshape(T, n_heads * head_dim), lse


def attention_backward(q, k, v, do, n_heads, n_kv, head_dim):
    """(dq [T][H dh], dk, dv [T][KV dh]) of one sample from dL/do."""
    T = q.shape[0]
    qh, kh, vh = _heads(q, n_heads, head_dim), _heads(k, n_kv, head_dim), _heads(v, n_kv, head_dim)
    doh = _heads(do, n_heads, head_dim)
    grp = n_heads // n_kv
    scale = 1.0 / np.sqrt(head_dim)
    mask = np.triu(np.ones((T, T), dtype=bool), 1)
    dq = np.zeros_like(qh)
    dk = np.zeros_like(kh)
    dv = np.zeros_like(vh)
    for h in range(n_heads):
        g = h // grp
        S = (qh[:, h, :] @ kh[:, g, :].T) * scale
        S[mask] = -np.inf
        P = np.exp(S - S.max(axis=1, keepdims=True))
        P /= P.sum(axis=1, keepdims=True)
        O = P @ vh[:, g, :]
        dv[:, g, :] += P.T @ doh[:, h, :]
        dP = doh[:, h, :] @ vh[:, g, :].T
        dS = P * (dP - np.sum(doh[:, h, :] * O, axis=1, keepdims=True))
        dq[:, h, :] = dS @ kh[:, g, :] * scale
        dk[:, g, :] += dS.T @ qh[:, h, :] * scale
    return (dq.reshape(T, n_heads * head_dim), dk.reshape(T, n_kv * head_dim),
            dv.reshape(T, n_kv * head_dim))


def attn_forward(x, gamma, Wq, Wk, Wv, Wo, eps, n_heads, n_kv, head_dim, base):
    """Every activation of the block for x [B][T][d] (fp64 dict)."""
    xhat, y, rstd = rmsnorm_forward(x, gamma, eps)
    q0, k0, v = linear_forward(y, Wq), linear_forward(y, Wk), linear_forward(y, Wv)
    q, k = rope(q0, n_heads, head_dim, base), rope(k0, n_kv, head_dim, base)
    B = q.shape[0]
    outs = [attention_forward(q[i], k[i], v[i], n_heads, n_kv, head_dim) for i in range(B)]
    o = np.stack([a for a, _ in outs])
    lse = np.stack([b for _, b in outs])
    out = linear_forward(o, Wo, residual=x)
    return {"xhat": xhat, "y": y, "rstd": rstd, "q": q, "k": k, "v": v, "o": o, "lse": lse,
            "out": out}


def attn_backward(x, gamma, Wq, Wk, Wv, Wo, eps, n_heads, n_kv, head_dim, base, dout, fwd=None):
    """Backward pass 1 (fp64 dict): G_q, G_k, G_v, G_o, dy, dx."""
    if fwd is None:
        fwd = attn_forward(x, gamma, Wq, Wk, Wv, Wo, eps, n_heads, n_kv, head_dim, base)
    R = to_f64(dout)
    do = R @ to_f64(Wo)
    B = R.shape[0]
    grads = [attention_backward(fwd["q"][i], fwd["k"][i], fwd["v"][i], do[i], n_heads, n_kv,
                                head_dim) for i in range(B)]
    dq = np.stack([g[0] for g in grads])
    dk = np.stack([g[1] for g in grads])
    dv = np.stack([g[2] for g in grads])
    Gq = rope(dq, n_heads, head_dim, base, inverse=True)
    Gk = rope(dk, n_kv, head_dim, base, inverse=True)
    dy = Gq @ to_f64(Wq) + Gk @ to_f64(Wk) + dv @ to_f64(Wv)
    dx = rmsnorm_backward(x, gamma, dy, R, eps)
    return {"do": do, "G_q": Gq, "G_k": Gk, "G_v": dv, "G_o": R, "dy": dy, "dx": dx}


def attn_per_sample_grads(fwd, bwd):
    """Sample i's gradient in each parameter: {name: [B][...]}."""
    return {
        "W_q": np.einsum("btp,btd->bpd", bwd["G_q"], fwd["y"]),
        "W_k": np.einsum("btp,btd->bpd", bwd["G_k"], fwd["y"]),
        "W_v": np.einsum("btp,btd->bpd", bwd["G_v"], fwd["y"]),
        "W_o": np.einsum("btp,btd->bpd", bwd["G_o"], fwd["o"]),
        "gamma": np.einsum("btd,btd->bd", fwd["xhat"], bwd["dy"]),
    }


# Parameter order and the layer ids that key their probes and noise.
ATTN_LAYERS = (("W_q", 0), ("W_k", 1), ("W_v", 2), ("W_o", 3), ("gamma", 4))


def attn_dp_step(acts, gamma, weights, method, k, C, sigma, eta, seed_norm, seed_noise,
                 layer_base=0):
    """One DP-SGD-RC step of the block ([RC] アルゴリズム的フロー steps 3-5) from its
    activations and output gradients ``acts`` (y, o, xhat, G_q, G_k, G_v, G_o, dy)
    and the fp32 parameters ``weights`` {W_q, W_k, W_v, W_o}: one clip factor per
    sample from the summed squared norms of all five parameters, then clipped
    sums, noise and updates.  Returns (n [B], c [B], {name: updated parameter})."""
    lin = {"W_q": ("y", "G_q"), "W_k": ("y", "G_k"), "W_v": ("y", "G_v"), "W_o": ("o", "G_o")}
    ids = {name: layer_base + i for name, i in ATTN_LAYERS}
    n = rmsnorm_norm_sq(acts["xhat"], acts["dy"])
    for name, (a, g) in lin.items():
        n = n + norm_est(method, acts[a], acts[g], k=k, seed=seed_norm, layer=ids[name])
    c, _flag = clip_factors(n, C)
    B = len(n)
    new = {}
    for name, (a, g) in lin.items():
        new[name] = noise_update(to_f64(weights[name]), aggregate(acts[a], acts[g], c), sigma, C,
                                 eta, B, seed_noise, ids[name])
    S_g = rmsnorm_aggregate(acts["xhat"], acts["dy"], c)
    new["gamma"] = noise_update(to_f64(gamma)[None, :], S_g[None, :], sigma, C, eta, B,
                                seed_noise, ids["gamma"])[0]
    return n, c, new


def layer_forward(x, attn_p, mlp_p, eps, n_heads, n_kv, head_dim, base):
    """A Llama decoder layer: the attention block, then the MLP block on its output.
    attn_p = (gamma, Wq, Wk, Wv, Wo), mlp_p = (gamma, W_gate, W_up, W_down)."""
    from .mlp_block import mlp_forward
    fa = attn_forward(x, *attn_p, eps, n_heads, n_kv, head_dim, base)
    fm = mlp_forward(fa["out"], *mlp_p, eps)
    return fa, fm


def layer_backward(x, attn_p, mlp_p, eps, n_heads, n_kv, head_dim, base, dout, fwd=None):
    """Backward pass 1 through the layer: the MLP block from R = dL/d(out), then the
    attention block from the MLP block's dL/d(input)."""
    from .mlp_block import mlp_backward
    fa, fm = layer_forward(x, attn_p, mlp_p, eps, n_heads, n_kv, head_dim, base) if fwd is None \
        else fwd
    bm = mlp_backward(fa["out"], *mlp_p, eps, dout, fm)
    ba = attn_backward(x, *attn_p, eps, n_heads, n_kv, head_dim, base, bm["dx"], fa)
    return ba, bm


def layer_dp_step(a_acts, m_acts, attn_p, mlp_p, method, k, C, sigma, eta, seed_norm,
                  seed_noise):
    """One DP-SGD-RC step of the whole layer: the squared norms of all eleven
    parameters (seven linears, two gains) summed per sample, one clip factor per
    sample, then every parameter's clipped sum, noise and update.  Layer ids: the
    attention block's parameters 0..4, the MLP block's 5..8 (ATTN_LAYERS, then
    MLP_LAYERS shifted by 5).  Returns (n, c, {name: updated})."""
    from .mlp_block import MLP_LAYERS
    lin = {"W_q": (a_acts, "y", "G_q", attn_p[1]), "W_k": (a_acts, "y", "G_k", attn_p[2]),
           "W_v": (a_acts, "y", "G_v", attn_p[3]), "W_o": (a_acts, "o", "G_o", attn_p[4]),
           "W_gate": (m_acts, "y", "G_gate", mlp_p[1]), "W_up": (m_acts, "y", "G_up", mlp_p[2]),
           "W_down": (m_acts, "h", "G_down", mlp_p[3])}
    ids = dict(ATTN_LAYERS)
    ids.update({("mlp_" + n if n == "gamma" else n): 5 + i for n, i in MLP_LAYERS})
    n = rmsnorm_norm_sq(a_acts["xhat"], a_acts["dy"]) + rmsnorm_norm_sq(m_acts["xhat"],
                                                                          m_acts["dy"])
    for name, (acts, a, g, _W) in lin.items():
        n = n + norm_est(method, acts[a], acts[g], k=k, seed=seed_norm, layer=ids[name])
    c, _flag = clip_factors(n, C)
    B = len(n)
    new = {}
    for name, (acts, a, g, W) in lin.items():
        new[name] = noise_update(to_f64(W), aggregate(acts[a], acts[g], c), sigma, C, eta, B,
                                 seed_noise, ids[name])
    for name, acts, gamma in (("gamma", a_acts, attn_p[0]), ("mlp_gamma", m_acts, mlp_p[0])):
        S_g = rmsnorm_aggregate(acts["xhat"], acts["dy"], c)
        new[name] = noise_update(to_f64(gamma)[None, :], S_g[None, :], sigma, C, eta, B,
                                 seed_noise, ids[name])[0]
    return n, c, new
