"""Forward pass and backward pass 1 of a Llama-shaped MLP block, and the block's
whole DP-SGD-RC step.

TEST INFRASTRUCTURE ONLY (see the package docstring).

[RC] section アルゴリズム的フロー: step 1 (forward) computes the activations,
step 2 (backward pass 1) the per-sample output gradients of every layer; steps
3-5 then estimate the norms, rescale and run backward pass 2 with noise.  The
pages fix neither the network nor the loss; the block here is the MLP half of
a Llama decoder layer (the model the pages fine-tune, section 実証結果), with
its usual definitions (readings, listed with the design notes):

  rstd_t = 1 / sqrt(mean_q x_{t,q}^2 + eps)      RMSNorm
  xhat   = x * rstd,  y = gamma * xhat
  g = y W_gate^T,  u = y W_up^T                  [T][f]
  h = silu(g) * u,  silu(z) = z * sigmoid(z)     SwiGLU
  out = x + h W_down^T                           residual

The block sits inside a network, so its loss enters through the output
gradient dL/d(out) = R that the layers above hand back; the tests take R as a
seeded input (equivalently, the per-sample loss L_i = sum_t <R_{i,t}, out_{i,t}>).
Backward pass 1, written out from the chain rule:

  G_down = R                     (output gradient of the down projection; A_down = h)
  dh = R W_down
  G_gate = dh * u * silu'(g),  silu'(z) = sigmoid(z) (1 + z (1 - sigmoid(z)))
  G_up   = dh * silu(g)          (A_gate = A_up = y)
  dy = G_gate W_gate + G_up W_up (the output gradient of the RMSNorm; its gain
                                  gradient is sum_t xhat_t * dy_t)
  dx = rstd * (gamma*dy - xhat * mean_q(gamma*dy*xhat)) + R
"""

import numpy as np

from .norms import norm_est, to_f64
from .other_layers import rmsnorm_aggregate, rmsnorm_norm_sq
from .step import aggregate, clip_factors, noise_update


def _sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def rmsnorm_forward(x, gamma, eps):
    """(xhat, y, rstd) of an RMSNorm over the last axis."""
    x = to_f64(x)
    rstd = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    xhat = x * rstd
    return xhat, to_f64(gamma) * xhat, rstd[..., 0]


def linear_forward(a, W, residual=None):
    """a W^T (+ residual): a [..][d], W [p][d]."""
    out = to_f64(a) @ to_f64(W).T
    return out if residual is None else out + to_f64(residual)


def swiglu_forward(g, u):
    g, u = to_f64(g), to_f64(u)
    return g * _sigmoid(g) * to_f64(u)


def swiglu_backward(dh, g, u):
    """(dL/dg, dL/du) from dL/dh."""
    dh, g, u = to_f64(dh), to_f64(g), to_f64(u)
    s = _sigmoid(g)
    return dh * u * s * (1.0 + g * (1.0 - s)), dh * g * s


def rmsnorm_backward(x, gamma, dy, dout, eps):
    """dL/dx of out = x + (block of y), y = gamma * RMSNorm(x), given dL/dy and
    the residual's dL/dout."""
    x, dy = to_f64(x), to_f64(dy)
    xhat, _, rstd = rmsnorm_forward(x, gamma, eps)
    gdy = to_f64(gamma) * dy
    mean = np.mean(gdy * xhat, axis=-1, keepdims=True)
    return rstd[..., None] * (gdy - xhat * mean) + to_f64(dout)


def mlp_forward(x, gamma, Wg, Wu, Wd, eps):
    """Every activation of the block, as a dict (fp64)."""
    xhat, y, rstd = rmsnorm_forward(x, gamma, eps)
    g = linear_forward(y, Wg)
    u = linear_forward(y, Wu)
    h = swiglu_forward(g, u)
    out = linear_forward(h, Wd, residual=x)
    return {"xhat": xhat, "y": y, "rstd": rstd, "g": g, "u": u, "h": h, "out": out}


def mlp_backward(x, gamma, Wg, Wu, Wd, eps, dout, fwd=None):
    """Backward pass 1: the output gradients of the three linears, the RMSNorm's
    dL/dy and dL/dx (fp64 dict)."""
    fwd = mlp_forward(x, gamma, Wg, Wu, Wd, eps) if fwd is None else fwd
    R = to_f64(dout)
    dh = R @ to_f64(Wd)
    dg, du = swiglu_backward(dh, fwd["g"], fwd["u"])
    dy = dg @ to_f64(Wg) + du @ to_f64(Wu)
    dx = rmsnorm_backward(x, gamma, dy, R, eps)
    return {"dh": dh, "G_gate": dg, "G_up": du, "G_down": R, "dy": dy, "dx": dx}


def mlp_per_sample_grads(fwd, bwd):
    """Sample i's gradient in each parameter: {name: [B][...]}."""
    return {
        "W_gate": np.einsum("btp,btd->bpd", bwd["G_gate"], fwd["y"]),
        "W_up": np.einsum("btp,btd->bpd", bwd["G_up"], fwd["y"]),
        "W_down": np.einsum("btp,btd->bpd", bwd["G_down"], fwd["h"]),
        "gamma": np.einsum("btd,btd->bd", fwd["xhat"], bwd["dy"]),
    }


# Parameter order and the layer ids that key their probes and noise.
MLP_LAYERS = (("W_gate", 0), ("W_up", 1), ("W_down", 2), ("gamma", 3))


def mlp_dp_step(x, gamma, Wg, Wu, Wd, eps, dout, method, k, C, sigma, eta, seed_norm, seed_noise,
                acts=None, layer_base=0):
    """One DP-SGD-RC step of the block ([RC] アルゴリズム的フロー steps 1-5).

    The norm of sample i's whole gradient is the sum over the three linears of
    the estimator's value (``method``) and the gain's exact squared norm; one
    clip factor per sample; then every parameter gets its clipped sum, noise and
    update.  ``acts`` optionally replaces the fp64 forward/backward with given
    activations and output gradients (a dict with y, h, xhat, G_gate, G_up,
    G_down, dy), so that the step can be checked on a GPU's own intermediates.
    Returns (n [B], c [B], {name: updated parameter}).
    """
    if acts is None:
        fwd = mlp_forward(x, gamma, Wg, Wu, Wd, eps)
        bwd = mlp_backward(x, gamma, Wg, Wu, Wd, eps, dout, fwd)
        acts = {**fwd, **bwd}
    lin = {"W_gate": (acts["y"], acts["G_gate"], Wg), "W_up": (acts["y"], acts["G_up"], Wu),
           "W_down": (acts["h"], acts["G_down"], Wd)}
    ids = {name: layer_base + i for name, i in MLP_LAYERS}
    n = rmsnorm_norm_sq(acts["xhat"], acts["dy"])
    for name, (A, G, _W) in lin.items():
        n = n + norm_est(method, A, G, k=k, seed=seed_norm, layer=ids[name])
    c, _flag = clip_factors(n, C)
    B = len(n)
    new = {}
    for name, (A, G, W) in lin.items():
        new[name] = noise_update(to_f64(W), aggregate(A, G, c), sigma, C, eta, B, seed_noise,
                                 ids[name])
    S_g = rmsnorm_aggregate(acts["xhat"], acts["dy"], c)
    new["gamma"] = noise_update(to_f64(gamma)[None, :], S_g[None, :], sigma, C, eta, B,
                                seed_noise, ids["gamma"])[0]
    return n, c, new
