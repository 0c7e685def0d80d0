"""Pins for the MLP block's forward pass, backward pass 1 and whole step (CPU).

What fixes them, other than the functions themselves:
  * every per-sample parameter gradient and dL/dx against central finite
    differences of the per-sample loss L_i = sum_t <R_{i,t}, out_{i,t}>;
  * the SwiGLU derivative against finite differences of SwiGLU itself;
  * RMSNorm with eps = 0: unit mean square and invariance under x -> c x;
  * W_down = 0: the block is the identity and the gate/up gradients vanish;
  * the step with no clipping and no noise is plain SGD on the batch loss
    (finite differences again), and its FGC norm is the sum of the squared
    per-sample gradient norms.
Planted mistakes in the oracle (a dropped residual, a wrong SwiGLU derivative,
a flipped sign in the RMSNorm backward) fail the finite-difference pins.
"""

import numpy as np
import pytest

from oracle import mlp_block as mb

EPS = 1e-5


def _block(seed, B=2, T=3, d=4, f=6):
    r = np.random.default_rng(seed)
    x = r.standard_normal((B, T, d))
    gamma = 1.0 + 0.3 * r.standard_normal(d)
    Wg = r.standard_normal((f, d)) / np.sqrt(d)
    Wu = r.standard_normal((f, d)) / np.sqrt(d)
    Wd = r.standard_normal((d, f)) / np.sqrt(f)
    R = r.standard_normal((B, T, d))
    return x, gamma, Wg, Wu, Wd, R


def _loss(i, x, gamma, Wg, Wu, Wd, R):
    out = mb.mlp_forward(x, gamma, Wg, Wu, Wd, EPS)["out"]
    return float(np.sum(R[i] * out[i]))


def _fd_param_grads(i, params, R, h=1e-5, picks=4, seed=0):
    """Central differences of L_i in a few random entries of every parameter."""
    r = np.random.default_rng(seed)
    names = ["x", "gamma", "W_gate", "W_up", "W_down"]
    out = {}
    for pi, name in enumerate(names):
        P = params[pi]
        got = []
        for _ in range(picks):
            idx = tuple(r.integers(0, s) for s in P.shape)
            Pp, Pm = P.copy(), P.copy()
            Pp[idx] += h
            Pm[idx] -= h
            pp = list(params)
            pm = list(params)
            pp[pi], pm[pi] = Pp, Pm
            got.append((idx, (_loss(i, *pp, R) - _loss(i, *pm, R)) / (2 * h)))
        out[name] = got
    return out


def _check_against_fd(seed, rtol=1e-6, atol=1e-8):
    x, gamma, Wg, Wu, Wd, R = _block(seed)
    fwd = mb.mlp_forward(x, gamma, Wg, Wu, Wd, EPS)
    bwd = mb.mlp_backward(x, gamma, Wg, Wu, Wd, EPS, R, fwd)
    grads = mb.mlp_per_sample_grads(fwd, bwd)
    bad = []
    for i in range(x.shape[0]):
        fd = _fd_param_grads(i, (x, gamma, Wg, Wu, Wd), R, seed=seed + i)
        for name, entries in fd.items():
            for idx, v in entries:
                if name == "x":
                    if idx[0] != i:
                        continue
                    an = bwd["dx"][idx]
                else:
                    an = grads[name][i][idx]
                if not np.isclose(an, v, rtol=rtol, atol=atol):
                    bad.append((name, idx, an, v))
    return bad


def test_backward_matches_finite_differences():
    assert _check_against_fd(11) == []
    assert _check_against_fd(12) == []


def test_swiglu_derivative_by_finite_differences():
    r = np.random.default_rng(3)
    g, u = 3 * r.standard_normal(50), r.standard_normal(50)
    h = 1e-6
    dg, du = mb.swiglu_backward(np.ones(50), g, u)
    assert np.allclose(dg, (mb.swiglu_forward(g + h, u) - mb.swiglu_forward(g - h, u)) / (2 * h),
                       rtol=1e-7, atol=1e-9)
    assert np.allclose(du, (mb.swiglu_forward(g, u + h) - mb.swiglu_forward(g, u - h)) / (2 * h),
                       rtol=1e-7, atol=1e-9)


def test_rmsnorm_unit_mean_square_and_scale_invariance():
    r = np.random.default_rng(4)
    x = r.standard_normal((3, 5, 16))
    xhat, y, rstd = mb.rmsnorm_forward(x, np.ones(16), 0.0)
    assert np.allclose(np.mean(xhat * xhat, axis=-1), 1.0, rtol=1e-14)
    assert np.allclose(mb.rmsnorm_forward(7.5 * x, np.ones(16), 0.0)[0], xhat, rtol=1e-13)
    assert np.allclose(rstd, 1.0 / np.sqrt(np.mean(x * x, axis=-1)), rtol=1e-14)


def test_zero_down_projection_is_the_identity():
    x, gamma, Wg, Wu, Wd, R = _block(5)
    Wd = np.zeros_like(Wd)
    fwd = mb.mlp_forward(x, gamma, Wg, Wu, Wd, EPS)
    bwd = mb.mlp_backward(x, gamma, Wg, Wu, Wd, EPS, R, fwd)
    assert np.array_equal(fwd["out"], x)
    assert not np.any(bwd["G_gate"]) and not np.any(bwd["G_up"]) and not np.any(bwd["dy"])
    assert np.array_equal(bwd["dx"], R)


@pytest.mark.parametrize("plant", ["no_residual", "swiglu_deriv", "rms_sign"])
def test_planted_mistakes_fail(monkeypatch, plant):
    if plant == "no_residual":
        orig = mb.rmsnorm_backward
        monkeypatch.setattr(mb, "rmsnorm_backward",
                            lambda x, gamma, dy, dout, eps: orig(x, gamma, dy, 0.0 * dout, eps))
    elif plant == "swiglu_deriv":
        def wrong(dh, g, u):
            s = 1.0 / (1.0 + np.exp(-g))
            return dh * u * s, dh * g * s  # sigmoid in place of silu'
        monkeypatch.setattr(mb, "swiglu_backward", wrong)
    else:
        def wrong(x, gamma, dy, dout, eps):
            xhat, _, rstd = mb.rmsnorm_forward(x, gamma, eps)
            gdy = gamma * dy
            return rstd[..., None] * (gdy + xhat * np.mean(gdy * xhat, axis=-1, keepdims=True)) + dout
        monkeypatch.setattr(mb, "rmsnorm_backward", wrong)
    assert _check_against_fd(11) != []


def test_step_without_clipping_or_noise_is_sgd_on_the_batch_loss():
    x, gamma, Wg, Wu, Wd, R = _block(21)
    eta, B = 0.3, x.shape[0]
    n, c, new = mb.mlp_dp_step(x, gamma, Wg, Wu, Wd, EPS, R, "fgc", 0, 1e6, 0.0, eta, 1, 2)
    assert np.all(c == 1.0)
    fwd = mb.mlp_forward(x, gamma, Wg, Wu, Wd, EPS)
    bwd = mb.mlp_backward(x, gamma, Wg, Wu, Wd, EPS, R, fwd)
    grads = mb.mlp_per_sample_grads(fwd, bwd)
    # the FGC norm is the sum over parameters of the squared per-sample gradient norms
    n_ref = sum(np.sum(grads[k].reshape(B, -1) ** 2, axis=1) for k in grads)
    assert np.allclose(n, n_ref, rtol=1e-12)
    # theta' = theta - eta/B * (gradient of sum_i L_i), checked by finite differences
    r = np.random.default_rng(0)
    h = 1e-5
    params = {"gamma": gamma, "W_gate": Wg, "W_up": Wu, "W_down": Wd}
    order = ["gamma", "W_gate", "W_up", "W_down"]
    for name, P in params.items():
        for _ in range(3):
            idx = tuple(r.integers(0, s) for s in P.shape)
            Pp, Pm = P.copy(), P.copy()
            Pp[idx] += h
            Pm[idx] -= h
            args_p = [params[o] if o != name else Pp for o in order]
            args_m = [params[o] if o != name else Pm for o in order]
            fd = sum(_loss(i, x, *args_p, R) - _loss(i, x, *args_m, R) for i in range(B)) / (2 * h)
            assert np.isclose(new[name][idx], P[idx] - eta / B * fd, rtol=1e-8, atol=1e-10)


def test_step_clips_the_whole_gradient():
    """With a small C every sample's clipped gradient over all four parameters
    has norm C: the clipped sum of a one-sample batch has norm exactly C."""
    x, gamma, Wg, Wu, Wd, R = _block(22, B=1)
    C = 1e-3
    n, c, new = mb.mlp_dp_step(x, gamma, Wg, Wu, Wd, EPS, R, "fgc", 0, C, 0.0, 1.0, 1, 2)
    assert c[0] < 1.0
    delta = np.concatenate([(p0 - new[k]).ravel() for k, p0 in
                            (("W_gate", Wg), ("W_up", Wu), ("W_down", Wd), ("gamma", gamma))])
    assert np.isclose(np.linalg.norm(delta), C, rtol=1e-10)
