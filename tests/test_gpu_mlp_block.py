"""GPU parity of the MLP block's forward pass and backward pass 1, and of its
whole DP-SGD-RC step, against the fp64 oracle.

Every kernel is checked on its own against the oracle applied to the GPU's own
bf16 inputs of that stage, within a bound derived from the arithmetic: a bf16
result is within 2^-8 |ref| of its fp32 value, an fp32 sum of K products
within K 2^-24 sum |a b| of the exact one, and the fp32 elementwise code
within 1e-5 of the magnitudes it combines.  SwiGLU runs in the products'
epilogues on the fp32 sums, so h (and dL/dg, dL/du) carry the sums' error
through the first derivatives.  End to end (fp64 oracle from the
same inputs, no bf16 intermediates) the bound is normwise, 2e-2.  At the full
Llama-3.2-1B width (d 2048, f 8192, 32768 tokens) sampled token rows are
checked one by one (every row of the block depends only on its own token).
"""

import numpy as np
import pytest
import torch

import oracle
from sample_gradient_clipping_amd import binding as dp
from sample_gradient_clipping_amd.inputs import mlp_block_inputs
from tests.gpu_util import device, f64, max_rel_normwise, report

pytestmark = pytest.mark.gpu

U8 = 2.0 ** -8   # bf16 unit roundoff
U24 = 2.0 ** -24  # fp32 unit roundoff
EPS = 1e-5


@pytest.fixture(scope="module")
def dev():
    d = device()
    dp.load_library()
    return d


def _bf16_f64(t):
    return t.detach().cpu().float().double().numpy()


def gemm_bound(A, W, ref, K):
    """|C - ref| bound for C = bf16(fp32 sum of K bf16 products (+ residual))."""
    return U8 * np.abs(ref) + (1 + U8) * K * U24 * (np.abs(A) @ np.abs(W).T) * 1.01 + 1e-30


def assert_within(name, got, ref, bound):
    excess = np.abs(got - ref) - bound
    worst = float(np.max(excess / np.maximum(bound, 1e-300)))
    report(name, max_rel=max_rel_normwise(got, ref), worst_over_bound=worst)
    assert np.all(excess <= 0), f"{name}: {int(np.sum(excess > 0))} elements beyond the bound"


GEMM_CASES = [  # (M, N, K, residual)
    (256, 256, 32, False),    # one stage
    (300, 512, 96, True),     # ragged m tail, three stages
    (1, 256, 64, False),      # a single row
    (513, 256, 2048, True),   # 64 stages, tail of one row
    (1024, 768, 160, False),  # several tiles each way, 5 stages
]


@pytest.mark.parametrize("M,N,K,resid", GEMM_CASES)
def test_linear_forward_matches_matmul(dev, M, N, K, resid):
    r = np.random.default_rng(M * 7 + K)
    A = torch.from_numpy(r.standard_normal((M, K), dtype=np.float32)).to(torch.bfloat16)
    W = torch.from_numpy(r.standard_normal((N, K), dtype=np.float32)).to(torch.bfloat16)
    R = torch.from_numpy(r.standard_normal((M, N), dtype=np.float32)).to(torch.bfloat16)
    C = dp.dp_linear_forward(A.to(dev), W.to(dev), R.to(dev) if resid else None)
    torch.cuda.synchronize()
    Af, Wf = _bf16_f64(A), _bf16_f64(W)
    ref = oracle.linear_forward(Af, Wf, residual=_bf16_f64(R) if resid else None)
    assert_within(f"linear M={M} N={N} K={K}", _bf16_f64(C), ref, gemm_bound(Af, Wf, ref, K))


def test_weights_bf16_is_rounding_and_transpose(dev):
    r = np.random.default_rng(5)
    theta = torch.from_numpy(r.standard_normal((192, 320), dtype=np.float32))
    theta[0, :4] = torch.tensor([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -0.0, 65504.0])  # ties, -0
    W, Wt = dp.dp_weights_bf16(theta.to(dev))
    torch.cuda.synchronize()
    ref = theta.to(torch.bfloat16)  # round to nearest even
    assert torch.equal(W.cpu().view(torch.int16), ref.view(torch.int16))
    assert torch.equal(Wt.cpu().view(torch.int16), ref.t().contiguous().view(torch.int16))


def _block(dev, B, T, d, f, seed):
    x, gamma, thetas, R = mlp_block_inputs(B, T, d, f, seed)
    Wb = {k: dp.dp_weights_bf16(v.to(dev)) for k, v in thetas.items()}
    torch.cuda.synchronize()
    return x, gamma, thetas, R, Wb


BLOCK_CASES = [(2, 128, 256, 512), (3, 100, 512, 768)]  # the second: 300 rows, ragged tail


@pytest.mark.parametrize("B,T,d,f", BLOCK_CASES)
def test_mlp_forward_stagewise_and_end_to_end(dev, B, T, d, f):
    x, gamma, thetas, R, Wb = _block(dev, B, T, d, f, 71)
    acts = dp.dp_mlp_forward(x.to(dev), gamma.to(dev), Wb["W_gate"][0], Wb["W_up"][0],
                             Wb["W_down"][0], eps=EPS)
    torch.cuda.synchronize()
    xf = _bf16_f64(x).reshape(-1, d)
    gm = gamma.double().numpy()
    W = {k: _bf16_f64(v[0]) for k, v in Wb.items()}
    got = {k: (f64(v) if k == "rstd" else _bf16_f64(v)).reshape(B * T, -1) for k, v in acts.items()}
    # RMSNorm
    xhat_r, y_r, rstd_r = oracle.rmsnorm_forward(xf, gm, EPS)
    assert np.allclose(got["rstd"][:, 0], rstd_r, rtol=1e-5, atol=0)
    assert_within("rmsnorm xhat", got["xhat"], xhat_r, (U8 + 2e-5) * np.abs(xhat_r))
    assert_within("rmsnorm y", got["y"], y_r, (U8 + 2e-5) * np.abs(y_r))
    # gate, up on the GPU's y
    for name, key in (("g", "W_gate"), ("u", "W_up")):
        ref = oracle.linear_forward(got["y"], W[key])
        assert_within(f"forward {name}", got[name], ref, gemm_bound(got["y"], W[key], ref, d))
    # h comes from the fp32 sums of g and u (the product's epilogue), before they are
    # rounded: compare with SwiGLU of the exact products, the sums' error carried
    # through the first derivatives
    g_ex, u_ex = oracle.linear_forward(got["y"], W["W_gate"]), oracle.linear_forward(got["y"], W["W_up"])
    h_r = oracle.swiglu_forward(g_ex, u_ex)
    acc_g = 1.01 * d * U24 * (np.abs(got["y"]) @ np.abs(W["W_gate"]).T)
    acc_u = 1.01 * d * U24 * (np.abs(got["y"]) @ np.abs(W["W_up"]).T)
    sg = 1.0 / (1.0 + np.exp(-g_ex))
    dev1 = np.abs(u_ex * sg * (1.0 + g_ex * (1.0 - sg))) * acc_g + np.abs(g_ex * sg) * acc_u
    assert_within("swiglu h", got["h"], h_r, (U8 + 1e-5) * (np.abs(h_r) + dev1) + 1.01 * dev1 + 1e-30)
    out_r = oracle.linear_forward(got["h"], W["W_down"], residual=xf)
    assert_within("forward out", got["out"], out_r, gemm_bound(got["h"], W["W_down"], out_r, f))
    # end to end, fp64 throughout
    ref = oracle.mlp_forward(xf, gm, W["W_gate"], W["W_up"], W["W_down"], EPS)
    for k in ("y", "g", "u", "h", "out"):
        e = max_rel_normwise(got[k], ref[k])
        report(f"forward end-to-end {k}", max_rel=e)
        assert e <= 2e-2


def _swiglu_bwd_bound(dh_r, dh_bound, g, u, ref_dg, ref_du):
    s = 1.0 / (1.0 + np.exp(-g))
    a_g = u * s * (1.0 + g * (1.0 - s))
    a_u = g * s
    dh_abs = np.abs(dh_r) + dh_bound
    bg = np.abs(a_g) * dh_bound + (U8 + 1e-5) * (np.abs(ref_dg) + np.abs(a_g) * dh_bound) \
        + 1e-5 * dh_abs * np.abs(u) * s * (1.0 + np.abs(g)) + 1e-30
    bu = np.abs(a_u) * dh_bound + (U8 + 1e-5) * (np.abs(ref_du) + np.abs(a_u) * dh_bound) + 1e-30
    return bg, bu


@pytest.mark.parametrize("B,T,d,f", BLOCK_CASES)
def test_mlp_backward_stagewise_and_end_to_end(dev, B, T, d, f):
    x, gamma, thetas, R, Wb = _block(dev, B, T, d, f, 73)
    xd, gd, Rd = x.to(dev), gamma.to(dev), R.to(dev)
    acts = dp.dp_mlp_forward(xd, gd, Wb["W_gate"][0], Wb["W_up"][0], Wb["W_down"][0], eps=EPS)
    grads = dp.dp_mlp_backward(xd, acts["rstd"], gd, acts["g"], acts["u"], Wb["W_gate"][1],
                               Wb["W_up"][1], Wb["W_down"][1], Rd)
    torch.cuda.synchronize()
    M = B * T
    xf, Rf = _bf16_f64(x).reshape(M, d), _bf16_f64(R).reshape(M, d)
    gm = gamma.double().numpy()
    W = {k: _bf16_f64(v[0]) for k, v in Wb.items()}
    g_, u_ = _bf16_f64(acts["g"]).reshape(M, f), _bf16_f64(acts["u"]).reshape(M, f)
    got = {k: _bf16_f64(v).reshape(M, -1) for k, v in grads.items()}
    # dh = R W_down (not stored), then the SwiGLU backward
    dh_r = Rf @ W["W_down"]
    dh_b = gemm_bound(Rf, W["W_down"].T, dh_r, d)
    dg_r, du_r = oracle.swiglu_backward(dh_r, g_, u_)
    bg, bu = _swiglu_bwd_bound(dh_r, dh_b, g_, u_, dg_r, du_r)
    assert_within("backward G_gate", got["G_gate"], dg_r, bg)
    assert_within("backward G_up", got["G_up"], du_r, bu)
    # dy = G_gate W_gate + G_up W_up on the GPU's G
    Gcat = np.concatenate([got["G_gate"], got["G_up"]], axis=1)
    Wcat = np.concatenate([W["W_gate"], W["W_up"]], axis=0).T  # [d][2f]
    dy_r = Gcat @ Wcat.T
    assert_within("backward dy", got["dy"], dy_r, gemm_bound(Gcat, Wcat, dy_r, 2 * f))
    # RMSNorm backward on the GPU's dy
    dx_r = oracle.rmsnorm_backward(xf, gm, got["dy"], Rf, EPS)
    xhat, _, rs = oracle.rmsnorm_forward(xf, gm, EPS)
    gdy = np.abs(gm * got["dy"])
    mag = rs[:, None] * (gdy + np.abs(xhat) * np.mean(gdy * np.abs(xhat), axis=1, keepdims=True)) \
        + np.abs(Rf)
    assert_within("backward dx", got["dx"], dx_r, U8 * np.abs(dx_r) + 1e-5 * mag + 1e-30)
    # end to end, fp64 throughout
    fwd = oracle.mlp_forward(xf, gm, W["W_gate"], W["W_up"], W["W_down"], EPS)
    ref = oracle.mlp_backward(xf, gm, W["W_gate"], W["W_up"], W["W_down"], EPS, Rf, fwd)
    for k in ("G_gate", "G_up", "dy", "dx"):
        e = max_rel_normwise(got[k], ref[k])
        report(f"backward end-to-end {k}", max_rel=e)
        assert e <= 2e-2


def _gpu_block_step(dev, x, gamma, thetas, R, Wb, method, k, C, sigma, eta, seed_n, seed_z):
    """Forward, backward pass 1 and the DP step of the block, all on the GPU."""
    B, T, d = x.shape
    xd, gd, Rd = x.to(dev), gamma.to(dev), R.to(dev)
    acts = dp.dp_mlp_forward(xd, gd, Wb["W_gate"][0], Wb["W_up"][0], Wb["W_down"][0], eps=EPS)
    grads = dp.dp_mlp_backward(xd, acts["rstd"], gd, acts["g"], acts["u"], Wb["W_gate"][1],
                               Wb["W_up"][1], Wb["W_down"][1], Rd)
    lin = {"W_gate": (acts["y"], grads["G_gate"]), "W_up": (acts["y"], grads["G_up"]),
           "W_down": (acts["h"], Rd)}
    ids = dict(oracle.MLP_LAYERS)
    n = torch.zeros(B, dtype=torch.float32, device=dev)
    v = torch.empty(B, d, dtype=torch.float32, device=dev)
    dp.dp_rmsnorm_norm(acts["xhat"], grads["dy"], n, v=v)
    for name, (A, G) in lin.items():
        dp.dp_norm_est(method, A, G, k, seed_n, ids[name], n, flags=dp.DP_ACCUMULATE)
    theta = {name: t.to(dev).clone() for name, t in thetas.items()}
    for name, (A, G) in lin.items():
        dp.dp_clip_aggregate_update(A, G, n, C, sigma, eta, seed_z, ids[name], theta[name])
    gam = gd.clone()
    dp.dp_rmsnorm_clip_aggregate_update(v, n, C, sigma, eta, seed_z, ids["gamma"], gam)
    torch.cuda.synchronize()
    host = {"y": acts["y"], "h": acts["h"], "xhat": acts["xhat"], "G_gate": grads["G_gate"],
            "G_up": grads["G_up"], "G_down": Rd, "dy": grads["dy"]}
    host = {k_: _bf16_f64(t) for k_, t in host.items()}
    return f64(n), {**{k_: f64(t) for k_, t in theta.items()}, "gamma": f64(gam)}, host


def test_mlp_block_dp_step_fgc_matches_oracle(dev):
    B, T, d, f = 3, 128, 256, 512
    x, gamma, thetas, R, Wb = _block(dev, B, T, d, f, 79)
    # sigma small enough that the clipped sum, not the noise, dominates the update,
    # and eta large enough that the update, not the fp32 rounding of theta', sets
    # the difference
    C, sigma, eta = 0.01, 2e-3, 50.0
    n, new, acts = _gpu_block_step(dev, x, gamma, thetas, R, Wb, "fgc", 0, C, sigma, eta, 11, 13)
    n_r, c_r, new_r = oracle.mlp_dp_step(None, gamma.double().numpy(),
                                         thetas["W_gate"].double().numpy(),
                                         thetas["W_up"].double().numpy(),
                                         thetas["W_down"].double().numpy(), EPS, None, "fgc", 0, C,
                                         sigma, eta, 11, 13, acts=acts)
    assert np.all(c_r < 1.0)  # every sample clipped: the step's clip factors are exercised
    e_n = float(np.max(np.abs(n - n_r) / n_r))
    report("block step fgc n", max_rel=e_n)
    assert e_n <= 1e-5
    for name in new_r:
        # theta' - theta is the part that depends on the step; compare it normwise
        base = (gamma.double().numpy() if name == "gamma" else thetas[name].double().numpy())
        e = max_rel_normwise(new[name] - base, new_r[name] - base)
        report(f"block step fgc {name}", max_rel=e)
        assert e <= 1e-4


def test_mlp_block_dp_step_hutch_norms(dev):
    B, T, d, f = 2, 256, 256, 512
    x, gamma, thetas, R, Wb = _block(dev, B, T, d, f, 83)
    n, _new, acts = _gpu_block_step(dev, x, gamma, thetas, R, Wb, "hutch", 16, 1.0, 1.0, 0.1, 17,
                                    19)
    n_r = oracle.rmsnorm_norm_sq(acts["xhat"], acts["dy"])
    for name, A, G in (("W_gate", "y", "G_gate"), ("W_up", "y", "G_up"), ("W_down", "h", "G_down")):
        n_r = n_r + oracle.norm_est("hutch", acts[A], acts[G], k=16, seed=17,
                                    layer=dict(oracle.MLP_LAYERS)[name])
    e = float(np.max(np.abs(n - n_r) / n_r))
    report("block step hutch n", max_rel=e)
    assert e <= 2e-2


def test_mlp_block_full_width_sampled_rows(dev):
    """B 8, T 4096, d 2048, f 8192: 48 sampled token rows of every output against
    the fp64 oracle run on those rows alone."""
    B, T, d, f = 8, 4096, 2048, 8192
    x, gamma, thetas, R, Wb = _block(dev, B, T, d, f, 89)
    xd, gd, Rd = x.to(dev), gamma.to(dev), R.to(dev)
    acts = dp.dp_mlp_forward(xd, gd, Wb["W_gate"][0], Wb["W_up"][0], Wb["W_down"][0], eps=EPS)
    grads = dp.dp_mlp_backward(xd, acts["rstd"], gd, acts["g"], acts["u"], Wb["W_gate"][1],
                               Wb["W_up"][1], Wb["W_down"][1], Rd)
    torch.cuda.synchronize()
    rows = np.random.default_rng(3).choice(B * T, size=48, replace=False)
    rows[:2] = [0, B * T - 1]
    idx = torch.from_numpy(rows).to(dev)
    pick = lambda t: _bf16_f64(t.reshape(B * T, -1).index_select(0, idx))  # noqa: E731
    xf, Rf = pick(xd), pick(Rd)
    gm = gamma.double().numpy()
    W = {k: _bf16_f64(v[0]) for k, v in Wb.items()}
    fwd = oracle.mlp_forward(xf, gm, W["W_gate"], W["W_up"], W["W_down"], EPS)
    bwd = oracle.mlp_backward(xf, gm, W["W_gate"], W["W_up"], W["W_down"], EPS, Rf, fwd)
    for k in ("y", "g", "u", "h", "out"):
        e = max_rel_normwise(pick(acts[k]), fwd[k])
        report(f"full-width forward {k}", max_rel=e)
        assert e <= 2e-2
    for k in ("G_gate", "G_up", "dy", "dx"):
        e = max_rel_normwise(pick(grads[k]), bwd[k])
        report(f"full-width backward {k}", max_rel=e)
        assert e <= 2e-2
