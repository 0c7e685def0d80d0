"""GPU parity of a whole Llama decoder layer (the attention block feeding the
MLP block): forward pass, backward pass 1 through both blocks, and the layer's
DP-SGD-RC step with one clip factor per sample over all eleven parameters.

The library's block entry points are chained exactly as a training step chains
them (the MLP block's dL/d(input) is the attention block's dL/d(out)).  End to
end against the fp64 oracle (no bf16 intermediates) the bound is normwise 2e-2,
as for each block; the step is checked against the oracle's step on the GPU's
own activations and output gradients: for FGC squared norms within 1e-5 (fp32
accumulation) and updates within 1e-4 normwise; for Hutch and Hutch++ (bf16
probes and sketches) both within 2e-2.
"""

import numpy as np
import pytest
import torch

import oracle
from sample_gradient_clipping_amd import binding as dp
from sample_gradient_clipping_amd.inputs import mlp_block_inputs
from tests.gpu_util import device, f64, max_rel_normwise, report

pytestmark = pytest.mark.gpu

EPS, BASE = 1e-5, 500000.0


@pytest.fixture(scope="module")
def dev():
    d = device()
    dp.load_library()
    return d


def _bf(t):
    return t.detach().cpu().float().double().numpy()


def _layer(dev, B, T, d, f, H, KV, seed):
    x, g_mlp, th_mlp, R = mlp_block_inputs(B, T, d, f, seed)
    r = np.random.default_rng(seed + 1)
    g_attn = torch.from_numpy((1.0 + 0.1 * r.standard_normal(d)).astype(np.float32))
    th_attn = {"W_q": 0.02 * r.standard_normal((64 * H, d)),
               "W_k": 0.02 * r.standard_normal((64 * KV, d)),
               "W_v": 0.02 * r.standard_normal((64 * KV, d)),
               "W_o": 0.02 * r.standard_normal((d, 64 * H))}
    th_attn = {k_: torch.from_numpy(v_.astype(np.float32)) for k_, v_ in th_attn.items()}
    thetas = {**th_attn, **th_mlp}
    Wb = {k_: dp.dp_weights_bf16(v_.to(dev)) for k_, v_ in thetas.items()}
    torch.cuda.synchronize()
    return x, g_attn, g_mlp, thetas, R, Wb


def _gpu_layer(dev, x, g_attn, g_mlp, R, Wb, H, KV):
    xd, gad, gmd, Rd = x.to(dev), g_attn.to(dev), g_mlp.to(dev), R.to(dev)
    a_acts = dp.dp_attn_forward(xd, gad, Wb["W_q"][0], Wb["W_k"][0], Wb["W_v"][0], Wb["W_o"][0],
                                H, KV, eps=EPS, rope_base=BASE)
    h1 = a_acts["out"]
    m_acts = dp.dp_mlp_forward(h1, gmd, Wb["W_gate"][0], Wb["W_up"][0], Wb["W_down"][0], eps=EPS)
    m_grads = dp.dp_mlp_backward(h1, m_acts["rstd"], gmd, m_acts["g"], m_acts["u"],
                                 Wb["W_gate"][1], Wb["W_up"][1], Wb["W_down"][1], Rd)
    a_grads = dp.dp_attn_backward(xd, a_acts, gad, Wb["W_q"][1], Wb["W_k"][1], Wb["W_v"][1],
                                  Wb["W_o"][1], m_grads["dx"], H, KV, rope_base=BASE)
    return xd, gad, gmd, Rd, a_acts, m_acts, a_grads, m_grads


LAYER_CASES = [(2, 128, 256, 512, 8, 4), (1, 256, 512, 768, 8, 8)]


@pytest.mark.parametrize("B,T,d,f,H,KV", LAYER_CASES)
def test_layer_forward_backward_end_to_end(dev, B, T, d, f, H, KV):
    x, g_attn, g_mlp, thetas, R, Wb = _layer(dev, B, T, d, f, H, KV, 201)
    _, _, _, _, a_acts, m_acts, a_grads, m_grads = _gpu_layer(dev, x, g_attn, g_mlp, R, Wb, H, KV)
    torch.cuda.synchronize()
    W = {k_: _bf(v_[0]) for k_, v_ in Wb.items()}
    attn_p = (g_attn.double().numpy(), W["W_q"], W["W_k"], W["W_v"], W["W_o"])
    mlp_p = (g_mlp.double().numpy(), W["W_gate"], W["W_up"], W["W_down"])
    xf, Rf = _bf(x), _bf(R)
    fa, fm = oracle.layer_forward(xf, attn_p, mlp_p, EPS, H, KV, 64, BASE)
    ba, bm = oracle.layer_backward(xf, attn_p, mlp_p, EPS, H, KV, 64, BASE, Rf, (fa, fm))
    checks = [("attn out", a_acts["out"], fa["out"]), ("mlp out", m_acts["out"], fm["out"]),
              ("mlp h", m_acts["h"], fm["h"]), ("G_gate", m_grads["G_gate"], bm["G_gate"]),
              ("G_up", m_grads["G_up"], bm["G_up"]), ("mlp dx", m_grads["dx"], bm["dx"]),
              ("G_q", a_grads["G_q"], ba["G_q"]), ("G_k", a_grads["G_k"], ba["G_k"]),
              ("G_v", a_grads["G_v"], ba["G_v"]), ("dy", a_grads["dy"], ba["dy"]),
              ("dx", a_grads["dx"], ba["dx"])]
    for name, got, ref in checks:
        e = max_rel_normwise(_bf(got), ref)
        report(f"layer end-to-end {name} B={B} T={T} d={d} f={f} H={H} KV={KV}", max_rel=e)
        assert e <= 2e-2, name


@pytest.mark.parametrize("method,k", [("fgc", 0), ("hutch", 6), ("hutchpp", 9)])
def test_layer_dp_step_matches_oracle(dev, method, k):
    B, T, d, f, H, KV = 3, 128, 256, 512, 8, 4
    x, g_attn, g_mlp, thetas, R, Wb = _layer(dev, B, T, d, f, H, KV, 203)
    xd, gad, gmd, Rd, a_acts, m_acts, a_grads, m_grads = _gpu_layer(dev, x, g_attn, g_mlp, R, Wb,
                                                                    H, KV)
    # sigma small enough that the clipped sum, not the noise, dominates the update,
    # and eta large enough that the update, not the fp32 rounding of theta', sets
    # the difference
    C, sigma, eta, seed_n, seed_z = 0.01, 2e-3, 50.0, 17, 19
    ids = dict(oracle.ATTN_LAYERS)
    ids.update({("mlp_" + n_ if n_ == "gamma" else n_): 5 + i for n_, i in oracle.MLP_LAYERS})
    lin = {"W_q": (a_acts["y"], a_grads["G_q"]), "W_k": (a_acts["y"], a_grads["G_k"]),
           "W_v": (a_acts["y"], a_grads["G_v"]), "W_o": (a_acts["o"], m_grads["dx"]),
           "W_gate": (m_acts["y"], m_grads["G_gate"]), "W_up": (m_acts["y"], m_grads["G_up"]),
           "W_down": (m_acts["h"], Rd)}
    n = torch.zeros(B, dtype=torch.float32, device=dev)
    va = torch.empty(B, d, dtype=torch.float32, device=dev)
    vm = torch.empty(B, d, dtype=torch.float32, device=dev)
    dp.dp_rmsnorm_norm(a_acts["xhat"], a_grads["dy"], n, v=va)
    dp.dp_rmsnorm_norm(m_acts["xhat"], m_grads["dy"], n, v=vm, flags=dp.DP_ACCUMULATE)
    for name, (A, G) in lin.items():
        dp.dp_norm_est(method, A, G, k, seed_n, ids[name], n, flags=dp.DP_ACCUMULATE)
    theta = {name: t.to(dev).clone() for name, t in thetas.items()}
    for name, (A, G) in lin.items():
        dp.dp_clip_aggregate_update(A, G, n, C, sigma, eta, seed_z, ids[name], theta[name])
    ga, gm = gad.clone(), gmd.clone()
    dp.dp_rmsnorm_clip_aggregate_update(va, n, C, sigma, eta, seed_z, ids["gamma"], ga)
    dp.dp_rmsnorm_clip_aggregate_update(vm, n, C, sigma, eta, seed_z, ids["mlp_gamma"], gm)
    torch.cuda.synchronize()
    a_host = {"y": a_acts["y"], "o": a_acts["o"], "xhat": a_acts["xhat"], "G_q": a_grads["G_q"],
              "G_k": a_grads["G_k"], "G_v": a_grads["G_v"], "G_o": m_grads["dx"],
              "dy": a_grads["dy"]}
    m_host = {"y": m_acts["y"], "h": m_acts["h"], "xhat": m_acts["xhat"],
              "G_gate": m_grads["G_gate"], "G_up": m_grads["G_up"], "G_down": Rd,
              "dy": m_grads["dy"]}
    a_host = {k_: _bf(t) for k_, t in a_host.items()}
    m_host = {k_: _bf(t) for k_, t in m_host.items()}
    th64 = {k_: t.double().numpy() for k_, t in thetas.items()}
    attn_p = (g_attn.double().numpy(), th64["W_q"], th64["W_k"], th64["W_v"], th64["W_o"])
    mlp_p = (g_mlp.double().numpy(), th64["W_gate"], th64["W_up"], th64["W_down"])
    n_r, c_r, new_r = oracle.layer_dp_step(a_host, m_host, attn_p, mlp_p, method, k, C, sigma,
                                           eta, seed_n, seed_z)
    assert np.all(c_r < 1.0)
    # fp32 accumulation for FGC; the sketches' bf16 probes and intermediates for
    # Hutch and Hutch++ (relative error of n ~1e-3, its half in c and the update)
    tol_n, tol_u = (1e-5, 1e-4) if method == "fgc" else (2e-2, 2e-2)
    e_n = float(np.max(np.abs(f64(n) - n_r) / n_r))
    report(f"layer step {method} n", max_rel=e_n)
    assert e_n <= tol_n
    got = {**{k_: f64(t) for k_, t in theta.items()}, "gamma": f64(ga), "mlp_gamma": f64(gm)}
    for name in new_r:
        base = (g_attn if name == "gamma" else g_mlp if name == "mlp_gamma"
                else thetas[name]).double().numpy()
        e = max_rel_normwise(got[name] - base, new_r[name] - base)
        report(f"layer step {method} {name}", max_rel=e)
        assert e <= tol_u, name
