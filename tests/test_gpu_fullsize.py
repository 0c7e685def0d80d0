"""GPU parity at the workloads' full sizes (the shapes and calls bench.py times).

Per-sample norms are compared for every sample, for the workload's estimator,
for the other estimators its configuration compares it with, and for the exact
ghost and FGC baselines (against the oracle's materialised ||A_i^T G_i||^2 of
every sample); the clipped sum and the update are compared on seeded sampled
rows of the (p, d) outputs, which the oracle computes row by row.  The
112-layer stack is covered per layer shape (one layer of each distinct (d, p),
norms accumulated over them), since its inputs (46 GB) cannot be drawn on the
host in a test.
Tolerances: bf16-input norms 2e-2 relative per sample; S within 1e-4 of its
max (fp32 accumulation of exact bf16 products); theta' within 1e-5.
"""

import numpy as np
import pytest
import torch

import oracle
from sample_gradient_clipping_amd import binding as dp
from sample_gradient_clipping_amd.configs import workloads
from sample_gradient_clipping_amd.inputs import linear_inputs
from tests.gpu_util import device, f64, max_rel_elementwise, max_rel_normwise, report

pytestmark = pytest.mark.gpu

WL = workloads()


@pytest.fixture(scope="module")
def dev():
    d = device()
    dp.load_library()
    return d


def _step_and_check(dev, wl, layers, method, rows_per_layer=24, baselines=(), estimators=()):
    """Norms over `layers` (accumulated), clip + aggregate + update per layer;
    compare to the oracle on all norms and on sampled rows.  Then, on the first
    layer, the other `estimators` (same probes as the oracle's) and the exact
    `baselines` on every sample."""
    B, T, k = wl.B, wl.T, wl.k
    host = []
    n = torch.zeros(B, dtype=torch.float32, device=dev)
    for li, l in enumerate(layers):
        A, G = linear_inputs(B, T, l.d, l.p, wl.dtype, wl.recipe, wl.data_seed, l.layer_id)
        host.append((l, A, G))
        Ad, Gd = A.to(dev), G.to(dev)
        dp.dp_norm_est(method, Ad, Gd, k, wl.method_seed, l.layer_id, n,
                       flags=dp.DP_ACCUMULATE if li else 0)
        del Ad, Gd
    torch.cuda.synchronize()
    n_gpu = f64(n)
    n_ref = sum(oracle.norm_est(method, A, G, k=k, seed=wl.method_seed, layer=l.layer_id)
                for l, A, G in host)
    err_n = max_rel_elementwise(n_gpu, n_ref)
    report(f"{wl.name} norms {method}", max_rel=err_n)
    assert err_n <= 2e-2
    # clip + aggregate + update from the GPU norms (the same n both sides)
    c_ref, _ = oracle.clip_factors(n_gpu, wl.C)
    rng = np.random.default_rng(wl.data_seed)
    for l, A, G in host:
        Ad, Gd = A.to(dev), G.to(dev)
        S = torch.empty(l.p, l.d, dtype=torch.float32, device=dev)
        c = torch.empty(B, dtype=torch.float32, device=dev)
        dp.dp_clip_aggregate(Ad, Gd, n, wl.C, S, c_out=c)
        theta = torch.zeros(l.p, l.d, dtype=torch.float32, device=dev)
        dp.dp_noise_update(theta, S, wl.sigma, wl.C, wl.eta, B, wl.noise_seed, l.layer_id)
        torch.cuda.synchronize()
        assert max_rel_elementwise(f64(c), c_ref) <= 1e-5
        rows = np.sort(rng.choice(l.p, size=min(rows_per_layer, l.p), replace=False))
        S_rows = oracle.aggregate_rows(A, G, c_ref, rows)
        es = max_rel_normwise(f64(S)[rows], S_rows)
        th_ref = oracle.noise_update(np.zeros((len(rows), l.d)), S_rows, wl.sigma, wl.C, wl.eta, B,
                                     wl.noise_seed, l.layer_id, rows=rows)
        et = max_rel_normwise(f64(theta)[rows], th_ref)
        report(f"{wl.name} layer {l.name}", S_err=es, theta_err=et)
        assert es <= 1e-4
        assert et <= 1e-5
        del Ad, Gd, S, theta
    l, A, G = host[0]
    for est in estimators:  # another estimator, same seeded probes as the oracle's
        ne = torch.zeros(B, dtype=torch.float32, device=dev)
        dp.dp_norm_est(est, A.to(dev), G.to(dev), k, wl.method_seed, l.layer_id, ne)
        torch.cuda.synchronize()
        ref = oracle.norm_est(est, A, G, k=k, seed=wl.method_seed, layer=l.layer_id)
        e = max_rel_elementwise(f64(ne), ref)
        report(f"{wl.name} layer {l.name} {est} every sample", max_rel=e)
        assert e <= 2e-2
    if baselines:  # exact baselines against the materialised ||A_i^T G_i||^2 of every sample
        exact = np.array([oracle.fgc_norm_sq(oracle.to_f64(A[i]), oracle.to_f64(G[i]))
                          for i in range(B)])
        for bl in baselines:
            nb = torch.zeros(B, dtype=torch.float32, device=dev)
            dp.dp_norm_est(bl, A.to(dev), G.to(dev), 0, 0, 0, nb)
            torch.cuda.synchronize()
            e = max_rel_elementwise(f64(nb), exact)
            report(f"{wl.name} layer {l.name} {bl} every sample", max_rel=e)
            assert e <= 2e-2


def test_attention_projection(dev):
    wl = WL["attn_proj_b8_t4096_d2048"]
    _step_and_check(dev, wl, wl.layers, "hutch", baselines=("ghost", "fgc"))


@pytest.mark.parametrize("name", ["mlp_up_b8_t4096_d2048_p8192", "mlp_down_b8_t4096_d8192_p2048"])
def test_mlp_hutchpp(dev, name):
    wl = WL[name]
    _step_and_check(dev, wl, wl.layers, "hutchpp", baselines=("ghost", "fgc"),
                    estimators=("hutch",))


def test_long_context(dev):
    wl = WL["long_ctx_b2_t16384_d2048_p8192"]
    _step_and_check(dev, wl, wl.layers, "hutch", rows_per_layer=8, baselines=("ghost", "fgc"),
                    estimators=("hutchpp",))


def test_llama_stack_layer_shapes(dev):
    wl = WL["llama1b_stack_b8_t4096"]
    seen, layers = set(), []
    for l in wl.layers:  # one layer of each distinct shape: q, k, gate, down
        if (l.d, l.p) not in seen:
            seen.add((l.d, l.p))
            layers.append(l)
    _step_and_check(dev, wl, layers, "hutch", rows_per_layer=16)
