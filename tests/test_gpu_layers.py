"""GPU tests of the batched calls over a step's linear layers
(dp_norm_est_layers, dp_clip_aggregate_update_layers).

They compute what the per-layer calls compute: the norm summed over the
layers (checked against the oracle's sum over layers, and against the
per-layer calls on the GPU with the same probes), and each layer's update
(bit-identical to the per-layer fused call, the same clip factors formed
once).  Shapes cover the batched Hutch path (every layer with at least 256
column blocks of the projection), the per-layer fallback (fp32, shapes off the
MFMA tiles, other methods), more layers than one probe launch takes (64), the
probe flags, accumulation and the status word.
Tolerances: norms 2e-2 relative per sample against the oracle (bf16 inputs),
1e-5 against the per-layer GPU calls (the same products; only the order of
the fp64 / fp32 sums over layers differs); fp32 inputs 1e-5 against the oracle.
"""

import numpy as np
import pytest
import torch

import oracle
from sample_gradient_clipping_amd import binding as dp
from sample_gradient_clipping_amd.inputs import linear_inputs
from tests.gpu_util import device, f64, max_rel_elementwise, max_rel_normwise, report

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    d = device()
    dp.load_library()
    return d


def _make(B, T, shapes, dtype, seed, recipe="llama_logu"):
    host, devl = [], []
    for i, (d, p, lid) in enumerate(shapes):
        A, G = linear_inputs(B, T, d, p, dtype, recipe, seed + 31 * i, lid)
        host.append((A, G, lid))
        devl.append((A.to(torch.device("cuda:0")), G.to(torch.device("cuda:0")), lid))
    return host, devl


def _per_layer(method, devl, k, seed, B, dev, flags=0):
    n = torch.zeros(B, dtype=torch.float32, device=dev)
    for i, (A, G, lid) in enumerate(devl):
        f = flags | (dp.DP_ACCUMULATE if i else 0)
        dp.dp_norm_est(method, A, G, k, seed, lid, n, flags=f)
    torch.cuda.synchronize()
    return f64(n)


# the batched Hutch path: B d / 64 >= 256 for every layer (64-column blocks need
# T % 256 == 0, 128-column blocks T % 128 == 0)
FUSED_SHAPES = [(2048, 2048, 3), (2048, 512, 4), (4096, 1024, 9)]


def test_norm_layers_batched_hutch(dev):
    B, T, k, seed = 8, 256, 32, 4242
    host, devl = _make(B, T, FUSED_SHAPES, "bf16", 5)
    n = torch.full((B,), -1.0, dtype=torch.float32, device=dev)
    dp.dp_norm_est_layers("hutch", devl, k, seed, n)
    torch.cuda.synchronize()
    ref = sum(oracle.norm_est("hutch", A, G, k=k, seed=seed, layer=lid) for A, G, lid in host)
    e_or = max_rel_elementwise(f64(n), ref)
    e_pl = max_rel_elementwise(f64(n), _per_layer("hutch", devl, k, seed, B, dev))
    report("norm layers batched hutch", oracle=e_or, per_layer=e_pl)
    assert e_or <= 2e-2
    assert e_pl <= 1e-5


@pytest.mark.parametrize("shapes", [
    [(2048, 2048, 0), (2048, 512, 1)],   # q, k: 64-token sketches, 64-column projections
    [(2048, 8192, 5), (8192, 2048, 6)],  # up, down: 128-token sketch, 128-column projection
], ids=["q_k", "up_down"])
def test_norm_layers_batched_full_width(dev, shapes):
    """The batched norm call at the stack's width and token count (B 8, T 4096,
    Llama 3.2 1B projections): the grouped sketch and fused projection-and-square
    launches that the step over the stack runs, every per-sample norm against
    the oracle and against the per-layer calls."""
    B, T, k, seed = 8, 4096, 32, 515
    host, devl = _make(B, T, shapes, "bf16", 14)
    n = torch.zeros(B, dtype=torch.float32, device=dev)
    dp.dp_norm_est_layers("hutch", devl, k, seed, n)
    torch.cuda.synchronize()
    ref = sum(oracle.norm_est("hutch", A, G, k=k, seed=seed, layer=lid) for A, G, lid in host)
    e_or = max_rel_elementwise(f64(n), ref)
    e_pl = max_rel_elementwise(f64(n), _per_layer("hutch", devl, k, seed, B, dev))
    report("norm layers batched full width", oracle=e_or, per_layer=e_pl)
    assert e_or <= 2e-2
    # same kernels per layer: only the order of the sums over layers differs
    assert e_pl <= 1e-5


@pytest.mark.parametrize("flags", [dp.DP_PROBE_SHARED, dp.DP_PROBE_RADEMACHER,
                                   dp.DP_PROBE_SHARED | dp.DP_PROBE_RADEMACHER])
def test_norm_layers_probe_flags(dev, flags):
    B, T, k, seed = 8, 256, 16, 77
    host, devl = _make(B, T, FUSED_SHAPES[:2], "bf16", 6)
    n = torch.zeros(B, dtype=torch.float32, device=dev)
    dp.dp_norm_est_layers("hutch", devl, k, seed, n, flags=flags)
    torch.cuda.synchronize()
    e_pl = max_rel_elementwise(f64(n), _per_layer("hutch", devl, k, seed, B, dev, flags=flags))
    shared = bool(flags & dp.DP_PROBE_SHARED)
    rad = bool(flags & dp.DP_PROBE_RADEMACHER)
    ref = sum(oracle.norm_est("hutch", A, G, k=k, seed=seed, layer=lid, shared=shared,
                              rademacher=rad) for A, G, lid in host)
    e_or = max_rel_elementwise(f64(n), ref)
    report(f"norm layers flags={flags}", oracle=e_or, per_layer=e_pl)
    assert e_pl <= 1e-5
    assert e_or <= 2e-2


def test_norm_layers_accumulate(dev):
    B, T, k, seed = 8, 256, 32, 91
    host, devl = _make(B, T, FUSED_SHAPES[:2], "bf16", 7)
    base = torch.linspace(1.0, 8.0, B, dtype=torch.float32, device=dev)
    n = base.clone()
    dp.dp_norm_est_layers("hutch", devl, k, seed, n, flags=dp.DP_ACCUMULATE)
    torch.cuda.synchronize()
    ref = f64(base) + sum(oracle.norm_est("hutch", A, G, k=k, seed=seed, layer=lid)
                          for A, G, lid in host)
    e = max_rel_elementwise(f64(n), ref)
    report("norm layers accumulate", max_rel=e)
    assert e <= 2e-2


def test_norm_layers_more_than_one_probe_launch(dev):
    # 70 layers (two probe launches) sharing two inputs under distinct layer ids
    B, T, k, seed = 8, 256, 8, 13
    _, devl = _make(B, T, [(2048, 256, 0), (2048, 512, 1)], "bf16", 8)
    layers = [(devl[i % 2][0], devl[i % 2][1], 1000 + i) for i in range(70)]
    n = torch.zeros(B, dtype=torch.float32, device=dev)
    dp.dp_norm_est_layers("hutch", layers, k, seed, n)
    torch.cuda.synchronize()
    e = max_rel_elementwise(f64(n), _per_layer("hutch", layers, k, seed, B, dev))
    report("norm layers x70", per_layer=e)
    assert e <= 1e-5


@pytest.mark.parametrize("method,dtype,shapes", [
    ("hutch", "f32", [(48, 40, 1), (24, 64, 2)]),        # generic kernels
    ("hutchpp", "bf16", [(256, 512, 1), (512, 256, 2)]),  # Hutch++ on MFMA, per layer
    ("hutch", "bf16", [(256, 512, 1), (512, 256, 2)]),    # MFMA Hutch with split projections
    ("ghost", "bf16", [(256, 512, 1), (512, 256, 2)]),
])
def test_norm_layers_fallback_matches_per_layer(dev, method, dtype, shapes):
    B, T, k, seed = 3, 128, 12, 21
    host, devl = _make(B, T, shapes, dtype, 9, recipe="unit_u0.1_3" if dtype == "f32" else "llama_logu")
    n = torch.zeros(B, dtype=torch.float32, device=dev)
    kk = 0 if method == "ghost" else k
    dp.dp_norm_est_layers(method, devl, kk, seed, n)
    torch.cuda.synchronize()
    per = _per_layer(method, devl, kk, seed, B, dev)
    assert np.array_equal(f64(n), per)  # the same calls in the same order
    ref = sum(oracle.norm_est(method, A, G, k=kk, seed=seed, layer=lid) for A, G, lid in host)
    e = max_rel_elementwise(per, ref)
    report(f"norm layers fallback {method} {dtype}", oracle=e)
    assert e <= (1e-5 if dtype == "f32" else 2e-2)


@pytest.mark.parametrize("dtype,B,T,shapes", [
    # MFMA contractions with token splits, each alone in its tile count (16 and
    # 64 tiles of 256 x 256), and one of 256 tiles (no splits)
    ("bf16", 8, 256, [(2048, 512, 4), (2048, 2048, 3), (4096, 4096, 5)]),
    ("f32", 3, 40, [(24, 20, 1), (16, 12, 2)]),        # generic kernels
])
def test_update_layers_bit_identical_to_per_layer(dev, dtype, B, T, shapes):
    _, devl = _make(B, T, shapes, dtype, 10, recipe="unit_u0.1_3" if dtype == "f32" else "llama_logu")
    n = torch.linspace(0.5, 40.0, B, dtype=torch.float32, device=dev)
    C, sigma, eta, seed = 2.0, 0.7, 1e-3, 99
    th_b = [torch.randn(G.shape[2], A.shape[2], device=dev) for A, G, _ in devl]
    th_p = [t.clone() for t in th_b]
    c_b = torch.empty(B, dtype=torch.float32, device=dev)
    dp.dp_clip_aggregate_update_layers([(A, G, lid, th) for (A, G, lid), th in zip(devl, th_b)],
                                       n, C, sigma, eta, seed, c_out=c_b)
    c_p = torch.empty(B, dtype=torch.float32, device=dev)
    for (A, G, lid), th in zip(devl, th_p):
        dp.dp_clip_aggregate_update(A, G, n, C, sigma, eta, seed, lid, th, c_out=c_p)
    torch.cuda.synchronize()
    assert torch.equal(c_b, c_p)
    for a, b in zip(th_b, th_p):
        assert torch.equal(a, b)
    c_ref, _ = oracle.clip_factors(f64(n), C)
    assert max_rel_elementwise(f64(c_b), c_ref) <= 1e-6


def test_update_layers_status_word(dev):
    B, T = 4, 128
    _, devl = _make(B, T, [(256, 256, 1), (256, 512, 2)], "bf16", 11)
    thetas = [torch.zeros(G.shape[2], A.shape[2], device=dev) for A, G, _ in devl]
    layers = [(A, G, lid, th) for (A, G, lid), th in zip(devl, thetas)]
    ws = dp.clip_workspace(dp.dp_clip_aggregate_update_layers_workspace("bf16", B, T, layers), dev)
    good = torch.tensor([4.0, 0.5, 2.0, 9.0], dtype=torch.float32, device=dev)
    bad = torch.tensor([4.0, float("inf"), 2.0, 9.0], dtype=torch.float32, device=dev)
    dp.dp_clip_aggregate_update_layers(layers, good, 1.0, 1.0, 1e-4, 5, ws=ws)
    assert dp.dp_read_device_status(ws) == 0
    dp.dp_clip_aggregate_update_layers(layers, bad, 1.0, 1.0, 1e-4, 5, ws=ws)
    assert dp.dp_read_device_status(ws) == dp.DP_STATUS_NONFINITE_NORM
    assert dp.dp_read_device_status(ws) == 0


def _tiles(d, p):
    return (p // 256) * (d // 256)


@pytest.mark.parametrize("B,T,shapes,alone", [
    # two 64-tile layers of different shapes: one launch of 128 tiles, 2 token splits
    (8, 256, [(2048, 2048, 3), (4096, 1024, 9)], []),
    # four 64-tile layers: 256 tiles, no splits
    (4, 256, [(2048, 2048, 20 + i) for i in range(4)], []),
    # sixteen 16-tile layers: 256 tiles, no splits
    (4, 128, [(2048, 512, 40 + i) for i in range(16)], []),
    # two 16-tile layers sharing a launch (with token splits), four 64-tile layers
    # in a full group, and a fifth 64-tile layer alone (the per-layer path)
    (4, 128, [(2048, 512, 70), (2048, 2048, 71), (2048, 2048, 72), (2048, 2048, 73),
              (2048, 512, 74), (2048, 2048, 75), (2048, 2048, 76)], [6]),
    # the stack's two grouped launches at full width (B 8, T 4096: 1024 stages a
    # workgroup): four q/o-shaped layers, and sixteen k/v-shaped ones
    (8, 4096, [(2048, 2048, 100 + i) for i in range(4)], []),
    (8, 4096, [(2048, 512, 120 + i) for i in range(16)], []),
])
def test_update_layers_grouped_contraction(dev, B, T, shapes, alone):
    """Layers whose tile counts divide 256 share contraction launches: theta matches
    the per-layer calls to fp32 rounding (bit for bit for a layer left alone) and
    the oracle on sampled rows."""
    host, devl = _make(B, T, shapes, "bf16", 12)
    n = torch.linspace(0.5, 40.0, B, dtype=torch.float32, device=dev)
    C, sigma, eta, seed = 2.0, 2e-3, 50.0, 123
    th0 = [torch.randn(G.shape[2], A.shape[2], device=dev) * 1e-2 for A, G, _ in devl]
    th_b = [t.clone() for t in th0]
    th_p = [t.clone() for t in th0]
    c_b = torch.empty(B, dtype=torch.float32, device=dev)
    dp.dp_clip_aggregate_update_layers([(A, G, lid, th) for (A, G, lid), th in zip(devl, th_b)],
                                       n, C, sigma, eta, seed, c_out=c_b)
    for (A, G, lid), th in zip(devl, th_p):
        dp.dp_clip_aggregate_update(A, G, n, C, sigma, eta, seed, lid, th)
    torch.cuda.synchronize()
    c_ref, _ = oracle.clip_factors(f64(n), C)
    assert max_rel_elementwise(f64(c_b), c_ref) <= 1e-6
    worst_p = worst_o = 0.0
    for i, ((A, G, lid), t0, tb, tp) in enumerate(zip(host, th0, th_b, th_p)):
        if i in alone:
            assert torch.equal(tb, tp)
        e_p = max_rel_normwise(f64(tb) - f64(t0), f64(tp) - f64(t0))
        rows = np.sort(np.random.default_rng(i).choice(tb.shape[0], size=8, replace=False))
        S_rows = oracle.aggregate_rows(A, G, c_ref, rows)
        t_ref = oracle.noise_update(f64(t0)[rows], S_rows, sigma, C, eta, B, seed, lid, rows=rows)
        e_o = max_rel_normwise(f64(tb)[rows] - f64(t0)[rows], t_ref - f64(t0)[rows])
        worst_p, worst_o = max(worst_p, e_p), max(worst_o, e_o)
    report(f"update layers grouped x{len(shapes)}", per_layer=worst_p, oracle=worst_o)
    assert worst_p <= 1e-5
    assert worst_o <= 1e-4


def test_update_layers_grouped_timed_pairs_add_up(dev):
    # a shared launch is timed in its first layer's pair; the others' pairs are empty
    B, T = 4, 1024  # 137 GFLOP in the shared launch: far longer than an empty pair
    _, devl = _make(B, T, [(2048, 2048, 80 + i) for i in range(4)], "bf16", 13)
    thetas = [torch.zeros(G.shape[2], A.shape[2], device=dev) for A, G, _ in devl]
    layers = [(A, G, lid, th) for (A, G, lid), th in zip(devl, thetas)]
    n = torch.full((B,), 4.0, dtype=torch.float32, device=dev)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in layers]
    eu = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in layers]
    dp.dp_clip_aggregate_update_layers(layers, n, 1.0, 1.0, 1e-3, 5, agg_events=ev, upd_events=eu)
    torch.cuda.synchronize()
    t = [a.elapsed_time(b) for a, b in ev]
    report("update layers grouped timed pairs", first_ms=t[0], others_max_ms=max(t[1:]))
    assert t[0] > 0.0
    assert all(abs(x) < 0.2 * t[0] for x in t[1:])
    assert all(a.elapsed_time(b) > 0.0 for a, b in eu)
