"""dp_norm_est_noalloc: dp_norm_est on the library's per-GPU scratch array, for
callers that cannot allocate.  Checked through the C ABI against dp_norm_est on
a caller workspace (bit-identical: the same kernels on the same inputs) and
against the oracle (1e-5 fp32, 2e-2 bf16), on two calls in a row whose second
is smaller than the first, so that the second runs on the scratch contents the
first left behind."""

import numpy as np
import pytest
import torch

import oracle
from sample_gradient_clipping_amd import binding as dp
from sample_gradient_clipping_amd.inputs import linear_inputs
from tests.gpu_util import device, f64, max_rel_elementwise, report

pytestmark = pytest.mark.gpu

# (method, dtype, B, T, d, p, k): large then small, per method
PAIRS = [
    (("hutch", "bf16", 8, 2048, 2048, 2048, 32), ("hutch", "bf16", 3, 256, 256, 512, 32)),
    (("hutchpp", "bf16", 4, 1024, 2048, 2048, 32), ("hutchpp", "bf16", 2, 256, 256, 512, 12)),
    (("hutch", "f32", 4, 96, 80, 120, 16), ("hutch", "f32", 3, 37, 50, 70, 5)),
    (("ghost", "bf16", 4, 1024, 512, 512, 0), ("ghost", "bf16", 2, 256, 256, 256, 0)),
]


@pytest.fixture(scope="module")
def dev():
    d = device()
    dp.load_library()
    return d


def _one(dev, method, dtype, B, T, d, p, k, seed):
    recipe = "unit_u0.1_3" if dtype == "f32" else "llama_logu"
    A, G = linear_inputs(B, T, d, p, dtype, recipe, seed=seed)
    Ad, Gd = A.to(dev), G.to(dev)
    n_free = torch.full((B,), -1.0, dtype=torch.float32, device=dev)
    n_ws = torch.full((B,), -2.0, dtype=torch.float32, device=dev)
    dp.dp_norm_est_noalloc(method, Ad, Gd, k, 4321, 3, n_free)
    dp.dp_norm_est(method, Ad, Gd, k, 4321, 3, n_ws)
    torch.cuda.synchronize()
    ref = oracle.norm_est(method, A, G, k=k, seed=4321, layer=3)
    err = max_rel_elementwise(f64(n_free), ref)
    report(f"noalloc {method} {dtype} B{B} T{T} d{d} p{p} k{k}", max_rel=err)
    assert torch.equal(n_free, n_ws)
    assert err <= (1e-5 if dtype == "f32" else 2e-2)


@pytest.mark.parametrize("pair", PAIRS, ids=[f"{a[0]}_{a[1]}" for a, _ in PAIRS])
def test_noalloc_matches_workspace_call_twice(dev, pair):
    big, small = pair
    _one(dev, *big, seed=31)
    _one(dev, *small, seed=32)


def test_noalloc_accumulates_over_layers(dev):
    A, G = linear_inputs(3, 256, 256, 512, "bf16", "llama_logu", seed=33)
    Ad, Gd = A.to(dev), G.to(dev)
    n = torch.zeros(3, dtype=torch.float32, device=dev)
    dp.dp_norm_est_noalloc("hutch", Ad, Gd, 8, 5, 0, n)
    dp.dp_norm_est_noalloc("hutch", Ad, Gd, 8, 5, 1, n, flags=dp.DP_ACCUMULATE)
    torch.cuda.synchronize()
    ref = (oracle.norm_est("hutch", A, G, k=8, seed=5, layer=0)
           + oracle.norm_est("hutch", A, G, k=8, seed=5, layer=1))
    assert max_rel_elementwise(f64(n), ref) <= 2e-2


def test_noalloc_rejects_oversized_calls(dev):
    # FGC materialises B d p fp32: 8 x 2048 x 2048 x 4 = 128 MiB > the 64 MiB scratch
    need = dp.dp_norm_est_workspace("fgc", "bf16", 8, 128, 2048, 2048, 0)
    assert need > dp.DP_NOALLOC_SCRATCH_BYTES
    A = torch.zeros(8, 128, 2048, dtype=torch.bfloat16, device=dev)
    n = torch.full((8,), 3.0, dtype=torch.float32, device=dev)
    with pytest.raises(dp.DprcError) as e:
        dp.dp_norm_est_noalloc("fgc", A, A, 0, 0, 0, n)
    assert e.value.status == dp.DP_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.all(n == 3.0).item()  # nothing was enqueued
