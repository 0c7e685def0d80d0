"""GPU parity for the parameters that are not linear layers: RMSNorm gains.

v_i and n_i against the oracle's definitions (fp32 accumulation over the
tokens on the GPU; bf16 inputs are exact in fp32, so only the order of the
sums differs), and the clipped, noised update of gamma.
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


RMS_CASES = [
    # (name, dtype, B, T, d, tol)
    ("ragged_d_f32", "f32", 3, 37, 50, 1e-5),     # d % 8 != 0: element loads
    ("vec_f32", "f32", 2, 64, 64, 1e-5),
    ("one_token_bf16", "bf16", 2, 1, 24, 1e-6),
    ("bf16_tiles", "bf16", 4, 512, 2048, 3e-5),
]


def _rms_inputs(case, seed):
    name, dtype, B, T, d, tol = case
    X, D = linear_inputs(B, T, d, d, dtype, "unit_u0.1_3" if dtype == "f32" else "llama_logu",
                         seed=seed)
    return X, D


@pytest.mark.parametrize("case", RMS_CASES, ids=[c[0] for c in RMS_CASES])
def test_rmsnorm_norm_parity(dev, case):
    name, dtype, B, T, d, tol = case
    X, D = _rms_inputs(case, 71 + T)
    n = torch.full((B,), -1.0, dtype=torch.float32, device=dev)
    v = torch.full((B, d), -1.0, dtype=torch.float32, device=dev)
    dp.dp_rmsnorm_norm(X.to(dev), D.to(dev), n, v=v)
    torch.cuda.synchronize()
    v_ref = oracle.rmsnorm_grad(X, D)
    n_ref = oracle.rmsnorm_norm_sq(X, D)
    e_v = max_rel_normwise(f64(v), v_ref)
    e_n = max_rel_elementwise(f64(n), n_ref)
    report(f"rmsnorm {name}", v=e_v, n=e_n)
    assert e_v <= tol and e_n <= tol


def test_rmsnorm_accumulate_and_empty(dev):
    X, D = linear_inputs(2, 40, 16, 16, "f32", "unit_u0.1_3", seed=5)
    n = torch.tensor([1.5, 2.5], dtype=torch.float32, device=dev)
    dp.dp_rmsnorm_norm(X.to(dev), D.to(dev), n, flags=dp.DP_ACCUMULATE)
    torch.cuda.synchronize()
    ref = np.array([1.5, 2.5]) + oracle.rmsnorm_norm_sq(X, D)
    assert max_rel_elementwise(f64(n), ref) <= 1e-5
    # T = 0: v = 0 and n unchanged under accumulation, 0 otherwise
    X0 = torch.zeros(2, 0, 16, dtype=torch.float32, device=dev)
    v = torch.full((2, 16), 7.0, dtype=torch.float32, device=dev)
    dp.dp_rmsnorm_norm(X0, X0, n, v=v, flags=dp.DP_ACCUMULATE)
    torch.cuda.synchronize()
    assert max_rel_elementwise(f64(n), ref) <= 1e-5 and torch.count_nonzero(v) == 0
    dp.dp_rmsnorm_norm(X0, X0, n)
    torch.cuda.synchronize()
    assert torch.count_nonzero(n) == 0


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_rmsnorm_clip_aggregate_update(dev, dtype):
    B, T, d = 4, 96, 200
    X, D = linear_inputs(B, T, d, d, dtype, "unit_u0.1_3", seed=9)
    n = torch.zeros(B, dtype=torch.float32, device=dev)
    v = torch.zeros(B, d, dtype=torch.float32, device=dev)
    dp.dp_rmsnorm_norm(X.to(dev), D.to(dev), n, v=v)
    # the other layers' share of the norms, then a clip level that clips some samples
    n_tot = n + torch.tensor([0.0, 5.0, 50.0, 500.0], device=dev)
    C, sigma, eta, seed, layer = float(torch.sqrt(n_tot.median()).item()), 0.7, 0.05, 3007, 900
    gamma = torch.ones(d, dtype=torch.float32, device=dev)
    S = torch.zeros(d, dtype=torch.float32, device=dev)
    c_out = torch.zeros(B, dtype=torch.float32, device=dev)
    dp.dp_rmsnorm_clip_aggregate_update(v, n_tot, C, sigma, eta, seed, layer, gamma, S=S,
                                        c_out=c_out)
    torch.cuda.synchronize()
    c_ref, _ = oracle.clip_factors(f64(n_tot), C)
    assert max_rel_elementwise(f64(c_out), c_ref) <= 1e-6
    assert np.any(c_ref < 1) and np.any(c_ref == 1)
    S_ref = c_ref @ f64(v)
    assert max_rel_normwise(f64(S), S_ref) <= 1e-6
    g_ref = oracle.noise_update(np.ones((1, d)), S_ref[None, :], sigma, C, eta, B, seed, layer)[0]
    e = max_rel_normwise(f64(gamma), g_ref)
    report(f"rmsnorm update {dtype}", gamma=e)
    assert e <= 1e-5


def test_rmsnorm_full_size(dev):
    """B8 T4096 d2048 bf16 (a Llama-3.2-1B norm layer): every sample's n and v."""
    from sample_gradient_clipping_amd.inputs import linear_inputs_device
    B, T, d = 8, 4096, 2048
    X, D = linear_inputs_device(B, T, d, d, "bf16", "llama_logu", 81, 0, dev)
    n = torch.zeros(B, dtype=torch.float32, device=dev)
    v = torch.zeros(B, d, dtype=torch.float32, device=dev)
    dp.dp_rmsnorm_norm(X, D, n, v=v)
    torch.cuda.synchronize()
    v_ref = oracle.rmsnorm_grad(X.float().cpu(), D.float().cpu())
    n_ref = np.sum(v_ref * v_ref, axis=1)
    e_v, e_n = max_rel_normwise(f64(v), v_ref), max_rel_elementwise(f64(n), n_ref)
    report("rmsnorm full size", v=e_v, n=e_n)
    assert e_v <= 1e-4 and e_n <= 1e-4


# ---------------------------------------------------------------------------
# embedding tables
# ---------------------------------------------------------------------------
def _emb_inputs(B, T, d, V, dtype, seed, zipf=True):
    """Token ids with a Zipf-like law (repeats within a sequence, as in text)
    and delta rows from the input recipe."""
    r = np.random.default_rng(seed)
    if zipf:
        ids = np.minimum(r.zipf(1.3, size=(B, T)) - 1, V - 1).astype(np.int32)
    else:
        ids = r.integers(0, V, size=(B, T)).astype(np.int32)
    _, D = linear_inputs(B, T, 8, d, dtype, "unit_u0.1_3", seed=seed)
    return torch.from_numpy(ids), D


EMB_CASES = [
    # (name, dtype, B, T, d, V)
    ("tiny_f32", "f32", 3, 40, 24, 17),
    ("ragged_d_f32", "f32", 2, 100, 50, 1000),    # d % 8 != 0
    ("bf16", "bf16", 4, 1000, 256, 3000),
    ("one_token_f32", "f32", 2, 1, 16, 5),
]


@pytest.mark.parametrize("case", EMB_CASES, ids=[c[0] for c in EMB_CASES])
def test_embedding_norm_parity(dev, case):
    name, dtype, B, T, d, V = case
    ids, D = _emb_inputs(B, T, d, V, dtype, 101 + T)
    n = torch.full((B,), -1.0, dtype=torch.float32, device=dev)
    dp.dp_embedding_norm(ids.to(dev), D.to(dev), n)
    torch.cuda.synchronize()
    ref = oracle.embedding_norm_sq(ids.numpy(), D)
    e = max_rel_elementwise(f64(n), ref)
    report(f"embedding norm {name}", distinct=len(np.unique(ids[0].numpy())), max_rel=e)
    assert e <= 1e-5


def test_embedding_norm_edge_cases(dev):
    B, T, d = 3, 64, 32
    D = torch.randn(B, T, d, dtype=torch.float32)
    ids = torch.stack([torch.arange(T, dtype=torch.int32),             # all distinct
                       torch.full((T,), 7, dtype=torch.int32),          # one id repeated
                       torch.arange(T, dtype=torch.int32).flip(0) % 5])  # few ids, unsorted
    n = torch.tensor([0.5, 0.5, 0.5], dtype=torch.float32, device=dev)
    dp.dp_embedding_norm(ids.to(dev), D.to(dev), n, flags=dp.DP_ACCUMULATE)
    torch.cuda.synchronize()
    ref = 0.5 + oracle.embedding_norm_sq(ids.numpy(), D)
    assert max_rel_elementwise(f64(n), ref) <= 1e-5
    # a long sequence at the sort's limit
    Dl = torch.randn(1, 16384, 8, dtype=torch.float32)
    idl = torch.from_numpy(np.random.default_rng(3).integers(0, 700, size=(1, 16384)).astype(np.int32))
    nl = torch.zeros(1, dtype=torch.float32, device=dev)
    dp.dp_embedding_norm(idl.to(dev), Dl.to(dev), nl)
    torch.cuda.synchronize()
    assert max_rel_elementwise(f64(nl), oracle.embedding_norm_sq(idl.numpy(), Dl)) <= 1e-5
    # T = 0
    z = torch.zeros(2, 0, 8, dtype=torch.float32, device=dev)
    n0 = torch.full((2,), 3.0, dtype=torch.float32, device=dev)
    dp.dp_embedding_norm(torch.zeros(2, 0, dtype=torch.int32, device=dev), z, n0)
    torch.cuda.synchronize()
    assert torch.count_nonzero(n0) == 0


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_embedding_clip_aggregate_update(dev, dtype):
    B, T, d, V = 4, 300, 72, 500
    ids, D = _emb_inputs(B, T, d, V, dtype, 55)
    n = torch.zeros(B, dtype=torch.float32, device=dev)
    dp.dp_embedding_norm(ids.to(dev), D.to(dev), n)
    n_tot = n + torch.tensor([0.0, 1.0, 10.0, 100.0], device=dev)
    C, sigma, eta, seed, layer = float(torch.sqrt(n_tot.median()).item()), 0.8, 0.05, 3011, 901
    E0 = torch.from_numpy(np.random.default_rng(2).standard_normal((V, d)).astype(np.float32) * 0.02)
    E = E0.clone().to(dev)
    c_out = torch.zeros(B, dtype=torch.float32, device=dev)
    dp.dp_embedding_clip_aggregate_update(ids.to(dev), D.to(dev), n_tot, C, sigma, eta, seed, layer,
                                          E, c_out=c_out)
    torch.cuda.synchronize()
    c_ref, _ = oracle.clip_factors(f64(n_tot), C)
    assert np.any(c_ref < 1) and np.any(c_ref == 1)
    assert max_rel_elementwise(f64(c_out), c_ref) <= 1e-6
    S_ref = oracle.embedding_aggregate(ids.numpy(), D, c_ref, V)
    E_ref = oracle.noise_update(E0.double().numpy(), S_ref, sigma, C, eta, B, seed, layer)
    err = max_rel_normwise(f64(E), E_ref)
    report(f"embedding update {dtype}", E=err)
    assert err <= 1e-5
    # rows that no token uses moved by the noise alone
    unused = np.setdiff1d(np.arange(V), np.unique(ids.numpy()))
    assert unused.size > 0
    noise_only = oracle.noise_update(E0.double().numpy(), np.zeros((V, d)), sigma, C, eta, B,
                                     seed, layer)
    assert np.allclose(f64(E)[unused], noise_only[unused], rtol=1e-5, atol=1e-7)
