"""GPU parity of Poisson subsampling and of ragged (zero-padded) batches.

Poisson membership is an integer decision on the same Philox words on both
sides, so the indices and |B| must match the oracle bit for bit.  A ragged
batch is given to the GPU padded to T tokens with zero rows of G in the pad
(and finite junk in A's pad rows); its norms, clip factors, clipped sum and
update must match the oracle computed on the truncated sequences, at the
tolerances of the dense parity tests.
"""

import numpy as np
import pytest
import torch

import oracle
from sample_gradient_clipping_amd import binding as dp
from sample_gradient_clipping_amd.inputs import linear_inputs, ragged_lengths
from tests.gpu_util import device, f64, max_rel_elementwise, max_rel_normwise, report

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-5
TOL_BF16 = 2e-2


@pytest.fixture(scope="module")
def dev():
    d = device()
    dp.load_library()
    return d


def _sample(dev, seed, step, N, q, cap=None):
    cap = N if cap is None else cap
    idx = torch.full((max(cap, 1),), -7, dtype=torch.int64, device=dev)[:cap]
    count = torch.full((1,), -1, dtype=torch.int64, device=dev)
    dp.dp_poisson_sample(seed, step, N, q, idx, count)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), int(count.item())


@pytest.mark.parametrize("N,q", [(0, 0.5), (1, 1.0), (5, 0.5), (4095, 0.3), (4096, 0.125),
                                 (4097, 0.9), (100003, 0.01), (1 << 20, 0.001), (50000, 0.0),
                                 (50000, 1.0)])
def test_poisson_indices_bit_exact(dev, N, q):
    seed, step = 0xA5A5_0001, 17
    idx, count = _sample(dev, seed, step, N, q)
    ref = oracle.poisson_sample(seed, step, N, q)
    report(f"poisson N={N} q={q}", count=count, expected=len(ref))
    assert count == len(ref)
    assert np.array_equal(idx[:count], ref)


def test_poisson_capacity_and_determinism(dev):
    seed, step, N, q = 77, 3, 20000, 0.2
    ref = oracle.poisson_sample(seed, step, N, q)
    cap = len(ref) // 2
    idx, count = _sample(dev, seed, step, N, q, cap=cap)
    assert count == len(ref)                 # the true |B|, beyond the capacity
    assert np.array_equal(idx, ref[:cap])     # the first cap indices, nothing past the buffer
    idx0, count0 = _sample(dev, seed, step, N, q, cap=0)
    assert count0 == len(ref) and idx0.size == 0
    a, _ = _sample(dev, seed, step, N, q)
    b, _ = _sample(dev, seed, step, N, q)
    assert np.array_equal(a, b)
    c, _ = _sample(dev, seed, step + 1, N, q)
    assert not np.array_equal(a[:100], c[:100])


def test_poisson_high_step_and_seed_words(dev):
    for seed, step in ((2**64 - 1, 2**32 - 1), (1 << 40, 0)):
        idx, count = _sample(dev, seed, step, 9000, 0.25)
        ref = oracle.poisson_sample(seed, step, 9000, 0.25)
        assert count == len(ref) and np.array_equal(idx[:count], ref)


RAGGED_CASES = [
    # (name, dtype, B, T, d, p, k)
    ("ragged_f32", "f32", 4, 40, 24, 30, 6),
    ("ragged_bf16_tiles", "bf16", 4, 512, 256, 256, 32),   # MFMA kernels
]


def _ragged_inputs(case, seed):
    name, dtype, B, T, d, p, k = case
    A, G = linear_inputs(B, T, d, p, dtype, "llama_logu" if dtype == "bf16" else "unit_u0.1_3",
                         seed=seed)
    lengths = ragged_lengths(B, T, seed, min_len=0)
    G = G.clone()
    for i, Ti in enumerate(lengths):
        G[i, Ti:] = 0
    return A, G, lengths


@pytest.mark.parametrize("method", ["hutch", "hutchpp", "ghost", "fgc"])
@pytest.mark.parametrize("case", RAGGED_CASES, ids=[c[0] for c in RAGGED_CASES])
def test_ragged_norms_match_truncated(dev, method, case):
    name, dtype, B, T, d, p, k = case
    A, G, lengths = _ragged_inputs(case, 41)
    n = torch.full((B,), -1.0, dtype=torch.float32, device=dev)
    dp.dp_norm_est(method, A.to(dev), G.to(dev), k, 901, 3, n)
    torch.cuda.synchronize()
    ref = oracle.norm_est_ragged(method, A, G, lengths, k=k, seed=901, layer=3)
    got = f64(n)
    assert np.all(got[ref == 0] == 0)
    err = max_rel_elementwise(got[ref > 0], ref[ref > 0])
    report(f"ragged norm {method} {name}", lengths=str(lengths), max_rel=err)
    assert err <= (TOL_F32 if dtype == "f32" else TOL_BF16)


@pytest.mark.parametrize("case", RAGGED_CASES, ids=[c[0] for c in RAGGED_CASES])
def test_ragged_clip_aggregate_update_matches_truncated(dev, case):
    name, dtype, B, T, d, p, k = case
    A, G, lengths = _ragged_inputs(case, 43)
    C, sigma, eta, seed_z, layer = 1.0, 0.5, 0.05, 3003, 2
    n = torch.from_numpy(oracle.norm_est_ragged("fgc", A, G, lengths).astype(np.float32)).to(dev)
    theta = torch.zeros(p, d, dtype=torch.float32, device=dev)
    S = torch.zeros(p, d, dtype=torch.float32, device=dev)
    c_out = torch.zeros(B, dtype=torch.float32, device=dev)
    dp.dp_clip_aggregate_update(A.to(dev), G.to(dev), n, C, sigma, eta, seed_z, layer, theta,
                                S=S, c_out=c_out)
    torch.cuda.synchronize()
    c_ref, _ = oracle.clip_factors(f64(n), C)
    S_ref = oracle.aggregate_ragged(A, G, c_ref, lengths)
    th_ref = oracle.noise_update(np.zeros((p, d)), S_ref, sigma, C, eta, B, seed_z, layer)
    tol = TOL_F32 if dtype == "f32" else 1e-4
    assert max_rel_elementwise(f64(c_out), c_ref) <= TOL_F32
    e_s = max_rel_normwise(f64(S), S_ref)
    e_t = max_rel_normwise(f64(theta), th_ref)
    report(f"ragged update {name}", S=e_s, theta=e_t)
    assert e_s <= tol and e_t <= tol


def test_poisson_then_step_end_to_end(dev):
    """Sample a minibatch on the GPU, gather it, and take one step; the update
    divides by the realized |B| (the page's G/|B|)."""
    N, T, d, p, k, q = 48, 64, 32, 40, 8, 0.2
    seed_s, step = 515, 9
    A_all, G_all = linear_inputs(N, T, d, p, "f32", "unit_u0.1_3", seed=61)
    idx, count = _sample(dev, seed_s, step, N, q)
    sel = idx[:count]
    assert np.array_equal(sel, oracle.poisson_sample(seed_s, step, N, q)) and count > 0
    A, G = A_all[torch.from_numpy(sel)], G_all[torch.from_numpy(sel)]
    Ad, Gd = A.contiguous().to(dev), G.contiguous().to(dev)
    n = torch.zeros(count, dtype=torch.float32, device=dev)
    dp.dp_norm_est("hutch", Ad, Gd, k, 2001, 0, n)
    theta = torch.zeros(p, d, dtype=torch.float32, device=dev)
    dp.dp_clip_aggregate_update(Ad, Gd, n, 1.0, 1.0, 0.1, 3001, 0, theta)
    torch.cuda.synchronize()
    n_ref, c_ref, S_ref, th_ref = oracle.dp_step([(0, A, G, np.zeros((p, d)))], "hutch", k, 1.0,
                                                 1.0, 0.1, 2001, 3001)
    assert max_rel_elementwise(f64(n), n_ref) <= TOL_F32
    assert max_rel_normwise(f64(theta), th_ref[0]) <= TOL_F32
