"""GPU parity of every hot-path call against the CPU oracle (small and ragged sizes).

All calls go through the C ABI (ctypes binding).  Tolerances: Philox words
bit-exact; normals 2e-6 max(1, |z|); fp32-input norms, clip factors, clipped
sums and updates 1e-5 relative; bf16-input norms 2e-2 relative per sample.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from sample_gradient_clipping_amd import binding as dp
from sample_gradient_clipping_amd.inputs import linear_inputs, theta_init
from tests.gpu_util import device, f64, max_rel_elementwise, max_rel_normwise, report

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-5
TOL_BF16 = 2e-2


@pytest.fixture(scope="module")
def dev():
    d = device()
    dp.load_library()
    return d


# ---------------------------------------------------------------------------
# random streams
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("seed", [0, 1, 2002, 2**64 - 1, 0x123456789ABCDEF])
def test_philox_words_bit_exact(dev, seed):
    rng = np.random.default_rng(seed & 0xFFFF)
    ctr = rng.integers(0, 2**32, size=(4099, 4), dtype=np.uint64)
    ctr[:8] = [[0, 0, 0, 0], [1, 0, 0, 0], [0xFFFFFFFF] * 4, [5, 31, 7, 111], [2047, 3, 0, 1],
               [123, 0, 0xFFFFFFFF, 42], [0, 1, 0xFFFFFFFF, 0], [7, 9, 11, 13]]
    ct = torch.from_numpy(ctr.astype(np.uint32).view(np.int32)).to(dev)
    out = torch.empty_like(ct)
    dp.dp_philox_u32(seed, ct, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint32)
    want = oracle.philox4x32_10(ctr[:, 0], ctr[:, 1], ctr[:, 2], ctr[:, 3], seed)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("seed,layer,sample,p,k", [(2002, 0, 0, 2048, 32), (5, 3, 7, 37, 5),
                                                   (2**63 + 11, 111, 2, 8192, 3)])
def test_probe_normals(dev, seed, layer, sample, p, k):
    Pt = torch.empty(k, p, dtype=torch.float32, device=dev)
    dp.dp_probe_fill(seed, layer, sample, p, k, Pt)
    torch.cuda.synchronize()
    ref = oracle.probe_matrix(seed, layer, sample, p, k).T
    err = np.abs(f64(Pt) - ref) / np.maximum(1.0, np.abs(ref))
    report("probe", p=p, k=k, max_err=float(err.max()))
    assert err.max() <= 2e-6


@pytest.mark.parametrize("offset,n", [(0, 4096), (3, 1001), ((1 << 33) + 1, 777)])
def test_noise_normals(dev, offset, n):
    xi = torch.empty(n, dtype=torch.float32, device=dev)
    dp.dp_noise_fill(3002, 9, offset, xi)
    torch.cuda.synchronize()
    ref = oracle.noise_vector(3002, 9, n, offset=offset)
    err = np.abs(f64(xi) - ref) / np.maximum(1.0, np.abs(ref))
    assert err.max() <= 2e-6


# ---------------------------------------------------------------------------
# per-sample norms
# ---------------------------------------------------------------------------
NORM_CASES = [
    # (name, dtype, B, T, d, p, k)
    ("tiny_f32", "f32", 4, 64, 64, 64, 8),
    ("ragged_f32", "f32", 3, 37, 50, 70, 5),
    ("ragged_bf16", "bf16", 3, 37, 50, 70, 5),
    ("tiles_bf16", "bf16", 3, 256, 256, 512, 32),
    ("tiles_bf16_wide_d", "bf16", 2, 384, 512, 256, 32),
    ("tiles_bf16_k7", "bf16", 2, 128, 128, 256, 7),
    ("wide_sketch_f32", "f32", 2, 64, 48, 300, 60),   # s = 20 > 16 sketch columns, ragged p
    ("rank_deficient_f32", "f32", 2, 4, 30, 40, 24),  # T = 4 < s = 8: dead pivots in the QR
    # probe-count edge cases.  Generic kernels: fp32 or shapes off the MFMA tiles;
    # MFMA kernels: bf16 with T % 128 == 0, p % 256 == 0, d % 256 == 0, k <= 32
    # (Hutch++: s + r <= 32), where the probe block is padded to 32 columns.
    ("k1_f32", "f32", 3, 40, 24, 20, 1),              # one probe, generic
    ("k1_bf16_mfma", "bf16", 2, 256, 256, 512, 1),    # one probe, 31 padded columns
    ("kp_f32", "f32", 2, 30, 20, 12, 12),             # k = p, generic (Hutch++: s = r = 4)
    ("kp_bf16", "bf16", 2, 37, 50, 24, 24),           # k = p, generic bf16 kernels
    ("k3_f32", "f32", 2, 64, 48, 40, 3),              # Hutch++ s = r = 1 with T > s, generic
    ("k3_bf16_mfma", "bf16", 2, 256, 256, 512, 3),    # Hutch++ s = r = 1 with T > s, MFMA
    # MFMA projection with the weighted square taken in the same kernel (at least 256
    # column blocks): 64-column blocks (B d / 64 = 256), 128-column blocks (B d / 128 = 256)
    ("fused_sq64_bf16", "bf16", 8, 256, 2048, 256, 32),
    ("fused_sq128_bf16", "bf16", 4, 128, 8192, 256, 32),
    # one sample: token splits of the projection and the chunked finish at B = 1
    ("single_sample_bf16", "bf16", 1, 512, 1024, 512, 32),
]


@pytest.mark.parametrize("method", ["hutch", "hutchpp", "ghost", "fgc"])
@pytest.mark.parametrize("case", NORM_CASES, ids=[c[0] for c in NORM_CASES])
def test_norm_parity(dev, method, case):
    name, dtype, B, T, d, p, k = case
    if method == "hutchpp" and k < 3:
        pytest.skip("Hutch++ needs k >= 3")
    recipe = "unit_u0.1_3" if dtype == "f32" else "llama_logu"
    A, G = linear_inputs(B, T, d, p, dtype, recipe, seed=11 + T)
    n = torch.full((B,), -1.0, dtype=torch.float32, device=dev)
    dp.dp_norm_est(method, A.to(dev), G.to(dev), k, 777, 5, n)
    torch.cuda.synchronize()
    ref = oracle.norm_est(method, A, G, k=k, seed=777, layer=5)
    err = max_rel_elementwise(f64(n), ref)
    report(f"norm {method} {name}", max_rel=err)
    assert err <= (TOL_F32 if dtype == "f32" else TOL_BF16)


GHOST_CASES = [
    # (name, B, T, d, p): the MFMA ghost kernel deals super-tiles of 4 x 8 blocks
    # (256-token S blocks by 128-token t blocks) to the XCDs, one per XCD per round.
    # Several super-tile rows with 9 super-tiles in all (the second round almost
    # empty), and a last S block that T cuts in half in every sample.
    ("ghost_rows_b3_t2048", 3, 2048, 64, 128),
    ("ghost_ragged_b2_t1152", 2, 1152, 128, 64),
]


@pytest.mark.parametrize("case", GHOST_CASES, ids=[c[0] for c in GHOST_CASES])
def test_ghost_tile_dealing(dev, case):
    """The exact ghost norm on bf16 inputs against the oracle's fp64 Grams of the
    same inputs: only the fp32 accumulation of each Gram entry (d + p <= 192
    products) differs, so the bound is 1e-4 relative, tighter than the 2e-2 of
    the estimators."""
    name, B, T, d, p = case
    A, G = linear_inputs(B, T, d, p, "bf16", "llama_logu", seed=23 + T)
    n = torch.full((B,), -1.0, dtype=torch.float32, device=dev)
    dp.dp_norm_est("ghost", A.to(dev), G.to(dev), 0, 0, 0, n)
    torch.cuda.synchronize()
    ref = oracle.norm_est("ghost", A, G)
    err = max_rel_elementwise(f64(n), ref)
    report(f"ghost dealing {name}", max_rel=err)
    assert err <= 1e-4


LOWRANK_CASES = [
    # (name, dtype, B, T, d, p, k): rank-8 signal plus noise (decaying spectrum)
    ("lowrank_f32", "f32", 3, 96, 64, 80, 12),
    ("lowrank_bf16", "bf16", 2, 256, 256, 512, 32),  # MFMA path
]


@pytest.mark.parametrize("method", ["hutch", "hutchpp", "ghost", "fgc"])
@pytest.mark.parametrize("case", LOWRANK_CASES, ids=[c[0] for c in LOWRANK_CASES])
def test_norm_parity_lowrank(dev, method, case):
    name, dtype, B, T, d, p, k = case
    A, G = linear_inputs(B, T, d, p, dtype, "lowrank", seed=17 + T)
    n = torch.full((B,), -1.0, dtype=torch.float32, device=dev)
    dp.dp_norm_est(method, A.to(dev), G.to(dev), k, 779, 2, n)
    torch.cuda.synchronize()
    ref = oracle.norm_est(method, A, G, k=k, seed=779, layer=2)
    err = max_rel_elementwise(f64(n), ref)
    report(f"norm {method} {name}", max_rel=err)
    assert err <= (TOL_F32 if dtype == "f32" else TOL_BF16)


def test_hutchpp_more_accurate_on_lowrank(dev):
    # On a decaying spectrum the sketch captures the head of tr(O) exactly and
    # only the small tail is estimated; on i.i.d. data (flat spectrum) the
    # plain estimator with all k probes on the trace has the smaller error.
    B, T, d, p, k = 4, 512, 256, 256, 32

    def rel_rms(recipe, method):
        A, G = linear_inputs(B, T, d, p, "bf16", recipe, seed=5)
        A, G = A.to(dev), G.to(dev)
        exact = torch.zeros(B, dtype=torch.float32, device=dev)
        dp.dp_norm_est("fgc", A, G, 0, 0, 0, exact)
        errs = []
        for s in range(8):
            n = torch.zeros(B, dtype=torch.float32, device=dev)
            dp.dp_norm_est(method, A, G, k, 100 + s, 2, n)
            errs.append(f64(n) / f64(exact) - 1.0)
        return float(np.sqrt(np.mean(np.square(errs))))

    lr = {m: rel_rms("lowrank", m) for m in ("hutch", "hutchpp")}
    iid = {m: rel_rms("llama_logu", m) for m in ("hutch", "hutchpp")}
    report("rel rms lowrank", **lr)
    report("rel rms iid", **iid)
    assert lr["hutchpp"] < 1e-2 * lr["hutch"]
    assert iid["hutch"] < iid["hutchpp"]


# ---------------------------------------------------------------------------
# sign (Rademacher) probes
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("seed,layer,sample,p,k", [(5, 3, 7, 37, 5), (2002, 0, 1, 2048, 32)])
def test_rademacher_probe_bit_exact(dev, seed, layer, sample, p, k):
    Pt = torch.zeros(k, p, dtype=torch.float32, device=dev)
    dp.dp_probe_fill(seed, layer, sample, p, k, Pt, rademacher=True)
    torch.cuda.synchronize()
    ref = oracle.rademacher_probe_matrix(seed, layer, sample, p, k).T
    assert np.array_equal(f64(Pt), ref)


@pytest.mark.parametrize("method", ["hutch", "hutchpp"])
@pytest.mark.parametrize("case", NORM_CASES, ids=[c[0] for c in NORM_CASES])
def test_norm_parity_rademacher(dev, method, case):
    name, dtype, B, T, d, p, k = case
    if method == "hutchpp" and k < 3:
        pytest.skip("Hutch++ needs k >= 3")
    recipe = "unit_u0.1_3" if dtype == "f32" else "llama_logu"
    A, G = linear_inputs(B, T, d, p, dtype, recipe, seed=13 + T)
    n = torch.full((B,), -1.0, dtype=torch.float32, device=dev)
    dp.dp_norm_est(method, A.to(dev), G.to(dev), k, 778, 6, n, flags=dp.DP_PROBE_RADEMACHER)
    torch.cuda.synchronize()
    ref = oracle.norm_est(method, A, G, k=k, seed=778, layer=6, rademacher=True)
    err = max_rel_elementwise(f64(n), ref)
    report(f"norm {method} rademacher {name}", max_rel=err)
    assert err <= (TOL_F32 if dtype == "f32" else TOL_BF16)


def test_rademacher_exact_on_diagonal_O(dev):
    # A = I (T = d), G = U diag(s) with orthonormal U: O = diag(s^2), and sign
    # probes give tr(O) for every seed (fp32 rounding only).
    d, p = 64, 48
    r = np.random.default_rng(8)
    U, _ = np.linalg.qr(r.standard_normal((d, p)))
    sv = r.uniform(0.5, 3.0, size=p)
    A = torch.eye(d, dtype=torch.float32).reshape(1, d, d).repeat(2, 1, 1)
    G = torch.from_numpy((U * sv[None, :]).astype(np.float32)).reshape(1, d, p).repeat(2, 1, 1)
    exact = oracle.norm_est("fgc", A, G)
    for seed in range(3):
        n = torch.zeros(2, dtype=torch.float32, device=dev)
        dp.dp_norm_est("hutch", A.to(dev), G.to(dev), 4, seed, 0, n, flags=dp.DP_PROBE_RADEMACHER)
        torch.cuda.synchronize()
        assert max_rel_elementwise(f64(n), exact) <= TOL_F32


@pytest.mark.parametrize("dtype,shape", [("f32", (3, 40, 24, 20)), ("bf16", (2, 256, 256, 256))])
def test_norm_flags_shared_and_accumulate(dev, dtype, shape):
    B, T, d, p = shape
    k = 6
    A, G = linear_inputs(B, T, d, p, dtype, "llama_logu", seed=5)
    Ad, Gd = A.to(dev), G.to(dev)
    n = torch.zeros(B, dtype=torch.float32, device=dev)
    dp.dp_norm_est("hutch", Ad, Gd, k, 9, 1, n, flags=dp.DP_PROBE_SHARED)
    dp.dp_norm_est("fgc", Ad, Gd, 0, 0, 0, n, flags=dp.DP_ACCUMULATE)
    dp.dp_norm_est("hutch", Ad, Gd, k, 9, 2, n, flags=dp.DP_ACCUMULATE)
    torch.cuda.synchronize()
    ref = (oracle.norm_est("hutch", A, G, k=k, seed=9, layer=1, shared=True)
           + oracle.norm_est("fgc", A, G)
           + oracle.norm_est("hutch", A, G, k=k, seed=9, layer=2))
    tol = TOL_F32 if dtype == "f32" else TOL_BF16
    assert max_rel_elementwise(f64(n), ref) <= tol


def test_norm_empty_inputs(dev):
    A = torch.zeros(3, 0, 8, dtype=torch.float32, device=dev)
    G = torch.zeros(3, 0, 6, dtype=torch.float32, device=dev)
    for method in ("hutch", "hutchpp", "ghost", "fgc"):
        n = torch.full((3,), 5.0, dtype=torch.float32, device=dev)
        dp.dp_norm_est(method, A, G, 3, 1, 0, n)
        torch.cuda.synchronize()
        assert torch.all(n == 0).item(), method
    n0 = torch.zeros(0, dtype=torch.float32, device=dev)
    dp.dp_norm_est("hutch", A[:0], G[:0], 3, 1, 0, n0)


def test_norm_deterministic(dev):
    A, G = linear_inputs(3, 256, 256, 512, "bf16", "llama_logu", seed=3)
    Ad, Gd = A.to(dev), G.to(dev)
    outs = []
    for _ in range(2):
        n = torch.zeros(3, dtype=torch.float32, device=dev)
        dp.dp_norm_est("hutch", Ad, Gd, 32, 4, 0, n)
        torch.cuda.synchronize()
        outs.append(n.cpu())
    assert torch.equal(outs[0], outs[1])


# ---------------------------------------------------------------------------
# clip + aggregation
# ---------------------------------------------------------------------------
AGG_CASES = [
    ("tiny_f32", "f32", 4, 64, 64, 64),
    ("ragged_f32", "f32", 3, 37, 50, 70),
    ("ragged_bf16", "bf16", 3, 37, 50, 70),
    ("tiles_bf16", "bf16", 3, 256, 256, 512),
    ("tiles_bf16_b5", "bf16", 5, 128, 512, 256),
    ("split_spans_samples_bf16", "bf16", 8, 128, 2048, 2048),
]


@pytest.mark.parametrize("case", AGG_CASES, ids=[c[0] for c in AGG_CASES])
def test_clip_aggregate_parity(dev, case):
    name, dtype, B, T, d, p = case
    recipe = "unit_u0.1_3" if dtype == "f32" else "llama_logu"
    A, G = linear_inputs(B, T, d, p, dtype, recipe, seed=21 + B)
    exact = oracle.norm_est("fgc", A, G)
    n32 = torch.tensor(exact, dtype=torch.float32)
    C = float(np.median(np.sqrt(exact)))  # both branches of the clip
    c = torch.zeros(B, dtype=torch.float32, device=dev)
    S = torch.full((p, d), float("nan"), dtype=torch.float32, device=dev)
    ws = dp.clip_workspace(dp.dp_clip_aggregate_workspace(dtype, B, T, d, p), dev)
    dp.dp_clip_aggregate(A.to(dev), G.to(dev), n32.to(dev), C, S, c_out=c, ws=ws)
    status = dp.dp_read_device_status(ws)
    c_ref, flag = oracle.clip_factors(n32.double().numpy(), C)
    S_ref = oracle.aggregate(A, G, c_ref)
    ec = max_rel_elementwise(f64(c), c_ref)
    es = max_rel_normwise(f64(S), S_ref)
    report(f"aggregate {name}", c_err=ec, S_err=es)
    assert status == 0 and not flag
    assert np.any(c_ref < 1) and np.any(c_ref == 1)
    assert ec <= TOL_F32
    assert es <= (TOL_F32 if dtype == "f32" else 1e-4)


@pytest.mark.parametrize("dtype,shape", [("f32", (4, 33, 20, 30)), ("bf16", (4, 64, 256, 256)),
                                         ("bf16", (4, 128, 256, 256))])
def test_clip_nonfinite_dropped_and_flagged(dev, dtype, shape):
    B, T, d, p = shape
    A, G = linear_inputs(B, T, d, p, dtype, "llama_logu", seed=8)
    n = torch.tensor([4.0, float("nan"), 0.25, float("inf")], dtype=torch.float32)
    c = torch.zeros(B, dtype=torch.float32, device=dev)
    S = torch.empty(p, d, dtype=torch.float32, device=dev)
    ws = dp.clip_workspace(dp.dp_clip_aggregate_workspace(dtype, B, T, d, p), dev)
    dp.dp_clip_aggregate(A.to(dev), G.to(dev), n.to(dev), 1.0, S, c_out=c, ws=ws)
    status = dp.dp_read_device_status(ws)
    c_ref, flag = oracle.clip_factors(n.double().numpy(), 1.0)
    assert flag and status == dp.DP_STATUS_NONFINITE_NORM
    assert np.array_equal(f64(c), c_ref)
    S_ref = oracle.aggregate(A, G, c_ref)
    assert max_rel_normwise(f64(S), S_ref) <= (TOL_F32 if dtype == "f32" else 1e-4)


def test_device_status_sticky_until_read(dev):
    """A NaN norm sets the workspace's status flag; calls with finite norms that
    reuse the workspace leave it set; dp_read_device_status reports it once and
    clears it.  The same word serves the fused call and the gain update."""
    B, T, d, p = 4, 64, 256, 256
    A, G = linear_inputs(B, T, d, p, "bf16", "llama_logu", seed=12)
    Ad, Gd = A.to(dev), G.to(dev)
    good = torch.tensor([4.0, 0.5, 2.0, 9.0], dtype=torch.float32, device=dev)
    bad = torch.tensor([4.0, float("nan"), 2.0, 9.0], dtype=torch.float32, device=dev)
    S = torch.empty(p, d, dtype=torch.float32, device=dev)
    ws = dp.clip_workspace(dp.dp_clip_aggregate_update_workspace("bf16", B, T, d, p), dev)
    dp.dp_clip_aggregate(Ad, Gd, good, 1.0, S, ws=ws)
    assert dp.dp_read_device_status(ws) == 0
    dp.dp_clip_aggregate(Ad, Gd, bad, 1.0, S, ws=ws)
    dp.dp_clip_aggregate(Ad, Gd, good, 1.0, S, ws=ws)  # a later clean call keeps the flag
    assert dp.dp_read_device_status(ws) == dp.DP_STATUS_NONFINITE_NORM
    assert dp.dp_read_device_status(ws) == 0          # cleared by the read
    theta = torch.zeros(p, d, dtype=torch.float32, device=dev)
    dp.dp_clip_aggregate_update(Ad, Gd, bad, 1.0, 1.0, 1e-4, 5, 0, theta, ws=ws)
    assert dp.dp_read_device_status(ws) == dp.DP_STATUS_NONFINITE_NORM
    v = torch.ones(B, d, dtype=torch.float32, device=dev)
    gamma = torch.zeros(d, dtype=torch.float32, device=dev)
    wg = dp.clip_workspace(dp.load_library().dp_rmsnorm_update_workspace(B, d), dev)
    dp.dp_rmsnorm_clip_aggregate_update(v, good, 1.0, 1.0, 1e-4, 5, 1, gamma, ws=wg)
    assert dp.dp_read_device_status(wg) == 0
    dp.dp_rmsnorm_clip_aggregate_update(v, bad, 1.0, 1.0, 1e-4, 5, 1, gamma, ws=wg)
    assert dp.dp_read_device_status(wg) == dp.DP_STATUS_NONFINITE_NORM


@pytest.mark.parametrize("dtype,shape", [("f32", (3, 40, 24, 20)), ("bf16", (3, 256, 256, 512))])
def test_clip_none_clipped_gives_batch_gradient(dev, dtype, shape):
    # C above every sample's norm: c = 1 for all, and S is the batch gradient G^T A
    B, T, d, p = shape
    A, G = linear_inputs(B, T, d, p, dtype, "llama_logu", seed=14)
    exact = oracle.norm_est("fgc", A, G)
    C = 2.0 * float(np.sqrt(exact.max()))
    c = torch.zeros(B, dtype=torch.float32, device=dev)
    S = torch.empty(p, d, dtype=torch.float32, device=dev)
    dp.dp_clip_aggregate(A.to(dev), G.to(dev), torch.tensor(exact, dtype=torch.float32).to(dev), C, S,
                         c_out=c)
    torch.cuda.synchronize()
    assert torch.all(c == 1.0).item()
    Af, Gf = oracle.to_f64(A), oracle.to_f64(G)
    batch = Gf.reshape(-1, p).T @ Af.reshape(-1, d)
    assert max_rel_normwise(f64(S), batch) <= (TOL_F32 if dtype == "f32" else 1e-4)


def test_clip_all_dropped_gives_zero_sum(dev):
    A, G = linear_inputs(2, 128, 256, 256, "bf16", "llama_logu", seed=9)
    n = torch.tensor([float("nan"), float("nan")], dtype=torch.float32, device=dev)
    S = torch.full((256, 256), 7.0, dtype=torch.float32, device=dev)
    dp.dp_clip_aggregate(A.to(dev), G.to(dev), n, 1.0, S)
    torch.cuda.synchronize()
    assert torch.count_nonzero(S).item() == 0


def test_aggregate_deterministic(dev):
    A, G = linear_inputs(3, 256, 256, 512, "bf16", "llama_logu", seed=10)
    Ad, Gd = A.to(dev), G.to(dev)
    n = torch.tensor([10.0, 0.5, 3.0], dtype=torch.float32, device=dev)
    outs = []
    for _ in range(2):
        S = torch.empty(512, 256, dtype=torch.float32, device=dev)
        dp.dp_clip_aggregate(Ad, Gd, n, 1.0, S)
        torch.cuda.synchronize()
        outs.append(S.cpu())
    assert torch.equal(outs[0], outs[1])


# ---------------------------------------------------------------------------
# clip + aggregation + noise + update in one call
# ---------------------------------------------------------------------------
FUSED_CASES = [
    ("tiny_f32", "f32", 4, 64, 64, 64),              # generic contraction
    ("ragged_bf16", "bf16", 3, 37, 50, 70),          # generic contraction, bf16
    ("one_split_bf16", "bf16", 2, 1024, 2048, 8192),  # MFMA, single token split
    ("splits_bf16", "bf16", 8, 128, 2048, 2048),     # MFMA, token splits summed in the update
]


@pytest.mark.parametrize("case", FUSED_CASES, ids=[c[0] for c in FUSED_CASES])
def test_clip_aggregate_update_matches_separate_calls(dev, case):
    """The fused call equals dp_clip_aggregate + dp_noise_update bit for bit,
    with and without the clipped sum stored, and matches the oracle."""
    name, dtype, B, T, d, p = case
    recipe = "unit_u0.1_3" if dtype == "f32" else "llama_logu"
    A, G = linear_inputs(B, T, d, p, dtype, recipe, seed=31 + B)
    Ad, Gd = A.to(dev), G.to(dev)
    exact = oracle.norm_est("fgc", A, G) if T * d * p <= (1 << 26) else None
    n32 = (torch.tensor(exact, dtype=torch.float32) if exact is not None
           else torch.linspace(0.5, 50.0, B, dtype=torch.float32))
    C = float(np.median(np.sqrt(n32.double().numpy())))
    sigma, eta, seed, layer = 0.8, 0.05, 4004, 9
    th0 = theta_init(p, d, seed=5).to(dev)
    # separate calls
    S1 = torch.empty(p, d, dtype=torch.float32, device=dev)
    c1 = torch.empty(B, dtype=torch.float32, device=dev)
    dp.dp_clip_aggregate(Ad, Gd, n32.to(dev), C, S1, c_out=c1)
    th1 = th0.clone()
    dp.dp_noise_update(th1, S1, sigma, C, eta, B, seed, layer)
    # fused, storing S; fused, S not stored
    S2 = torch.full((p, d), float("nan"), dtype=torch.float32, device=dev)
    c2 = torch.empty(B, dtype=torch.float32, device=dev)
    th2 = th0.clone()
    dp.dp_clip_aggregate_update(Ad, Gd, n32.to(dev), C, sigma, eta, seed, layer, th2, S=S2,
                                c_out=c2)
    th3 = th0.clone()
    dp.dp_clip_aggregate_update(Ad, Gd, n32.to(dev), C, sigma, eta, seed, layer, th3)
    torch.cuda.synchronize()
    assert torch.equal(c1, c2)
    assert torch.equal(S1, S2)
    assert torch.equal(th1, th2) and torch.equal(th1, th3)
    # against the oracle on sampled rows
    c_ref, _ = oracle.clip_factors(n32.double().numpy(), C)
    rows = np.sort(np.random.default_rng(B).choice(p, size=min(16, p), replace=False))
    S_rows = oracle.aggregate_rows(A, G, c_ref, rows)
    th_ref = oracle.noise_update(f64(th0)[rows], S_rows, sigma, C, eta, B, seed, layer, rows=rows)
    es = max_rel_normwise(f64(S2)[rows], S_rows)
    et = max_rel_normwise(f64(th2)[rows] - f64(th0)[rows], th_ref - f64(th0)[rows])
    report(f"fused update {name}", S_err=es, dtheta_err=et)
    assert es <= (TOL_F32 if dtype == "f32" else 1e-4)
    assert et <= (TOL_F32 if dtype == "f32" else 1e-4)


# ---------------------------------------------------------------------------
# noise + update
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("p,d", [(64, 64), (37, 29), (512, 384)])
def test_noise_update_parity(dev, p, d):
    rng = np.random.default_rng(p * d)
    S = torch.from_numpy(rng.standard_normal((p, d)).astype(np.float32))
    theta = torch.zeros(p, d, dtype=torch.float32)
    th = theta.to(dev)
    dp.dp_noise_update(th, S.to(dev), 1.0, 1.0, 0.1, 4, 3001, 7)
    torch.cuda.synchronize()
    ref = oracle.noise_update(np.zeros((p, d)), S.double().numpy(), 1.0, 1.0, 0.1, 4, 3001, 7)
    err = max_rel_normwise(f64(th), ref)
    report("update", p=p, d=d, err=err)
    assert err <= TOL_F32


def test_noise_update_sigma_zero_and_rmw(dev):
    p, d = 96, 80
    rng = np.random.default_rng(1)
    S = torch.from_numpy(rng.standard_normal((p, d)).astype(np.float32))
    th0 = theta_init(p, d, seed=4)
    th = th0.to(dev)
    dp.dp_noise_update(th, S.to(dev), 0.0, 1.0, 0.05, 8, 1, 0)
    torch.cuda.synchronize()
    ref = oracle.noise_update(th0.double().numpy(), S.double().numpy(), 0.0, 1.0, 0.05, 8, 1, 0)
    assert np.max(np.abs(f64(th) - ref)) <= 2 * np.spacing(np.float32(np.max(np.abs(ref))))
    th = th0.to(dev)
    dp.dp_noise_update(th, S.to(dev), 1.3, 0.7, 0.05, 8, 2, 3)
    torch.cuda.synchronize()
    ref = oracle.noise_update(th0.double().numpy(), S.double().numpy(), 1.3, 0.7, 0.05, 8, 2, 3)
    delta_ref = ref - th0.double().numpy()
    ulp = np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(f64(th) - ref) <= TOL_F32 * np.max(np.abs(delta_ref)) + ulp)


def test_noise_update_statistics(dev):
    p, d = 1024, 1024
    S = torch.zeros(p, d, dtype=torch.float32, device=dev)
    th = torch.zeros(p, d, dtype=torch.float32, device=dev)
    sigma, C, eta, B = 1.1, 0.9, 0.01, 16
    dp.dp_noise_update(th, S, sigma, C, eta, B, 77, 1)
    torch.cuda.synchronize()
    noise = -(B / eta) * f64(th).ravel()
    N = noise.size
    assert abs(noise.mean()) < 5 * sigma * C / math.sqrt(N)
    assert abs(noise.var() / (sigma * C) ** 2 - 1) < 5 * math.sqrt(2 / N)


# ---------------------------------------------------------------------------
# one whole step, two layers, flat clipping
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_whole_step(dev, dtype):
    B, T = 3, 128
    shapes = [(256, 256), (256, 512)]
    layers = []
    for lid, (d, p) in enumerate(shapes):
        A, G = linear_inputs(B, T, d, p, dtype, "llama_logu", seed=40, layer_id=lid)
        layers.append((lid, A, G, np.zeros((p, d))))
    k, C, sigma, eta = 8, 1.0, 1.0, 1e-3
    n = torch.zeros(B, dtype=torch.float32, device=dev)
    for lid, A, G, _ in layers:
        dp.dp_norm_est("hutch", A.to(dev), G.to(dev), k, 50, lid, n, flags=dp.DP_ACCUMULATE)
    thetas, Ss = [], []
    for lid, A, G, th0 in layers:
        p, d = th0.shape
        S = torch.empty(p, d, dtype=torch.float32, device=dev)
        dp.dp_clip_aggregate(A.to(dev), G.to(dev), n, C, S)
        th = torch.zeros(p, d, dtype=torch.float32, device=dev)
        dp.dp_noise_update(th, S, sigma, C, eta, B, 60, lid)
        thetas.append(th)
        Ss.append(S)
    torch.cuda.synchronize()
    n_ref, c_ref, S_ref, th_ref = oracle.dp_step(layers, "hutch", k, C, sigma, eta, 50, 60)
    tol_n = TOL_F32 if dtype == "f32" else TOL_BF16
    assert max_rel_elementwise(f64(n), n_ref) <= tol_n
    # aggregation and update from the GPU's own norms
    c_gpu, _ = oracle.clip_factors(f64(n), C)
    for (lid, A, G, th0), S, th in zip(layers, Ss, thetas):
        S_r = oracle.aggregate(A, G, c_gpu)
        assert max_rel_normwise(f64(S), S_r) <= (TOL_F32 if dtype == "f32" else 1e-4)
        t_r = oracle.noise_update(th0, S_r, sigma, C, eta, B, 60, lid)
        assert max_rel_normwise(f64(th), t_r) <= TOL_F32


@pytest.mark.parametrize("nbytes,nblocks", [(16, 1), (4096 * 16 + 48, 7), (3 << 20, 2048)])
def test_stream_read_reads_every_word(dev, nbytes, nblocks):
    # the measurement hook touches every 32-bit word once: the XOR of its
    # workgroups' results is the XOR of the whole buffer (ragged last round)
    g = torch.Generator().manual_seed(nbytes)
    host = torch.randint(-2**31, 2**31 - 1, (nbytes // 4,), dtype=torch.int32, generator=g)
    out = torch.zeros(nblocks, dtype=torch.int32, device=dev)
    dp.dp_stream_read(host.to(dev), out)
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(host.numpy().view(np.uint32))
    got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
    assert int(got) == int(want)
