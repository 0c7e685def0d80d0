"""GPU parity of the attention block's forward pass and backward pass 1, and of
its whole DP-SGD-RC step, against the fp64 oracle.

Each kernel is checked against the oracle applied to the GPU's own bf16 inputs
of that stage, within a bound derived from its arithmetic:
  * RoPE: fp64 angles, fp32 rotation, one bf16 rounding: 2^-8 |ref| + 1e-6 |x|;
  * attention: the probabilities enter the second product as bf16, so
    |o - ref| <= 2^-8 |ref| + (2^-8 + 1e-4) (P |v|) (P from the oracle's own
    normaliser), and lse within 1e-5 (1 + |lse|);
  * the products as for the MLP block.
End to end against the fp64 oracle (no bf16 intermediates) the bound is
normwise, 2e-2.  At Llama-3.2-1B's attention shape (d 2048, 32 query and 8
key/value heads of 64, T 4096) sampled (token, head) pairs are checked one by
one from the GPU's q, k and v.
"""

import numpy as np
import pytest
import torch

import oracle
from sample_gradient_clipping_amd import binding as dp
from tests.gpu_util import device, f64, max_rel_normwise, report

pytestmark = pytest.mark.gpu

U8 = 2.0 ** -8
U24 = 2.0 ** -24
EPS, BASE = 1e-5, 500000.0


@pytest.fixture(scope="module")
def dev():
    d = device()
    dp.load_library()
    return d


def _bf(t):
    return t.detach().cpu().float().double().numpy()


def _rand_bf16(r, shape, scale=1.0):
    return torch.from_numpy((scale * r.standard_normal(shape)).astype(np.float32)).to(torch.bfloat16)


def assert_within(name, got, ref, bound):
    excess = np.abs(got - ref) - bound
    worst = float(np.max(excess / np.maximum(bound, 1e-300)))
    report(name, max_rel=max_rel_normwise(got, ref), worst_over_bound=worst)
    assert np.all(excess <= 0), f"{name}: {int(np.sum(excess > 0))} elements beyond the bound"


@pytest.mark.parametrize("inverse", [False, True])
@pytest.mark.parametrize("T,nh,base", [(128, 4, BASE), (64, 2, 10.0), (300, 1, 10000.0)])
def test_rope(dev, T, nh, base, inverse):
    r = np.random.default_rng(T + nh)
    x = _rand_bf16(r, (2, T, 64 * nh))
    y = dp.dp_rope(x.to(dev).clone(), T, nh, base=base, inverse=inverse)
    torch.cuda.synchronize()
    ref = np.stack([oracle.rope(_bf(x[i]), nh, 64, base, inverse=inverse) for i in range(2)])
    assert_within(f"rope T={T} nh={nh} inverse={inverse}", _bf(y), ref,
                  U8 * np.abs(ref) + 1e-6 * np.max(np.abs(_bf(x))) + 1e-30)


def _attn_ref_bound(q, k, v, H, KV, o_ref, lse_ref):
    """(P |v|) for every query row and head, P from the oracle's normaliser."""
    T = q.shape[0]
    qh, kh, vh = q.reshape(T, H, 64), k.reshape(T, KV, 64), v.reshape(T, KV, 64)
    pv = np.zeros((T, H, 64))
    mask = np.triu(np.ones((T, T), dtype=bool), 1)
    for h in range(H):
        g = h // (H // KV)
        S = qh[:, h] @ kh[:, g].T / 8.0
        S[mask] = -np.inf
        P = np.exp(S - lse_ref[h][:, None])
        pv[:, h] = P @ np.abs(vh[:, g])
    return pv.reshape(T, H * 64)


@pytest.mark.parametrize("B,T,H,KV", [(2, 128, 8, 2), (1, 128, 4, 4), (2, 384, 4, 1), (1, 640, 32, 8)])
def test_attention_forward(dev, B, T, H, KV):
    r = np.random.default_rng(T * 3 + H)
    q = _rand_bf16(r, (B, T, 64 * H), 0.5)
    k = _rand_bf16(r, (B, T, 64 * KV), 0.5)
    v = _rand_bf16(r, (B, T, 64 * KV))
    o, lse = dp.dp_attention_forward(q.to(dev), k.to(dev), v.to(dev), H, KV)
    torch.cuda.synchronize()
    for i in range(B):
        qf, kf, vf = _bf(q[i]), _bf(k[i]), _bf(v[i])
        o_ref, lse_ref = oracle.attention_forward(qf, kf, vf, H, KV, 64)
        pv = _attn_ref_bound(qf, kf, vf, H, KV, o_ref, lse_ref)
        assert_within(f"attention o B={B} T={T} H={H} KV={KV} sample {i}", _bf(o[i]), o_ref,
                      (U8 + 1e-5) * np.abs(o_ref) + (U8 + 1e-4) * pv + 1e-30)
        assert np.all(np.abs(f64(lse[i]) - lse_ref) <= 1e-5 * (1 + np.abs(lse_ref)))


def _weights(r, d, H, KV):
    th = {"W_q": 0.02 * r.standard_normal((64 * H, d)), "W_k": 0.02 * r.standard_normal((64 * KV, d)),
          "W_v": 0.02 * r.standard_normal((64 * KV, d)), "W_o": 0.02 * r.standard_normal((d, 64 * H))}
    return {k_: torch.from_numpy(v_.astype(np.float32)) for k_, v_ in th.items()}


def _block(dev, B, T, d, H, KV, seed):
    r = np.random.default_rng(seed)
    x = _rand_bf16(r, (B, T, d))
    gamma = torch.from_numpy((1.0 + 0.1 * r.standard_normal(d)).astype(np.float32))
    thetas = _weights(r, d, H, KV)
    R = torch.from_numpy((0.01 * r.standard_normal((B, T, d))).astype(np.float32)).to(torch.bfloat16)
    Wb = {k_: dp.dp_weights_bf16(v_.to(dev)) for k_, v_ in thetas.items()}
    torch.cuda.synchronize()
    return x, gamma, thetas, R, Wb


BLOCK_CASES = [(2, 128, 256, 4, 4), (1, 256, 512, 8, 4)]


@pytest.mark.parametrize("B,T,d,H,KV", BLOCK_CASES)
def test_attn_block_forward(dev, B, T, d, H, KV):
    x, gamma, thetas, R, Wb = _block(dev, B, T, d, H, KV, 101)
    acts = dp.dp_attn_forward(x.to(dev), gamma.to(dev), Wb["W_q"][0], Wb["W_k"][0], Wb["W_v"][0],
                              Wb["W_o"][0], H, KV, eps=EPS, rope_base=BASE)
    torch.cuda.synchronize()
    W = {k_: _bf(v_[0]) for k_, v_ in Wb.items()}
    xf, gm = _bf(x), gamma.double().numpy()
    got = {k_: (f64(v_) if k_ in ("rstd", "lse") else _bf(v_)) for k_, v_ in acts.items()}
    # attention and the output product on the GPU's own q, k, v and o
    for i in range(B):
        o_ref, lse_ref = oracle.attention_forward(got["q"][i], got["k"][i], got["v"][i], H, KV, 64)
        pv = _attn_ref_bound(got["q"][i], got["k"][i], got["v"][i], H, KV, o_ref, lse_ref)
        assert_within(f"block attention sample {i}", got["o"][i], o_ref,
                      (U8 + 1e-5) * np.abs(o_ref) + (U8 + 1e-4) * pv + 1e-30)
    o2 = got["o"].reshape(B * T, -1)
    out_r = oracle.linear_forward(o2, W["W_o"], residual=xf.reshape(B * T, -1))
    bound = U8 * np.abs(out_r) + (1 + U8) * 64 * H * U24 * (np.abs(o2) @ np.abs(W["W_o"]).T) * 1.01
    assert_within("block out", got["out"].reshape(B * T, -1), out_r, bound + 1e-30)
    # end to end, fp64 throughout
    ref = oracle.attn_forward(xf, gm, W["W_q"], W["W_k"], W["W_v"], W["W_o"], EPS, H, KV, 64, BASE)
    for k_ in ("y", "q", "k", "v", "o", "out"):
        e = max_rel_normwise(got[k_], ref[k_])
        report(f"attn forward end-to-end {k_}", max_rel=e)
        assert e <= 2e-2
    assert np.all(np.abs(got["lse"] - ref["lse"]) <= 2e-2 * (1 + np.abs(ref["lse"])))


@pytest.mark.parametrize("B,T,H,KV", [(2, 128, 8, 2), (1, 128, 4, 4), (2, 384, 4, 1), (1, 640, 32, 8)])
def test_attention_backward(dev, B, T, H, KV):
    r = np.random.default_rng(T * 5 + H)
    q = _rand_bf16(r, (B, T, 64 * H), 0.5).to(dev)
    k = _rand_bf16(r, (B, T, 64 * KV), 0.5).to(dev)
    v = _rand_bf16(r, (B, T, 64 * KV)).to(dev)
    dO = _rand_bf16(r, (B, T, 64 * H)).to(dev)
    o, lse = dp.dp_attention_forward(q, k, v, H, KV)
    dq, dk, dv = dp.dp_attention_backward(q, k, v, o, lse, dO, H, KV)
    torch.cuda.synchronize()
    for i in range(B):
        ref = oracle.attention_backward(_bf(q[i]), _bf(k[i]), _bf(v[i]), _bf(dO[i]), H, KV, 64)
        for name, got, rf in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
            e = max_rel_normwise(_bf(got[i]), rf)
            report(f"attention backward {name} B={B} T={T} H={H} KV={KV} sample {i}", max_rel=e)
            assert e <= 2e-2


def _gpu_attn_block(dev, x, gamma, R, Wb, H, KV):
    xd, gd, Rd = x.to(dev), gamma.to(dev), R.to(dev)
    acts = dp.dp_attn_forward(xd, gd, Wb["W_q"][0], Wb["W_k"][0], Wb["W_v"][0], Wb["W_o"][0], H, KV,
                              eps=EPS, rope_base=BASE)
    grads = dp.dp_attn_backward(xd, acts, gd, Wb["W_q"][1], Wb["W_k"][1], Wb["W_v"][1],
                                Wb["W_o"][1], Rd, H, KV, rope_base=BASE)
    return xd, gd, Rd, acts, grads


@pytest.mark.parametrize("B,T,d,H,KV", BLOCK_CASES)
def test_attn_block_backward(dev, B, T, d, H, KV):
    x, gamma, thetas, R, Wb = _block(dev, B, T, d, H, KV, 103)
    _, _, _, acts, grads = _gpu_attn_block(dev, x, gamma, R, Wb, H, KV)
    torch.cuda.synchronize()
    W = {k_: _bf(v_[0]) for k_, v_ in Wb.items()}
    xf, gm, Rf = _bf(x), gamma.double().numpy(), _bf(R)
    got = {k_: _bf(v_) for k_, v_ in grads.items()}
    M = B * T
    # dy on the GPU's G (one product over three k ranges)
    Gcat = np.concatenate([got["G_q"].reshape(M, -1), got["G_k"].reshape(M, -1),
                           got["G_v"].reshape(M, -1)], axis=1)
    Wcat = np.concatenate([W["W_q"], W["W_k"], W["W_v"]], axis=0).T  # [d][64 (H + 2 KV)]
    dy_r = Gcat @ Wcat.T
    K = Gcat.shape[1]
    assert_within("attn backward dy", got["dy"].reshape(M, -1), dy_r,
                  U8 * np.abs(dy_r) + (1 + U8) * K * U24 * (np.abs(Gcat) @ np.abs(Wcat).T) * 1.01
                  + 1e-30)
    # end to end, fp64 throughout
    fwd = oracle.attn_forward(xf, gm, W["W_q"], W["W_k"], W["W_v"], W["W_o"], EPS, H, KV, 64, BASE)
    ref = oracle.attn_backward(xf, gm, W["W_q"], W["W_k"], W["W_v"], W["W_o"], EPS, H, KV, 64,
                               BASE, Rf, fwd)
    for k_ in ("G_q", "G_k", "G_v", "dy", "dx"):
        e = max_rel_normwise(got[k_], ref[k_])
        report(f"attn backward end-to-end {k_}", max_rel=e)
        assert e <= 2e-2


def test_attn_block_dp_step_fgc_matches_oracle(dev):
    B, T, d, H, KV = 3, 128, 256, 4, 4
    x, gamma, thetas, R, Wb = _block(dev, B, T, d, H, KV, 107)
    xd, gd, Rd, acts, grads = _gpu_attn_block(dev, x, gamma, R, Wb, H, KV)
    # sigma small enough that the clipped sum, not the noise, dominates the update,
    # and eta large enough that the update, not the fp32 rounding of theta', sets
    # the difference
    C, sigma, eta, seed_n, seed_z = 0.01, 2e-3, 50.0, 11, 13
    ids = dict(oracle.ATTN_LAYERS)
    lin = {"W_q": (acts["y"], grads["G_q"]), "W_k": (acts["y"], grads["G_k"]),
           "W_v": (acts["y"], grads["G_v"]), "W_o": (acts["o"], Rd)}
    n = torch.zeros(B, dtype=torch.float32, device=dev)
    v = torch.empty(B, d, dtype=torch.float32, device=dev)
    dp.dp_rmsnorm_norm(acts["xhat"], grads["dy"], n, v=v)
    for name, (A, G) in lin.items():
        dp.dp_norm_est("fgc", A, G, 0, seed_n, ids[name], n, flags=dp.DP_ACCUMULATE)
    theta = {name: t.to(dev).clone() for name, t in thetas.items()}
    for name, (A, G) in lin.items():
        dp.dp_clip_aggregate_update(A, G, n, C, sigma, eta, seed_z, ids[name], theta[name])
    gam = gd.clone()
    dp.dp_rmsnorm_clip_aggregate_update(v, n, C, sigma, eta, seed_z, ids["gamma"], gam)
    torch.cuda.synchronize()
    host = {"y": acts["y"], "o": acts["o"], "xhat": acts["xhat"], "G_q": grads["G_q"],
            "G_k": grads["G_k"], "G_v": grads["G_v"], "G_o": Rd, "dy": grads["dy"]}
    host = {k_: _bf(t) for k_, t in host.items()}
    n_r, c_r, new_r = oracle.attn_dp_step(host, gamma.double().numpy(),
                                          {k_: t.double().numpy() for k_, t in thetas.items()},
                                          "fgc", 0, C, sigma, eta, seed_n, seed_z)
    assert np.all(c_r < 1.0)
    e_n = float(np.max(np.abs(f64(n) - n_r) / n_r))
    report("attn block step fgc n", max_rel=e_n)
    assert e_n <= 1e-5
    got = {**{k_: f64(t) for k_, t in theta.items()}, "gamma": f64(gam)}
    for name in new_r:
        base = gamma.double().numpy() if name == "gamma" else thetas[name].double().numpy()
        e = max_rel_normwise(got[name] - base, new_r[name] - base)
        report(f"attn block step fgc {name}", max_rel=e)
        assert e <= 1e-4


def test_attn_block_full_width_sampled_rows(dev):
    """Llama-3.2-1B attention at full width (B 2, T 4096, d 2048, 32 query and 8
    key/value heads): the block forward and the attention backward on sampled
    (token, head) pairs and sampled keys.  The references are the oracle's
    attention forward (o and lse) and backward (dq, dk, dv) of each whole
    sample, run on the GPU's bf16 q, k, v and the seeded dO: the attention
    stage checked on its own inputs, with nothing else taken from the GPU."""
    B, T, d, H, KV = 2, 4096, 2048, 32, 8
    x, gamma, thetas, R, Wb = _block(dev, B, T, d, H, KV, 109)
    xd, gd, Rd, acts, grads = _gpu_attn_block(dev, x, gamma, R, Wb, H, KV)
    r = np.random.default_rng(7)
    dO = _rand_bf16(r, (B, T, 64 * H)).to(dev)
    dq, dk, dv = dp.dp_attention_backward(acts["q"], acts["k"], acts["v"], acts["o"], acts["lse"],
                                          dO, H, KV)
    torch.cuda.synchronize()
    Wo = _bf(Wb["W_o"][0])
    ref = {}
    for b in range(B):
        q, k, v, do = (_bf(acts["q"][b]), _bf(acts["k"][b]), _bf(acts["v"][b]), _bf(dO[b]))
        o_r, lse_r = oracle.attention_forward(q, k, v, H, KV, 64)
        dq_r, dk_r, dv_r = oracle.attention_backward(q, k, v, do, H, KV, 64)
        ref[b] = {"o": o_r, "lse": lse_r, "dq": dq_r, "dk": dk_r, "dv": dv_r}
    picks = [(0, 0, 0), (B - 1, T - 1, H - 1)] + [
        (int(r.integers(B)), int(r.integers(T)), int(r.integers(H))) for _ in range(22)]
    for b, t, h in picks:
        cols = slice(64 * h, 64 * h + 64)
        assert max_rel_normwise(_bf(acts["o"][b, t, cols]), ref[b]["o"][t, cols]) <= 2e-2, (b, t, h)
        lse_r = ref[b]["lse"][h, t]
        assert abs(float(acts["lse"][b, h, t]) - lse_r) <= 1e-4 * (1 + abs(lse_r)), (b, t, h)
        assert max_rel_normwise(_bf(dq[b, t, cols]), ref[b]["dq"][t, cols]) <= 2e-2, (b, t, h)
        # out row of the block: the o projection and residual on the GPU's o row
        out_ref = oracle.linear_forward(_bf(acts["o"][b, t])[None], Wo, residual=_bf(x[b, t])[None])
        assert max_rel_normwise(_bf(acts["out"][b, t]), out_ref[0]) <= 2e-2
    # dk, dv of sampled keys (summed over the group's query heads by both sides)
    for b, tk, g in [(0, 0, 0), (B - 1, T - 1, KV - 1)] + [
            (int(r.integers(B)), int(r.integers(T)), int(r.integers(KV))) for _ in range(10)]:
        cols = slice(64 * g, 64 * g + 64)
        assert max_rel_normwise(_bf(dk[b, tk, cols]), ref[b]["dk"][tk, cols]) <= 2e-2, (b, tk, g)
        assert max_rel_normwise(_bf(dv[b, tk, cols]), ref[b]["dv"][tk, cols]) <= 2e-2, (b, tk, g)
    report("attn full-width sampled rows", rows=len(picks))
