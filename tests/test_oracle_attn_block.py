"""Pins for the attention block's forward pass, backward pass 1 and whole step (CPU).

What fixes them, other than the functions themselves:
  * every per-sample parameter gradient and dL/dx against central finite
    differences of the per-sample loss L_i = sum_t <R_{i,t}, out_{i,t}>, with
    grouped heads (2 query heads per key/value head);
  * causality: changing x at position t' leaves out[:t'] unchanged;
  * softmax rows sum to one: constant value rows come back unchanged;
  * RoPE is a rotation: norms are kept, the inverse undoes it, and the dot
    product of rotated q and k depends only on the distance of their positions;
  * the step without clipping or noise is SGD on the batch loss.
Planted mistakes in the oracle (the rowsum term of the softmax backward
dropped, RoPE's forward in place of its transpose in the backward, the grouped
heads' gradients overwritten instead of summed) fail the finite-difference pin.
"""

import numpy as np
import pytest

from oracle import attn_block as ab

EPS, BASE = 1e-5, 500000.0
H, KV, DH = 4, 2, 4


def _block(seed, B=2, T=5, d=8):
    r = np.random.default_rng(seed)
    x = r.standard_normal((B, T, d))
    gamma = 1.0 + 0.3 * r.standard_normal(d)
    Wq = r.standard_normal((H * DH, d)) / np.sqrt(d)
    Wk = r.standard_normal((KV * DH, d)) / np.sqrt(d)
    Wv = r.standard_normal((KV * DH, d)) / np.sqrt(d)
    Wo = r.standard_normal((d, H * DH)) / np.sqrt(H * DH)
    R = r.standard_normal((B, T, d))
    return x, gamma, Wq, Wk, Wv, Wo, R


def _out(x, gamma, Wq, Wk, Wv, Wo, base=BASE):
    return ab.attn_forward(x, gamma, Wq, Wk, Wv, Wo, EPS, H, KV, DH, base)["out"]


def _loss(i, params, R):
    return float(np.sum(R[i] * _out(*params)[i]))


def _check_against_fd(seed, base=BASE, rtol=1e-6, atol=1e-8, picks=4):
    x, gamma, Wq, Wk, Wv, Wo, R = _block(seed)
    params = [x, gamma, Wq, Wk, Wv, Wo]
    fwd = ab.attn_forward(x, gamma, Wq, Wk, Wv, Wo, EPS, H, KV, DH, base)
    bwd = ab.attn_backward(x, gamma, Wq, Wk, Wv, Wo, EPS, H, KV, DH, base, R, fwd)
    grads = ab.attn_per_sample_grads(fwd, bwd)
    names = ["x", "gamma", "W_q", "W_k", "W_v", "W_o"]
    r = np.random.default_rng(seed)
    h = 1e-5
    bad = []
    for i in range(x.shape[0]):
        for pi, name in enumerate(names):
            P = params[pi]
            for _ in range(picks):
                idx = tuple(int(r.integers(0, s)) for s in P.shape)
                if name == "x":
                    idx = (i,) + idx[1:]
                Pp, Pm = P.copy(), P.copy()
                Pp[idx] += h
                Pm[idx] -= h
                pp, pm = list(params), list(params)
                pp[pi], pm[pi] = Pp, Pm
                fd = (float(np.sum(R[i] * _out(*pp, base=base)[i]))
                      - float(np.sum(R[i] * _out(*pm, base=base)[i]))) / (2 * h)
                an = bwd["dx"][idx] if name == "x" else grads[name][i][idx]
                if not np.isclose(an, fd, rtol=rtol, atol=atol):
                    bad.append((name, idx, an, fd))
    return bad


def test_backward_matches_finite_differences():
    assert _check_against_fd(31) == []
    assert _check_against_fd(32, base=10.0) == []  # large rotation angles


def test_causal():
    x, gamma, Wq, Wk, Wv, Wo, R = _block(33, B=1, T=6)
    out = _out(x, gamma, Wq, Wk, Wv, Wo)
    x2 = x.copy()
    x2[0, 4] += 1.0
    out2 = _out(x2, gamma, Wq, Wk, Wv, Wo)
    assert np.array_equal(out[0, :4], out2[0, :4])
    assert not np.allclose(out[0, 4:], out2[0, 4:])


def test_softmax_rows_sum_to_one():
    r = np.random.default_rng(34)
    T = 7
    q = r.standard_normal((T, H * DH))
    k = r.standard_normal((T, KV * DH))
    v = np.tile(r.standard_normal((1, KV * DH)), (T, 1))  # every key has the same value row
    o, lse = ab.attention_forward(q, k, v, H, KV, DH)
    for h in range(H):
        g = h // (H // KV)
        assert np.allclose(o[:, h * DH:(h + 1) * DH], v[:, g * DH:(g + 1) * DH], rtol=1e-13)
    # first row attends only to itself: its normaliser is exp(score)
    s00 = q[0, :DH] @ k[0, :DH] / np.sqrt(DH)
    assert np.isclose(lse[0, 0], s00, rtol=1e-13)


def test_rope_is_a_rotation_with_relative_positions():
    r = np.random.default_rng(35)
    T = 9
    x = r.standard_normal((T, H * DH))
    y = ab.rope(x, H, DH, BASE)
    assert np.allclose(np.linalg.norm(y.reshape(T, H, DH), axis=-1),
                       np.linalg.norm(x.reshape(T, H, DH), axis=-1), rtol=1e-13)
    assert np.allclose(ab.rope(y, H, DH, BASE, inverse=True), x, rtol=1e-12, atol=1e-13)
    assert np.allclose(y[0], x[0])  # position 0 is not rotated
    qv, kv = r.standard_normal(DH), r.standard_normal(DH)
    Q = ab.rope(np.tile(qv, (T, 1)), 1, DH, 100.0)
    K = ab.rope(np.tile(kv, (T, 1)), 1, DH, 100.0)
    assert np.isclose(Q[5] @ K[2], Q[7] @ K[4], rtol=1e-12)
    assert np.isclose(Q[3] @ K[3], qv @ kv, rtol=1e-12)


@pytest.mark.parametrize("plant", ["no_rowsum", "rope_forward", "gqa_overwrite"])
def test_planted_mistakes_fail(monkeypatch, plant):
    if plant == "no_rowsum":
        def wrong(q, k, v, do, n_heads, n_kv, head_dim):
            T = q.shape[0]
            qh, kh, vh = (a.reshape(T, -1, head_dim) for a in (q, k, v))
            doh = do.reshape(T, n_heads, head_dim)
            grp = n_heads // n_kv
            scale = 1.0 / np.sqrt(head_dim)
            mask = np.triu(np.ones((T, T), dtype=bool), 1)
            dq, dk, dv = np.zeros_like(qh), np.zeros_like(kh), np.zeros_like(vh)
            for hh in range(n_heads):
                g = hh // grp
                S = (qh[:, hh] @ kh[:, g].T) * scale
                S[mask] = -np.inf
                P = np.exp(S - S.max(axis=1, keepdims=True))
                P /= P.sum(axis=1, keepdims=True)
                dv[:, g] += P.T @ doh[:, hh]
                dS = P * (doh[:, hh] @ vh[:, g].T)  # rowsum term dropped
                dq[:, hh] = dS @ kh[:, g] * scale
                dk[:, g] += dS.T @ qh[:, hh] * scale
            return dq.reshape(T, -1), dk.reshape(T, -1), dv.reshape(T, -1)
        monkeypatch.setattr(ab, "attention_backward", wrong)
    elif plant == "rope_forward":
        orig = ab.rope
        monkeypatch.setattr(ab, "rope", lambda x, n, dh, base, inverse=False: orig(x, n, dh, base))
    else:
        orig = ab.attention_backward

        def wrong(q, k, v, do, n_heads, n_kv, head_dim):
            # only the last query head of each group reaches dk, dv
            T = q.shape[0]
            grp = n_heads // n_kv
            dq, dk, dv = orig(q, k, v, do, n_heads, n_kv, head_dim)
            keep = np.zeros((T, n_heads, head_dim))
            keep[:, grp - 1::grp] = do.reshape(T, n_heads, head_dim)[:, grp - 1::grp]
            _, dk1, dv1 = orig(q, k, v, keep.reshape(T, -1), n_heads, n_kv, head_dim)
            return dq, dk1, dv1
        monkeypatch.setattr(ab, "attention_backward", wrong)
    assert _check_against_fd(31) != []


def test_step_without_clipping_or_noise_is_sgd_on_the_batch_loss():
    x, gamma, Wq, Wk, Wv, Wo, R = _block(36)
    eta, B = 0.3, x.shape[0]
    fwd = ab.attn_forward(x, gamma, Wq, Wk, Wv, Wo, EPS, H, KV, DH, BASE)
    bwd = ab.attn_backward(x, gamma, Wq, Wk, Wv, Wo, EPS, H, KV, DH, BASE, R, fwd)
    weights = {"W_q": Wq, "W_k": Wk, "W_v": Wv, "W_o": Wo}
    n, c, new = ab.attn_dp_step({**fwd, **bwd}, gamma, weights, "fgc", 0, 1e6, 0.0, eta, 1, 2)
    assert np.all(c == 1.0)
    grads = ab.attn_per_sample_grads(fwd, bwd)
    assert np.allclose(n, sum(np.sum(g.reshape(B, -1) ** 2, axis=1) for g in grads.values()),
                       rtol=1e-12)
    params = {"gamma": gamma, **weights}
    order = ["gamma", "W_q", "W_k", "W_v", "W_o"]
    r = np.random.default_rng(1)
    h = 1e-5
    for name, P in params.items():
        for _ in range(2):
            idx = tuple(int(r.integers(0, s)) for s in P.shape)
            Pp, Pm = P.copy(), P.copy()
            Pp[idx] += h
            Pm[idx] -= h
            ap = [x] + [params[o] if o != name else Pp for o in order]
            am = [x] + [params[o] if o != name else Pm for o in order]
            fd = sum(_loss(i, ap, R) - _loss(i, am, R) for i in range(B)) / (2 * h)
            assert np.isclose(new[name][idx], P[idx] - eta / B * fd, rtol=1e-8, atol=1e-10)


def test_layer_backward_matches_finite_differences():
    """The attention block feeding the MLP block: every parameter of both halves
    and dL/dx against central differences of the layer's per-sample loss."""
    from oracle import mlp_block as mb
    x, gamma, Wq, Wk, Wv, Wo, R = _block(41)
    r = np.random.default_rng(42)
    d, f = x.shape[-1], 6
    mlp_p = (1.0 + 0.3 * r.standard_normal(d), r.standard_normal((f, d)) / np.sqrt(d),
             r.standard_normal((f, d)) / np.sqrt(d), r.standard_normal((d, f)) / np.sqrt(f))
    attn_p = (gamma, Wq, Wk, Wv, Wo)
    fa, fm = ab.layer_forward(x, attn_p, mlp_p, EPS, H, KV, DH, BASE)
    ba, bm = ab.layer_backward(x, attn_p, mlp_p, EPS, H, KV, DH, BASE, R, (fa, fm))
    ga = ab.attn_per_sample_grads(fa, ba)
    gm = mb.mlp_per_sample_grads(fm, bm)

    def loss(i, xx, ap, mp):
        return float(np.sum(R[i] * ab.layer_forward(xx, ap, mp, EPS, H, KV, DH, BASE)[1]["out"][i]))

    h = 1e-5
    for i in range(x.shape[0]):
        checks = [("x", None, None)] + [("attn", j, n) for j, n in enumerate(
            ["gamma", "W_q", "W_k", "W_v", "W_o"])] + [("mlp", j, n) for j, n in enumerate(
                ["gamma", "W_gate", "W_up", "W_down"])]
        for part, j, name in checks:
            P = x if part == "x" else (attn_p[j] if part == "attn" else mlp_p[j])
            for _ in range(2):
                idx = tuple(int(r.integers(0, s)) for s in P.shape)
                if part == "x":
                    idx = (i,) + idx[1:]
                Pp, Pm = P.copy(), P.copy()
                Pp[idx] += h
                Pm[idx] -= h
                if part == "x":
                    fd = (loss(i, Pp, attn_p, mlp_p) - loss(i, Pm, attn_p, mlp_p)) / (2 * h)
                    an = ba["dx"][idx]
                elif part == "attn":
                    ap_, am_ = list(attn_p), list(attn_p)
                    ap_[j], am_[j] = Pp, Pm
                    fd = (loss(i, x, ap_, mlp_p) - loss(i, x, am_, mlp_p)) / (2 * h)
                    an = ga[name][i][idx]
                else:
                    mp_, mm_ = list(mlp_p), list(mlp_p)
                    mp_[j], mm_[j] = Pp, Pm
                    fd = (loss(i, x, attn_p, mp_) - loss(i, x, attn_p, mm_)) / (2 * h)
                    an = gm[name][i][idx]
                assert np.isclose(an, fd, rtol=1e-6, atol=1e-8), (part, name, idx, an, fd)


def test_layer_step_clips_the_whole_layer_gradient():
    """With a small C the one-sample update of all eleven parameters together has
    norm exactly C (one clip factor for the whole layer)."""
    x, gamma, Wq, Wk, Wv, Wo, R = _block(43, B=1)
    r = np.random.default_rng(44)
    d, f = x.shape[-1], 6
    mlp_p = (1.0 + 0.3 * r.standard_normal(d), r.standard_normal((f, d)) / np.sqrt(d),
             r.standard_normal((f, d)) / np.sqrt(d), r.standard_normal((d, f)) / np.sqrt(f))
    attn_p = (gamma, Wq, Wk, Wv, Wo)
    fa, fm = ab.layer_forward(x, attn_p, mlp_p, EPS, H, KV, DH, BASE)
    ba, bm = ab.layer_backward(x, attn_p, mlp_p, EPS, H, KV, DH, BASE, R, (fa, fm))
    C = 1e-3
    n, c, new = ab.layer_dp_step({**fa, **ba}, {**fm, **bm}, attn_p, mlp_p, "fgc", 0, C, 0.0, 1.0,
                                 1, 2)
    assert c[0] < 1.0
    old = {"W_q": Wq, "W_k": Wk, "W_v": Wv, "W_o": Wo, "gamma": gamma, "W_gate": mlp_p[1],
           "W_up": mlp_p[2], "W_down": mlp_p[3], "mlp_gamma": mlp_p[0]}
    delta = np.concatenate([(old[k_] - new[k_]).ravel() for k_ in old])
    assert np.isclose(np.linalg.norm(delta), C, rtol=1e-10)
