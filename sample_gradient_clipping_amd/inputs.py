"""Seeded synthetic inputs shared by the tests, the bench and the checker.

This module holds no arithmetic of the method: it only draws seeded random
activations A [B][T][d], output gradients G [B][T][p] and parameters theta
[p][d], in the dtype the GPU reads.  Both the HIP path and the CPU reference
consume the same bytes.

Recipes (the value distributions of the five workloads):
  * "unit_u0.1_3": A, G i.i.d. N(0, 1); each G_i scaled by s_i ~ U(0.1, 3).
  * "llama_logu":  A ~ N(0, 1) (RMSNorm-like activations); G ~ N(0, 1e-4)
    (variance 1e-4, std 0.01) times a per-sample scale s_i = 10^U(-1, 1),
    log-uniform over [0.1, 10].
  * "lowrank":     A = U_a V_a^T + 0.05 N and G likewise, rank-8 signal plus
    noise, for estimator-accuracy checks on a decaying spectrum.
  * MLP block (``mlp_block_inputs``): x ~ N(0, 1) (the residual stream),
    gamma = 1 + 0.1 N(0, 1), weights N(0, 0.02^2) in fp32 (as theta_init), and
    the output gradient R = dL/d(out) ~ N(0, 1e-4) times s_i = 10^U(-1, 1).
Ragged batches (``ragged_lengths``): per-sample lengths T_i <= T; the caller
zeroes G's rows from T_i on (the pad), as a masked backward pass leaves them.
Host draws use numpy's PCG64 seeded with (seed, layer_id, tensor_tag); values
are drawn in fp32 and rounded to nearest-even bf16 when the dtype is bf16.
"""

import numpy as np
import torch

TAG_A, TAG_G, TAG_SCALE, TAG_THETA, TAG_LEN = 0, 1, 2, 3, 4
TAG_GAMMA = 5


def _rng(seed, layer_id, tag):
    return np.random.default_rng([int(seed), int(layer_id), int(tag)])


def torch_dtype(dtype):
    return {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]


def sample_scales(B, recipe, seed, layer_id=0):
    rng = _rng(seed, layer_id, TAG_SCALE)
    if recipe == "unit_u0.1_3":
        return rng.uniform(0.1, 3.0, size=B)
    if recipe in ("llama_logu", "lowrank"):
        return 10.0 ** rng.uniform(-1.0, 1.0, size=B)
    raise ValueError(recipe)


def _lowrank(rng, B, T, n, rank=8, noise=0.05):
    U = rng.standard_normal((B, T, rank), dtype=np.float32)
    V = rng.standard_normal((B, rank, n), dtype=np.float32) / np.float32(np.sqrt(rank))
    E = rng.standard_normal((B, T, n), dtype=np.float32)
    return np.matmul(U, V) + np.float32(noise) * E


def linear_inputs(B, T, d, p, dtype, recipe, seed, layer_id=0):
    """(A [B][T][d], G [B][T][p]) as CPU torch tensors of ``dtype``."""
    ra = _rng(seed, layer_id, TAG_A)
    rg = _rng(seed, layer_id, TAG_G)
    s = sample_scales(B, recipe, seed, layer_id).astype(np.float32)
    if recipe == "lowrank":
        A = _lowrank(ra, B, T, d)
        G = _lowrank(rg, B, T, p) * np.float32(0.01)
    else:
        A = ra.standard_normal((B, T, d), dtype=np.float32)
        G = rg.standard_normal((B, T, p), dtype=np.float32)
        if recipe == "llama_logu":
            G *= np.float32(0.01)
    G *= s[:, None, None]
    td = torch_dtype(dtype)
    return torch.from_numpy(A).to(td), torch.from_numpy(G).to(td)


def ragged_lengths(B, T, seed, min_len=1):
    """Per-sample sequence lengths T_i for a ragged batch padded to T tokens:
    sample 0 has the full T, the last sample min_len, the others are uniform
    on [min_len, T] (numpy PCG64 seeded with (seed, 0, TAG_LEN))."""
    r = _rng(seed, 0, TAG_LEN)
    lengths = r.integers(min_len, T, endpoint=True, size=B)
    lengths[0] = T
    if B > 1:
        lengths[-1] = min_len
    return [int(x) for x in lengths]


def theta_init(p, d, seed, layer_id=0, std=0.02, zero=False):
    """fp32 parameters theta [p][d]: zeros, or N(0, std^2)."""
    if zero:
        return torch.zeros(p, d, dtype=torch.float32)
    r = _rng(seed, layer_id, TAG_THETA)
    return torch.from_numpy(r.standard_normal((p, d), dtype=np.float32) * np.float32(std))


def linear_inputs_device(B, T, d, p, dtype, recipe, seed, layer_id, device):
    """Device-side draws of the same shapes and law (bench only: the host
    generator is too slow for tens of GB).  Not bit-identical to
    :func:`linear_inputs`; nothing is compared against a host reference."""
    gen = torch.Generator(device=device)
    gen.manual_seed((int(seed) * 1_000_003 + int(layer_id)) & 0x7FFFFFFFFFFFFFFF)
    td = torch_dtype(dtype)
    s = torch.from_numpy(sample_scales(B, recipe, seed, layer_id).astype(np.float32)).to(device)
    if recipe == "lowrank":
        def lowrank(n, rank=8, noise=0.05):
            U = torch.randn((B, T, rank), generator=gen, device=device, dtype=torch.float32)
            V = torch.randn((B, rank, n), generator=gen, device=device,
                            dtype=torch.float32) / float(np.sqrt(rank))
            E = torch.randn((B, T, n), generator=gen, device=device, dtype=torch.float32)
            return torch.bmm(U, V) + noise * E
        A = lowrank(d).to(td)
        G = lowrank(p) * 0.01
    else:
        A = torch.randn((B, T, d), generator=gen, device=device, dtype=torch.float32).to(td)
        G = torch.randn((B, T, p), generator=gen, device=device, dtype=torch.float32)
        if recipe == "llama_logu":
            G *= 0.01
    G = (G * s[:, None, None]).to(td)
    return A, G


def mlp_block_inputs(B, T, d, f, seed, block=0):
    """(x [B][T][d] bf16, gamma [d] fp32, {"W_gate": [f][d], "W_up": [f][d],
    "W_down": [d][f]} fp32, R [B][T][d] bf16) on the CPU; the three weights use
    layer ids 7 block + {0, 1, 2} of the theta stream."""
    x = _rng(seed, 7 * block, TAG_A).standard_normal((B, T, d), dtype=np.float32)
    gamma = 1.0 + 0.1 * _rng(seed, 7 * block, TAG_GAMMA).standard_normal(d, dtype=np.float32)
    thetas = {name: theta_init(shape[0], shape[1], seed, 7 * block + i)
              for i, (name, shape) in enumerate((("W_gate", (f, d)), ("W_up", (f, d)),
                                                 ("W_down", (d, f))))}
    s = sample_scales(B, "llama_logu", seed, 7 * block).astype(np.float32)
    R = _rng(seed, 7 * block, TAG_G).standard_normal((B, T, d), dtype=np.float32)
    R *= np.float32(0.01) * s[:, None, None]
    return (torch.from_numpy(x).to(torch.bfloat16), torch.from_numpy(gamma.astype(np.float32)),
            thetas, torch.from_numpy(R).to(torch.bfloat16))


def mlp_block_inputs_device(B, T, d, f, seed, device):
    """The same shapes and law drawn on the device (bench only; not bit-identical
    to :func:`mlp_block_inputs`)."""
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed) & 0x7FFFFFFFFFFFFFFF)

    def randn(*shape):
        return torch.randn(shape, generator=gen, device=device, dtype=torch.float32)

    x = randn(B, T, d).to(torch.bfloat16)
    gamma = 1.0 + 0.1 * randn(d)
    thetas = {"W_gate": 0.02 * randn(f, d), "W_up": 0.02 * randn(f, d), "W_down": 0.02 * randn(d, f)}
    s = torch.from_numpy(sample_scales(B, "llama_logu", seed).astype(np.float32)).to(device)
    R = (0.01 * randn(B, T, d) * s[:, None, None]).to(torch.bfloat16)
    return x, gamma, thetas, R
