"""Shared helpers for the GPU parity tests (imported by tests only)."""

import numpy as np
import pytest
import torch


def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def f64(t):
    return t.detach().cpu().double().numpy()


def max_rel_elementwise(x, ref):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.maximum(np.abs(ref), 1e-300)
    return float(np.max(np.abs(x - ref) / den)) if ref.size else 0.0


def max_rel_normwise(x, ref):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    scale = float(np.max(np.abs(ref)))
    return float(np.max(np.abs(x - ref))) / (scale if scale > 0 else 1.0)


def report(name, **vals):
    print(f"[parity] {name} " + " ".join(f"{k}={v:.3e}" if isinstance(v, float) else f"{k}={v}"
                                         for k, v in vals.items()), flush=True)
