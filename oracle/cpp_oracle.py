"""ctypes wrapper of the plain C++ fp64 oracle (oracle/cpp/oracle_fp64.cpp).

TEST INFRASTRUCTURE ONLY: used by tests/ and by bench.py's CPU baseline; the
product path never imports it.  build() compiles the library in-tree with g++
(C++17, -O3, std::thread, no BLAS); load() raises if it has not been built.
Inputs are the exact bytes the GPU reads (fp32 or raw bf16), passed by
pointer; results are fp64 numpy arrays.
"""

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "cpp", "oracle_fp64.cpp")
LIB = os.path.join(HERE, "cpp", "liboracle_fp64.so")
# x86-64-v3 (AVX2 + FMA) rather than -march=native: the library is built here
# and may run on another host of the same family.  No contraction of a * b + c
# into one fused rounding, so every expression rounds as it is written.
FLAGS = ["-O3", "-march=x86-64-v3", "-ffp-contract=off", "-std=c++17", "-pthread", "-shared", "-fPIC",
         "-Wall"]

_lib = None


def build():
    """Compile liboracle_fp64.so (always)."""
    tmp = LIB + ".tmp"
    r = subprocess.run(["g++"] + FLAGS + ["-o", tmp, SRC], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"g++ failed for the C++ oracle:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


def load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB):
        raise FileNotFoundError(f"{LIB} is missing: run __graft_entry__.build()")
    L = ctypes.CDLL(LIB)
    i32, i64, u32, u64, dbl, p = (ctypes.c_int, ctypes.c_int64, ctypes.c_uint32, ctypes.c_uint64,
                                  ctypes.c_double, ctypes.c_void_p)
    L.oc_hardware_concurrency.restype = i32
    L.oc_philox.argtypes = [u64, p, p, i64]
    L.oc_probe.argtypes = [u64, u32, u32, i32, i32, p]
    L.oc_hutch_norms.argtypes = [i32] * 6 + [p, p, u64, u32, i32, i32, p]
    L.oc_clip.argtypes = [i32, p, dbl, p]
    L.oc_clip.restype = i32
    L.oc_aggregate.argtypes = [i32] * 5 + [p, p, p, i32, p]
    L.oc_noise_update.argtypes = [i64, i64, p, p, dbl, dbl, dbl, i32, u64, u32, i32]
    _lib = L
    return L


def hardware_concurrency():
    return int(load().oc_hardware_concurrency())


def _raw(x):
    """(dtype code, contiguous numpy array of the raw bytes) of an fp32 or bf16 tensor/array."""
    if hasattr(x, "detach"):  # torch tensor
        import torch
        t = x.detach().to("cpu").contiguous()
        if t.dtype == torch.bfloat16:
            return 1, t.view(torch.int16).numpy()
        if t.dtype == torch.float32:
            return 0, t.numpy()
        raise TypeError(f"unsupported dtype {t.dtype}")
    a = np.ascontiguousarray(x, dtype=np.float32)
    return 0, a


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def philox(seed, ctr):
    """Philox4x32-10 words [n][4] of counters ctr [n][4] (uint32)."""
    ctr = np.ascontiguousarray(ctr, dtype=np.uint32).reshape(-1, 4)
    out = np.empty_like(ctr)
    load().oc_philox(int(seed) & (2**64 - 1), _ptr(ctr), _ptr(out), ctr.shape[0])
    return out


def probe(seed, layer, sample, p, k):
    P = np.empty((p, k), dtype=np.float64)
    load().oc_probe(int(seed) & (2**64 - 1), int(layer), int(sample), p, k, _ptr(P))
    return P


def hutch_norms(A, G, k, seed, layer, n=None, threads=0):
    """n[i] (=, or += when n is given) Hutch estimate ||A_i^T (G_i P_i)||^2 / k."""
    ta, a = _raw(A)
    tg, g = _raw(G)
    assert ta == tg
    B, T, d = a.shape
    p = g.shape[2]
    acc = n is not None
    n = np.zeros(B) if n is None else np.ascontiguousarray(n, dtype=np.float64)
    load().oc_hutch_norms(ta, B, T, d, p, k, _ptr(a), _ptr(g), int(seed) & (2**64 - 1),
                          int(layer), int(acc), threads, _ptr(n))
    return n


def clip_factors(n, C):
    n = np.ascontiguousarray(n, dtype=np.float64)
    c = np.empty_like(n)
    flag = load().oc_clip(len(n), _ptr(n), float(C), _ptr(c))
    return c, bool(flag)


def aggregate(A, G, c, threads=0):
    """S [p][d] = sum_i c_i G_i^T A_i."""
    ta, a = _raw(A)
    tg, g = _raw(G)
    assert ta == tg
    B, T, d = a.shape
    p = g.shape[2]
    c = np.ascontiguousarray(c, dtype=np.float64)
    S = np.empty((p, d), dtype=np.float64)
    load().oc_aggregate(ta, B, T, d, p, _ptr(a), _ptr(g), _ptr(c), threads, _ptr(S))
    return S


def noise_update(theta, S, sigma, C, eta, B, seed, layer, offset=0, threads=0):
    """theta - (eta / B) (S + sigma C xi) for flat elements offset .. offset + theta.size - 1."""
    th = np.array(theta, dtype=np.float64, order="C", copy=True)
    S = np.ascontiguousarray(S, dtype=np.float64)
    load().oc_noise_update(int(offset), th.size, _ptr(th), _ptr(S), float(sigma), float(C),
                           float(eta), int(B), int(seed) & (2**64 - 1), int(layer), threads)
    return th
