"""Pins for the oracle's random streams (CPU only).

Philox4x32-10 is checked bit for bit against an independent implementation
(PyTorch's open-source engine header, compiled here with g++); the Gaussian
transform against the mathematics of Box-Muller and the N(0, 1) law.
"""

import math
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest
from scipy import stats

import oracle
from oracle.philox import NOISE_C2

HERE = os.path.dirname(os.path.abspath(__file__))


def _torch_include():
    try:
        import torch
    except ImportError:
        return None
    inc = os.path.join(os.path.dirname(torch.__file__), "include")
    hdr = os.path.join(inc, "ATen", "core", "PhiloxRNGEngine.h")
    return inc if os.path.exists(hdr) else None


@pytest.fixture(scope="module")
def philox_ref_bin():
    inc = _torch_include()
    if inc is None or shutil.which("g++") is None:
        pytest.skip("PyTorch Philox header or g++ not available")
    tmp = tempfile.mkdtemp(prefix="philox_ref_")
    exe = os.path.join(tmp, "philox_ref")
    subprocess.run(["g++", "-std=c++17", "-O1", "-I", inc,
                    os.path.join(HERE, "philox_ref.cpp"), "-o", exe], check=True)
    yield exe
    shutil.rmtree(tmp, ignore_errors=True)


def _ref_words(exe, triples):
    text = "".join(f"{s} {sub} {off}\n" for s, sub, off in triples)
    out = subprocess.run([exe], input=text, capture_output=True, text=True, check=True).stdout
    return np.array([[int(w) for w in line.split()] for line in out.strip().splitlines()],
                    dtype=np.uint64)


def test_philox_matches_independent_engine(philox_ref_bin):
    rng = np.random.default_rng(7)
    cases = []
    # random full-width counters and keys
    for _ in range(200):
        seed = int(rng.integers(0, 2**63)) * 2 + int(rng.integers(0, 2))
        c = [int(x) for x in rng.integers(0, 2**32, size=4, dtype=np.uint64)]
        cases.append((seed, c))
    # the counter layouts the method uses: probes (r>>2, j, i, layer) and noise
    for seed in (0, 1, 2002, 2**64 - 1):
        for c in ([0, 0, 0, 0], [5, 31, 7, 111], [2047, 3, 0, 1],
                  [0xFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF],
                  [123456, 0, NOISE_C2, 42], [7, 1, NOISE_C2, 0]):
            cases.append((seed, c))
    triples = [(s, c[2] | (c[3] << 32), c[0] | (c[1] << 32)) for s, c in cases]
    ref = _ref_words(philox_ref_bin, triples)
    for (seed, c), want in zip(cases, ref):
        got = oracle.philox4x32_10(c[0], c[1], c[2], c[3], seed)
        assert np.array_equal(got.astype(np.uint64), want), (seed, c)


def test_philox_vectorised_equals_scalar():
    c0 = np.arange(50, dtype=np.uint64)
    batch = oracle.philox4x32_10(c0, 3, 9, 4, 12345)
    for i in range(50):
        assert np.array_equal(batch[i], oracle.philox4x32_10(i, 3, 9, 4, 12345))


def test_uniforms_are_exact_24bit():
    w = np.array([0, 255, 256, 0xFFFFFFFF, 0x80000000], dtype=np.uint64)
    u1, u2 = oracle.uniforms_from_words(w, w)
    m = (w >> np.uint64(8)).astype(np.float64)
    assert np.all(u1 * 2**24 == m + 1)
    assert np.all(u2 * 2**24 == m)
    assert u1.min() > 0 and u1.max() == 1.0
    assert u2.min() == 0.0 and u2.max() < 1.0
    # fp32 represents every value exactly
    assert np.all(u1.astype(np.float32).astype(np.float64) == u1)
    assert np.all(u2.astype(np.float32).astype(np.float64) == u2)


def test_box_muller_polar_identities():
    words = oracle.philox4x32_10(np.arange(4096, dtype=np.uint64), 1, 2, 3, 99)
    z = oracle.box_muller(words)
    for a in (0, 2):
        u1, u2 = oracle.uniforms_from_words(words[:, a], words[:, a + 1])
        r2 = z[:, a] ** 2 + z[:, a + 1] ** 2
        np.testing.assert_allclose(r2, -2.0 * np.log(u1), rtol=1e-12, atol=1e-14)
        ang = np.mod(np.arctan2(z[:, a + 1], z[:, a]), 2 * np.pi)
        want = np.mod(2 * np.pi * u2, 2 * np.pi)
        d = np.abs(ang - want)
        d = np.minimum(d, 2 * np.pi - d)
        big = r2 > 1e-12
        assert np.all(d[big] < 1e-9)


def test_normal_law_of_probes():
    P = oracle.probe_matrix(seed=5, layer=3, sample=1, p=4096, k=64)  # 262144 draws
    z = P.ravel()
    assert abs(z.mean()) < 5 / math.sqrt(z.size)
    assert abs(z.var() - 1.0) < 5 * math.sqrt(2.0 / z.size)
    assert np.abs(z).max() <= math.sqrt(2 * 24 * math.log(2)) + 1e-12
    assert stats.kstest(z, "norm").pvalue > 1e-4
    # columns and rows are uncorrelated
    corr = np.corrcoef(P[:, :8].T)
    assert np.abs(corr - np.eye(8)).max() < 5 / math.sqrt(4096)


def test_probe_layout_and_independence():
    P = oracle.probe_matrix(seed=11, layer=2, sample=3, p=10, k=5)
    for r in range(10):
        for j in range(5):
            z = oracle.normals_from_counters(r >> 2, j, 3, 2, 11)
            assert P[r, j] == z[r & 3]
    # prefix property: a smaller p is a prefix of a larger one
    P12 = oracle.probe_matrix(seed=11, layer=2, sample=3, p=12, k=5)
    assert np.array_equal(P12[:10], P)
    # samples, layers and seeds give different matrices
    assert not np.allclose(P, oracle.probe_matrix(11, 2, 4, 10, 5))
    assert not np.allclose(P, oracle.probe_matrix(11, 3, 3, 10, 5))
    assert not np.allclose(P, oracle.probe_matrix(12, 2, 3, 10, 5))


def test_noise_stream_split_equals_whole():
    whole = oracle.noise_vector(seed=77, layer=5, n=1003)
    parts = np.concatenate([oracle.noise_vector(77, 5, 1, 0), oracle.noise_vector(77, 5, 400, 1),
                            oracle.noise_vector(77, 5, 602, 401)])
    assert np.array_equal(whole, parts)
    # element e is lane e mod 4 of counter (e >> 2, 0, NOISE_C2, layer)
    for e in (0, 1, 2, 3, 4, 1002):
        z = oracle.normals_from_counters(e >> 2, 0, NOISE_C2, 5, 77)
        assert whole[e] == z[e & 3]
    big = oracle.noise_vector(77, 5, 4, offset=(1 << 34) + 8)
    z = oracle.normals_from_counters(((1 << 34) + 8) >> 2 & 0xFFFFFFFF, ((1 << 34) + 8) >> 34,
                                     NOISE_C2, 5, 77)
    assert np.array_equal(big, z)


def test_noise_law():
    xi = oracle.noise_vector(seed=3, layer=0, n=1 << 18)
    assert abs(xi.mean()) < 5 / math.sqrt(xi.size)
    assert abs(xi.var() - 1.0) < 5 * math.sqrt(2.0 / xi.size)
    assert stats.kstest(xi, "norm").pvalue > 1e-4
