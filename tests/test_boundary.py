"""The C ABI on the host (no GPU needed): the library loads, exports every
function include/dprc.h declares, and rejects bad arguments before anything
is enqueued (every case here returns before the first HIP call)."""

import ctypes
import os
import re

import pytest

from sample_gradient_clipping_amd import binding as dp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dprc.h")

FAKE = ctypes.c_void_p(0x100000)      # aligned, never dereferenced on these paths
FAKE_MIS = ctypes.c_void_p(0x100004)  # 4-byte aligned, not 16
NULL = ctypes.c_void_p(0)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(dp.lib_path()):
        pytest.fail("libdprc.so not built (run __graft_entry__.build())")
    return dp.load_library()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dp_\w+)\s*\(", text)))


def test_exports_every_declared_function(lib):
    names = _declared_functions()
    assert "dp_norm_est" in names and "dp_clip_aggregate" in names and "dp_noise_update" in names
    for n in names:
        assert hasattr(lib, n), f"{n} declared in dprc.h but not exported"


def test_abi_version_and_status_strings(lib):
    assert dp.dp_abi_version() == 4
    for s in range(5):
        assert dp.dp_status_string(s).startswith("DP_")
    assert "unknown" in dp.dp_status_string(99)


def test_workspace_queries(lib):
    assert dp.dp_norm_est_workspace("hutch", "bf16", 8, 4096, 2048, 2048, 32) > 0
    assert dp.dp_norm_est_workspace("hutch", "f32", 4, 64, 64, 64, 8) > 0
    assert dp.dp_norm_est_workspace("ghost", "f32", 4, 64, 64, 64, 0) > 0
    # invalid: k > p, k < 3 for Hutch++, bad method/dtype, negative sizes
    assert dp.dp_norm_est_workspace("hutch", "f32", 4, 64, 64, 64, 65) is None
    assert dp.dp_norm_est_workspace("hutchpp", "f32", 4, 64, 64, 64, 2) is None
    # Hutch++ column limits: s = k/3 <= 32 and r = k - 2s <= 32
    assert dp.dp_norm_est_workspace("hutchpp", "f32", 2, 64, 64, 128, 96) > 0
    assert dp.dp_norm_est_workspace("hutchpp", "f32", 2, 64, 64, 128, 95) is None
    assert dp.dp_norm_est_workspace("hutchpp", "f32", 2, 64, 64, 128, 97) is None
    assert dp.load_library().dp_norm_est_workspace(9, 0, 1, 1, 1, 1, 1) == ctypes.c_size_t(-1).value
    assert dp.load_library().dp_norm_est_workspace(0, 7, 1, 1, 1, 1, 1) == ctypes.c_size_t(-1).value
    assert dp.dp_norm_est_workspace("hutch", "f32", -1, 64, 64, 64, 8) is None
    assert dp.dp_norm_est_workspace("hutch", "f32", 4, 64, 0, 64, 8) is None
    assert dp.dp_clip_aggregate_workspace("bf16", 8, 4096, 2048, 2048) > 0
    assert dp.dp_clip_aggregate_workspace("f32", 4, 64, 0, 64) is None


def _norm(lib, method=0, dtype=0, B=2, T=8, d=8, p=8, k=4, A=FAKE, G=FAKE, flags=0, n=FAKE,
          ws=FAKE, ws_bytes=1 << 30):
    return lib.dp_norm_est(method, dtype, B, T, d, p, k, A, G, 1, 0, flags, n, ws, ws_bytes, NULL)


def test_norm_est_rejects_bad_arguments(lib):
    E, W = dp.DP_ERR_INVALID_ARG, dp.DP_ERR_WORKSPACE
    assert _norm(lib, method=7) == E
    assert _norm(lib, dtype=3) == E
    assert _norm(lib, k=0) == E
    assert _norm(lib, k=9) == E            # k > p
    assert _norm(lib, method=1, k=2) == E  # Hutch++ needs k >= 3
    assert _norm(lib, d=0) == E
    assert _norm(lib, B=-1) == E
    assert _norm(lib, flags=8) == E
    assert _norm(lib, flags=dp.DP_PROBE_RADEMACHER | 16) == E
    assert _norm(lib, A=NULL) == E
    assert _norm(lib, G=FAKE_MIS) == E
    assert _norm(lib, n=NULL) == E
    assert _norm(lib, ws=NULL) == E
    assert _norm(lib, ws_bytes=16) == W
    assert _norm(lib, B=0) == dp.DP_OK    # empty batch: nothing to do


def test_norm_est_noalloc_rejects_before_any_hip_call(lib):
    # invalid sizes, and calls whose workspace exceeds the scratch array, return
    # before the array's address is looked up
    f = lambda method=0, dtype=1, B=8, T=128, d=2048, p=2048, k=32: lib.dp_norm_est_noalloc(
        method, dtype, B, T, d, p, k, FAKE, FAKE, 1, 0, 0, FAKE, NULL)
    assert f(method=7) == dp.DP_ERR_INVALID_ARG
    assert f(k=0) == dp.DP_ERR_INVALID_ARG
    assert f(d=0) == dp.DP_ERR_INVALID_ARG
    assert dp.dp_norm_est_workspace("fgc", "bf16", 8, 128, 2048, 2048, 0) > dp.DP_NOALLOC_SCRATCH_BYTES
    assert f(method=dp.DP_NORM_FGC, k=0) == dp.DP_ERR_WORKSPACE
    assert dp.DP_NOALLOC_SCRATCH_BYTES == 64 << 20  # the header's DP_NOALLOC_SCRATCH_BYTES
    assert "((size_t)64 << 20)" in open(HEADER).read()


def _agg(lib, dtype=0, B=2, T=8, d=8, p=8, A=FAKE, G=FAKE, n=FAKE, C=1.0, S=FAKE, ws=FAKE,
         ws_bytes=1 << 30, c_out=NULL):
    return lib.dp_clip_aggregate(dtype, B, T, d, p, A, G, n, C, c_out, S, ws, ws_bytes, NULL)


def test_clip_aggregate_rejects_bad_arguments(lib):
    E = dp.DP_ERR_INVALID_ARG
    assert _agg(lib, C=0.0) == E
    assert _agg(lib, C=-1.0) == E
    assert _agg(lib, C=float("inf")) == E
    assert _agg(lib, C=float("nan")) == E
    assert _agg(lib, S=NULL) == E
    assert _agg(lib, S=FAKE_MIS) == E
    assert _agg(lib, n=NULL) == E
    assert _agg(lib, A=NULL) == E
    assert _agg(lib, dtype=5) == E
    assert _agg(lib, p=0) == E
    assert _agg(lib, c_out=ctypes.c_void_p(0x100002)) == E
    assert _agg(lib, ws_bytes=0) == dp.DP_ERR_WORKSPACE


def test_noise_update_rejects_bad_arguments(lib):
    E = dp.DP_ERR_INVALID_ARG
    f = lambda **kw: lib.dp_noise_update(kw.get("d", 8), kw.get("p", 8), kw.get("th", FAKE),
                                         kw.get("S", ctypes.c_void_p(0x200000)),
                                         kw.get("sigma", 1.0), kw.get("C", 1.0),
                                         kw.get("eta", 0.1), kw.get("B", 4), 1, 0, NULL)
    assert f(B=0) == E
    assert f(sigma=-1.0) == E
    assert f(sigma=float("nan")) == E
    assert f(C=0.0) == E
    assert f(eta=float("inf")) == E
    assert f(d=0) == E
    assert f(th=NULL) == E
    assert f(th=FAKE_MIS) == E
    assert f(S=ctypes.c_void_p(0x100000 + 64)) == E  # overlaps theta


def _aggu(lib, dtype=0, B=2, T=8, d=8, p=8, A=FAKE, G=FAKE, n=FAKE, C=1.0, sigma=1.0, eta=0.1,
          th=ctypes.c_void_p(0x400000), S=NULL, ws=ctypes.c_void_p(0x800000), ws_bytes=1 << 20):
    return lib.dp_clip_aggregate_update(dtype, B, T, d, p, A, G, n, C, sigma, eta, 1, 0, th, S,
                                        NULL, ws, ws_bytes, NULL)


def test_clip_aggregate_update_rejects_bad_arguments(lib):
    E = dp.DP_ERR_INVALID_ARG
    assert _aggu(lib, B=0) == E                      # |B| = 0 has no update
    assert _aggu(lib, C=0.0) == E
    assert _aggu(lib, sigma=-1.0) == E
    assert _aggu(lib, eta=float("nan")) == E
    assert _aggu(lib, th=NULL) == E
    assert _aggu(lib, th=ctypes.c_void_p(0x400004)) == E   # misaligned theta
    assert _aggu(lib, S=ctypes.c_void_p(0x400000 + 64)) == E  # S overlaps theta
    assert _aggu(lib, ws=ctypes.c_void_p(0x400000 + 64)) == E  # workspace overlaps theta
    assert _aggu(lib, n=NULL) == E
    assert _aggu(lib, d=0) == E
    assert _aggu(lib, ws_bytes=0) == dp.DP_ERR_WORKSPACE
    need = dp.dp_clip_aggregate_update_workspace("f32", 2, 8, 8, 8)
    assert need >= dp.dp_clip_aggregate_workspace("f32", 2, 8, 8, 8) + 8 * 8 * 4
    assert dp.dp_clip_aggregate_update_workspace("f32", 2, 8, 0, 8) is None


def _layers(specs):
    """ctypes dp_linear_layer_t array from (d, p, layer, A, G, theta) with raw addresses."""
    arr = (dp.DpLinearLayer * len(specs))()
    for i, (d, p, lid, A, G, th) in enumerate(specs):
        arr[i].d, arr[i].p, arr[i].layer = d, p, lid
        arr[i].A, arr[i].G, arr[i].theta = A, G, th
    return arr


def test_batched_workspace_queries(lib):
    SZ = ctypes.c_size_t(-1).value
    two = _layers([(2048, 2048, 0, 0x100000, 0x100000, None), (2048, 512, 1, 0x100000, 0x100000, None)])
    # fused Hutch: the probes of both layers, one Y buffer, the partial row per sample
    n = lib.dp_norm_est_layers_workspace(0, 1, 8, 4096, 32, 2, two)
    assert n >= 8 * 32 * (2048 + 512) * 2 + 8 * 32 * 4096 * 2
    # the per-layer fallback needs the largest per-layer workspace
    n = lib.dp_norm_est_layers_workspace(0, 0, 4, 64, 8, 2, two)
    assert n == max(dp.dp_norm_est_workspace("hutch", "f32", 4, 64, 2048, 2048, 8),
                    dp.dp_norm_est_workspace("hutch", "f32", 4, 64, 2048, 512, 8))
    assert lib.dp_norm_est_layers_workspace(0, 1, 8, 4096, 32, 0, two) == SZ    # no layers
    assert lib.dp_norm_est_layers_workspace(0, 1, 8, 4096, 32, 2, None) == SZ
    assert lib.dp_norm_est_layers_workspace(0, 1, 8, 4096, 600, 2, two) == SZ  # k > p of layer 1
    bad = _layers([(2048, 2048, 0, 0x100000, 0x100000, None), (0, 512, 1, 0x100000, 0x100000, None)])
    assert lib.dp_norm_est_layers_workspace(0, 1, 8, 4096, 32, 2, bad) == SZ
    u = lib.dp_clip_aggregate_update_layers_workspace(1, 8, 4096, 2, two)
    assert u == max(dp.dp_clip_aggregate_update_workspace("bf16", 8, 4096, 2048, 2048),
                    dp.dp_clip_aggregate_update_workspace("bf16", 8, 4096, 2048, 512))
    assert lib.dp_clip_aggregate_update_layers_workspace(1, 8, 4096, 0, two) == SZ
    assert lib.dp_clip_aggregate_update_layers_workspace(1, 8, 4096, 2, bad) == SZ
    # 64- and 16-tile layers with no partner of their tile count: two launches
    assert lib.dp_clip_aggregate_update_layers_launches(1, 8, 4096, 2, two) == 2
    assert lib.dp_clip_aggregate_update_layers_launches(1, 8, 4096, 0, two) == -1
    assert lib.dp_clip_aggregate_update_layers_launches(1, 8, 4096, 2, bad) == -1


def test_batched_update_groups_small_contractions(lib):
    # layers whose 256 x 256 tile count divides 256 share launches, 256 / tiles per
    # launch: a full group is unsplit and needs one p x d fp32 sum per layer
    F = 0x100000
    qo = [(2048, 2048, i, F, F, None) for i in range(4)]      # 64 tiles each
    kv = [(2048, 512, 10 + i, F, F, None) for i in range(16)]  # 16 tiles each
    per_q = dp.dp_clip_aggregate_update_workspace("bf16", 8, 4096, 2048, 2048)
    for specs, one in ((qo, 2048 * 2048 * 4), (kv, 2048 * 512 * 4)):
        arr = _layers(specs)
        assert lib.dp_clip_aggregate_update_layers_launches(1, 8, 4096, len(specs), arr) == 1
        u = lib.dp_clip_aggregate_update_layers_workspace(1, 8, 4096, len(specs), arr)
        assert len(specs) * one <= u < len(specs) * one + 4096
    assert lib.dp_clip_aggregate_update_layers_workspace(1, 8, 4096, 4, _layers(qo)) < per_q
    # the stack's order: q k v o per block, then gate up down (256 tiles, never grouped)
    block = lambda b: [(2048, 2048, 0, F, F, None), (2048, 512, 1, F, F, None),
                       (2048, 512, 2, F, F, None), (2048, 2048, 3, F, F, None),
                       (2048, 8192, 4, F, F, None), (2048, 8192, 5, F, F, None),
                       (8192, 2048, 6, F, F, None)]
    stack = [ly for b in range(16) for ly in block(b)]
    assert lib.dp_clip_aggregate_update_layers_launches(1, 8, 4096, 112, _layers(stack)) == 8 + 2 + 48
    # a fifth 64-tile layer has no partner: the per-layer path and its workspace
    five = qo + [(2048, 2048, 9, F, F, None)]
    assert lib.dp_clip_aggregate_update_layers_launches(1, 8, 4096, 5, _layers(five)) == 2
    assert lib.dp_clip_aggregate_update_layers_workspace(1, 8, 4096, 5, _layers(five)) == per_q
    # fp32 layers never share a launch
    assert lib.dp_clip_aggregate_update_layers_launches(0, 8, 4096, 4, _layers(qo)) == 4


def test_batched_calls_reject_bad_arguments(lib):
    E, W = dp.DP_ERR_INVALID_ARG, dp.DP_ERR_WORKSPACE
    ok = [(8, 8, 0, 0x100000, 0x100000, 0x400000), (8, 8, 1, 0x100000, 0x100000, 0x500000)]
    norm = lambda specs, n=FAKE, flags=0, ws=FAKE, ws_bytes=1 << 30, k=4, nl=None: \
        lib.dp_norm_est_layers(0, 0, 2, 8, k, len(specs) if nl is None else nl, _layers(specs),
                               1, flags, n, ws, ws_bytes, NULL)
    assert norm(ok, nl=0) == E
    assert norm(ok, k=9) == E                                   # k > p
    assert norm(ok, flags=8) == E
    assert norm(ok, n=NULL) == E
    assert norm([ok[0], (8, 8, 1, 0, 0x100000, None)]) == E     # layer 1 has no A
    assert norm([ok[0], (8, 8, 1, 0x100004, 0x100000, None)]) == E  # misaligned A
    assert norm(ok, ws_bytes=16) == W
    upd = lambda specs, n=FAKE, C=1.0, sigma=1.0, ws=ctypes.c_void_p(0x800000), ws_bytes=1 << 20: \
        lib.dp_clip_aggregate_update_layers(0, 2, 8, len(specs), _layers(specs), n, C, sigma, 0.1,
                                            1, NULL, ws, ws_bytes, NULL)
    assert upd(ok, C=0.0) == E
    assert upd(ok, sigma=-1.0) == E
    assert upd(ok, n=NULL) == E
    assert upd([ok[0], (8, 8, 1, 0x100000, 0x100000, None)]) == E        # no theta
    assert upd([ok[0], (8, 8, 1, 0x100000, 0x100000, 0x400000 + 64)]) == E  # thetas overlap
    assert upd(ok, ws=ctypes.c_void_p(0x500000)) == E                     # ws overlaps a theta
    assert upd(ok, ws_bytes=0) == W


def test_stream_read_rejects_bad_arguments(lib):
    E = dp.DP_ERR_INVALID_ARG
    f = lambda buf=FAKE, nbytes=1024, out=FAKE, nblocks=4: lib.dp_stream_read(buf, nbytes, out, nblocks, NULL)
    assert f(nbytes=0) == dp.DP_OK
    assert f(buf=NULL) == E
    assert f(buf=FAKE_MIS) == E
    assert f(out=NULL) == E
    assert f(nbytes=1000) == E       # not a multiple of 16
    assert f(nblocks=0) == E
    assert f(nblocks=65537) == E


def test_read_device_status_rejects_bad_arguments(lib):
    E = dp.DP_ERR_INVALID_ARG
    flags = ctypes.c_uint32(77)
    assert lib.dp_read_device_status(NULL, ctypes.byref(flags), NULL) == E
    assert lib.dp_read_device_status(FAKE, None, NULL) == E
    assert lib.dp_read_device_status(FAKE_MIS, ctypes.byref(flags), NULL) == E
    assert flags.value == 77  # untouched on an argument error


def test_clip_workspaces_hold_the_status_word(lib):
    # the status word sits in the first 8 bytes, so every clip workspace has them
    assert dp.dp_clip_aggregate_workspace("f32", 1, 1, 1, 1) >= 8
    assert dp.dp_clip_aggregate_update_workspace("f32", 1, 1, 1, 1) >= 8
    assert lib.dp_rmsnorm_update_workspace(1, 1) >= 8
    assert lib.dp_embedding_update_workspace(0, 1, 0, 1, 1) >= 8


def test_test_hooks_reject_bad_arguments(lib):
    E = dp.DP_ERR_INVALID_ARG
    assert lib.dp_philox_u32(1, NULL, FAKE, 4, NULL) == E
    assert lib.dp_philox_u32(1, FAKE, FAKE, 0, NULL) == dp.DP_OK
    assert lib.dp_probe_fill(1, 0, 0, 0, 4, FAKE, NULL) == E
    assert lib.dp_probe_fill(1, 0, 0, 4, 4, NULL, NULL) == E
    assert lib.dp_noise_fill(1, 0, 0, 4, NULL, NULL) == E
    assert lib.dp_probe_fill_ex(1, 0, 0, 4, 4, 8, FAKE, NULL) == E  # unknown flag
    assert lib.dp_probe_fill_ex(1, 0, 0, 4, 4, dp.DP_PROBE_SHARED, FAKE, NULL) == E
    assert lib.dp_probe_fill_ex(1, 0, 0, 0, 4, dp.DP_PROBE_RADEMACHER, FAKE, NULL) == E
    assert lib.dp_noise_fill(1, 0, 2**64 - 2, 4, FAKE, NULL) == E


def test_poisson_sample_rejects_bad_arguments(lib):
    E, W = dp.DP_ERR_INVALID_ARG, dp.DP_ERR_WORKSPACE
    assert dp.dp_poisson_sample_workspace(0) > 0
    assert dp.dp_poisson_sample_workspace(4096) == 8
    assert dp.dp_poisson_sample_workspace(4097) == 16
    assert dp.dp_poisson_sample_workspace(-1) is None
    assert dp.dp_poisson_sample_workspace((1 << 40) + 1) is None

    def call(N=10, q=0.5, idx=FAKE, cap=4, count=FAKE, ws=FAKE, ws_bytes=1 << 20):
        return lib.dp_poisson_sample(1, 0, N, q, idx, cap, count, ws, ws_bytes, NULL)

    assert call(N=-1) == E
    assert call(q=-0.1) == E
    assert call(q=1.5) == E
    assert call(q=float("nan")) == E
    assert call(cap=-1) == E
    assert call(idx=NULL) == E            # capacity without a buffer
    assert call(count=NULL) == E
    assert call(count=FAKE_MIS) == E      # int64 needs 8-byte alignment
    assert call(ws=NULL) == E
    assert call(ws_bytes=0) == W


def test_rmsnorm_entry_points_reject_bad_arguments(lib):
    E, W = dp.DP_ERR_INVALID_ARG, dp.DP_ERR_WORKSPACE
    assert lib.dp_rmsnorm_norm_workspace(0, 2, 8, 8) > 0
    assert lib.dp_rmsnorm_norm_workspace(5, 2, 8, 8) == ctypes.c_size_t(-1).value
    assert lib.dp_rmsnorm_norm_workspace(0, 2, 8, 0) == ctypes.c_size_t(-1).value

    def norm(dtype=0, B=2, T=8, d=8, x=FAKE, dl=FAKE, flags=0, n=FAKE, v=NULL, ws=FAKE,
             ws_bytes=1 << 20):
        return lib.dp_rmsnorm_norm(dtype, B, T, d, x, dl, flags, n, v, ws, ws_bytes, NULL)

    assert norm(dtype=3) == E
    assert norm(flags=dp.DP_PROBE_SHARED) == E   # only DP_ACCUMULATE applies
    assert norm(x=FAKE_MIS) == E
    assert norm(n=NULL) == E
    assert norm(ws=NULL) == E
    assert norm(ws_bytes=0) == W

    def upd(B=2, d=8, v=FAKE, n=FAKE, C=1.0, sigma=1.0, eta=0.1, gamma=FAKE, ws=FAKE,
            ws_bytes=1 << 20):
        return lib.dp_rmsnorm_clip_aggregate_update(B, d, v, n, C, sigma, eta, 1, 0, gamma, NULL,
                                                    NULL, ws, ws_bytes, NULL)

    assert upd(B=0) == E
    assert upd(C=0.0) == E
    assert upd(sigma=-1.0) == E
    assert upd(gamma=FAKE_MIS) == E
    assert upd(v=NULL) == E
    assert upd(ws_bytes=0) == W


def test_embedding_entry_points_reject_bad_arguments(lib):
    E, W = dp.DP_ERR_INVALID_ARG, dp.DP_ERR_WORKSPACE
    inv = ctypes.c_size_t(-1).value
    assert lib.dp_embedding_norm_workspace(0, 2, 16384, 8) > 0
    assert lib.dp_embedding_norm_workspace(0, 2, 16385, 8) == inv   # the per-sample sort's limit
    assert lib.dp_embedding_update_workspace(0, 2, 8, 8, 0) == inv

    def norm(dtype=0, B=2, T=8, d=8, ids=FAKE, dl=FAKE, flags=0, n=FAKE, ws=FAKE,
             ws_bytes=1 << 20):
        return lib.dp_embedding_norm(dtype, B, T, d, ids, dl, flags, n, ws, ws_bytes, NULL)

    assert norm(T=16385) == E
    assert norm(flags=dp.DP_PROBE_RADEMACHER) == E
    assert norm(ids=NULL) == E
    assert norm(dl=FAKE_MIS) == E
    assert norm(ws_bytes=0) == W

    def upd(B=2, T=8, d=8, V=16, C=1.0, Ep=FAKE, ws_bytes=1 << 20):
        return lib.dp_embedding_clip_aggregate_update(0, B, T, d, V, FAKE, FAKE, FAKE, C, 1.0, 0.1,
                                                      1, 0, Ep, NULL, FAKE, ws_bytes, NULL)

    assert upd(V=0) == E
    assert upd(B=0) == E
    assert upd(C=-1.0) == E
    assert upd(Ep=FAKE_MIS) == E
    assert upd(ws_bytes=16) == W


def _addr(i):
    """Distinct, well separated fake device addresses (never dereferenced)."""
    return ctypes.c_void_p(0x10000000 + i * 0x10000000)


def test_mlp_block_entry_points_reject_bad_arguments(lib):
    E = dp.DP_ERR_INVALID_ARG
    assert lib.dp_weights_bf16(64, 100, FAKE, _addr(1), _addr(2), NULL) == E     # d % 64
    assert lib.dp_weights_bf16(0, 64, FAKE, FAKE, FAKE, NULL) == dp.DP_OK       # empty: no-op
    assert lib.dp_weights_bf16(64, 64, FAKE_MIS, _addr(1), _addr(2), NULL) == E
    assert lib.dp_weights_bf16(64, 64, _addr(0), _addr(1), _addr(1), NULL) == E  # W, Wt overlap

    def lin(M=512, N=256, K=64, A=_addr(0), W=_addr(1), R=NULL, C=_addr(2)):
        return lib.dp_linear_forward(M, N, K, A, W, R, C, NULL)

    assert lin(N=300) == E
    assert lin(K=48) == E
    assert lin(M=-1) == E
    assert lin(M=0) == dp.DP_OK
    assert lin(C=_addr(0)) == E                           # C overlaps A
    assert lin(A=FAKE_MIS) == E
    assert lin(R=ctypes.c_void_p(_addr(2).value + 2)) == E  # residual overlaps C, not equal

    def fwd(B=2, T=128, d=256, f=512, eps=1e-5, out=_addr(11), x=_addr(0)):
        return lib.dp_mlp_forward(B, T, d, f, eps, x, _addr(1), _addr(2), _addr(3), _addr(4),
                                  _addr(5), _addr(6), _addr(7), _addr(8), _addr(9), _addr(10), out,
                                  NULL)

    assert fwd(d=200) == E
    assert fwd(f=384) == E
    assert fwd(eps=-1.0) == E
    assert fwd(eps=float("nan")) == E
    assert fwd(out=_addr(5)) == E                         # out overlaps xhat
    assert fwd(B=0) == dp.DP_OK

    def bwd(B=2, T=128, d=256, f=512, dx=_addr(16), G=_addr(13)):
        return lib.dp_mlp_backward(B, T, d, f, _addr(0), _addr(1), _addr(2), _addr(3), _addr(4),
                                   _addr(5), _addr(6), _addr(7), _addr(8), G, _addr(14), _addr(15),
                                   dx, NULL)

    assert bwd(d=128) == E
    assert bwd(dx=_addr(8)) == E                          # dx overlaps dout
    assert bwd(G=FAKE_MIS) == E
    assert bwd(T=0) == dp.DP_OK


def test_kernel_path_queries(lib):
    """Which kernels serve a call, decided on the host: the MFMA kernels for bf16
    on their tiles, the generic ones otherwise, -1 for invalid arguments."""
    # the stack's shapes and the long-context layer take the MFMA kernels
    for method, k in (("hutch", 32), ("hutchpp", 32), ("ghost", 0), ("fgc", 0)):
        assert dp.dp_norm_est_uses_mfma(method, "bf16", 8, 4096, 2048, 8192, k) == 1
        assert dp.dp_norm_est_uses_mfma(method, "bf16", 2, 16384, 2048, 8192, k) == 1
    assert dp.dp_clip_aggregate_uses_mfma("bf16", 8, 4096, 8192, 2048) == 1
    # fp32, more than 32 probes, off-tile widths and token counts: generic
    assert dp.dp_norm_est_uses_mfma("hutch", "f32", 8, 4096, 2048, 2048, 32) == 0
    assert dp.dp_norm_est_uses_mfma("hutch", "bf16", 8, 4096, 2048, 2048, 48) == 0
    assert dp.dp_norm_est_uses_mfma("hutch", "bf16", 8, 4096, 2048, 2000, 32) == 0
    assert dp.dp_norm_est_uses_mfma("fgc", "bf16", 8, 4000, 2048, 2048, 0) == 0
    assert dp.dp_norm_est_uses_mfma("ghost", "bf16", 4, 64, 64, 64, 0) == 0
    assert dp.dp_clip_aggregate_uses_mfma("f32", 4, 64, 64, 64) == 0
    assert dp.dp_clip_aggregate_uses_mfma("bf16", 8, 4096, 2048, 2000) == 0
    # invalid arguments
    assert dp.dp_norm_est_uses_mfma("hutch", "bf16", 8, 4096, 2048, 2048, 0) == -1
    assert dp.dp_norm_est_uses_mfma("hutchpp", "bf16", 8, 4096, 2048, 2048, 2) == -1
    assert dp.dp_clip_aggregate_uses_mfma("bf16", -1, 4096, 2048, 2048) == -1
