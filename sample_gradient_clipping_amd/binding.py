"""ctypes binding of libdprc.so: the C ABI of include/dprc.h with the same names.

Argument marshalling only.  Tensors are torch tensors on the GPU (torch is
used for device memory and streams); every step of the computation runs in
the library's HIP kernels.  Work is enqueued on torch's current stream.  If
the library is missing, loading raises: there is no fallback.
"""

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))

DP_OK, DP_ERR_INVALID_ARG, DP_ERR_UNSUPPORTED, DP_ERR_WORKSPACE, DP_ERR_HIP = range(5)
DP_F32, DP_BF16 = 0, 1
DP_NORM_HUTCH, DP_NORM_HUTCHPP, DP_NORM_GHOST, DP_NORM_FGC = range(4)
DP_ACCUMULATE = 1
DP_PROBE_SHARED = 2
DP_PROBE_RADEMACHER = 4
DP_STATUS_NONFINITE_NORM = 1
METHODS = {"hutch": DP_NORM_HUTCH, "hutchpp": DP_NORM_HUTCHPP, "ghost": DP_NORM_GHOST,
           "fgc": DP_NORM_FGC}
_SIZE_INVALID = ctypes.c_size_t(-1).value


class DprcError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {dp_status_string(status)} (status {status})")


_lib = None


def lib_path():
    return os.environ.get("DPRC_LIB", os.path.join(_PKG, "libdprc.so"))


class DpLinearLayer(ctypes.Structure):
    """dp_linear_layer_t: one linear layer of a batched call."""
    _fields_ = [("d", ctypes.c_int), ("p", ctypes.c_int), ("layer", ctypes.c_uint32),
                ("A", ctypes.c_void_p), ("G", ctypes.c_void_p), ("theta", ctypes.c_void_p)]


def _layer_array(layers):
    """ctypes array of dp_linear_layer_t from (A, G, layer_id[, theta]) tuples."""
    arr = (DpLinearLayer * len(layers))()
    for i, ly in enumerate(layers):
        A, G, lid = ly[0], ly[1], ly[2]
        theta = ly[3] if len(ly) > 3 else None
        arr[i].d = A.shape[2]
        arr[i].p = G.shape[2]
        arr[i].layer = int(lid)
        arr[i].A = A.data_ptr()
        arr[i].G = G.data_ptr()
        arr[i].theta = None if theta is None else theta.data_ptr()
    return arr


def load_library():
    """Load libdprc.so once and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    path = lib_path()
    if not os.path.exists(path):
        raise FileNotFoundError(
            f"{path} is missing: build it with `python -m sample_gradient_clipping_amd.build`")
    L = ctypes.CDLL(path)
    c_int, c_u32, c_u64, c_sz, c_f, c_p = (ctypes.c_int, ctypes.c_uint32, ctypes.c_uint64,
                                           ctypes.c_size_t, ctypes.c_float, ctypes.c_void_p)
    L.dp_abi_version.restype = c_int
    L.dp_norm_est_uses_mfma.argtypes = [c_int] * 7
    L.dp_norm_est_uses_mfma.restype = c_int
    L.dp_clip_aggregate_uses_mfma.argtypes = [c_int] * 5
    L.dp_clip_aggregate_uses_mfma.restype = c_int
    L.dp_status_string.argtypes = [c_int]
    L.dp_status_string.restype = ctypes.c_char_p
    L.dp_norm_est_workspace.argtypes = [c_int] * 7
    L.dp_norm_est_workspace.restype = c_sz
    L.dp_norm_est.argtypes = [c_int] * 7 + [c_p, c_p, c_u64, c_u32, c_u32, c_p, c_p, c_sz, c_p]
    L.dp_norm_est.restype = c_int
    L.dp_norm_est_noalloc.argtypes = [c_int] * 7 + [c_p, c_p, c_u64, c_u32, c_u32, c_p, c_p]
    L.dp_norm_est_noalloc.restype = c_int
    L.dp_clip_aggregate_workspace.argtypes = [c_int] * 5
    L.dp_clip_aggregate_workspace.restype = c_sz
    L.dp_clip_aggregate.argtypes = [c_int] * 5 + [c_p, c_p, c_p, c_f, c_p, c_p, c_p, c_sz, c_p]
    L.dp_clip_aggregate.restype = c_int
    L.dp_noise_update.argtypes = [c_int, c_int, c_p, c_p, c_f, c_f, c_f, c_int, c_u64, c_u32, c_p]
    L.dp_noise_update.restype = c_int
    L.dp_norm_est_timed.argtypes = L.dp_norm_est.argtypes + [c_p, c_p]
    L.dp_norm_est_timed.restype = c_int
    L.dp_clip_aggregate_timed.argtypes = L.dp_clip_aggregate.argtypes + [c_p, c_p]
    L.dp_clip_aggregate_timed.restype = c_int
    L.dp_noise_update_timed.argtypes = L.dp_noise_update.argtypes + [c_p, c_p]
    L.dp_noise_update_timed.restype = c_int
    L.dp_clip_aggregate_update_workspace.argtypes = [c_int] * 5
    L.dp_clip_aggregate_update_workspace.restype = c_sz
    L.dp_clip_aggregate_update.argtypes = ([c_int] * 5 + [c_p, c_p, c_p, c_f, c_f, c_f, c_u64, c_u32]
                                           + [c_p, c_p, c_p, c_p, c_sz, c_p])
    L.dp_clip_aggregate_update.restype = c_int
    L.dp_read_device_status.argtypes = [c_p, ctypes.POINTER(c_u32), c_p]
    L.dp_read_device_status.restype = c_int
    L.dp_clip_aggregate_update_timed.argtypes = L.dp_clip_aggregate_update.argtypes + [c_p] * 4
    L.dp_clip_aggregate_update_timed.restype = c_int
    LP = ctypes.POINTER(DpLinearLayer)
    L.dp_norm_est_layers_workspace.argtypes = [c_int] * 6 + [LP]
    L.dp_norm_est_layers_workspace.restype = c_sz
    L.dp_norm_est_layers.argtypes = [c_int] * 6 + [LP, c_u64, c_u32, c_p, c_p, c_sz, c_p]
    L.dp_norm_est_layers.restype = c_int
    L.dp_norm_est_layers_timed.argtypes = L.dp_norm_est_layers.argtypes + [c_p, c_p]
    L.dp_norm_est_layers_timed.restype = c_int
    L.dp_clip_aggregate_update_layers_workspace.argtypes = [c_int] * 4 + [LP]
    L.dp_clip_aggregate_update_layers_workspace.restype = c_sz
    L.dp_clip_aggregate_update_layers_launches.argtypes = [c_int] * 4 + [LP]
    L.dp_clip_aggregate_update_layers_launches.restype = c_int
    L.dp_clip_aggregate_update_layers.argtypes = ([c_int] * 4 + [LP, c_p, c_f, c_f, c_f, c_u64, c_p,
                                                                 c_p, c_sz, c_p])
    L.dp_clip_aggregate_update_layers.restype = c_int
    L.dp_clip_aggregate_update_layers_timed.argtypes = (L.dp_clip_aggregate_update_layers.argtypes
                                                        + [ctypes.POINTER(c_p)] * 4)
    L.dp_clip_aggregate_update_layers_timed.restype = c_int
    L.dp_stream_read.argtypes = [c_p, c_sz, c_p, c_int, c_p]
    L.dp_stream_read.restype = c_int
    L.dp_philox_u32.argtypes = [c_u64, c_p, c_p, c_sz, c_p]
    L.dp_philox_u32.restype = c_int
    L.dp_probe_fill.argtypes = [c_u64, c_u32, c_u32, c_int, c_int, c_p, c_p]
    L.dp_probe_fill.restype = c_int
    L.dp_probe_fill_ex.argtypes = [c_u64, c_u32, c_u32, c_int, c_int, c_u32, c_p, c_p]
    L.dp_probe_fill_ex.restype = c_int
    L.dp_noise_fill.argtypes = [c_u64, c_u32, c_u64, c_sz, c_p, c_p]
    L.dp_noise_fill.restype = c_int
    c_i64, c_dbl = ctypes.c_int64, ctypes.c_double
    L.dp_poisson_sample_workspace.argtypes = [c_i64]
    L.dp_poisson_sample_workspace.restype = c_sz
    L.dp_poisson_sample.argtypes = [c_u64, c_u32, c_i64, c_dbl, c_p, c_i64, c_p, c_p, c_sz, c_p]
    L.dp_poisson_sample.restype = c_int
    L.dp_rmsnorm_norm_workspace.argtypes = [c_int] * 4
    L.dp_rmsnorm_norm_workspace.restype = c_sz
    L.dp_rmsnorm_norm.argtypes = [c_int] * 4 + [c_p, c_p, c_u32, c_p, c_p, c_p, c_sz, c_p]
    L.dp_rmsnorm_norm.restype = c_int
    L.dp_rmsnorm_update_workspace.argtypes = [c_int, c_int]
    L.dp_rmsnorm_update_workspace.restype = c_sz
    L.dp_rmsnorm_clip_aggregate_update.argtypes = [c_int, c_int, c_p, c_p, c_f, c_f, c_f, c_u64,
                                                   c_u32, c_p, c_p, c_p, c_p, c_sz, c_p]
    L.dp_rmsnorm_clip_aggregate_update.restype = c_int
    L.dp_embedding_norm_workspace.argtypes = [c_int] * 4
    L.dp_embedding_norm_workspace.restype = c_sz
    L.dp_embedding_norm.argtypes = [c_int] * 4 + [c_p, c_p, c_u32, c_p, c_p, c_sz, c_p]
    L.dp_embedding_norm.restype = c_int
    L.dp_embedding_update_workspace.argtypes = [c_int] * 5
    L.dp_embedding_update_workspace.restype = c_sz
    L.dp_embedding_clip_aggregate_update.argtypes = ([c_int] * 5 + [c_p, c_p, c_p, c_f, c_f, c_f,
                                                                    c_u64, c_u32, c_p, c_p, c_p,
                                                                    c_sz, c_p])
    L.dp_embedding_clip_aggregate_update.restype = c_int
    L.dp_weights_bf16.argtypes = [c_int, c_int, c_p, c_p, c_p, c_p]
    L.dp_weights_bf16.restype = c_int
    L.dp_linear_forward.argtypes = [c_i64, c_int, c_int, c_p, c_p, c_p, c_p, c_p]
    L.dp_linear_forward.restype = c_int
    L.dp_mlp_forward.argtypes = [c_int] * 4 + [c_f] + [c_p] * 12 + [c_p]
    L.dp_mlp_forward.restype = c_int
    L.dp_mlp_backward.argtypes = [c_int] * 4 + [c_p] * 13 + [c_p]
    L.dp_mlp_backward.restype = c_int
    L.dp_rope.argtypes = [c_i64, c_int, c_int, c_dbl, c_int, c_p, c_p]
    L.dp_rope.restype = c_int
    L.dp_attention_forward.argtypes = [c_int] * 4 + [c_p] * 6
    L.dp_attention_forward.restype = c_int
    L.dp_attn_forward.argtypes = [c_int] * 5 + [c_f, c_dbl] + [c_p] * 15 + [c_p]
    L.dp_attn_forward.restype = c_int
    L.dp_attention_backward_workspace.argtypes = [c_int] * 3
    L.dp_attention_backward_workspace.restype = c_sz
    L.dp_attention_backward.argtypes = [c_int] * 4 + [c_p] * 10 + [c_sz, c_p]
    L.dp_attention_backward.restype = c_int
    L.dp_attn_backward_workspace.argtypes = [c_int] * 3
    L.dp_attn_backward_workspace.restype = c_sz
    L.dp_attn_backward.argtypes = [c_int] * 5 + [c_dbl] + [c_p] * 19 + [c_sz, c_p]
    L.dp_attn_backward.restype = c_int
    _lib = L
    return L


def dp_abi_version():
    return load_library().dp_abi_version()


def dp_norm_est_uses_mfma(method, dtype, B, T, d, p, k):
    """1 if the MFMA kernels serve this dp_norm_est call, 0 if the generic ones, -1 if invalid."""
    return load_library().dp_norm_est_uses_mfma(_method_code(method), _dtype_name_code(dtype), B, T,
                                                d, p, k)


def dp_clip_aggregate_uses_mfma(dtype, B, T, d, p):
    """1 if the MFMA contraction serves this dp_clip_aggregate call, 0 if the generic one, -1 if invalid."""
    return load_library().dp_clip_aggregate_uses_mfma(_dtype_name_code(dtype), B, T, d, p)


def dp_status_string(status):
    return load_library().dp_status_string(int(status)).decode()


def _check(status, where):
    if status != DP_OK:
        raise DprcError(status, where)


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _event(ev):
    """Raw hipEvent_t of a torch.cuda.Event (recorded once so that it exists)."""
    if ev is None:
        return None
    if ev.cuda_event == 0:
        ev.record()
    return ctypes.c_void_p(ev.cuda_event)


def _dtype_code(t):
    if t.dtype == torch.float32:
        return DP_F32
    if t.dtype == torch.bfloat16:
        return DP_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _method_code(method):
    return METHODS[method] if isinstance(method, str) else int(method)


def _dtype_name_code(dtype):
    return dtype if isinstance(dtype, int) else {"f32": DP_F32, "bf16": DP_BF16}[dtype]


def _workspace(nbytes, device, ws, zeroed=False):
    """The caller's workspace, or a new one of nbytes (zeroed for the calls that
    keep a status word in it)."""
    if nbytes == _SIZE_INVALID:
        return None
    if ws is not None:
        return ws
    alloc = torch.zeros if zeroed else torch.empty
    return alloc(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def clip_workspace(nbytes, device):
    """A zeroed workspace for the calls that form clip factors (its first word is
    the sticky status word read by dp_read_device_status)."""
    return torch.zeros(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def dp_read_device_status(ws, stream=None):
    """The DP_STATUS_* flags ORed into ``ws`` by the clip-factor calls since the
    last read; clears them.  Synchronises the stream."""
    flags = ctypes.c_uint32(0)
    _check(load_library().dp_read_device_status(_ptr(ws), ctypes.byref(flags), _stream(stream)),
           "dp_read_device_status")
    return int(flags.value)


def dp_norm_est_workspace(method, dtype, B, T, d, p, k):
    """Workspace bytes, or None for invalid arguments."""
    code = dtype if isinstance(dtype, int) else {"f32": DP_F32, "bf16": DP_BF16}[dtype]
    n = load_library().dp_norm_est_workspace(_method_code(method), code, B, T, d, p, k)
    return None if n == _SIZE_INVALID else n


def dp_norm_est(method, A, G, k, seed, layer, n_sq, flags=0, ws=None, stream=None, events=None):
    """n_sq[i] (=, or += with DP_ACCUMULATE) squared-norm estimate of sample i.

    A [B][T][d], G [B][T][p]: contiguous device tensors, fp32 or bf16.
    n_sq: fp32 [B] device tensor.  ``ws``: optional uint8 device workspace.
    ``events``: optional (begin, end) torch.cuda.Event pair -> dp_norm_est_timed.
    """
    L = load_library()
    B, T, d = A.shape
    p = G.shape[2]
    dt = _dtype_code(A)
    m = _method_code(method)
    k = int(k or 0)
    nbytes = L.dp_norm_est_workspace(m, dt, B, T, d, p, k)
    ws_t = _workspace(nbytes, A.device, ws)
    args = [m, dt, B, T, d, p, k, _ptr(A), _ptr(G), int(seed) & (2**64 - 1), int(layer),
            int(flags), _ptr(n_sq), _ptr(ws_t), 0 if ws_t is None else ws_t.numel(),
            _stream(stream)]
    if events is None:
        st = L.dp_norm_est(*args)
    else:
        st = L.dp_norm_est_timed(*args, _event(events[0]), _event(events[1]))
    _check(st, "dp_norm_est")
    return n_sq


DP_NOALLOC_SCRATCH_BYTES = 64 << 20


def dp_norm_est_noalloc(method, A, G, k, seed, layer, n_sq, flags=0, stream=None):
    """dp_norm_est on the library's own per-GPU scratch array (no workspace, no
    allocation); raises DprcError(DP_ERR_WORKSPACE) when the call needs more
    than DP_NOALLOC_SCRATCH_BYTES."""
    L = load_library()
    B, T, d = A.shape
    p = G.shape[2]
    st = L.dp_norm_est_noalloc(_method_code(method), _dtype_code(A), B, T, d, p, int(k or 0),
                               _ptr(A), _ptr(G), int(seed) & (2**64 - 1), int(layer), int(flags),
                               _ptr(n_sq), _stream(stream))
    _check(st, "dp_norm_est_noalloc")
    return n_sq


def dp_clip_aggregate_workspace(dtype, B, T, d, p):
    code = dtype if isinstance(dtype, int) else {"f32": DP_F32, "bf16": DP_BF16}[dtype]
    n = load_library().dp_clip_aggregate_workspace(code, B, T, d, p)
    return None if n == _SIZE_INVALID else n


def dp_clip_aggregate(A, G, n_sq, C, S, c_out=None, ws=None, stream=None, events=None):
    """Clip factors from n_sq and S[o][q] = sum_i c_i sum_t G_i[t][o] A_i[t][q]."""
    L = load_library()
    B, T, d = A.shape
    p = G.shape[2]
    dt = _dtype_code(A)
    nbytes = L.dp_clip_aggregate_workspace(dt, B, T, d, p)
    ws_t = _workspace(nbytes, A.device, ws, zeroed=True)
    args = [dt, B, T, d, p, _ptr(A), _ptr(G), _ptr(n_sq), float(C), _ptr(c_out), _ptr(S),
            _ptr(ws_t), 0 if ws_t is None else ws_t.numel(), _stream(stream)]
    if events is None:
        st = L.dp_clip_aggregate(*args)
    else:
        st = L.dp_clip_aggregate_timed(*args, _event(events[0]), _event(events[1]))
    _check(st, "dp_clip_aggregate")
    return S


def dp_clip_aggregate_update_workspace(dtype, B, T, d, p):
    code = dtype if isinstance(dtype, int) else {"f32": DP_F32, "bf16": DP_BF16}[dtype]
    n = load_library().dp_clip_aggregate_update_workspace(code, B, T, d, p)
    return None if n == _SIZE_INVALID else n


def dp_clip_aggregate_update(A, G, n_sq, C, sigma, eta, seed, layer, theta, S=None, c_out=None,
                             ws=None, stream=None, events=None):
    """Clip factors, clipped sum, noise and update of theta [p][d] in one call
    (|B| = A.shape[0]); S, if given, receives the clipped sum.  ``events``: optional
    ((agg_begin, agg_end), (upd_begin, upd_end)) torch.cuda.Event pairs."""
    L = load_library()
    B, T, d = A.shape
    p = G.shape[2]
    dt = _dtype_code(A)
    nbytes = L.dp_clip_aggregate_update_workspace(dt, B, T, d, p)
    ws_t = _workspace(nbytes, A.device, ws, zeroed=True)
    args = [dt, B, T, d, p, _ptr(A), _ptr(G), _ptr(n_sq), float(C), float(sigma), float(eta),
            int(seed) & (2**64 - 1), int(layer), _ptr(theta), _ptr(S), _ptr(c_out),
            _ptr(ws_t), 0 if ws_t is None else ws_t.numel(), _stream(stream)]
    if events is None:
        st = L.dp_clip_aggregate_update(*args)
    else:
        ea, eu = events  # either pair may be None
        a0, a1 = ea if ea is not None else (None, None)
        u0, u1 = eu if eu is not None else (None, None)
        st = L.dp_clip_aggregate_update_timed(*args, _event(a0), _event(a1), _event(u0),
                                              _event(u1))
    _check(st, "dp_clip_aggregate_update")
    return theta


def dp_noise_update(theta, S, sigma, C, eta, B, seed, layer, stream=None, events=None):
    """theta <- theta - (eta / B) (S + sigma C xi) in place; theta, S fp32 [p][d]."""
    p, d = theta.shape
    L = load_library()
    args = [d, p, _ptr(theta), _ptr(S), float(sigma), float(C), float(eta), int(B),
            int(seed) & (2**64 - 1), int(layer), _stream(stream)]
    if events is None:
        st = L.dp_noise_update(*args)
    else:
        st = L.dp_noise_update_timed(*args, _event(events[0]), _event(events[1]))
    _check(st, "dp_noise_update")
    return theta


def dp_norm_est_layers_workspace(method, dtype, B, T, k, layers):
    """Workspace bytes of dp_norm_est_layers for (A, G, layer_id) tuples, or None."""
    code = dtype if isinstance(dtype, int) else {"f32": DP_F32, "bf16": DP_BF16}[dtype]
    n = load_library().dp_norm_est_layers_workspace(_method_code(method), code, B, T, int(k or 0),
                                                    len(layers), _layer_array(layers))
    return None if n == _SIZE_INVALID else n


def dp_norm_est_layers(method, layers, k, seed, n_sq, flags=0, ws=None, stream=None,
                       events=None):
    """n_sq[i] (= or += with DP_ACCUMULATE) the estimate summed over ``layers``, a list
    of (A, G, layer_id) with A [B][T][d_l] and G [B][T][p_l] of one dtype.
    ``events``: optional (begin, end) pair -> dp_norm_est_layers_timed."""
    L = load_library()
    A0 = layers[0][0]
    B, T = A0.shape[0], A0.shape[1]
    dt = _dtype_code(A0)
    m = _method_code(method)
    k = int(k or 0)
    arr = _layer_array(layers)
    nbytes = L.dp_norm_est_layers_workspace(m, dt, B, T, k, len(layers), arr)
    ws_t = _workspace(nbytes, A0.device, ws)
    args = [m, dt, B, T, k, len(layers), arr, int(seed) & (2**64 - 1), int(flags), _ptr(n_sq),
            _ptr(ws_t), 0 if ws_t is None else ws_t.numel(), _stream(stream)]
    if events is None:
        st = L.dp_norm_est_layers(*args)
    else:
        st = L.dp_norm_est_layers_timed(*args, _event(events[0]), _event(events[1]))
    _check(st, "dp_norm_est_layers")
    return n_sq


def dp_clip_aggregate_update_layers_workspace(dtype, B, T, layers):
    """Workspace bytes of dp_clip_aggregate_update_layers, or None."""
    code = dtype if isinstance(dtype, int) else {"f32": DP_F32, "bf16": DP_BF16}[dtype]
    n = load_library().dp_clip_aggregate_update_layers_workspace(code, B, T, len(layers),
                                                                 _layer_array(layers))
    return None if n == _SIZE_INVALID else n


def dp_clip_aggregate_update_layers_launches(dtype, B, T, layers):
    """Contraction launches the batched update makes for ``layers`` (None if invalid)."""
    code = dtype if isinstance(dtype, int) else {"f32": DP_F32, "bf16": DP_BF16}[dtype]
    n = load_library().dp_clip_aggregate_update_layers_launches(code, B, T, len(layers),
                                                                _layer_array(layers))
    return None if n < 0 else n


def dp_clip_aggregate_update_layers(layers, n_sq, C, sigma, eta, seed, c_out=None, ws=None,
                                    stream=None, agg_events=None, upd_events=None):
    """dp_clip_aggregate_update over ``layers``, a list of (A, G, layer_id, theta), with
    the clip factors formed once.  ``agg_events`` / ``upd_events``: optional lists of
    (begin, end) pairs, one per layer (or None), around each layer's contraction /
    noise + update; a contraction launch shared by several layers is timed in the
    first one's pair, the others' pairs are empty."""
    L = load_library()
    A0 = layers[0][0]
    B, T = A0.shape[0], A0.shape[1]
    dt = _dtype_code(A0)
    arr = _layer_array(layers)
    nbytes = L.dp_clip_aggregate_update_layers_workspace(dt, B, T, len(layers), arr)
    ws_t = _workspace(nbytes, A0.device, ws, zeroed=True)
    args = [dt, B, T, len(layers), arr, _ptr(n_sq), float(C), float(sigma), float(eta),
            int(seed) & (2**64 - 1), _ptr(c_out), _ptr(ws_t), 0 if ws_t is None else ws_t.numel(),
            _stream(stream)]
    if agg_events is None and upd_events is None:
        st = L.dp_clip_aggregate_update_layers(*args)
    else:
        n = len(layers)

        def arrays(evs):
            if evs is None:
                return None, None
            b = (ctypes.c_void_p * n)(*[_event(e[0]).value if e is not None else None for e in evs])
            f = (ctypes.c_void_p * n)(*[_event(e[1]).value if e is not None else None for e in evs])
            return b, f

        ab, ae = arrays(agg_events)
        ub, ue = arrays(upd_events)
        st = L.dp_clip_aggregate_update_layers_timed(*args, ab, ae, ub, ue)
    _check(st, "dp_clip_aggregate_update_layers")
    return n_sq


def dp_stream_read(buf, out, stream=None):
    """Measurement hook: stream every byte of the device tensor ``buf`` (size a
    multiple of 16); out (int32 [nblocks]) receives each workgroup's XOR."""
    st = load_library().dp_stream_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(out),
                                       out.numel(), _stream(stream))
    _check(st, "dp_stream_read")
    return out


def dp_philox_u32(seed, ctr, out, stream=None):
    """out[n][4] = Philox4x32-10 words of counters ctr[n][4] (uint32-valued int32 tensors)."""
    n = ctr.numel() // 4
    st = load_library().dp_philox_u32(int(seed) & (2**64 - 1), _ptr(ctr), _ptr(out), n,
                                      _stream(stream))
    _check(st, "dp_philox_u32")
    return out


def dp_probe_fill(seed, layer, sample, p, k, Pt, stream=None, rademacher=False):
    """Pt [k][p] fp32 = probe entries P[r][j] of (seed, layer, sample);
    ``rademacher`` gives the +-1 sign probe."""
    L = load_library()
    if rademacher:
        st = L.dp_probe_fill_ex(int(seed) & (2**64 - 1), int(layer), int(sample), int(p), int(k),
                                DP_PROBE_RADEMACHER, _ptr(Pt), _stream(stream))
    else:
        st = L.dp_probe_fill(int(seed) & (2**64 - 1), int(layer), int(sample), int(p), int(k),
                             _ptr(Pt), _stream(stream))
    _check(st, "dp_probe_fill")
    return Pt


def dp_noise_fill(seed, layer, offset, xi, stream=None):
    """xi[n] fp32 = noise normals of flat indices offset .. offset + n - 1."""
    st = load_library().dp_noise_fill(int(seed) & (2**64 - 1), int(layer), int(offset),
                                      xi.numel(), _ptr(xi), _stream(stream))
    _check(st, "dp_noise_fill")
    return xi


def dp_poisson_sample_workspace(N):
    """Workspace bytes for dp_poisson_sample over N examples, or None if N is out of range."""
    n = load_library().dp_poisson_sample_workspace(int(N))
    return None if n == _SIZE_INVALID else n


def dp_poisson_sample(seed, step, N, q, idx, count, ws=None, stream=None):
    """Poisson-subsampled minibatch of step ``step``: ascending indices into
    ``idx`` (int64 device tensor; its length is the capacity) and |B| into
    ``count`` (int64 device tensor of one element).  ``ws``: optional uint8
    device workspace (allocated here when omitted)."""
    import torch
    L = load_library()
    if ws is None:
        nbytes = dp_poisson_sample_workspace(N)
        if nbytes is None:
            raise ValueError(f"N = {N} out of range")
        ws = torch.empty(nbytes, dtype=torch.uint8, device=count.device)
    st = L.dp_poisson_sample(int(seed) & (2**64 - 1), int(step) & 0xFFFFFFFF, int(N), float(q),
                             _ptr(idx) if idx is not None and idx.numel() else None,
                             idx.numel() if idx is not None else 0, _ptr(count), _ptr(ws),
                             ws.numel(), _stream(stream))
    _check(st, "dp_poisson_sample")
    return idx, count


def dp_rmsnorm_norm(xhat, delta, n_sq, v=None, flags=0, ws=None, stream=None):
    """RMSNorm gain: v[i] = sum_t xhat[i,t] * delta[i,t] (if ``v`` is given, fp32 [B][d])
    and n_sq[i] (=, or += with DP_ACCUMULATE) ||v_i||^2.  xhat, delta: [B][T][d]."""
    L = load_library()
    B, T, d = xhat.shape
    dt = _dtype_code(xhat)
    ws_t = _workspace(L.dp_rmsnorm_norm_workspace(dt, B, T, d), xhat.device, ws)
    st = L.dp_rmsnorm_norm(dt, B, T, d, _ptr(xhat), _ptr(delta), int(flags), _ptr(n_sq), _ptr(v),
                           _ptr(ws_t), 0 if ws_t is None else ws_t.numel(), _stream(stream))
    _check(st, "dp_rmsnorm_norm")
    return n_sq


def dp_rmsnorm_clip_aggregate_update(v, n_sq, C, sigma, eta, seed, layer, gamma, S=None,
                                     c_out=None, ws=None, stream=None):
    """gamma[d] <- gamma - (eta / B) (sum_i c_i v_i + sigma C xi), c_i = min(1, C / sqrt(n_i))."""
    L = load_library()
    B, d = v.shape
    ws_t = _workspace(L.dp_rmsnorm_update_workspace(B, d), v.device, ws, zeroed=True)
    st = L.dp_rmsnorm_clip_aggregate_update(B, d, _ptr(v), _ptr(n_sq), float(C), float(sigma),
                                            float(eta), int(seed) & (2**64 - 1), int(layer),
                                            _ptr(gamma), _ptr(S), _ptr(c_out), _ptr(ws_t), 0 if ws_t is None else ws_t.numel(),
                                            _stream(stream))
    _check(st, "dp_rmsnorm_clip_aggregate_update")
    return gamma


def dp_embedding_norm(ids, delta, n_sq, flags=0, ws=None, stream=None):
    """Embedding table: n_sq[i] (=, or += with DP_ACCUMULATE) = sum over the distinct ids
    of sample i of ||sum of its delta rows||^2.  ids: int32 [B][T]; delta: [B][T][d]."""
    L = load_library()
    B, T, d = delta.shape
    dt = _dtype_code(delta)
    ws_t = _workspace(L.dp_embedding_norm_workspace(dt, B, T, d), delta.device, ws)
    st = L.dp_embedding_norm(dt, B, T, d, _ptr(ids), _ptr(delta), int(flags), _ptr(n_sq),
                             _ptr(ws_t), 0 if ws_t is None else ws_t.numel(), _stream(stream))
    _check(st, "dp_embedding_norm")
    return n_sq


def dp_embedding_clip_aggregate_update(ids, delta, n_sq, C, sigma, eta, seed, layer, E,
                                       c_out=None, ws=None, stream=None):
    """E [V][d] <- E - (eta / B) (sum_i c_i grad_i + sigma C xi) over every row of E."""
    L = load_library()
    B, T, d = delta.shape
    V = E.shape[0]
    dt = _dtype_code(delta)
    ws_t = _workspace(L.dp_embedding_update_workspace(dt, B, T, d, V), delta.device, ws,
                      zeroed=True)
    st = L.dp_embedding_clip_aggregate_update(dt, B, T, d, V, _ptr(ids), _ptr(delta), _ptr(n_sq),
                                              float(C), float(sigma), float(eta),
                                              int(seed) & (2**64 - 1), int(layer), _ptr(E),
                                              _ptr(c_out), _ptr(ws_t),
                                              0 if ws_t is None else ws_t.numel(),
                                              _stream(stream))
    _check(st, "dp_embedding_clip_aggregate_update")
    return E


def dp_weights_bf16(theta, W=None, Wt=None, stream=None):
    """(W, Wt): bf16 copies of fp32 parameters theta [p][d] and of their transpose."""
    L = load_library()
    p, d = theta.shape
    W = torch.empty(p, d, dtype=torch.bfloat16, device=theta.device) if W is None else W
    Wt = torch.empty(d, p, dtype=torch.bfloat16, device=theta.device) if Wt is None else Wt
    _check(L.dp_weights_bf16(p, d, _ptr(theta), _ptr(W), _ptr(Wt), _stream(stream)),
           "dp_weights_bf16")
    return W, Wt


def dp_linear_forward(A, W, residual=None, C=None, stream=None):
    """C = bf16(A W^T (+ residual)); A [..][K], W [N][K] bf16."""
    L = load_library()
    K = A.shape[-1]
    M = A.numel() // K if K else 0
    N = W.shape[0]
    C = torch.empty(*A.shape[:-1], N, dtype=torch.bfloat16, device=A.device) if C is None else C
    _check(L.dp_linear_forward(M, N, K, _ptr(A), _ptr(W), _ptr(residual), _ptr(C),
                               _stream(stream)), "dp_linear_forward")
    return C


MLP_FORWARD_OUTPUTS = ("xhat", "y", "rstd", "g", "u", "h", "out")
MLP_BACKWARD_OUTPUTS = ("G_gate", "G_up", "dy", "dx")


def dp_mlp_forward(x, gamma, Wg, Wu, Wd, eps=1e-5, acts=None, stream=None):
    """Forward of the MLP block: x [B][T][d] bf16; gamma [d] fp32; Wg, Wu [f][d],
    Wd [d][f] bf16.  Returns (and fills ``acts`` if given) a dict with xhat, y,
    rstd [B][T] fp32, g, u, h [B][T][f] and out."""
    L = load_library()
    B, T, d = x.shape
    f = Wg.shape[0]
    acts = {} if acts is None else acts
    for name in MLP_FORWARD_OUTPUTS:
        if name not in acts:
            width = f if name in ("g", "u", "h") else d
            acts[name] = (torch.empty(B, T, dtype=torch.float32, device=x.device) if name == "rstd"
                          else torch.empty(B, T, width, dtype=torch.bfloat16, device=x.device))
    st = L.dp_mlp_forward(B, T, d, f, float(eps), _ptr(x), _ptr(gamma), _ptr(Wg), _ptr(Wu),
                          _ptr(Wd), *(_ptr(acts[n]) for n in MLP_FORWARD_OUTPUTS),
                          _stream(stream))
    _check(st, "dp_mlp_forward")
    return acts


def dp_mlp_backward(x, rstd, gamma, g, u, WgT, WuT, WdT, dout, grads=None, stream=None):
    """Backward pass 1 of the MLP block: dict with G_gate, G_up [B][T][f], dy and
    dx [B][T][d] (bf16) from the forward's x, rstd, g, u, the transposed bf16
    weights and dout = dL/d(out)."""
    L = load_library()
    B, T, d = x.shape
    f = g.shape[-1]
    grads = {} if grads is None else grads
    for name in MLP_BACKWARD_OUTPUTS:
        if name not in grads:
            width = f if name in ("G_gate", "G_up") else d
            grads[name] = torch.empty(B, T, width, dtype=torch.bfloat16, device=x.device)
    st = L.dp_mlp_backward(B, T, d, f, _ptr(x), _ptr(rstd), _ptr(gamma), _ptr(g), _ptr(u),
                           _ptr(WgT), _ptr(WuT), _ptr(WdT), _ptr(dout),
                           *(_ptr(grads[n]) for n in MLP_BACKWARD_OUTPUTS), _stream(stream))
    _check(st, "dp_mlp_backward")
    return grads


def dp_rope(x, T, n_heads, base=500000.0, inverse=False, stream=None):
    """In place RoPE of x [..][64 n_heads] bf16 (row index % T is the position)."""
    L = load_library()
    M = x.numel() // (64 * n_heads)
    _check(L.dp_rope(M, int(T), int(n_heads), float(base), 1 if inverse else 0, _ptr(x),
                     _stream(stream)), "dp_rope")
    return x


def dp_attention_forward(q, k, v, n_heads, n_kv, o=None, lse=None, stream=None):
    """Causal grouped-query attention: q [B][T][64 H], k, v [B][T][64 KV] bf16 ->
    (o [B][T][64 H] bf16, lse [B][H][T] fp32)."""
    L = load_library()
    B, T = q.shape[0], q.shape[1]
    o = torch.empty_like(q) if o is None else o
    lse = torch.empty(B, n_heads, T, dtype=torch.float32, device=q.device) if lse is None else lse
    _check(L.dp_attention_forward(B, T, n_heads, n_kv, _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                  _ptr(lse), _stream(stream)), "dp_attention_forward")
    return o, lse


ATTN_FORWARD_OUTPUTS = ("xhat", "y", "rstd", "q", "k", "v", "o", "lse", "out")


def dp_attn_forward(x, gamma, Wq, Wk, Wv, Wo, n_heads, n_kv, eps=1e-5, rope_base=500000.0,
                    acts=None, stream=None):
    """Forward of the attention block: x [B][T][d] bf16; gamma [d] fp32; Wq [64 H][d],
    Wk, Wv [64 KV][d], Wo [d][64 H] bf16.  Returns (and fills ``acts``) a dict with
    xhat, y, rstd, q, k, v (after RoPE), o, lse [B][H][T] and out."""
    L = load_library()
    B, T, d = x.shape
    acts = {} if acts is None else acts
    shapes = {"xhat": (B, T, d), "y": (B, T, d), "rstd": (B, T), "q": (B, T, 64 * n_heads),
              "k": (B, T, 64 * n_kv), "v": (B, T, 64 * n_kv), "o": (B, T, 64 * n_heads),
              "lse": (B, n_heads, T), "out": (B, T, d)}
    for name in ATTN_FORWARD_OUTPUTS:
        if name not in acts:
            dt = torch.float32 if name in ("rstd", "lse") else torch.bfloat16
            acts[name] = torch.empty(shapes[name], dtype=dt, device=x.device)
    st = L.dp_attn_forward(B, T, d, n_heads, n_kv, float(eps), float(rope_base), _ptr(x),
                           _ptr(gamma), _ptr(Wq), _ptr(Wk), _ptr(Wv), _ptr(Wo),
                           *(_ptr(acts[n]) for n in ATTN_FORWARD_OUTPUTS), _stream(stream))
    _check(st, "dp_attn_forward")
    return acts


def dp_attention_backward(q, k, v, o, lse, dO, n_heads, n_kv, ws=None, stream=None):
    """(dq, dk, dv) of causal grouped-query attention from dO [B][T][64 H]."""
    L = load_library()
    B, T = q.shape[0], q.shape[1]
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws_t = _workspace(L.dp_attention_backward_workspace(B, T, n_heads), q.device, ws)
    _check(L.dp_attention_backward(B, T, n_heads, n_kv, _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                   _ptr(lse), _ptr(dO), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws_t),
                                   0 if ws_t is None else ws_t.numel(), _stream(stream)),
           "dp_attention_backward")
    return dq, dk, dv


ATTN_BACKWARD_OUTPUTS = ("G_q", "G_k", "G_v", "dy", "dx")


def dp_attn_backward(x, acts, gamma, WqT, WkT, WvT, WoT, dout, n_heads, n_kv,
                     rope_base=500000.0, grads=None, ws=None, stream=None):
    """Backward pass 1 of the attention block from the forward's ``acts`` (rstd, q, k,
    v, o, lse) and dout = dL/d(out): dict with G_q, G_k, G_v, dy and dx (bf16)."""
    L = load_library()
    B, T, d = x.shape
    grads = {} if grads is None else grads
    widths = {"G_q": 64 * n_heads, "G_k": 64 * n_kv, "G_v": 64 * n_kv, "dy": d, "dx": d}
    for name in ATTN_BACKWARD_OUTPUTS:
        if name not in grads:
            grads[name] = torch.empty(B, T, widths[name], dtype=torch.bfloat16, device=x.device)
    ws_t = _workspace(L.dp_attn_backward_workspace(B, T, n_heads), x.device, ws)
    st = L.dp_attn_backward(B, T, d, n_heads, n_kv, float(rope_base), _ptr(x), _ptr(acts["rstd"]),
                            _ptr(gamma), _ptr(acts["q"]), _ptr(acts["k"]), _ptr(acts["v"]),
                            _ptr(acts["o"]), _ptr(acts["lse"]), _ptr(WqT), _ptr(WkT), _ptr(WvT),
                            _ptr(WoT), _ptr(dout), *(_ptr(grads[n]) for n in ATTN_BACKWARD_OUTPUTS),
                            _ptr(ws_t), 0 if ws_t is None else ws_t.numel(), _stream(stream))
    _check(st, "dp_attn_backward")
    return grads
