"""DP-SGD with randomized clipping: the per-step hot path on MI355X (gfx950).

The compute lives in ``libdprc.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/dprc.h``).  ``sample_gradient_clipping_amd.binding`` is
the thin ctypes layer over it; its functions are re-exported here on first
use.  Importing the data helpers (``configs``, ``inputs``) does not load the
library; calling any compute entry point does, and raises if it is missing.
"""

_BINDING_NAMES = (
    "dp_abi_version", "dp_status_string", "dp_norm_est", "dp_norm_est_workspace",
    "dp_clip_aggregate", "dp_clip_aggregate_workspace", "dp_noise_update",
    "dp_clip_aggregate_update", "dp_clip_aggregate_update_workspace",
    "dp_philox_u32", "dp_probe_fill", "dp_noise_fill", "dp_poisson_sample",
    "dp_poisson_sample_workspace", "dp_rmsnorm_norm", "dp_rmsnorm_clip_aggregate_update",
    "dp_embedding_norm", "dp_embedding_clip_aggregate_update",
    "dp_weights_bf16", "dp_linear_forward", "dp_mlp_forward", "dp_mlp_backward",
    "dp_rope", "dp_attention_forward", "dp_attn_forward", "dp_attention_backward",
    "dp_attn_backward",
    "DprcError", "lib_path",
    "load_library", "METHODS", "DP_ACCUMULATE", "DP_PROBE_SHARED", "DP_PROBE_RADEMACHER",
)


def __getattr__(name):
    if name in _BINDING_NAMES:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
