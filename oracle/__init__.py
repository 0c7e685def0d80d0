"""Plain fp64 CPU oracle for the DP-SGD-RC hot path.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with
the HIP library and never imports it.

Sources it follows (cited by page title and section throughout):

* [RC] "技術的サマリー：ランダム化クリッピングを備えた LLM 向け効率的な DP-SGD"
  (technical summary of DP-SGD with randomized clipping):
  - section 手法 / 中核メカニズム (core mechanism): the trace identity
    ||A^T G||_F^2 = tr(G^T A A^T G) = tr(O), item 1 (Hutch: Gaussian
    P in R^{p x k}), item 2 (Hutch++: QR head + Hutchinson tail);
  - section アルゴリズム的フロー (algorithmic flow), steps 3-5
    (norm estimation, rescale by min(C / n_i, 1), backward-2 + noise + update);
  - section 問題定義 and 主要な貢献 / 1. 複雑性の削減 (problem statement and
    complexity): FGC materialises the per-sample gradient, GC works with
    T x T Gram products.
* [DPSGD] "DP-SGD（差分プライバシー確率的勾配降下法）とは？", section
  DP-SGDのアルゴリズム (algorithm), steps 3-5: clip, Gaussian noise
  N(0, sigma^2 C^2 I) added to the clipped sum, SGD update theta - eta G/|B|.
  Step 1 (Poisson subsampling of the minibatch) is in ``sampling.py``; the
  per-sample gradients of RMSNorm gains and embedding tables (the parameters
  that are not linear layers) in ``other_layers.py``; the forward pass and
  backward pass 1 of a Llama-shaped MLP block ([RC] アルゴリズム的フロー, steps
  1-2) and that block's whole step in ``mlp_block.py``; the attention half of
  the decoder layer (grouped heads, RoPE, causal softmax) in ``attn_block.py``,
  with the whole layer (attention block, then MLP block) and its step.
* Philox4x32-10: Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as
  easy as 1, 2, 3", SC'11 (the published counter-based generator).

Everything is float64 numpy; matrix products use numpy's matmul as a library
primitive.  Inputs are the exact bytes the GPU reads (fp32 or bf16), upcast
exactly to float64 by :func:`to_f64`.

Readings the pages leave open are stated where they are used; the same list
is kept with the design notes at the repository root.  Parity status: every
function here is pinned by a ``-m "not gpu"`` test against something other
than itself (see ``tests/test_oracle_*.py``); none is "parity unpinned".
"""

from .philox import (  # noqa: F401
    philox4x32_10,
    uniforms_from_words,
    box_muller,
    normals_from_counters,
    probe_matrix,
    rademacher_probe_matrix,
    noise_vector,
    PROBE_LANES,
)
from .norms import (  # noqa: F401
    to_f64,
    fgc_norm_sq,
    ghost_norm_sq,
    hutch_core,
    hutch_norm_sq,
    householder_thin_q,
    hutchpp_split,
    hutchpp_norm_sq,
    norm_est,
)
from .step import (  # noqa: F401
    clip_factors,
    aggregate,
    aggregate_rows,
    noise_update,
    dp_step,
)
from .other_layers import (  # noqa: F401
    rmsnorm_grad,
    rmsnorm_norm_sq,
    rmsnorm_aggregate,
    embedding_rows,
    embedding_norm_sq,
    embedding_aggregate,
)
from .sampling import (  # noqa: F401
    POISSON_C3,
    poisson_threshold,
    poisson_words,
    poisson_sample,
    norm_est_ragged,
    aggregate_ragged,
)
from .mlp_block import (  # noqa: F401
    rmsnorm_forward,
    rmsnorm_backward,
    linear_forward,
    swiglu_forward,
    swiglu_backward,
    mlp_forward,
    mlp_backward,
    mlp_per_sample_grads,
    mlp_dp_step,
    MLP_LAYERS,
)
from .attn_block import (  # noqa: F401
    rope,
    attention_forward,
    attention_backward,
    attn_forward,
    attn_backward,
    attn_per_sample_grads,
    attn_dp_step,
    ATTN_LAYERS,
    layer_forward,
    layer_backward,
    layer_dp_step,
)
