"""The workloads: five linear-layer configurations of the DP-SGD-RC step.

Shapes follow the pages' notation: B samples, T tokens per sample, a linear
layer of shape (p, d) (d inputs, p outputs), k probes, clip norm C, noise
multiplier sigma, learning rate eta.  The Llama-3.2-1B-shaped layers stand in
for the long-context fine-tuning workload of the randomized-clipping summary
(section 実証結果: Llama 3.2 1B, context >= 4096); the data are synthetic.
"""

from dataclasses import dataclass, field
from typing import List, Tuple


@dataclass(frozen=True)
class Layer:
    name: str
    layer_id: int
    d: int  # input width
    p: int  # output width


@dataclass
class Workload:
    name: str
    B: int
    T: int
    dtype: str  # "f32" | "bf16"
    layers: List[Layer]
    method: str  # estimator timed on the hot path
    k: int
    C: float
    sigma: float
    eta: float
    recipe: str  # value distribution, see inputs.py
    data_seed: int
    method_seed: int
    noise_seed: int
    baselines: Tuple[str, ...] = field(default_factory=tuple)

    @property
    def tokens(self):
        return self.B * self.T

    @property
    def n_params(self):
        return sum(l.d * l.p for l in self.layers)


def llama_1b_stack(blocks=16, hidden=2048, kv=512, ffn=8192):
    """Every linear layer of a Llama-3.2-1B-shaped decoder stack (no biases)."""
    shapes = [("q", hidden, hidden), ("k", hidden, kv), ("v", hidden, kv),
              ("o", hidden, hidden), ("gate", hidden, ffn), ("up", hidden, ffn),
              ("down", ffn, hidden)]
    out = []
    for b in range(blocks):
        for idx, (nm, d, p) in enumerate(shapes):
            out.append(Layer(f"blk{b}.{nm}", 7 * b + idx, d, p))
    return out


def workloads():
    """The workloads by name: five configurations and one spectrum-structured layer."""
    w = {}
    w["tiny_f32_b4_t64"] = Workload(
        "tiny_f32_b4_t64", B=4, T=64, dtype="f32",
        layers=[Layer("linear", 0, 64, 64)], method="hutch", k=8,
        C=1.0, sigma=1.0, eta=0.1, recipe="unit_u0.1_3",
        data_seed=1001, method_seed=2001, noise_seed=3001,
        baselines=("fgc", "ghost"))
    w["attn_proj_b8_t4096_d2048"] = Workload(
        "attn_proj_b8_t4096_d2048", B=8, T=4096, dtype="bf16",
        layers=[Layer("q_proj", 0, 2048, 2048)], method="hutch", k=32,
        C=1.0, sigma=1.0, eta=1e-4, recipe="llama_logu",
        data_seed=1002, method_seed=2002, noise_seed=3002,
        baselines=("ghost", "fgc"))
    w["mlp_up_b8_t4096_d2048_p8192"] = Workload(
        "mlp_up_b8_t4096_d2048_p8192", B=8, T=4096, dtype="bf16",
        layers=[Layer("up_proj", 0, 2048, 8192)], method="hutchpp", k=32,
        C=1.0, sigma=1.0, eta=1e-4, recipe="llama_logu",
        data_seed=1003, method_seed=2003, noise_seed=3003,
        baselines=("hutch", "ghost"))
    w["mlp_down_b8_t4096_d8192_p2048"] = Workload(
        "mlp_down_b8_t4096_d8192_p2048", B=8, T=4096, dtype="bf16",
        layers=[Layer("down_proj", 0, 8192, 2048)], method="hutchpp", k=32,
        C=1.0, sigma=1.0, eta=1e-4, recipe="llama_logu",
        data_seed=1013, method_seed=2013, noise_seed=3013,
        baselines=("hutch", "ghost"))
    w["long_ctx_b2_t16384_d2048_p8192"] = Workload(
        "long_ctx_b2_t16384_d2048_p8192", B=2, T=16384, dtype="bf16",
        layers=[Layer("up_proj", 0, 2048, 8192)], method="hutch", k=32,
        C=1.0, sigma=1.0, eta=1e-4, recipe="llama_logu",
        data_seed=1004, method_seed=2004, noise_seed=3004,
        baselines=("ghost", "fgc"))
    # a spectrum-structured layer (rank-8 signal + 5% noise in A and G): the
    # head that Hutch++ takes exactly carries most of tr(O)
    w["lowrank_attn_b8_t4096_d2048"] = Workload(
        "lowrank_attn_b8_t4096_d2048", B=8, T=4096, dtype="bf16",
        layers=[Layer("q_proj", 0, 2048, 2048)], method="hutchpp", k=32,
        C=1.0, sigma=1.0, eta=1e-4, recipe="lowrank",
        data_seed=1006, method_seed=2006, noise_seed=3006,
        baselines=("hutch", "fgc"))
    w["llama1b_stack_b8_t4096"] = Workload(
        "llama1b_stack_b8_t4096", B=8, T=4096, dtype="bf16",
        layers=llama_1b_stack(), method="hutch", k=32,
        C=1.0, sigma=1.0, eta=1e-4, recipe="llama_logu",
        data_seed=1005, method_seed=2005, noise_seed=3005)
    return w
