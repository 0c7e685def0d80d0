"""Algorithmic work of each kernel and the MI355X peaks it is measured against.

Bytes are the bytes a kernel must move (each input read once, each output
written once); flops are the multiply-adds of its contraction (x2).  E is the
input element size (2 for bf16, 4 for fp32).

Per layer of shape (p, d), batch B, T tokens per sample, k probes:
  Hutch passes   bytes B T (d + p) E                      flops 2 B T k (d + p)
  Hutch++        bytes 3 B T (d + p) E                    flops 2 B T (d + p)(3 s + r)
  ghost          bytes B T (d + p) E                      flops B T^2 (d + p)  (upper triangle)
  FGC            bytes B T (d + p) E + 4 B d p            flops 2 B T d p
  aggregation    bytes B T (d + p) E + 4 d p              flops 2 B T d p
  noise+update   bytes 12 d p  (theta read + write, S read)
The big-O costs the randomized-clipping summary quotes (section 主要な貢献,
1. 複雑性の削減): FGC O(B T p d), GC O(B T^2 (p + d)), RC O(B T k (p + d)).
"""

# MI355X published peaks.
PEAK_HBM_GBPS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
PEAK_FP32_TFLOPS = 157.3
PEAK_FP64_TFLOPS = 78.6


def elem_size(dtype):
    return {"f32": 4, "bf16": 2}[dtype]


def hutch_bytes(B, T, d, p, dtype):
    return B * T * (d + p) * elem_size(dtype)


def hutch_flops(B, T, d, p, k):
    return 2 * B * T * k * (d + p)


def hutchpp_bytes(B, T, d, p, dtype):
    return 3 * hutch_bytes(B, T, d, p, dtype)


def hutchpp_flops(B, T, d, p, k):
    s = k // 3
    r = k - 2 * s
    return 2 * B * T * (d + p) * (3 * s + r)


def ghost_flops(B, T, d, p):
    return B * T * T * (d + p)


def gemm_flops(B, T, d, p):
    return 2 * B * T * d * p


def aggregate_bytes(B, T, d, p, dtype):
    return B * T * (d + p) * elem_size(dtype) + 4 * d * p


def fgc_bytes(B, T, d, p, dtype):
    return B * T * (d + p) * elem_size(dtype) + 4 * B * d * p


def noise_bytes(d, p):
    return 12 * d * p


def big_o_flops(method, B, T, d, p, k):
    """The summary's big-O expressions with their constants dropped."""
    if method == "fgc":
        return B * T * p * d
    if method == "ghost":
        return B * T * T * (p + d)
    if method in ("hutch", "hutchpp"):
        return B * T * k * (p + d)
    raise ValueError(method)
