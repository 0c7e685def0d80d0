"""Values the pages print, checked against the accounting the bench uses."""

import json
import os

from sample_gradient_clipping_amd import roofline

HERE = os.path.dirname(os.path.abspath(__file__))


def test_gc_over_rc_flop_ratio_matches_page():
    g = json.load(open(os.path.join(HERE, "golden", "complexity_ratio.json")))
    T, k = g["T"], g["k"]
    for B, d, p in ((1, 2048, 2048), (8, 2048, 8192)):
        ratio = roofline.big_o_flops("ghost", B, T, d, p, k) / roofline.big_o_flops("hutch", B, T, d, p, k)
        assert ratio == g["gc_over_rc"]


def test_kernel_flop_counts_are_consistent():
    B, T, d, p, k = 8, 4096, 2048, 2048, 32
    # ghost counts the upper triangle of two T x T Grams: T^2 (d + p) per sample
    assert roofline.ghost_flops(B, T, d, p) == B * T * T * (d + p)
    # Hutch: two thin products, k columns each, 2 flops per multiply-add
    assert roofline.hutch_flops(B, T, d, p, k) == 2 * k * B * T * (d + p)
    # Hutch++ with k = 32: s = 10, r = 12; 3 s + r = 42 column-products per row
    assert roofline.hutchpp_flops(B, T, d, p, 32) == 2 * B * T * (d + p) * 42
    # the aggregation and FGC contract over all B T tokens
    assert roofline.gemm_flops(B, T, d, p) == 2 * B * T * d * p
    assert roofline.hutch_bytes(B, T, d, p, "bf16") == 268435456
