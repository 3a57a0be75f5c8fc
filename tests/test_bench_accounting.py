"""The algorithmic work bench.py divides by to report its roofline fractions, derived here
by hand from the layer's shapes (no GPU)."""
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import bench  # noqa: E402


def test_decode_layer_bytes():
    """One batch-1 layer of the decode workload (hidden 2048, 256 experts, top-8 + shared,
    inter 512, 4-bit codes, groups of 64 with an fp16 scale and bias each) must read the
    bf16 router matrix, the k routed experts and the shared one, and x, and write y."""
    H, I, E, K = 2048, 512, 256, 8
    router = E * H * 2                                      # bf16 [E][H]
    codes = (2 * I * H + H * I) * 4 // 8                    # [gate; up] rows and down rows, 4 bits each
    sb = (2 * I * (H // 64) + H * (I // 64)) * 2 * 2        # one fp16 scale and one fp16 bias per group
    expert = codes + sb
    assert expert == 1_769_472
    total = router + (K + 1) * expert + 2 * H * 2           # + x in and y out (bf16)
    assert total == 16_982_016
    assert bench.decode_layer_bytes(H, I, E, K, 4) == total
    assert bench.decode_layer_bytes(H, I, E, K, 4, shared=False) == total - expert


def test_prefill_layer_flops():
    """Prefill T = 4096: 2 T E H for the router, and per (token, expert) of the k routed
    and the shared one, 2 H 2I for [gate; up] plus 2 I H for down."""
    T, H, I, E, K = 4096, 2048, 512, 256, 8
    router = 2 * T * E * H
    experts = T * (K + 1) * (2 * H * 2 * I + 2 * I * H)
    assert router + experts == 236_223_201_280
    assert bench.layer_flops(T, H, I, E, K) == router + experts
    assert bench.layer_flops(4 * T, H, I, E, K) == 4 * (router + experts)


def test_q8_layer_bytes():
    """The Q8_0 layer of four projections reads 34 bytes per 32 weights of each matrix, its
    bf16 activation, and writes its bf16 output (the figure the bench reports)."""
    shapes = ((3072, 2048), (2048, 2048), (16384, 2048), (2048, 8192))
    weights = sum(n * k // 32 * 34 for n, k in shapes)
    assert weights == 64_618_496
    assert sum(bench.q8_weight_bytes(n, k) for n, k in shapes) == weights
    assert weights + sum(2 * k + 2 * n for n, k in shapes) == 64_694_272
