"""Seeded synthetic inputs for the quantized sparse MoE layer and the Q8_0 GEMV.

This module only draws random numbers and lays them out in the byte formats the
layer consumes.  It holds none of the layer's arithmetic: no dequantization, no
routing, no matrix products.  Both the HIP path's tests/benchmark and the CPU
oracle take their inputs from here.

Recipe (same distributions as the workloads the pages describe; no trained
weights exist here):

* activations ``x ~ N(0, 1)`` rounded to bfloat16;
* affine codes uniform over ``[0, 2^bits)`` (4-bit codes two per byte, so a
  uniform random byte is two uniform codes);
* per-group-of-64 scales ``s ~ U(0.005, 0.02)`` (divided by 16 for 8-bit codes so
  that the weight spread matches), stored as fp16 (or bf16: the checkpoint
  variant the pages print);
* biases ``b = fp16(s * (U(-0.5, 0.5) - 2^(bits-1)))``: centred, and not a
  multiple of ``s``, so a consumer that ignores the bias is visibly wrong;
* router weights ``N(0, std)`` rounded to bfloat16 (``std = 1/sqrt(hidden)``
  makes the logits roughly ``N(0, 1)``); the optional shared-expert gate vector the
  same way;
* optional Zipf router bias ``b_e = ln(r_e^-s / sum_j j^-s)`` with ``r`` a seeded
  permutation of ``1..E``, so a few experts receive many times the mean load;
* Q8_0 rows: ``q ~ U{-127..127}`` int8 and ``d ~ U(0.0005, 0.002)`` as fp16, in
  row-contiguous 34-byte blocks ``[fp16 d][32 x int8]``.

Every array is drawn from its own PCG64 stream keyed by ``(seed, stream id)`` so
that, e.g., changing ``T`` never changes the weights.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

GROUP = 64

# stream ids
_S_X, _S_ROUTER, _S_RBIAS, _S_GU, _S_DN, _S_SGU, _S_SDN, _S_Q8, _S_SGATE = range(9)


def _rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64([int(seed), int(stream)]))


def to_bf16_bits(a) -> np.ndarray:
    """Round float values to bfloat16 (nearest-even) and return the bit patterns."""
    f = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32 (for building inputs)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def to_f16_bits(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64).astype(np.float16).view(np.uint16)


@dataclasses.dataclass
class QMat:
    """A stack of affine-quantized matrices ``[n][rows][cols]`` (group 64 on cols).

    ``codes``  uint8 ``[n][rows][cols*bits/8]`` (4-bit: column 2i low nibble of byte i)
    ``scales`` uint16 fp16 bits ``[n][rows][cols/64]`` (bf16 bits when sb_dtype == "bf16")
    ``biases`` uint16, same format as the scales
    """

    codes: np.ndarray
    scales: np.ndarray
    biases: np.ndarray
    bits: int
    sb_dtype: str = "f16"

    @property
    def rows(self) -> int:
        return self.codes.shape[1]

    @property
    def cols(self) -> int:
        return self.scales.shape[2] * GROUP


@dataclasses.dataclass
class LayerInputs:
    """Weights of one MoE layer in the fused ``[gate; up]`` layout.

    ``gate_up``: ``[E][2*inter][hidden]`` (gate rows first, then up rows)
    ``down``:    ``[E][hidden][inter]``
    ``s_gate_up`` / ``s_down``: the shared expert, stacks of one matrix.
    """

    hidden: int
    inter: int
    n_experts: int
    top_k: int
    bits: int
    router_w: np.ndarray                 # uint16 bf16 bits [E][hidden]
    router_bias: Optional[np.ndarray]    # float32 [E] or None
    gate_up: QMat
    down: QMat
    has_shared: bool
    s_gate_up: Optional[QMat]
    s_down: Optional[QMat]
    seed: int = 0
    scale_dtype: str = "f16"                 # "f16" or "bf16" scales and biases
    shared_gate_w: Optional[np.ndarray] = None   # uint16 bf16 bits [hidden], or None

    @property
    def expert_bytes(self) -> int:
        """Bytes of one expert's weights (codes + fp16 scale + fp16 bias)."""
        H, I, b = self.hidden, self.inter, self.bits
        per_w = b / 8 + 4 / GROUP
        return int(round(3 * H * I * per_w))


def _qmat(rng: np.random.Generator, n: int, rows: int, cols: int, bits: int, sb: str = "f16",
          scale_range=None) -> QMat:
    assert cols % GROUP == 0 and bits in (4, 8) and sb in ("f16", "bf16")
    codes = rng.integers(0, 256, size=(n, rows, cols * bits // 8), dtype=np.uint8)
    if scale_range is None:
        s = rng.uniform(0.005, 0.02, size=(n, rows, cols // GROUP))
        if bits == 8:
            s = s / 16.0
    else:                                    # log-uniform over [lo, hi]
        lo, hi = scale_range
        s = np.exp(rng.uniform(np.log(lo), np.log(hi), size=(n, rows, cols // GROUP)))
    off = rng.uniform(-0.5, 0.5, size=s.shape) - 2.0 ** (bits - 1)
    if sb == "bf16":
        sbits = to_bf16_bits(s)
        bbits = to_bf16_bits(bf16_bits_to_f32(sbits).astype(np.float64) * off)
        return QMat(codes=codes, scales=sbits, biases=bbits, bits=bits, sb_dtype="bf16")
    s16 = s.astype(np.float16)
    b16 = (s16.astype(np.float64) * off).astype(np.float16)
    return QMat(codes=codes, scales=s16.view(np.uint16), biases=b16.view(np.uint16), bits=bits)


def zipf_router_bias(n_experts: int, s: float, seed: int) -> np.ndarray:
    r = _rng(seed, _S_RBIAS).permutation(np.arange(1, n_experts + 1))
    z = np.sum(np.arange(1, n_experts + 1, dtype=np.float64) ** (-s))
    return np.log(r.astype(np.float64) ** (-s) / z).astype(np.float32)


def make_layer(hidden: int, inter: int, n_experts: int, top_k: int, bits: int,
               seed: int = 0, router_std: Optional[float] = None,
               zipf_s: Optional[float] = None, has_shared: bool = True,
               scale_dtype: str = "f16", shared_gate: bool = False, scale_range=None) -> LayerInputs:
    """One layer's weights.  scale_dtype "bf16": scales and biases stored as bfloat16
    (the checkpoint format the pages print); shared_gate: a bf16 gate vector
    ``g ~ N(0, 1/hidden)`` whose sigmoid(g . x) scales the shared expert's output;
    scale_range (lo, hi): scales drawn log-uniformly over [lo, hi] instead."""
    if router_std is None:
        router_std = 1.0 / np.sqrt(hidden)
    rw = _rng(seed, _S_ROUTER).normal(0.0, router_std, size=(n_experts, hidden))
    rb = zipf_router_bias(n_experts, zipf_s, seed) if zipf_s is not None else None
    gu = _qmat(_rng(seed, _S_GU), n_experts, 2 * inter, hidden, bits, scale_dtype, scale_range)
    dn = _qmat(_rng(seed, _S_DN), n_experts, hidden, inter, bits, scale_dtype, scale_range)
    sgu = _qmat(_rng(seed, _S_SGU), 1, 2 * inter, hidden, bits, scale_dtype, scale_range) if has_shared else None
    sdn = _qmat(_rng(seed, _S_SDN), 1, hidden, inter, bits, scale_dtype, scale_range) if has_shared else None
    sg = None
    if shared_gate:
        assert has_shared
        sg = to_bf16_bits(_rng(seed, _S_SGATE).normal(0.0, 1.0 / np.sqrt(hidden), size=hidden))
    return LayerInputs(hidden=hidden, inter=inter, n_experts=n_experts, top_k=top_k,
                       bits=bits, router_w=to_bf16_bits(rw), router_bias=rb,
                       gate_up=gu, down=dn, has_shared=has_shared, s_gate_up=sgu,
                       s_down=sdn, seed=seed, scale_dtype=scale_dtype, shared_gate_w=sg)


def make_x(T: int, hidden: int, seed: int = 0, std: float = 1.0) -> np.ndarray:
    """bf16 bit patterns [T][hidden] of N(0, std^2) activations."""
    return to_bf16_bits(std * _rng(seed, _S_X).standard_normal((T, hidden)))


def make_q8_rows(N: int, K: int, seed: int = 0) -> np.ndarray:
    """Row-contiguous Q8_0 blocks, uint8 [N][K/32][34]."""
    assert K % 32 == 0
    rng = _rng(seed, _S_Q8)
    q = rng.integers(-127, 128, size=(N, K // 32, 32), dtype=np.int64).astype(np.int8)
    d = rng.uniform(0.0005, 0.002, size=(N, K // 32)).astype(np.float16)
    out = np.empty((N, K // 32, 34), dtype=np.uint8)
    out[:, :, 0:2] = d.view(np.uint8).reshape(N, K // 32, 2)
    out[:, :, 2:] = q.view(np.uint8)
    return out


# ----------------------------------------------------------------- named workloads
# Shapes of the workloads the pages describe (Qwen3.6-35B-A3B-style MoE layer:
# 256 experts, top-8, one shared expert; Llama-3.2-1B projections for Q8_0).

TINY = dict(hidden=256, inter=128, n_experts=16, top_k=2, bits=8, seed=0, router_std=0.02)
DECODE = dict(hidden=2048, inter=512, n_experts=256, top_k=8, bits=4, seed=0)
PREFILL = DECODE
SKEW = dict(hidden=2048, inter=512, n_experts=256, top_k=8, bits=8, seed=0, zipf_s=1.1)
TINY_T, DECODE_T, PREFILL_T, SKEW_T = 4, 1, 4096, 16384

# Llama-3.2-1B projections (N out, K in): fused QKV, O, fused gate/up, down
Q8_SHAPES = [(3072, 2048), (2048, 2048), (16384, 2048), (2048, 8192)]
