"""ctypes wrapper of the fp64 CPU oracle (``oracle.c``).

TEST INFRASTRUCTURE ONLY: the test-suite, the smoke check and the benchmark's
``cpu_baseline`` leg are the only users.  The product package never imports this.
It shares no code with the HIP library; the only thing both sides see is the
seeded inputs from ``qsmoe_synth``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.environ.get("QSMOE_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True, src: str = _SRC, out: str = None) -> str:
    """Compile liboracle.so with gcc (plain C, OpenMP, no fast-math)."""
    out = out or _LIB
    if force or not os.path.exists(out):
        tmp = out + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                               "-Wall", "-I", _HERE, "-o", tmp, src, "-lm"])
        os.replace(tmp, out)
    return out


class _QMat(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("biases", ctypes.c_void_p), ("mat_stride", ctypes.c_int64),
                ("sb_bf16", ctypes.c_int32)]


class _Layer(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("bits", ctypes.c_int32), ("group", ctypes.c_int32),
                ("router_w", ctypes.c_void_p), ("router_bias", ctypes.c_void_p),
                ("gate", _QMat), ("up", _QMat), ("down", _QMat),
                ("has_shared", ctypes.c_int32),
                ("s_gate", _QMat), ("s_up", _QMat), ("s_down", _QMat),
                ("shared_gate_w", ctypes.c_void_p)]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        L = ctypes.CDLL(_LIB)
        P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
        L.orc_f16_to_double.restype = ctypes.c_double
        L.orc_f16_to_double.argtypes = [ctypes.c_uint16]
        L.orc_bf16_to_double.restype = ctypes.c_double
        L.orc_bf16_to_double.argtypes = [ctypes.c_uint16]
        L.orc_f64_to_f16.argtypes = [P, I64, P]
        L.orc_dequant_matrix.argtypes = [P, I32, I64, I64, I64, P]
        L.orc_router_logits.argtypes = [P, P, I64, P]
        L.orc_route.argtypes = [P, P, I64, P, P, P]
        L.orc_layer_forward.argtypes = [P, P, I64, P, P, P]
        L.orc_layer_forward_with_routing.argtypes = [P, P, I64, P, P, P]
        L.orc_expert_mlp.argtypes = [P, P, P, P, I64, P, P]
        L.orc_q8_gemv.argtypes = [P, I64, I64, P, P]
        L.orc_q8_pack_rows16.argtypes = [P, I64, I64, P]
        L.orc_q8_unpack_rows16.argtypes = [P, I64, I64, P]
        L.orc_q8_quantize_row.argtypes = [P, I64, P]
        L.orc_q8_dequantize_row.argtypes = [P, I64, P]
        L.orc_q8_quantize_x.argtypes = [P, I64, P, P]
        L.orc_q8_gemv_q8x.argtypes = [P, I64, I64, P, P, P]
        L.orc_num_threads.restype = ctypes.c_int
        for f in ("orc_dequant_matrix", "orc_router_logits", "orc_route", "orc_layer_forward",
                  "orc_layer_forward_with_routing", "orc_expert_mlp", "orc_q8_gemv",
                  "orc_q8_pack_rows16", "orc_q8_unpack_rows16", "orc_q8_quantize_row",
                  "orc_q8_dequantize_row", "orc_q8_quantize_x", "orc_q8_gemv_q8x"):
            getattr(L, f).restype = None
        _lib = L
    return _lib


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


class OracleLayer:
    """Holds a ``qsmoe_synth.LayerInputs`` as the oracle's C descriptor.

    ``separate=True`` hands gate and up over as two distinct arrays (copies),
    otherwise as the two halves of the fused ``[gate; up]`` stack.
    """

    def __init__(self, layer, separate: bool = False):
        self.layer = layer
        self._keep = []
        E, I = layer.n_experts, layer.inter
        d = _Layer()
        d.hidden, d.inter, d.n_experts = layer.hidden, layer.inter, layer.n_experts
        d.top_k, d.bits, d.group = layer.top_k, layer.bits, 64
        rw = np.ascontiguousarray(layer.router_w, dtype=np.uint16)
        self._keep.append(rw)
        d.router_w = rw.ctypes.data
        if layer.router_bias is not None:
            rb = np.ascontiguousarray(layer.router_bias, dtype=np.float32)
            self._keep.append(rb)
            d.router_bias = rb.ctypes.data
        else:
            d.router_bias = None
        d.gate, d.up = self._gate_up(layer.gate_up, I, separate)
        d.down = self._mat(layer.down, 0, layer.down.rows)
        d.has_shared = 1 if layer.has_shared else 0
        if layer.has_shared:
            d.s_gate, d.s_up = self._gate_up(layer.s_gate_up, I, separate)
            d.s_down = self._mat(layer.s_down, 0, layer.s_down.rows)
        d.shared_gate_w = None
        if getattr(layer, "shared_gate_w", None) is not None:
            g = np.ascontiguousarray(layer.shared_gate_w, dtype=np.uint16)
            self._keep.append(g)
            d.shared_gate_w = g.ctypes.data
        self.desc = d

    def _mat(self, qm, row0: int, stride: int) -> _QMat:
        codes = np.ascontiguousarray(qm.codes)
        sc = np.ascontiguousarray(qm.scales)
        bi = np.ascontiguousarray(qm.biases)
        self._keep += [codes, sc, bi]
        cb = codes.shape[2]
        ng = sc.shape[2]
        return _QMat(codes.ctypes.data + row0 * cb, sc.ctypes.data + row0 * ng * 2,
                     bi.ctypes.data + row0 * ng * 2, stride, 1 if getattr(qm, "sb_dtype", "f16") == "bf16" else 0)

    def _gate_up(self, qm, I: int, separate: bool):
        if not separate:
            return self._mat(qm, 0, 2 * I), self._mat(qm, I, 2 * I)
        from qsmoe_synth import QMat
        g = QMat(qm.codes[:, :I].copy(), qm.scales[:, :I].copy(), qm.biases[:, :I].copy(), qm.bits)
        u = QMat(qm.codes[:, I:].copy(), qm.scales[:, I:].copy(), qm.biases[:, I:].copy(), qm.bits)
        return self._mat(g, 0, I), self._mat(u, 0, I)

    @property
    def ptr(self):
        return ctypes.addressof(self.desc)


def _x(x: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.uint16)


def router_logits(ol: OracleLayer, x: np.ndarray) -> np.ndarray:
    x = _x(x)
    T = x.shape[0]
    out = np.empty((T, ol.layer.n_experts), dtype=np.float64)
    lib().orc_router_logits(ol.ptr, x.ctypes.data, T, out.ctypes.data)
    return out


def route(ol: OracleLayer, x: np.ndarray):
    """Returns (idx [T,k] int32 ascending expert id, w [T,k] fp64, gap [T] fp64)."""
    x = _x(x)
    T, k = x.shape[0], ol.layer.top_k
    idx = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    gap = np.empty((T,), dtype=np.float64)
    lib().orc_route(ol.ptr, x.ctypes.data, T, idx.ctypes.data, w.ctypes.data, gap.ctypes.data)
    return idx, w, gap


def layer_forward(ol: OracleLayer, x: np.ndarray):
    """Returns (y [T,H] fp64, idx, w)."""
    x = _x(x)
    T, k, H = x.shape[0], ol.layer.top_k, ol.layer.hidden
    y = np.empty((T, H), dtype=np.float64)
    idx = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    lib().orc_layer_forward(ol.ptr, x.ctypes.data, T, y.ctypes.data, idx.ctypes.data,
                            w.ctypes.data)
    return y, idx, w


def layer_forward_with_routing(ol: OracleLayer, x: np.ndarray, idx: np.ndarray,
                               w: np.ndarray) -> np.ndarray:
    x = _x(x)
    T, H = x.shape[0], ol.layer.hidden
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    w = np.ascontiguousarray(w, dtype=np.float64)
    y = np.empty((T, H), dtype=np.float64)
    lib().orc_layer_forward_with_routing(ol.ptr, x.ctypes.data, T, idx.ctypes.data,
                                         w.ctypes.data, y.ctypes.data)
    return y


def dequant_matrix(qm, e: int, row0: int = 0, rows: Optional[int] = None,
                   stride: Optional[int] = None) -> np.ndarray:
    """fp64 W of matrix e of a QMat (rows row0 .. row0+rows)."""
    codes = np.ascontiguousarray(qm.codes)
    sc = np.ascontiguousarray(qm.scales)
    bi = np.ascontiguousarray(qm.biases)
    R, cb = codes.shape[1], codes.shape[2]
    ng = sc.shape[2]
    rows = R - row0 if rows is None else rows
    m = _QMat(codes.ctypes.data + row0 * cb, sc.ctypes.data + row0 * ng * 2,
              bi.ctypes.data + row0 * ng * 2, R if stride is None else stride,
              1 if getattr(qm, "sb_dtype", "f16") == "bf16" else 0)
    out = np.empty((rows, ng * 64), dtype=np.float64)
    lib().orc_dequant_matrix(ctypes.addressof(m), qm.bits, e, rows, ng * 64, out.ctypes.data)
    return out


def q8_gemv(rows: np.ndarray, N: int, K: int, x: np.ndarray) -> np.ndarray:
    rows = np.ascontiguousarray(rows, dtype=np.uint8)
    assert rows.size == N * (K // 32) * 34
    x = _x(x)
    y = np.empty((N,), dtype=np.float64)
    lib().orc_q8_gemv(rows.ctypes.data, N, K, x.ctypes.data, y.ctypes.data)
    return y


def q8_pack_rows16(rows: np.ndarray, N: int, K: int) -> np.ndarray:
    rows = np.ascontiguousarray(rows, dtype=np.uint8)
    out = np.empty((N // 16 * (K // 32) * 544,), dtype=np.uint8)
    lib().orc_q8_pack_rows16(rows.ctypes.data, N, K, out.ctypes.data)
    return out


def q8_unpack_rows16(tiles: np.ndarray, N: int, K: int) -> np.ndarray:
    tiles = np.ascontiguousarray(tiles, dtype=np.uint8)
    out = np.empty((N, K // 32, 34), dtype=np.uint8)
    lib().orc_q8_unpack_rows16(tiles.ctypes.data, N, K, out.ctypes.data)
    return out


def q8_quantize_row(v: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float32)
    K = v.shape[0]
    out = np.empty((K // 32, 34), dtype=np.uint8)
    lib().orc_q8_quantize_row(v.ctypes.data, K, out.ctypes.data)
    return out


def q8_dequantize_row(blocks: np.ndarray, K: int) -> np.ndarray:
    blocks = np.ascontiguousarray(blocks, dtype=np.uint8)
    out = np.empty((K,), dtype=np.float64)
    lib().orc_q8_dequantize_row(blocks.ctypes.data, K, out.ctypes.data)
    return out


def q8_quantize_x(x_bf16: np.ndarray):
    """Activation quantization (bf16 bits [K] -> int8 codes [K], fp16 scale bits [K/32])."""
    x = np.ascontiguousarray(x_bf16).view(np.uint16)
    K = x.shape[0]
    q = np.empty((K,), dtype=np.int8)
    d = np.empty((K // 32,), dtype=np.uint16)
    lib().orc_q8_quantize_x(x.ctypes.data, K, q.ctypes.data, d.ctypes.data)
    return q, d


def q8_gemv_q8x(rows: np.ndarray, N: int, K: int, xq: np.ndarray, xd: np.ndarray) -> np.ndarray:
    """GEMV over row-contiguous Q8_0 blocks with a quantized activation (fp64 result)."""
    rows = np.ascontiguousarray(rows, dtype=np.uint8)
    xq = np.ascontiguousarray(xq, dtype=np.int8)
    xd = np.ascontiguousarray(xd, dtype=np.uint16)
    y = np.empty((N,), dtype=np.float64)
    lib().orc_q8_gemv_q8x(rows.ctypes.data, N, K, xq.ctypes.data, xd.ctypes.data, y.ctypes.data)
    return y


def f16_to_double(h: int) -> float:
    return lib().orc_f16_to_double(int(h))


def f64_to_f16(v: np.ndarray) -> np.ndarray:
    """The oracle's binary64 -> binary16 encoder (used by its Q8_0 quantizers) over an
    array; returns the uint16 bit patterns."""
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty(v.shape, np.uint16)
    lib().orc_f64_to_f16(_p(v), v.size, _p(out))
    return out


def bf16_to_double(b: int) -> float:
    return lib().orc_bf16_to_double(int(b))


def num_threads() -> int:
    return lib().orc_num_threads()
