"""Python binding of libqsmoe, the MI355X (gfx950) quantized sparse MoE layer library.

Argument marshalling only: every step of the layer runs in the HIP kernels of
``libqsmoe.so`` behind the C ABI declared in ``include/qsmoe.h``.  PyTorch supplies
device memory and the current stream; outputs and workspaces the caller does not pass
are allocated here with torch.  The functions carry the names of the C entry points:

    moe_workspace_size, moe_workspace_status, moe_route, moe_layer_forward, q8_gemv,
    q8_quantize_x, q8_gemv_q8x, q8_gemv_qx, q8_pack_rows16

There is no fallback: if the shared library is missing, loading raises.
Build it with ``python -m quantized_sparse_moe_amd.build``.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqsmoe.so")

MOE_OK, MOE_ERR_INVALID, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_DEVICE = 0, -1, -2, -3, -4
MOE_BF16, MOE_F16, MOE_F32 = 0, 1, 2
MOE_WS_ERR_DECODE_WAIT, MOE_WS_ERR_GEMM_WAIT = 1, 2      # bits of the workspace error word

_lib = None


class QsmoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


class moe_qmat(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("biases", ctypes.c_void_p), ("mat_stride", ctypes.c_int64)]


class moe_layer_desc(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("bits", ctypes.c_int32), ("group", ctypes.c_int32),
                ("scale_dtype", ctypes.c_int32),
                ("router_w", ctypes.c_void_p), ("router_bias", ctypes.c_void_p),
                ("gate", moe_qmat), ("up", moe_qmat), ("down", moe_qmat),
                ("has_shared", ctypes.c_int32),
                ("s_gate", moe_qmat), ("s_up", moe_qmat), ("s_down", moe_qmat),
                ("shared_gate_w", ctypes.c_void_p)]


EXPORTS = ("moe_abi_version", "moe_status_string", "moe_workspace_size",
           "moe_workspace_size_chunked", "moe_workspace_status", "moe_route",
           "moe_layer_forward", "moe_layer_forward_static", "q8_gemv", "q8_quantize_x", "q8_gemv_q8x", "q8_gemv_qx",
           "q8_pack_rows16", "moe_calib_read", "moe_calib_mfma")


def lib() -> ctypes.CDLL:
    """Load libqsmoe.so (raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m quantized_sparse_moe_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        L.moe_abi_version.restype = ctypes.c_int
        L.moe_abi_version.argtypes = []
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_status_string.argtypes = [I32]
        L.moe_workspace_size.restype = SZ
        L.moe_workspace_size.argtypes = [P, I64]
        L.moe_workspace_size_chunked.restype = SZ
        L.moe_workspace_size_chunked.argtypes = [P, I64, I64]
        L.moe_workspace_status.restype = I32
        L.moe_workspace_status.argtypes = [P, SZ, P, I32, P]
        L.moe_route.restype = I32
        L.moe_route.argtypes = [P, P, I64, P, P, P, SZ, P]
        L.moe_layer_forward.restype = I32
        L.moe_layer_forward.argtypes = [P, P, I64, P, I32, P, P, P, SZ, P]
        L.moe_layer_forward_static.restype = I32
        L.moe_layer_forward_static.argtypes = [P, P, I64, P, I32, P, P, P]
        L.q8_gemv.restype = I32
        L.q8_gemv.argtypes = [P, I64, I64, P, P, I32, P]
        L.q8_quantize_x.restype = I32
        L.q8_quantize_x.argtypes = [P, I64, P, P, P]
        L.q8_gemv_q8x.restype = I32
        L.q8_gemv_q8x.argtypes = [P, I64, I64, P, P, P, I32, P]
        L.q8_gemv_qx.restype = I32
        L.q8_gemv_qx.argtypes = [P, I64, I64, P, P, I32, P]
        L.q8_pack_rows16.restype = I32
        L.q8_pack_rows16.argtypes = [P, I64, I64, P, P]
        L.moe_calib_read.restype = I32
        L.moe_calib_read.argtypes = [P, SZ, P]
        L.moe_calib_mfma.restype = I32
        L.moe_calib_mfma.argtypes = [I32, I32, P]
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().moe_status_string(int(status)).decode()


def abi_version() -> int:
    return lib().moe_abi_version()


def _check(status: int, where: str) -> None:
    if status != MOE_OK:
        raise QsmoeError(status, where)


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _alloc_stream(stream):
    """The stream that buffers allocated here for a call on `stream` belong to.

    torch's caching allocator hands a freed block only to later work on the stream it was
    allocated on, and torch.zeros fills on the current stream: allocating under the call's
    own stream orders the fill before the kernel and keeps the block from being reused
    while the kernel may still run.  A raw stream handle cannot be told to torch, so a
    call on one must pass every buffer itself."""
    import torch
    if stream is None or isinstance(stream, torch.cuda.Stream):
        return stream or torch.cuda.current_stream()
    raise QsmoeError(MOE_ERR_INVALID, "a raw stream handle needs caller-provided outputs and workspace")


# ---------------------------------------------------------------- layer descriptor
class LayerDesc:
    """A ``moe_layer_desc`` plus the device tensors it points into.

    ``gate``, ``up``, ``down`` (and ``s_gate``, ``s_up``, ``s_down`` for the shared
    expert) are ``(codes, scales, biases, mat_stride, row0)`` tuples of device tensors:
    matrix e, row r lives at row ``row0 + e*mat_stride + r`` of those tensors.
    """

    def __init__(self, hidden, inter, n_experts, top_k, bits, router_w, gate, up, down,
                 router_bias=None, shared=None, scale_dtype=MOE_F16, shared_gate_w=None):
        self.hidden, self.inter, self.n_experts, self.top_k, self.bits = hidden, inter, n_experts, top_k, bits
        self._keep = [router_w, router_bias, gate, up, down, shared, shared_gate_w]
        d = moe_layer_desc()
        d.hidden, d.inter, d.n_experts, d.top_k, d.bits, d.group = hidden, inter, n_experts, top_k, bits, 64
        d.scale_dtype = scale_dtype
        d.shared_gate_w = None if shared_gate_w is None else shared_gate_w.data_ptr()
        d.router_w = router_w.data_ptr()
        d.router_bias = None if router_bias is None else router_bias.data_ptr()
        d.gate, d.up = self._qmat(gate, hidden), self._qmat(up, hidden)
        d.down = self._qmat(down, inter)
        d.has_shared = 0 if shared is None else 1
        if shared is not None:
            d.s_gate, d.s_up, d.s_down = (self._qmat(shared[0], hidden), self._qmat(shared[1], hidden),
                                          self._qmat(shared[2], inter))
        self.desc = d

    def _qmat(self, m, cols: int) -> moe_qmat:
        codes, scales, biases, stride, row0 = m
        rb = cols * self.bits // 8
        ng = cols // 64
        return moe_qmat(codes.data_ptr() + row0 * rb, scales.data_ptr() + row0 * ng * 2,
                          biases.data_ptr() + row0 * ng * 2, stride)

    @property
    def ptr(self) -> int:
        return ctypes.addressof(self.desc)

    @classmethod
    def from_host(cls, layer, device="cuda", fused: bool = True) -> "LayerDesc":
        """Upload a host layer (numpy arrays laid out as ``qsmoe_synth.LayerInputs``).

        ``fused=True`` passes gate and up as the two halves of one [gate; up] stack;
        ``fused=False`` copies them into two separate stacks.
        """
        import numpy as np
        import torch

        def dev(a):
            a = np.ascontiguousarray(a)
            if a.dtype == np.uint16:
                a = a.view(np.int16)
            return torch.from_numpy(a).to(device)

        I = layer.inter

        def gate_up(qm):
            c, s, b = dev(qm.codes), dev(qm.scales), dev(qm.biases)
            if fused:
                return (c, s, b, 2 * I, 0), (c, s, b, 2 * I, I)
            g = (c[:, :I].contiguous(), s[:, :I].contiguous(), b[:, :I].contiguous(), I, 0)
            u = (c[:, I:].contiguous(), s[:, I:].contiguous(), b[:, I:].contiguous(), I, 0)
            return g, u

        g, u = gate_up(layer.gate_up)
        dn = (dev(layer.down.codes), dev(layer.down.scales), dev(layer.down.biases), layer.hidden, 0)
        shared = None
        if layer.has_shared:
            sg, su = gate_up(layer.s_gate_up)
            sd = (dev(layer.s_down.codes), dev(layer.s_down.scales), dev(layer.s_down.biases),
                  layer.hidden, 0)
            shared = (sg, su, sd)
        rb = None if layer.router_bias is None else dev(np.asarray(layer.router_bias, np.float32))
        sgw = getattr(layer, "shared_gate_w", None)
        return cls(layer.hidden, I, layer.n_experts, layer.top_k, layer.bits, dev(layer.router_w),
                   g, u, dn, router_bias=rb, shared=shared,
                   scale_dtype=MOE_BF16 if getattr(layer, "scale_dtype", "f16") == "bf16" else MOE_F16,
                   shared_gate_w=None if sgw is None else dev(sgw))


# ------------------------------------------------------------------- entry points
# tokens per prefill chunk inside one call (MOE_PREFILL_CHUNK in include/qsmoe.h)
PREFILL_CHUNK = 4096


def moe_workspace_size(desc: LayerDesc, T: int, chunk: Optional[int] = None) -> int:
    """Workspace bytes for T tokens; `chunk` (tokens per prefill chunk, T for none) as in
    moe_workspace_size_chunked, default MOE_PREFILL_CHUNK."""
    if chunk is None:
        n = lib().moe_workspace_size(desc.ptr, int(T))
    else:
        n = lib().moe_workspace_size_chunked(desc.ptr, int(T), int(chunk))
    if n == ctypes.c_size_t(-1).value:
        raise QsmoeError(MOE_ERR_UNSUPPORTED, "moe_workspace_size")
    return n


def new_workspace(desc: LayerDesc, T: int, chunk: Optional[int] = None, device="cuda", stream=None):
    """A zero-filled workspace for T tokens, allocated and filled on `stream`."""
    import torch
    with torch.cuda.stream(_alloc_stream(stream)):
        return torch.zeros(max(moe_workspace_size(desc, T, chunk), 256), dtype=torch.uint8, device=device)


def _workspace(desc: LayerDesc, T: int, workspace, device, stream):
    if workspace is None:
        # zero-filled: the start of the workspace holds decode state that must begin at zero
        workspace = new_workspace(desc, T, device=device, stream=stream)
    return workspace, workspace.numel() * workspace.element_size()


def _empty(shape, dtype, device, stream):
    import torch
    with torch.cuda.stream(_alloc_stream(stream)):
        return torch.empty(shape, dtype=dtype, device=device)


def moe_workspace_status(workspace, clear: bool = False, out=None, stream=None):
    """Enqueue a read of the workspace's error word (MOE_WS_ERR_* bits); returns a device
    uint32 tensor [1] (int32 view) that holds it once the stream reaches the read."""
    import torch
    if out is None:
        out = _empty((1,), torch.int32, workspace.device, stream)
    _check(lib().moe_workspace_status(_ptr(workspace), workspace.numel() * workspace.element_size(),
                                      _ptr(out), 1 if clear else 0, _stream(stream)), "moe_workspace_status")
    return out


def moe_route(desc: LayerDesc, x, topk_idx=None, topk_w=None, workspace=None,
              stream=None) -> Tuple["object", "object"]:
    """Router + top-k: returns (topk_idx int32 [T, k], topk_w fp32 [T, k])."""
    import torch
    T = x.shape[0]
    if topk_idx is None:
        topk_idx = _empty((T, desc.top_k), torch.int32, x.device, stream)
    if topk_w is None:
        topk_w = _empty((T, desc.top_k), torch.float32, x.device, stream)
    ws, nbytes = _workspace(desc, T, workspace, x.device, stream)
    _check(lib().moe_route(desc.ptr, _ptr(x), T, _ptr(topk_idx), _ptr(topk_w), _ptr(ws), nbytes,
                           _stream(stream)), "moe_route")
    return topk_idx, topk_w


def moe_layer_forward(desc: LayerDesc, x, y=None, y_dtype=None, topk_idx=None, topk_w=None,
                      workspace=None, stream=None):
    """The whole MoE layer on bf16 ``x`` [T, hidden]; returns ``y`` (fp32 or bf16)."""
    import torch
    T = x.shape[0]
    if y is None:
        y = _empty((T, desc.hidden), y_dtype or torch.float32, x.device, stream)
    code = MOE_F32 if y.dtype == torch.float32 else MOE_BF16 if y.dtype == torch.bfloat16 else None
    if code is None:
        raise QsmoeError(MOE_ERR_INVALID, "moe_layer_forward: y must be float32 or bfloat16")
    ws, nbytes = _workspace(desc, T, workspace, x.device, stream)
    _check(lib().moe_layer_forward(desc.ptr, _ptr(x), T, _ptr(y), code, _ptr(topk_idx), _ptr(topk_w),
                                   _ptr(ws), nbytes, _stream(stream)), "moe_layer_forward")
    return y


def moe_layer_forward_static(desc: LayerDesc, x, y=None, y_dtype=None, topk_idx=None, topk_w=None,
                             stream=None):
    """The whole layer without a workspace (the library's static per-GPU array); the C
    call allocates nothing -- pass ``y`` to allocate nothing here either."""
    import torch
    T = x.shape[0]
    if y is None:
        y = _empty((T, desc.hidden), y_dtype or torch.float32, x.device, stream)
    _check(lib().moe_layer_forward_static(desc.ptr, _ptr(x), T, _ptr(y), _out_code(y, "moe_layer_forward_static"),
                                          _ptr(topk_idx), _ptr(topk_w), _stream(stream)),
           "moe_layer_forward_static")
    return y


def _out_code(y, where):
    import torch
    code = MOE_F32 if y.dtype == torch.float32 else MOE_BF16 if y.dtype == torch.bfloat16 else None
    if code is None:
        raise QsmoeError(MOE_ERR_INVALID, f"{where}: y must be float32 or bfloat16")
    return code


def q8_gemv(w_tiles, N: int, K: int, x, y=None, y_dtype=None, stream=None):
    """Dense Q8_0 GEMV over 16-row packed tiles; returns ``y`` [N] (fp32 or bf16)."""
    import torch
    if y is None:
        y = _empty((N,), y_dtype or torch.float32, x.device, stream)
    _check(lib().q8_gemv(_ptr(w_tiles), N, K, _ptr(x), _ptr(y), _out_code(y, "q8_gemv"), _stream(stream)),
           "q8_gemv")
    return y


def q8_quantize_x(x, K: int = None, xq=None, xd=None, stream=None):
    """Q8_0 quantization of an activation ``x`` [K] (bf16 bits); returns (codes int8 [K],
    scales fp16 bits [K/32]), to be shared by the GEMVs that read ``x``."""
    import torch
    K = x.numel() if K is None else K
    if xq is None:
        xq = _empty((K,), torch.int8, x.device, stream)
    if xd is None:
        xd = _empty((K // 32,), torch.int16, x.device, stream)
    _check(lib().q8_quantize_x(_ptr(x), K, _ptr(xq), _ptr(xd), _stream(stream)), "q8_quantize_x")
    return xq, xd


def q8_gemv_q8x(w_tiles, N: int, K: int, xq, xd, y=None, y_dtype=None, stream=None):
    """Dense Q8_0 GEMV with a quantized activation (``q8_quantize_x``); returns ``y`` [N]."""
    import torch
    if y is None:
        y = _empty((N,), y_dtype or torch.float32, xq.device, stream)
    _check(lib().q8_gemv_q8x(_ptr(w_tiles), N, K, _ptr(xq), _ptr(xd), _ptr(y), _out_code(y, "q8_gemv_q8x"),
                             _stream(stream)), "q8_gemv_q8x")
    return y


def q8_gemv_qx(w_tiles, N: int, K: int, x, y=None, y_dtype=None, stream=None):
    """Dense Q8_0 GEMV quantizing ``x`` (bf16) inside the kernel; returns ``y`` [N]."""
    import torch
    if y is None:
        y = _empty((N,), y_dtype or torch.float32, x.device, stream)
    _check(lib().q8_gemv_qx(_ptr(w_tiles), N, K, _ptr(x), _ptr(y), _out_code(y, "q8_gemv_qx"), _stream(stream)),
           "q8_gemv_qx")
    return y


def q8_pack_rows16(w_rows, N: int, K: int, w_tiles=None, stream=None):
    """Row-contiguous Q8_0 blocks -> 16-row packed tiles (load-time, on the device)."""
    import torch
    if w_tiles is None:
        w_tiles = _empty((N // 16 * (K // 32) * 544,), torch.uint8, w_rows.device, stream)
    _check(lib().q8_pack_rows16(_ptr(w_rows), N, K, _ptr(w_tiles), _stream(stream)), "q8_pack_rows16")
    return w_tiles


def moe_calib_read(buf, stream=None):
    """Enqueue one read-only pass over the device buffer `buf` (measured HBM ceiling)."""
    _check(lib().moe_calib_read(_ptr(buf), buf.numel() * buf.element_size(), _stream(stream)), "moe_calib_read")


def moe_calib_mfma(iters: int, blocks: int, stream=None):
    """Enqueue the MFMA-only loop: blocks x 4 waves x iters x 8 MFMAs of 16384 flops."""
    _check(lib().moe_calib_mfma(iters, blocks, _stream(stream)), "moe_calib_mfma")
