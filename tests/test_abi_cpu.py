"""Host-side checks of the C ABI (no GPU): the library loads, exports every entry point
the header declares, and rejects invalid calls on the host before any HIP call.

Pointers passed here are fake, never dereferenced: every call below fails validation
(or is a T = 0 no-op), which the ABI guarantees happens before anything is enqueued.
"""
import ctypes
import os
import re
import subprocess

import pytest

import quantized_sparse_moe_amd as q

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qsmoe.h")
FAKE = 0x7F0000000000          # 256-byte aligned, never dereferenced


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_0-9]+)\s*\(", text)) - {"sizeof"})


def test_library_exports_every_declared_function():
    L = q.lib()
    declared = header_functions()
    assert set(declared) == set(q.EXPORTS)
    for name in declared:
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", q.LIB_PATH], capture_output=True, text=True).stdout
    for name in declared:
        assert re.search(rf"\bT {name}$", out, flags=re.M), name


def test_abi_version_and_status_strings():
    assert q.abi_version() == 3
    for s in (0, -1, -2, -3, -4):
        assert q.status_string(s) and q.status_string(s) != "unknown status"
    assert q.status_string(7) == "unknown status"


def desc(**kw):
    d = q.moe_layer_desc()
    d.hidden, d.inter, d.n_experts, d.top_k, d.bits, d.group = 2048, 512, 256, 8, 4, 64
    d.scale_dtype = q.MOE_F16
    d.router_w = FAKE
    d.router_bias = None
    rows_gu, rows_d = 512, 2048
    d.gate = q.moe_qmat(FAKE, FAKE, FAKE, 2 * rows_gu)
    d.up = q.moe_qmat(FAKE + 512 * 1024, FAKE, FAKE, 2 * rows_gu)
    d.down = q.moe_qmat(FAKE, FAKE, FAKE, rows_d)
    d.has_shared = 1
    d.s_gate = q.moe_qmat(FAKE, FAKE, FAKE, 2 * rows_gu)
    d.s_up = q.moe_qmat(FAKE, FAKE, FAKE, 2 * rows_gu)
    d.s_down = q.moe_qmat(FAKE, FAKE, FAKE, rows_d)
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def fwd(d, T=16, x=FAKE, y=FAKE, y_dtype=q.MOE_F32, ws=FAKE, ws_bytes=1 << 40, idx=None, w=None):
    return q.lib().moe_layer_forward(ctypes.byref(d), x, T, y, y_dtype, idx, w, ws, ws_bytes, None)


def route(d, T=16, x=FAKE, ws=FAKE, ws_bytes=1 << 40, idx=FAKE, w=FAKE):
    return q.lib().moe_route(ctypes.byref(d), x, T, idx, w, ws, ws_bytes, None)


@pytest.mark.parametrize("field,value,status", [
    ("bits", 3, q.MOE_ERR_UNSUPPORTED), ("bits", 2, q.MOE_ERR_UNSUPPORTED),
    ("group", 32, q.MOE_ERR_UNSUPPORTED), ("scale_dtype", q.MOE_F32, q.MOE_ERR_UNSUPPORTED),
    ("n_experts", 0, q.MOE_ERR_UNSUPPORTED), ("n_experts", 257, q.MOE_ERR_UNSUPPORTED),
    ("top_k", 0, q.MOE_ERR_UNSUPPORTED), ("top_k", 17, q.MOE_ERR_UNSUPPORTED),
    ("hidden", 2000, q.MOE_ERR_UNSUPPORTED), ("hidden", 32, q.MOE_ERR_UNSUPPORTED),
    ("hidden", 96, q.MOE_ERR_UNSUPPORTED), ("hidden", 8256, q.MOE_ERR_UNSUPPORTED),
    ("inter", 544, q.MOE_ERR_UNSUPPORTED), ("inter", 32, q.MOE_ERR_UNSUPPORTED),
    ("inter", 2112, q.MOE_ERR_UNSUPPORTED), ("router_w", None, q.MOE_ERR_INVALID),
    ("router_w", FAKE + 8, q.MOE_ERR_INVALID), ("has_shared", 2, q.MOE_ERR_INVALID),
    ("shared_gate_w", FAKE + 8, q.MOE_ERR_INVALID),
])
def test_descriptor_validation(field, value, status):
    d = desc(**{field: value})
    assert fwd(d) == status
    assert route(d) == status
    assert q.lib().moe_workspace_size(ctypes.byref(d), 16) == ctypes.c_size_t(-1).value


def test_checkpoint_variants_accepted():
    """bf16 scales and a shared-expert gate are valid descriptors (checked through the
    workspace query, which validates without enqueueing anything); a gate without the
    shared expert is not."""
    ws = lambda d: q.lib().moe_workspace_size(ctypes.byref(d), 16)
    bad = ctypes.c_size_t(-1).value
    assert ws(desc(scale_dtype=q.MOE_BF16)) != bad
    assert ws(desc(shared_gate_w=FAKE)) != bad
    d = desc(shared_gate_w=FAKE)
    d.has_shared = 0
    assert ws(d) == bad and fwd(d) == q.MOE_ERR_INVALID


def test_multiples_of_64_accepted():
    """hidden and inter need only be multiples of 64 (one quantization group)."""
    bad = ctypes.c_size_t(-1).value
    for h, i in ((64, 64), (192, 320), (8192, 2048 - 64), (2048 + 64, 576)):
        d = desc(hidden=h, inter=i)
        for m, rows in (("gate", 2 * i), ("up", 2 * i), ("down", h), ("s_gate", 2 * i), ("s_up", 2 * i),
                        ("s_down", h)):
            setattr(d, m, q.moe_qmat(FAKE, FAKE, FAKE, rows))
        assert q.lib().moe_workspace_size(ctypes.byref(d), 16) != bad, (h, i)


def test_top_k_above_experts_and_lds_limit():
    assert fwd(desc(n_experts=4, top_k=8)) == q.MOE_ERR_UNSUPPORTED
    assert fwd(desc(top_k=16, inter=2048)) == q.MOE_ERR_UNSUPPORTED     # (k+1)*inter > 24576


def test_qmat_validation():
    d = desc()
    d.gate = q.moe_qmat(None, FAKE, FAKE, 1024)
    assert fwd(d) == q.MOE_ERR_INVALID
    d = desc()
    d.up = q.moe_qmat(FAKE + 4, FAKE, FAKE, 1024)                      # codes misaligned
    assert fwd(d) == q.MOE_ERR_INVALID
    d = desc()
    d.down = q.moe_qmat(FAKE, FAKE, FAKE, 100)                         # stride < rows
    assert fwd(d) == q.MOE_ERR_INVALID
    d = desc()
    d.s_down = q.moe_qmat(FAKE, None, FAKE, 2048)
    assert fwd(d) == q.MOE_ERR_INVALID
    d.has_shared = 0                                                     # shared ignored
    assert fwd(d, T=0) == q.MOE_OK


def test_call_validation():
    d = desc()
    assert fwd(d, T=-1) == q.MOE_ERR_INVALID
    assert fwd(d, T=0) == q.MOE_OK                                     # no work, nothing enqueued
    assert fwd(d, T=0, x=None, y=None, ws=None) == q.MOE_OK
    assert fwd(d, x=None) == q.MOE_ERR_INVALID
    assert fwd(d, x=FAKE + 2) == q.MOE_ERR_INVALID
    assert fwd(d, y=None) == q.MOE_ERR_INVALID
    assert fwd(d, y_dtype=q.MOE_F16) == q.MOE_ERR_INVALID
    assert fwd(d, y=FAKE + 2, y_dtype=q.MOE_F32) == q.MOE_ERR_INVALID
    assert fwd(d, idx=FAKE + 1) == q.MOE_ERR_INVALID
    assert fwd(d, ws=None) == q.MOE_ERR_WORKSPACE
    assert fwd(d, ws=FAKE + 64) == q.MOE_ERR_WORKSPACE
    least = q.lib().moe_workspace_size_chunked(ctypes.byref(d), 16, 2)      # the smallest accepted
    assert fwd(d, ws_bytes=least - 1) == q.MOE_ERR_WORKSPACE
    assert fwd(d, T=(1 << 20) + 1) == q.MOE_ERR_UNSUPPORTED
    assert route(d, idx=None) == q.MOE_ERR_INVALID
    assert route(d, w=FAKE + 2) == q.MOE_ERR_INVALID
    assert route(d, T=0) == q.MOE_OK


def test_workspace_sizes():
    d = desc()
    f = lambda T: q.lib().moe_workspace_size(ctypes.byref(d), T)
    assert f(0) == 0 and f(-3) == 0
    assert 0 < f(1) <= 2 << 20                                           # decode: its 2 MiB state
    prev = f(2)
    for T in (3, 17, 64, 1000, 4096):
        assert f(T) >= prev
        prev = f(T)
    # the grouped path keeps x16, h (routed + shared) and the fp16 slots (routed + shared)
    T, H, I, K = 4096, 2048, 512, 8
    assert f(T) >= 2 * T * H + 2 * (T * K + T) * I + 2 * (T * K + T) * H
    assert f(T) < 400 * 2 ** 20
    # longer prompts run in chunks of MOE_PREFILL_CHUNK tokens: the size stops there
    assert q.PREFILL_CHUNK == 4096
    assert f(4095) < f(4096) == f(4097) == f(16384) == f(1 << 20)
    g = lambda T, c: q.lib().moe_workspace_size_chunked(ctypes.byref(d), T, c)
    assert g(16384, 0) == f(16384) and g(1, 16384) == f(1) and g(100, 4096) == f(100)
    assert g(16384, 16384) > g(16384, 8192) > g(16384, 4096) == f(16384)
    assert g(16384, -1) == ctypes.c_size_t(-1).value
    # a workspace sized for small chunks bounds memory: the calls accept any size from the
    # chunk-2 size up (and pick the largest chunk that fits); below it is an error
    assert g(16384, 1024) < f(16384) and g(16384, 1) == g(16384, 2) < g(16384, 1024)
    assert fwd(d, T=16384, ws_bytes=g(16384, 2) - 1) == q.MOE_ERR_WORKSPACE
    assert route(d, T=16384, ws_bytes=g(16384, 2) - 1) == q.MOE_ERR_WORKSPACE


def test_static_entry_validation():
    """The no-workspace entry point refuses bad calls on the host, before it looks up its
    device array (so these run without a GPU)."""
    L = q.lib()
    st = lambda d, T=16, x=FAKE, y=FAKE, y_dtype=q.MOE_F32: L.moe_layer_forward_static(
        ctypes.byref(d), x, T, y, y_dtype, None, None, None)
    assert st(desc(bits=3)) == q.MOE_ERR_UNSUPPORTED
    assert st(desc(), T=-1) == q.MOE_ERR_INVALID
    assert st(desc(), T=0) == q.MOE_OK
    assert st(desc(), x=None) == q.MOE_ERR_INVALID
    assert st(desc(), y=FAKE + 2) == q.MOE_ERR_INVALID
    assert st(desc(), y_dtype=q.MOE_F16) == q.MOE_ERR_INVALID
    assert st(desc(), T=(1 << 20) + 1) == q.MOE_ERR_UNSUPPORTED


def test_workspace_status_validation():
    L = q.lib()
    assert L.moe_workspace_status(None, 1 << 20, FAKE, 0, None) == q.MOE_ERR_INVALID
    assert L.moe_workspace_status(FAKE + 64, 1 << 20, FAKE, 0, None) == q.MOE_ERR_INVALID
    assert L.moe_workspace_status(FAKE, 1 << 20, None, 0, None) == q.MOE_ERR_INVALID
    assert L.moe_workspace_status(FAKE, 1 << 20, FAKE + 2, 0, None) == q.MOE_ERR_INVALID
    assert L.moe_workspace_status(FAKE, (2 << 20) - 1, FAKE, 1, None) == q.MOE_ERR_WORKSPACE


def test_binding_constants_match_header():
    import re
    hdr = open(os.path.join(ROOT, "include", "qsmoe.h")).read()
    for name in ("MOE_OK", "MOE_ERR_INVALID", "MOE_ERR_UNSUPPORTED", "MOE_ERR_WORKSPACE", "MOE_ERR_DEVICE",
                 "MOE_BF16", "MOE_F16", "MOE_F32", "MOE_WS_ERR_DECODE_WAIT", "MOE_WS_ERR_GEMM_WAIT",
                 "MOE_ABI_VERSION"):
        m = re.search(rf"#define {name}\s+(-?\d+)u?", hdr)
        assert m, name
        want = q.abi_version() if name == "MOE_ABI_VERSION" else getattr(q, name)
        assert int(m.group(1)) == want, name


def test_prefill_chunk_matches_header():
    import re
    hdr = open(os.path.join(ROOT, "include", "qsmoe.h")).read()
    assert int(re.search(r"#define MOE_PREFILL_CHUNK (\d+)", hdr).group(1)) == q.PREFILL_CHUNK


def test_q8_validation():
    L = q.lib()
    assert L.q8_gemv(FAKE, 2048, 2048, FAKE, FAKE, q.MOE_F16, None) == q.MOE_ERR_INVALID
    assert L.q8_gemv(FAKE, 2040, 2048, FAKE, FAKE, q.MOE_F32, None) == q.MOE_ERR_UNSUPPORTED
    assert L.q8_gemv(FAKE, 2048, 2050, FAKE, FAKE, q.MOE_F32, None) == q.MOE_ERR_UNSUPPORTED
    assert L.q8_gemv(FAKE, 2048, 8224, FAKE, FAKE, q.MOE_F32, None) == q.MOE_ERR_UNSUPPORTED
    assert L.q8_gemv(FAKE, -16, 2048, FAKE, FAKE, q.MOE_F32, None) == q.MOE_ERR_INVALID
    assert L.q8_gemv(None, 2048, 2048, FAKE, FAKE, q.MOE_F32, None) == q.MOE_ERR_INVALID
    assert L.q8_gemv(FAKE + 8, 2048, 2048, FAKE, FAKE, q.MOE_F32, None) == q.MOE_ERR_INVALID
    assert L.q8_pack_rows16(FAKE, 2048, 2040, FAKE, None) == q.MOE_ERR_UNSUPPORTED
    assert L.q8_pack_rows16(FAKE, 0, 2048, FAKE, None) == q.MOE_OK
    assert L.q8_pack_rows16(FAKE, 32, 64, FAKE + 64, None) == q.MOE_ERR_INVALID     # overlap
    assert L.q8_pack_rows16(None, 32, 64, FAKE, None) == q.MOE_ERR_INVALID


def test_q8_activation_validation():
    L = q.lib()
    assert L.q8_quantize_x(FAKE, 2050, FAKE, FAKE, None) == q.MOE_ERR_UNSUPPORTED
    assert L.q8_quantize_x(FAKE, 8224, FAKE, FAKE, None) == q.MOE_ERR_UNSUPPORTED
    assert L.q8_quantize_x(FAKE, -32, FAKE, FAKE, None) == q.MOE_ERR_INVALID
    assert L.q8_quantize_x(FAKE, 0, None, None, None) == q.MOE_OK            # nothing to do
    assert L.q8_quantize_x(FAKE, 64, FAKE + 2, FAKE, None) == q.MOE_ERR_INVALID   # codes 4-byte aligned
    assert L.q8_quantize_x(None, 64, FAKE, FAKE, None) == q.MOE_ERR_INVALID
    g = lambda *a: L.q8_gemv_q8x(*a, None)
    assert g(FAKE, 2048, 2048, FAKE, FAKE, FAKE, q.MOE_F16) == q.MOE_ERR_INVALID
    assert g(FAKE, 2040, 2048, FAKE, FAKE, FAKE, q.MOE_F32) == q.MOE_ERR_UNSUPPORTED
    assert g(FAKE, 2048, 2050, FAKE, FAKE, FAKE, q.MOE_F32) == q.MOE_ERR_UNSUPPORTED
    assert g(FAKE + 8, 2048, 2048, FAKE, FAKE, FAKE, q.MOE_F32) == q.MOE_ERR_INVALID
    assert g(FAKE, 2048, 2048, FAKE + 1, FAKE, FAKE, q.MOE_F32) == q.MOE_ERR_INVALID
    assert g(FAKE, 2048, 2048, FAKE, None, FAKE, q.MOE_F32) == q.MOE_ERR_INVALID
    h = lambda *a: L.q8_gemv_qx(*a, None)
    assert h(FAKE, 2048, 2048, FAKE, FAKE, q.MOE_F16) == q.MOE_ERR_INVALID
    assert h(FAKE, 2048, 2050, FAKE, FAKE, q.MOE_F32) == q.MOE_ERR_UNSUPPORTED
    assert h(FAKE, 2048, 2048, FAKE + 4, FAKE, q.MOE_F32) == q.MOE_ERR_INVALID   # x 8-byte aligned
    assert h(FAKE, 2048, 2048, FAKE, None, q.MOE_F32) == q.MOE_ERR_INVALID


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    monkeypatch.setattr(q, "_lib", None)
    monkeypatch.setattr(q, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        q.lib()
