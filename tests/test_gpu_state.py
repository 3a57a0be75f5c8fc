"""GPU tests of the workspace state the one-launch decode kernels keep between calls, the
error word that reports a bounded wait that gave up, and calls on a side stream.

The decode state at the start of a workspace (uint32 words): 0 = error word, 32 = the
bound on the polls of one wait (0: the default), 64 = the generation of the last
completed call.  Forcing a tiny bound makes the waits give up at once: every kernel
still runs to its end (a wait that gives up goes on with whatever it holds, every index
it uses is clamped into range), the error word says so, and the outputs of that call are
not used.
"""
import numpy as np
import pytest

import qsmoe_synth as syn
from gpu_util import to_dev

pytestmark = pytest.mark.gpu

CTL_ERR, CTL_SPIN, CTL_GEN = 0, 32, 64


@pytest.fixture(scope="module")
def torch():
    import torch as t
    assert t.cuda.is_available(), "GPU tests need a ROCm device"
    return t


@pytest.fixture(scope="module")
def qs():
    import quantized_sparse_moe_amd as q
    q.lib()
    return q


@pytest.fixture(scope="module")
def decode_layer(qs):
    L = syn.make_layer(**syn.DECODE)
    return L, qs.LayerDesc.from_host(L)


def status(qs, torch, ws, clear=False):
    out = qs.moe_workspace_status(ws, clear=clear)
    torch.cuda.synchronize()
    return int(out.cpu().numpy().view(np.uint32)[0])


def set_word(torch, ws, i, v):
    w = ws[:1 << 20].view(torch.int32)
    w[i] = int(np.uint32(v).view(np.int32))
    torch.cuda.synchronize()


def word(torch, ws, i):
    return int(ws[:1 << 20].view(torch.int32)[i].cpu().numpy().view(np.uint32))


def fresh(qs, torch, desc, x, T, route=False):
    ws = qs.new_workspace(desc, max(T, 64))
    if route:
        r = qs.moe_route(desc, x, workspace=ws)
    else:
        r = qs.moe_layer_forward(desc, x, workspace=ws)
    torch.cuda.synchronize()
    return r


def test_interleaved_calls_share_one_workspace(torch, qs, decode_layer):
    """T = 1, 3, 6, route-only and T = 40 calls interleaved on one workspace and one
    stream give the same bits as each call on a fresh workspace; no wait gave up."""
    L, desc = decode_layer
    xs = {T: to_dev(syn.make_x(T, L.hidden, seed=50 + T), torch) for T in (1, 3, 6, 40)}
    ref = {T: fresh(qs, torch, desc, xs[T], T) for T in xs}
    ref_route = {T: fresh(qs, torch, desc, xs[T], T, route=True) for T in (1, 3, 40)}
    ws = qs.new_workspace(desc, 64)
    order = [1, 3, "r1", 6, 40, 1, "r40", 3, 1, "r3", 40, 6, 1] * 3
    outs = []
    for c in order:
        if isinstance(c, str):
            T = int(c[1:])
            outs.append((c, qs.moe_route(desc, xs[T], workspace=ws)))
        else:
            outs.append((c, qs.moe_layer_forward(desc, xs[c], workspace=ws)))
    torch.cuda.synchronize()
    for c, r in outs:
        if isinstance(c, str):
            T = int(c[1:])
            assert torch.equal(r[0], ref_route[T][0]) and torch.equal(r[1], ref_route[T][1]), c
        else:
            assert torch.equal(r, ref[c]), c
    assert status(qs, torch, ws) == 0
    # the routing of the layer calls equals moe_route's
    for T in (1, 3, 40):
        idx = torch.empty((T, L.top_k), dtype=torch.int32, device="cuda")
        w = torch.empty((T, L.top_k), dtype=torch.float32, device="cuda")
        qs.moe_layer_forward(desc, xs[T], topk_idx=idx, topk_w=w, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(idx, ref_route[T][0]) and torch.equal(w, ref_route[T][1]), T


@pytest.mark.parametrize("T", [1, 3])
def test_generation_wrap_skips_the_zero_tag(torch, qs, decode_layer, T):
    """A workspace whose call counter is about to wrap: the next call must not take tag 0,
    the tag of the zeroed words nobody has written, or its readers would accept them."""
    L, desc = decode_layer
    x = to_dev(syn.make_x(T, L.hidden, seed=70 + T), torch)
    ref = fresh(qs, torch, desc, x, T)
    ws = qs.new_workspace(desc, 64)
    set_word(torch, ws, CTL_GEN, 0xFFFFFFFF)
    y = qs.moe_layer_forward(desc, x, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(y, ref)
    assert word(torch, ws, CTL_GEN) == 1
    assert status(qs, torch, ws) == 0


def test_forced_give_up_is_reported(torch, qs, decode_layer):
    """With a poll bound of 1 the waits of a T = 1 call give up: the kernel still ends,
    and the error word carries the decode bit; clearing it reads it once more and resets
    it.  A grouped-path call (T = 40) with the same bound ends too and sets at most the
    GEMM bit.  A workspace used this way is then discarded."""
    L, desc = decode_layer
    x1 = to_dev(syn.make_x(1, L.hidden, seed=90), torch)
    ws = qs.new_workspace(desc, 64)
    set_word(torch, ws, CTL_SPIN, 1)
    qs.moe_layer_forward(desc, x1, workspace=ws)
    torch.cuda.synchronize()
    st = status(qs, torch, ws, clear=True)
    assert st & qs.MOE_WS_ERR_DECODE_WAIT, st
    assert status(qs, torch, ws) == 0
    del ws
    x40 = to_dev(syn.make_x(40, L.hidden, seed=91), torch)
    ws = qs.new_workspace(desc, 64)
    set_word(torch, ws, CTL_SPIN, 1)
    qs.moe_layer_forward(desc, x40, workspace=ws)
    torch.cuda.synchronize()
    st = status(qs, torch, ws)
    assert st & ~qs.MOE_WS_ERR_GEMM_WAIT == 0, st
    print(f"[state] grouped call with poll bound 1: error word {st}", flush=True)
    del ws
    # a fresh workspace afterwards: normal results, no error
    ws = qs.new_workspace(desc, 64)
    y = qs.moe_layer_forward(desc, x1, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(y, fresh(qs, torch, desc, x1, 1))
    assert status(qs, torch, ws) == 0


@pytest.mark.parametrize("T", [1, 40])
def test_side_stream_call(torch, qs, decode_layer, T):
    """A call on a stream other than torch's current one, with the output and workspace
    allocated by the binding: allocated and zeroed on that stream, so the result equals
    the current-stream call bit for bit."""
    L, desc = decode_layer
    x = to_dev(syn.make_x(T, L.hidden, seed=110 + T), torch)
    ref = fresh(qs, torch, desc, x, T)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    y = qs.moe_layer_forward(desc, x, stream=s)
    idx, w = qs.moe_route(desc, x, stream=s)
    s.synchronize()
    assert torch.equal(y, ref)
    ri, rw = fresh(qs, torch, desc, x, T, route=True)
    assert torch.equal(idx, ri) and torch.equal(w, rw)
