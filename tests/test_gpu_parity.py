"""GPU parity of the HIP path (through the C ABI) against the fp64 CPU oracle.

Sizes: small cases the oracle finishes in seconds (several tiles plus ragged tails),
and the full workload sizes in the launch configuration the benchmark times (a
workspace for the whole T, bf16 output), checked on sampled tokens (tokens are
independent, so the oracle evaluates just those rows).
Bit-exact invariants: fused [gate; up] == separate gate and up, repeat calls,
token permutation and chunking.
"""
import dataclasses

import numpy as np
import pytest

import oracle
import qsmoe_synth as syn
from gpu_util import (TAU, W_TOL, check_output, check_routing, report, sample_tokens, to_dev, y_to_np)

pytestmark = pytest.mark.gpu


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


_LAYERS = {}


def layer(name, **over):
    key = (name, tuple(sorted(over.items())))
    if key not in _LAYERS:
        cfg = dict(getattr(syn, name)) if isinstance(name, str) else dict(name)
        cfg.update(over)
        _LAYERS.clear()                       # keep one big layer resident at a time
        _LAYERS[key] = syn.make_layer(**cfg)
    return _LAYERS[key]


def run_layer(torch, qs, L, x_np, fused=True, bf16_out=False, desc=None):
    desc = desc or qs.LayerDesc.from_host(L, fused=fused)
    x = to_dev(x_np, torch)
    T = x_np.shape[0]
    idx = torch.empty((T, L.top_k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, L.top_k), dtype=torch.float32, device="cuda")
    y = qs.moe_layer_forward(desc, x, y_dtype=torch.bfloat16 if bf16_out else torch.float32,
                             topk_idx=idx, topk_w=w)
    torch.cuda.synchronize()
    return y, idx.cpu().numpy(), w.cpu().numpy()


def oracle_check(L, x_np, y, idx, w, bf16_out, what, rows=None, torch=None):
    """Compare GPU (y, idx, w) with the oracle on `rows` (default: all tokens)."""
    rows = np.arange(x_np.shape[0]) if rows is None else rows
    ol = oracle.OracleLayer(L)
    xs = x_np[rows]
    idx_r, w_r, gap = oracle.route(ol, xs)
    amb, wmax = check_routing(idx[rows], w[rows], idx_r, w_r, gap)
    # evaluate the oracle on the GPU's routing where it is ambiguous, its own elsewhere
    use_idx = np.where(amb[:, None], idx[rows], idx_r)
    use_w = np.where(amb[:, None], w[rows].astype(np.float64), w_r)
    ref = oracle.layer_forward_with_routing(ol, xs, use_idx, use_w)
    rel = check_output(y[rows], ref, bf16_out, what)
    report(what, err_over_rms=rel, ambiguous=f"{int(amb.sum())}/{len(rows)}", w_err=wmax)
    return rel, int(amb.sum())


# ------------------------------------------------------------------------- routing
@pytest.mark.parametrize("cfg,T,nsample", [("TINY", 4, None), ("TINY", 200, None), ("DECODE", 1, None),
                                           ("PREFILL", 4096, 256), ("SKEW", 16384, 256)])
def test_route_parity(torch, qs, cfg, T, nsample):
    L = layer(cfg)
    x_np = syn.make_x(T, L.hidden, seed=11)
    desc = qs.LayerDesc.from_host(L)
    idx, w = qs.moe_route(desc, to_dev(x_np, torch))
    torch.cuda.synchronize()
    idx, w = idx.cpu().numpy(), w.cpu().numpy()
    rows = np.arange(T) if nsample is None else sample_tokens(T, nsample, seed=T)
    idx_r, w_r, gap = oracle.route(oracle.OracleLayer(L), x_np[rows])
    amb, wmax = check_routing(idx[rows], w[rows], idx_r, w_r, gap)
    report(f"route {cfg} T={T}", ambiguous=f"{int(amb.sum())}/{len(rows)}", w_err=wmax)
    assert ((idx >= 0) & (idx < L.n_experts)).all()


@pytest.mark.parametrize("cfg,k", [("TINY", 3), ("DECODE", 7)])
def test_route_exact_ties(torch, qs, cfg, k):
    """Router rows duplicated in pairs give exactly equal logits on both sides; with an
    odd k the last selected pair is split and its lower id must be taken.  x = 0 makes
    every logit 0: the k lowest ids, each with weight 1/k.  Decode (T = 1) and prefill
    routers both."""
    base = layer(cfg)
    rw = base.router_w.copy()
    rw[1::2] = rw[0::2]
    L = dataclasses.replace(base, top_k=k, router_w=rw, router_bias=None)
    desc = qs.LayerDesc.from_host(L)
    ol = oracle.OracleLayer(L)
    x_np = syn.make_x(64, L.hidden, seed=5)
    lg = oracle.router_logits(ol, x_np)                       # fp64, pairs exactly equal
    assert (lg[:, 1::2] == lg[:, 0::2]).all()
    idx_r, w_r, _ = oracle.route(ol, x_np)
    # unambiguous tokens: the split pair is at least TAU away from the pairs beside it
    pv = -np.sort(-lg[:, 0::2], axis=1)
    m = (k + 1) // 2
    ok = (pv[:, m - 2] - pv[:, m - 1] >= TAU) & (pv[:, m - 1] - pv[:, m] >= TAU)
    assert ok.sum() >= 48
    assert (idx_r % 2 == 0).sum(axis=1).tolist() == [m] * len(x_np)   # oracle: lower id of the split pair
    zero = np.zeros((1, L.hidden), np.uint16)
    for T in (1, 64):
        rows = range(0, 64, 8) if T == 1 else [slice(0, 64)]
        for r in rows:
            xs = x_np[r] if T == 64 else x_np[r:r + 1]
            idx, w = qs.moe_route(desc, to_dev(xs, torch))
            torch.cuda.synchronize()
            sel = np.arange(64)[r] if T == 64 else np.array([r])
            good = ok[sel]
            assert (idx.cpu().numpy()[good] == idx_r[sel][good]).all(), f"T={T} rows {r}"
            assert np.abs(w.cpu().numpy()[good] - w_r[sel][good]).max() <= W_TOL
        xz = np.repeat(zero, T, axis=0)
        idx, w = qs.moe_route(desc, to_dev(xz, torch))
        torch.cuda.synchronize()
        assert (idx.cpu().numpy() == np.arange(k)[None, :]).all(), f"x = 0, T={T}"
        assert np.abs(w.cpu().numpy() - 1.0 / k).max() <= 1e-7


# -------------------------------------------------------------------- whole layer
@pytest.mark.parametrize("bf16_out", [False, True])
def test_decode_parity(torch, qs, bf16_out):
    """T = 1 decode kernels at the decode workload, several tokens one at a time."""
    L = layer("DECODE")
    desc = qs.LayerDesc.from_host(L)
    xs = syn.make_x(6, L.hidden, seed=3)
    for t in range(xs.shape[0]):
        y, idx, w = run_layer(torch, qs, L, xs[t:t + 1], bf16_out=bf16_out, desc=desc)
        oracle_check(L, xs[t:t + 1], y_to_np(y, torch), idx, w, bf16_out, f"decode token {t}")


@pytest.mark.parametrize("bf16_out", [False, True])
def test_tiny_grouped_and_decode(torch, qs, bf16_out):
    """Tiny layer: T = 4 in one small-batch call and as 4 separate T = 1 calls."""
    L = layer("TINY")
    x_np = syn.make_x(4, L.hidden, seed=0)
    y, idx, w = run_layer(torch, qs, L, x_np, bf16_out=bf16_out)
    oracle_check(L, x_np, y_to_np(y, torch), idx, w, bf16_out, "tiny grouped")
    for t in range(4):
        y1, i1, w1 = run_layer(torch, qs, L, x_np[t:t + 1], bf16_out=bf16_out)
        oracle_check(L, x_np[t:t + 1], y_to_np(y1, torch), i1, w1, bf16_out, f"tiny decode {t}")


@pytest.mark.parametrize("cfg,T", [("DECODE", 2), ("DECODE", 40), ("DECODE", 97), ("SKEW", 64)])
def test_grouped_small_parity(torch, qs, cfg, T):
    """Grouped path, every token checked: small T spans many tiles and ragged tails."""
    L = layer(cfg)
    x_np = syn.make_x(T, L.hidden, seed=T)
    for bf16_out in (False, True):
        y, idx, w = run_layer(torch, qs, L, x_np, bf16_out=bf16_out)
        oracle_check(L, x_np, y_to_np(y, torch), idx, w, bf16_out, f"{cfg} T={T}")


@pytest.mark.parametrize("cfg,T", [("DECODE", 2), ("DECODE", 3), ("DECODE", 4), ("DECODE", 5), ("DECODE", 8),
                                   ("SKEW", 2), ("SKEW", 3), ("SKEW", 4), ("SKEW", 6), ("SKEW", 7)])
def test_small_batch_decode_parity(torch, qs, cfg, T):
    """Small-batch decode (T = 2..4 in one launch, 5..8 as two launches of ceil(T/2) and
    floor(T/2) tokens; 4- and 8-bit codes at hidden 2048): every token vs the oracle in
    both output types, and the routing of moe_route equal to the layer's; then T copies of
    one token, which share all their experts and must give T identical rows."""
    L = layer(cfg)
    x_np = syn.make_x(T, L.hidden, seed=100 + T)
    for bf16_out in (False, True):
        y, idx, w = run_layer(torch, qs, L, x_np, bf16_out=bf16_out)
        oracle_check(L, x_np, y_to_np(y, torch), idx, w, bf16_out, f"{cfg} small T={T}")
    ri, rw = qs.moe_route(qs.LayerDesc.from_host(L), to_dev(x_np, torch))
    assert (ri.cpu().numpy() == idx).all() and (rw.cpu().numpy() == w).all()
    if T > 4:                                 # the parts, called on their own, give the same bits
        y_all = run_layer(torch, qs, L, x_np)[0]
        for a, b in ((0, (T + 1) // 2), ((T + 1) // 2, T)):
            assert torch.equal(run_layer(torch, qs, L, x_np[a:b])[0], y_all[a:b]), (T, a, b)
    xd = np.repeat(x_np[:1], T, axis=0)
    y, idx, w = run_layer(torch, qs, L, xd)
    oracle_check(L, xd, y_to_np(y, torch), idx, w, False, f"{cfg} small T={T} repeated token")
    for t in range(1, T):
        assert torch.equal(y[t], y[0]) and (idx[t] == idx[0]).all() and (w[t] == w[0]).all()


@pytest.mark.parametrize("cfg,T", [("PREFILL", 4096), ("SKEW", 16384)])
def test_full_size_sampled(torch, qs, cfg, T):
    """Full workload size in the launch configuration the benchmark times: a workspace
    for the whole T (one unchunked pass), bf16 output as the benchmark writes it, and
    fp32 output; sampled tokens vs the oracle in both, a bit-identical repeat.  Then the
    same call with the default workspace (4096-token chunks: four for the skewed
    workload) must give the same bits."""
    L = layer(cfg)
    x_np = syn.make_x(T, L.hidden, seed=0)
    desc = qs.LayerDesc.from_host(L)
    x = to_dev(x_np, torch)
    rows = sample_tokens(T, 64, seed=1)
    ws_full = qs.new_workspace(desc, T, chunk=T)
    outs = {}
    for bf16_out in (True, False):
        idx = torch.empty((T, L.top_k), dtype=torch.int32, device="cuda")
        w = torch.empty((T, L.top_k), dtype=torch.float32, device="cuda")
        y = qs.moe_layer_forward(desc, x, y_dtype=torch.bfloat16 if bf16_out else torch.float32,
                                 topk_idx=idx, topk_w=w, workspace=ws_full)
        torch.cuda.synchronize()
        idx, w = idx.cpu().numpy(), w.cpu().numpy()
        oracle_check(L, x_np, y_to_np(y, torch), idx, w, bf16_out, f"{cfg} T={T} unchunked bf16={bf16_out}",
                     rows=rows)
        outs[bf16_out] = (y, idx, w)
    y2 = qs.moe_layer_forward(desc, x, y_dtype=torch.bfloat16, workspace=ws_full)
    torch.cuda.synchronize()
    assert torch.equal(y2, outs[True][0])
    del ws_full
    yc = qs.moe_layer_forward(desc, x, y_dtype=torch.bfloat16)            # default: chunks of 4096
    torch.cuda.synchronize()
    assert torch.equal(yc, outs[True][0]), "chunked != unchunked"
    # the bins were uneven as the workload intends
    idx = outs[True][1]
    counts = np.bincount(idx.reshape(-1), minlength=L.n_experts)
    assert counts.sum() == T * L.top_k
    if cfg == "SKEW":
        assert (counts > 10 * counts.mean()).sum() >= 3
    report(f"{cfg} T={T} bins", max_rows=int(counts.max()), empty=int((counts == 0).sum()))


def test_tiny_through_grouped_path(torch, qs):
    """The tiny layer (16 experts top-2, 8-bit) through the grouped path (T = 40, every
    token vs the oracle in both output types), next to its small-batch and T = 1 runs."""
    L = layer("TINY")
    x_np = syn.make_x(40, L.hidden, seed=0)
    for bf16_out in (False, True):
        y, idx, w = run_layer(torch, qs, L, x_np, bf16_out=bf16_out)
        oracle_check(L, x_np, y_to_np(y, torch), idx, w, bf16_out, f"tiny grouped T=40 bf16={bf16_out}")


def test_small_workspace_bounds_memory(torch, qs):
    """A workspace sized for 1024-token chunks (a quarter of the default) is accepted and
    gives the same bits as the default and the unchunked ones (8-bit, T = 4096 + 77)."""
    L = layer("SKEW")
    desc = qs.LayerDesc.from_host(L)
    T = 4096 + 77
    x = to_dev(syn.make_x(T, L.hidden, seed=3), torch)
    ys = []
    for chunk in (1024, None, T):
        ws = qs.new_workspace(desc, T, chunk=chunk)
        ys.append(qs.moe_layer_forward(desc, x, y_dtype=torch.bfloat16, workspace=ws))
        torch.cuda.synchronize()
        del ws
    assert torch.equal(ys[0], ys[1]) and torch.equal(ys[1], ys[2])


# ----------------------------------------------------------------- bit invariants
@pytest.mark.parametrize("cfg,T", [("DECODE", 1), ("DECODE", 40), ("TINY", 4), ("SKEW", 40)])
def test_fused_equals_separate_bit_exact(torch, qs, cfg, T):
    """oMLX fusion principle: [gate; up] as one stack == separate gate and up, bit for bit."""
    L = layer(cfg)
    x_np = syn.make_x(T, L.hidden, seed=5)
    ya, ia, wa = run_layer(torch, qs, L, x_np, fused=True)
    yb, ib, wb = run_layer(torch, qs, L, x_np, fused=False)
    assert torch.equal(ya, yb)
    assert (ia == ib).all() and (wa == wb).all()


def test_permutation_and_chunking_invariance(torch, qs):
    """Tokens are independent: permuting them permutes y bit for bit, and splitting the
    call into chunks gives the same bits (the chunked-prefill property)."""
    L = layer("DECODE")
    T = 256
    x_np = syn.make_x(T, L.hidden, seed=9)
    desc = qs.LayerDesc.from_host(L)
    y, idx, w = run_layer(torch, qs, L, x_np, desc=desc)
    perm = np.random.default_rng(0).permutation(T)
    yp, ip, wp = run_layer(torch, qs, L, x_np[perm], desc=desc)
    assert torch.equal(yp, y[torch.from_numpy(perm).cuda()])
    assert (ip == idx[perm]).all() and (wp == w[perm]).all()
    parts = [run_layer(torch, qs, L, x_np[a:a + 64], desc=desc)[0] for a in range(0, T, 64)]
    assert torch.equal(torch.cat(parts), y)


def test_chunked_prefill_bit_identical(torch, qs):
    """T = 2 * chunk + 100 tokens: with the default workspace one call runs three chunks;
    with a workspace for the whole T it runs unchunked; with one for 5000 tokens it runs
    5000 + 3292.  Outputs and routing must be identical bit for bit, and sampled tokens
    (both sides of each chunk boundary) must match the oracle."""
    L = layer("PREFILL")
    desc = qs.LayerDesc.from_host(L)
    C = qs.PREFILL_CHUNK
    T = 2 * C + 100
    x_np = syn.make_x(T, L.hidden, seed=17)
    x = to_dev(x_np, torch)
    outs = []
    for chunk in (None, T, 5000):
        ws = qs.new_workspace(desc, T, chunk=chunk)
        idx = torch.empty((T, L.top_k), dtype=torch.int32, device="cuda")
        w = torch.empty((T, L.top_k), dtype=torch.float32, device="cuda")
        y = qs.moe_layer_forward(desc, x, y_dtype=torch.bfloat16, topk_idx=idx, topk_w=w, workspace=ws)
        torch.cuda.synchronize()
        outs.append((y, idx.cpu().numpy(), w.cpu().numpy()))
        del ws
    for y, idx, w in outs[1:]:
        assert torch.equal(y, outs[0][0])
        assert (idx == outs[0][1]).all() and (w == outs[0][2]).all()
    y, idx, w = outs[0]
    rows = np.array([0, C - 1, C, 2 * C - 1, 2 * C, T - 1])
    oracle_check(L, x_np, y_to_np(y, torch), idx, w, True, "chunked prefill", rows=rows)


def _shifted_desc(torch, qs, base, shift):
    """The layer of `base` with every scale and bias array copied to an address `shift`
    fp16 elements past an allocation (2-byte or 4-byte aligned instead of 256-byte)."""
    made = {}

    def moved(t):
        if t.data_ptr() not in made:
            buf = torch.empty(t.numel() + shift, dtype=t.dtype, device=t.device)
            view = buf[shift:]
            view.copy_(t.reshape(-1))
            made[t.data_ptr()] = (buf, view.view(t.shape))
        return made[t.data_ptr()][1]

    def qm(m):
        codes, scales, biases, stride, row0 = m
        return (codes, moved(scales), moved(biases), stride, row0)

    rw, rb, g, u, d, sh, sgw = base._keep
    shared = None if sh is None else tuple(qm(m) for m in sh)
    desc = qs.LayerDesc(base.hidden, base.inter, base.n_experts, base.top_k, base.bits, rw, qm(g), qm(u), qm(d),
                        router_bias=rb, shared=shared, scale_dtype=base.desc.scale_dtype, shared_gate_w=sgw)
    desc._made = made
    return desc


@pytest.mark.parametrize("cfg,variant", [("PREFILL", False), ("SKEW", False), ("PREFILL", True)])
def test_scale_staging_paths_bit_identical(torch, qs, cfg, variant):
    """The grouped GEMM stages scales and biases 8, 2 or 1 groups per row at a time
    depending on their alignment; every path must give the same bits (T = 64 and T = 1),
    also with bf16 scales and the gated shared expert."""
    L = layer(cfg, scale_dtype="bf16", shared_gate=True) if variant else layer(cfg)
    base = qs.LayerDesc.from_host(L)
    x_np = syn.make_x(64, L.hidden, seed=29)
    ref = [run_layer(torch, qs, L, x_np[:T], desc=base)[0] for T in (64, 1)]
    for shift in (1, 2):                      # 2-byte and 4-byte aligned scales / biases
        desc = _shifted_desc(torch, qs, base, shift)
        for T, r in zip((64, 1), ref):
            y = run_layer(torch, qs, L, x_np[:T], desc=desc)[0]
            assert torch.equal(y, r), (cfg, shift, T)


def test_decode_repeat_bit_identical(torch, qs):
    """The one-launch decode kernel hands logits and h between workgroups through the
    workspace: many back-to-back calls, alternating inputs and two layers sharing one
    workspace, must reproduce the first results bit for bit (stale data would not)."""
    L = layer("DECODE")
    descs = [qs.LayerDesc.from_host(L), qs.LayerDesc.from_host(L, fused=False)]
    xs = [to_dev(syn.make_x(1, L.hidden, seed=s), torch) for s in (21, 22, 23)]
    ws = torch.zeros(qs.moe_workspace_size(descs[0], 1), dtype=torch.uint8, device="cuda")
    ref = [qs.moe_layer_forward(descs[0], x, workspace=ws) for x in xs]
    torch.cuda.synchronize()
    outs = []
    for i in range(60):
        outs.append((i % 3, qs.moe_layer_forward(descs[i % 2], xs[i % 3], workspace=ws)))
    torch.cuda.synchronize()
    for j, y in outs:
        assert torch.equal(y, ref[j])
    # decode state: no bounded wait gave up (error word), the generation counts the 63
    # calls made on this workspace, the completion counters (16 groups and a top counter,
    # one 256-byte line each) are back at zero
    w32 = ws[:1024 * 1024].cpu().numpy().view(np.uint32)
    assert w32[0] == 0
    assert w32[64] == 63
    cnt = 128 + 64 * np.arange(17)
    assert (w32[cnt] == 0).all()


def test_zero_tokens_is_a_no_op(torch, qs):
    L = layer("TINY")
    desc = qs.LayerDesc.from_host(L)
    x = torch.zeros((0, L.hidden), dtype=torch.int16, device="cuda")
    y = torch.full((0, L.hidden), 7.0, device="cuda")
    qs.moe_layer_forward(desc, x, y=y)
    torch.cuda.synchronize()


# ------------------------------------------------------------------- edge shapes
@pytest.mark.parametrize("shape", [
    dict(hidden=384, inter=384, n_experts=20, top_k=3, bits=4, router_std=0.05),
    dict(hidden=384, inter=256, n_experts=20, top_k=3, bits=8, router_std=0.05, has_shared=False),
    dict(hidden=640, inter=128, n_experts=70, top_k=1, bits=4, zipf_s=1.1),
    dict(hidden=256, inter=128, n_experts=256, top_k=16, bits=8, router_std=0.05),
    dict(hidden=128, inter=640, n_experts=2, top_k=2, bits=4, router_std=0.05),
])
@pytest.mark.parametrize("T", [1, 2, 33])
def test_edge_shapes(torch, qs, shape, T):
    L = syn.make_layer(seed=2, **shape)
    x_np = syn.make_x(T, L.hidden, seed=T + 1)
    y, idx, w = run_layer(torch, qs, L, x_np)
    oracle_check(L, x_np, y_to_np(y, torch), idx, w, False, f"{shape} T={T}")


# --------------------------------------------------------------------------- Q8_0
@pytest.mark.parametrize("N,K", syn.Q8_SHAPES + [(16, 32), (48, 96), (32, 8192), (160, 288), (128, 2048), (256, 4096), (128, 8192)])
def test_q8_pack_and_gemv(torch, qs, N, K):
    rows = syn.make_q8_rows(N, K, seed=N + K)
    x_np = syn.make_x(1, K, seed=K)[0]
    tiles = qs.q8_pack_rows16(to_dev(rows.reshape(-1), torch), N, K)
    torch.cuda.synchronize()
    assert np.array_equal(tiles.cpu().numpy(), oracle.q8_pack_rows16(rows, N, K))
    ref = oracle.q8_gemv(rows, N, K, x_np)
    x = to_dev(x_np, torch)
    y = qs.q8_gemv(tiles, N, K, x)
    yb = qs.q8_gemv(tiles, N, K, x, y_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    y = y.cpu().numpy().astype(np.float64)
    rms = np.sqrt(np.mean(ref ** 2))
    # fp32 accumulation of K products: bound well inside 1e-4 * RMS at these sizes
    assert np.max(np.abs(y - ref)) <= 1e-4 * rms
    check_output(y_to_np(yb, torch), ref, True, f"q8 bf16 {N}x{K}")


@pytest.mark.parametrize("N,K", syn.Q8_SHAPES + [(16, 32), (48, 96), (32, 8192), (160, 288), (128, 2048), (256, 4096), (128, 8192)])
def test_q8_activation_quantized_gemv(torch, qs, N, K):
    """[EMBER] one activation quantization shared by the projections: the activation's
    codes and scales bit for bit against the oracle (an integer decision taken in binary32
    on both sides, including an all-zero block and values on rounding halves), then the
    GEMV with exact int8 dots against the oracle's exact-integer version, the variant that
    quantizes inside the GEMV bit for bit equal to it; the distance to the
    exact-activation path stays inside the quantization bound."""
    rows = syn.make_q8_rows(N, K, seed=N + K)
    x_np = syn.make_x(1, K, seed=K)[0].copy()
    if K >= 64:                                                # an all-zero block, then
        x_np[:64] = 0                                          # block 1: d = 1, halves
        x_np[32:36] = np.array([127.0, 0.5, -2.5, 63.5], np.float32).view(np.uint32) >> 16
    tiles = qs.q8_pack_rows16(to_dev(rows.reshape(-1), torch), N, K)
    xq, xd = qs.q8_quantize_x(to_dev(x_np, torch))
    torch.cuda.synchronize()
    q_r, d_r = oracle.q8_quantize_x(x_np)
    assert np.array_equal(xq.cpu().numpy(), q_r)
    assert np.array_equal(xd.cpu().numpy().view(np.uint16), d_r)
    if K >= 64:
        assert xq[32:36].tolist() == [127, 1, -3, 64]
    ref = oracle.q8_gemv_q8x(rows, N, K, q_r, d_r)
    y = qs.q8_gemv_q8x(tiles, N, K, xq, xd)
    yb = qs.q8_gemv_q8x(tiles, N, K, xq, xd, y_dtype=torch.bfloat16)
    yf = qs.q8_gemv_qx(tiles, N, K, to_dev(x_np, torch))          # quantizing inside the GEMV
    torch.cuda.synchronize()
    assert torch.equal(yf, y)
    y = y.cpu().numpy().astype(np.float64)
    rms = np.sqrt(np.mean(ref ** 2))
    assert np.max(np.abs(y - ref)) <= 1e-5 * rms               # fp32 scaling and sums only
    check_output(y_to_np(yb, torch), ref, True, f"q8x bf16 {N}x{K}")
    exact = oracle.q8_gemv(rows, N, K, x_np)
    rel = np.max(np.abs(y - exact)) / np.sqrt(np.mean(exact ** 2))
    assert 0 < rel < 5e-2, rel                                 # quantized x: close, not equal


# ------------------------------------------------------------ checkpoint variants
@pytest.mark.parametrize("cfg,T", [("DECODE", 1), ("DECODE", 3), ("DECODE", 40), ("SKEW", 2), ("SKEW", 64)])
def test_checkpoint_variants_parity(torch, qs, cfg, T):
    """bf16 scales and biases together with the sigmoid-gated shared expert, on the T = 1
    kernel, the small-batch kernel and the grouped path, 4- and 8-bit, both output types;
    then the gate alone and bf16 alone at the same shape."""
    for sd, gate in (("bf16", True), ("f16", True), ("bf16", False)):
        L = layer(cfg, scale_dtype=sd, shared_gate=gate)
        x_np = syn.make_x(T, L.hidden, seed=200 + T)
        for bf16_out in (False, True):
            y, idx, w = run_layer(torch, qs, L, x_np, bf16_out=bf16_out)
            oracle_check(L, x_np, y_to_np(y, torch), idx, w, bf16_out, f"{cfg} T={T} {sd} gate={gate}")
