"""Benchmark of the MI355X quantized sparse MoE layer (one GPU).

A step is one pass of the MoE layer (router, top-k, binning for T >= 2, fused
[gate; up] + SwiGLU, down projection, weighted combine with the shared expert) over one
batch of synthetic input already resident in HBM.  The headline line reports the
batch-1 decode workload (hidden 2048, 256 experts top-8 + 1 shared, expert inter 512,
4-bit affine group-64 weights, T = 1): tokens/s, with the layer's algorithmic weight
bytes over HBM peak as the roofline.  Extra keys report the prefill (T = 4096), the
skewed long prefill (T = 16384, 8-bit, Zipf router bias), the dense Q8_0 GEMV, the
same GEMVs with a quantized activation (int8 dots, and their deviation from the exact
path) and (--only smallT) the decode layer at T = 1, 2, 4, 5, 8.

Decode cycles through 40 distinct copies of the layer (18 GB, far beyond the 256 MB
Infinity Cache) so every step streams its experts from HBM.  Steps are captured in one
HIP graph; HIP events on the replay stream bracket the timed region.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu] [--only decode,prefill,skew,q8,q8x,smallT,variant,copy]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_F16_PEAK_TFS = 2500.0     # MI355X dense fp16/bf16 MFMA, TFLOP/s
GROUP = 64

# HBM traffic of one decode-kernel launch: rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE
# (KiB per dispatch, median over the timed launches), each scaled by what the same
# counter reads for a plain 1 GiB device copy (FETCH_SIZE x 2.0, WRITE_SIZE x 1.0).  A
# figure holds only for the kernel sources it was measured on, identified by their
# sha256; once they change the traffic is reported as null until measured again.
DECODE_SOURCES = ("csrc/decode.hip", "csrc/decode_state.h", "csrc/common.h", "csrc/internal.h")
GEMM_SOURCES = ("csrc/gemm.hip", "csrc/common.h", "csrc/internal.h")
PREFILL_TRAFFIC = {"sources_sha256": "a1d683c4130b605d777143281266a3820d5ae4e79a84a41909bb194fcc1f9e12", "bytes": 1002660106}
DECODE_TRAFFIC = {"sources_sha256": "8886823710cf56d48e32cf7a72c37fe7ab5888a9605d6196767a04915e92ef1d", "bytes": 17974594}


# ----------------------------------------------------------- algorithmic accounting
def q8_weight_bytes(N: int, K: int) -> int:
    """Bytes of a Q8_0 matrix: 34 bytes (fp16 scale + 32 int8) per 32 weights."""
    return N * K // 32 * 34


def affine_matrix_bytes(rows: int, cols: int, bits: int) -> int:
    """codes + one fp16 scale and one fp16 bias per group of 64."""
    return rows * cols * bits // 8 + rows * (cols // GROUP) * 4


def expert_bytes(H: int, I: int, bits: int) -> int:
    return affine_matrix_bytes(2 * I, H, bits) + affine_matrix_bytes(H, I, bits)


def decode_layer_bytes(H: int, I: int, E: int, K: int, bits: int, shared: bool = True) -> int:
    """What one T = 1 layer must read/write: router weights, the k routed experts and the
    shared expert, x in and y out (bf16)."""
    return E * H * 2 + (K + (1 if shared else 0)) * expert_bytes(H, I, bits) + 2 * H * 2


def layer_flops(T: int, H: int, I: int, E: int, K: int, shared: bool = True) -> int:
    """2*T*E*H (router) + 2 * 3*H*I per (token, expert) over the k routed + shared."""
    return 2 * T * E * H + 2 * T * (K + (1 if shared else 0)) * 3 * H * I


def measured_traffic(sources, rec):
    """HBM bytes per launch from the committed counter runs, or None once the kernel's
    sources differ from the ones the counters were taken on."""
    import hashlib
    h = hashlib.sha256()
    pkg = os.path.join(os.path.dirname(os.path.abspath(__file__)), "quantized_sparse_moe_amd")
    for f in sources:
        with open(os.path.join(pkg, f), "rb") as fh:
            h.update(fh.read())
    return rec["bytes"] if h.hexdigest() == rec["sources_sha256"] else None


def decode_traffic():
    return measured_traffic(DECODE_SOURCES, DECODE_TRAFFIC)


# ------------------------------------------------------------------------- helpers
def _dev_layer_copies(qs, torch, L, copies: int):
    """Upload one layer and clone its device tensors `copies` times (distinct HBM)."""
    base = qs.LayerDesc.from_host(L, fused=True)
    descs = [base]
    for _ in range(copies - 1):
        k = base._keep
        clone = lambda m: tuple(t.clone() if hasattr(t, "clone") else t for t in m)
        router_w, router_bias, gate, up, down, shared, shared_gate_w = k
        c_codes, c_sc, c_bi = gate[0].clone(), gate[1].clone(), gate[2].clone()
        g = (c_codes, c_sc, c_bi, gate[3], gate[4])
        u = (c_codes, c_sc, c_bi, up[3], up[4])
        d = clone(down)
        sh = None
        if shared is not None:
            sg, su, sd = shared
            s_codes, s_sc, s_bi = sg[0].clone(), sg[1].clone(), sg[2].clone()
            sh = ((s_codes, s_sc, s_bi, sg[3], sg[4]), (s_codes, s_sc, s_bi, su[3], su[4]), clone(sd))
        descs.append(qs.LayerDesc(L.hidden, L.inter, L.n_experts, L.top_k, L.bits, router_w.clone(),
                                  g, u, d, router_bias=None if router_bias is None else router_bias.clone(),
                                  shared=sh, scale_dtype=base.desc.scale_dtype,
                                  shared_gate_w=None if shared_gate_w is None else shared_gate_w.clone()))
    return descs


def _graph_time(torch, fn_steps, steps: int, warmup: int):
    """Capture `steps` calls in a HIP graph, replay once untimed (after `warmup` eager
    steps), then time one replay with events on the replay stream. Returns ms/step."""
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for i in range(warmup):
            fn_steps(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for i in range(steps):
            fn_steps(i)
    torch.cuda.synchronize()
    g.replay()                      # untimed replay
    torch.cuda.synchronize()
    cur = torch.cuda.current_stream()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(cur)
    g.replay()
    end.record(cur)
    end.synchronize()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def cpu_cores() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except Exception:
        return os.cpu_count() or 1


def cpu_baseline_decode(L, ntok: int):
    """fp64 oracle on a bounded sample of decode tokens (baseline only)."""
    import oracle
    oracle.build(force=False)
    import qsmoe_synth as syn
    x = syn.make_x(ntok, L.hidden, seed=123)
    ol = oracle.OracleLayer(L)
    t = time.perf_counter()
    oracle.layer_forward(ol, x)
    dt = time.perf_counter() - t
    return {"value": ntok / dt, "unit": "tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{ntok} tokens of the decode workload, one layer, fp64, {dt:.1f} s"}


# ----------------------------------------------------------------------- workloads
def bench_decode(qs, torch, syn, steps, warmup, copies=40, **variant):
    L = syn.make_layer(**syn.DECODE, **variant)
    descs = _dev_layer_copies(qs, torch, L, copies)
    xs = [torch.from_numpy(syn.make_x(1, L.hidden, seed=100 + l).view(np.int16)).cuda() for l in range(copies)]
    ys = [torch.empty((1, L.hidden), dtype=torch.bfloat16, device="cuda") for _ in range(copies)]
    ws = torch.zeros(qs.moe_workspace_size(descs[0], 1), dtype=torch.uint8, device="cuda")

    def step(i):
        l = i % copies
        qs.moe_layer_forward(descs[l], xs[l], y=ys[l], workspace=ws)

    ms = _graph_time(torch, step, steps, warmup)
    nbytes = decode_layer_bytes(L.hidden, L.inter, L.n_experts, L.top_k, L.bits)
    return L, ms, nbytes


def bench_small_t(qs, torch, syn, steps, warmup, Ts=(1, 2, 4, 5, 8), copies=40):
    """Small batches of the decode layer (the verification / batched-decode shape): per T,
    the time per call and the bytes a call must read -- router weights, each expert that
    any of the T tokens selects (once), the shared expert, x and y -- per token."""
    L = syn.make_layer(**syn.DECODE)
    descs = _dev_layer_copies(qs, torch, L, copies)
    eb = expert_bytes(L.hidden, L.inter, L.bits)
    res = []
    for T in Ts:
        xs = [torch.from_numpy(syn.make_x(T, L.hidden, seed=1000 * T + l).view(np.int16)).cuda()
              for l in range(copies)]
        ys = [torch.empty((T, L.hidden), dtype=torch.bfloat16, device="cuda") for _ in range(copies)]
        ws = torch.zeros(qs.moe_workspace_size(descs[0], T), dtype=torch.uint8, device="cuda")
        union = []
        for l in range(copies):
            idx, _ = qs.moe_route(descs[l], xs[l], workspace=ws)
            union.append(len(np.unique(idx.cpu().numpy())))
        torch.cuda.synchronize()

        def step(i):
            l = i % copies
            qs.moe_layer_forward(descs[l], xs[l], y=ys[l], workspace=ws)

        ms = _graph_time(torch, step, steps, warmup)
        experts = float(np.mean(union))
        nbytes = L.n_experts * L.hidden * 2 + (experts + 1) * eb + 2 * T * L.hidden * 2
        res.append({"T": T, "us_per_call": ms * 1e3, "tokens_per_s": T / (ms * 1e-3),
                    "experts_read": experts, "bytes_per_token": nbytes / T,
                    "GB_per_s": nbytes / (ms * 1e-3) / 1e9})
        del ws
    return res


def bench_prefill(qs, torch, syn, cfg, T, steps, warmup, copies):
    L = syn.make_layer(**cfg)
    descs = _dev_layer_copies(qs, torch, L, copies)
    x = torch.from_numpy(syn.make_x(T, L.hidden, seed=0).view(np.int16)).cuda()
    y = torch.empty((T, L.hidden), dtype=torch.bfloat16, device="cuda")
    # a workspace for the whole T, so that the call runs unchunked (one pass over the
    # expert weights); with the default size a long prompt runs in 4096-token chunks
    ws = torch.zeros(qs.moe_workspace_size(descs[0], T, chunk=T), dtype=torch.uint8, device="cuda")

    def step(i):
        qs.moe_layer_forward(descs[i % copies], x, y=y, workspace=ws)

    ms = _graph_time(torch, step, steps, warmup)
    flops = layer_flops(T, L.hidden, L.inter, L.n_experts, L.top_k)
    return L, ms, flops


def bench_q8(qs, torch, syn, steps, warmup, layers=16):
    shapes = syn.Q8_SHAPES
    mats = []
    for (N, K) in shapes:
        rows = torch.from_numpy(syn.make_q8_rows(N, K, seed=N + K).reshape(-1)).cuda()
        tiles = qs.q8_pack_rows16(rows, N, K)
        mats.append([(tiles if l == 0 else tiles.clone()) for l in range(layers)])
    xs = {K: torch.from_numpy(syn.make_x(1, K, seed=K)[0].view(np.int16)).cuda() for _, K in shapes}
    ys = {N: torch.empty((N,), dtype=torch.bfloat16, device="cuda") for N, _ in shapes}
    torch.cuda.synchronize()

    def step(i):
        l = i % layers
        for j, (N, K) in enumerate(shapes):
            qs.q8_gemv(mats[j][l], N, K, xs[K], y=ys[N])

    ms = _graph_time(torch, step, steps, warmup)
    nbytes = sum(q8_weight_bytes(N, K) + 2 * K + 2 * N for N, K in shapes)
    return ms, nbytes


def bench_q8x(qs, torch, syn, steps, warmup, layers=16, fused=False):
    """The same four projections with the activation quantized once per projection input
    (q8_quantize_x) and int8-dot GEMVs (q8_gemv_q8x), or (fused) quantized inside the
    GEMV (q8_gemv_qx); also the largest deviation from the exact-activation GEMV,
    relative to that output's RMS."""
    shapes = syn.Q8_SHAPES
    mats = []
    for (N, K) in shapes:
        rows = torch.from_numpy(syn.make_q8_rows(N, K, seed=N + K).reshape(-1)).cuda()
        tiles = qs.q8_pack_rows16(rows, N, K)
        mats.append([(tiles if l == 0 else tiles.clone()) for l in range(layers)])
    xs = {K: torch.from_numpy(syn.make_x(1, K, seed=K)[0].view(np.int16)).cuda() for _, K in shapes}
    xqs = {K: torch.empty((K,), dtype=torch.int8, device="cuda") for _, K in shapes}
    xds = {K: torch.empty((K // 32,), dtype=torch.int16, device="cuda") for _, K in shapes}
    ys = [torch.empty((N,), dtype=torch.bfloat16, device="cuda") for N, _ in shapes]
    torch.cuda.synchronize()

    def step(i):
        l = i % layers
        for j, (N, K) in enumerate(shapes):
            if fused:
                qs.q8_gemv_qx(mats[j][l], N, K, xs[K], y=ys[j])
            else:
                qs.q8_quantize_x(xs[K], xq=xqs[K], xd=xds[K])
                qs.q8_gemv_q8x(mats[j][l], N, K, xqs[K], xds[K], y=ys[j])

    ms = _graph_time(torch, step, steps, warmup)
    err = 0.0
    for j, (N, K) in enumerate(shapes):
        xq, xd = qs.q8_quantize_x(xs[K])
        yq = qs.q8_gemv_q8x(mats[j][0], N, K, xq, xd).double()
        ye = qs.q8_gemv(mats[j][0], N, K, xs[K]).double()
        err = max(err, float((yq - ye).abs().max() / ye.pow(2).mean().sqrt()))
    nbytes = sum(q8_weight_bytes(N, K) + 2 * K + 2 * N for N, K in shapes)
    return ms, nbytes, err


def bench_copy(torch, steps, nbytes=1 << 30):
    """Plain device-to-device copy of `nbytes` (torch's copy kernel): the calibration
    workload for the HBM byte counters (it must read and write exactly `nbytes`)."""
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    b = torch.empty_like(a)
    ms = _graph_time(torch, lambda i: b.copy_(a), steps, 2)
    return ms, nbytes


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--only", default="decode,prefill,skew,q8,q8x")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); multi-GPU runs are "
              "not part of this build", file=sys.stderr)
        return 2
    import torch
    import qsmoe_synth as syn
    import quantized_sparse_moe_amd as qs
    qs.lib()
    only = set(args.only.split(","))
    out = {"metric": "MoE-layer tokens/s (decode T=1, prefill T=4096) + % HBM / MFMA roofline",
           "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
           "data": "synthetic"}
    Ld = None
    if "decode" in only:
        Ld, ms, nbytes = bench_decode(qs, torch, syn, args.steps, args.warmup)
        out["value"] = 1.0 / (ms * 1e-3)
        out["ms_per_step"] = ms
        out["config"] = {"workload": "decode MoE layer: hidden 2048, 256 experts top-8 + 1 shared, "
                                     "inter 512, 4-bit affine g64 (fp16 scale+bias), T=1, "
                                     "40 distinct layer copies",
                         "global_batch": 1, "seq_len": 1}
        gbs = nbytes / (ms * 1e-3) / 1e9
        out["roofline"] = {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": gbs / HBM_PEAK_GBS, "traffic": decode_traffic(),
                           "kernel": "decode layer (router+shared gate/up, routed gate/up, down+combine)",
                           "bytes_per_launch": nbytes}
    if "variant" in only:
        # same decode layer with bf16 scales / biases and the sigmoid-gated shared expert
        Lv, ms, nbytes = bench_decode(qs, torch, syn, args.steps, args.warmup, scale_dtype="bf16",
                                      shared_gate=True)
        out["decode_bf16_gated"] = {"ms_per_step": ms, "tokens_per_s": 1.0 / (ms * 1e-3),
                                    "GB_per_s": nbytes / (ms * 1e-3) / 1e9}
    if "prefill" in only:
        steps = max(4, args.steps // 100)
        L, ms, flops = bench_prefill(qs, torch, syn, syn.PREFILL, syn.PREFILL_T, steps,
                                     max(2, args.warmup // 10), copies=4)
        tf = flops / (ms * 1e-3) / 1e12
        out["prefill"] = {"tokens_per_s": syn.PREFILL_T / (ms * 1e-3), "ms_per_step": ms, "T": syn.PREFILL_T,
                          "steps": steps,
                          "roofline": {"bound": "mfma", "achieved": tf, "peak": MFMA_F16_PEAK_TFS,
                                       "unit": "TFLOP/s", "frac": tf / MFMA_F16_PEAK_TFS,
                                       "traffic": measured_traffic(GEMM_SOURCES, PREFILL_TRAFFIC),
                                       "flops_per_step": flops}}
    if "skew" in only:
        steps = max(2, args.steps // 400)
        L, ms, flops = bench_prefill(qs, torch, syn, syn.SKEW, syn.SKEW_T, steps, 1, copies=1)
        tf = flops / (ms * 1e-3) / 1e12
        out["skew"] = {"tokens_per_s": syn.SKEW_T / (ms * 1e-3), "ms_per_step": ms, "T": syn.SKEW_T,
                       "steps": steps, "tflops": tf, "frac_mfma": tf / MFMA_F16_PEAK_TFS}
    if "smallT" in only:
        out["small_t"] = bench_small_t(qs, torch, syn, max(40, args.steps // 10), args.warmup)
    if "q8" in only:
        steps = max(16, args.steps // 4)
        ms, nbytes = bench_q8(qs, torch, syn, steps, args.warmup)
        gbs = nbytes / (ms * 1e-3) / 1e9
        out["q8"] = {"layers_per_s": 1.0 / (ms * 1e-3), "ms_per_layer": ms, "GB_per_s": gbs,
                     "frac_hbm": gbs / HBM_PEAK_GBS, "bytes_per_layer": nbytes}
    if "q8x" in only:
        steps = max(16, args.steps // 4)
        for key, fused in (("q8x", False), ("q8qx", True)):
            ms, nbytes, err = bench_q8x(qs, torch, syn, steps, args.warmup, fused=fused)
            gbs = nbytes / (ms * 1e-3) / 1e9
            out[key] = {"layers_per_s": 1.0 / (ms * 1e-3), "ms_per_layer": ms, "GB_per_s": gbs,
                        "frac_hbm": gbs / HBM_PEAK_GBS, "bytes_per_layer": nbytes,
                        "max_err_vs_exact_over_rms": err}
    if "copy" in only:
        ms, nbytes = bench_copy(torch, 8)
        out["copy"] = {"bytes_each_way": nbytes, "ms": ms, "GB_per_s": 2 * nbytes / (ms * 1e-3) / 1e9}
    if not args.no_cpu and Ld is not None:
        out["cpu_baseline"] = cpu_baseline_decode(Ld, 1024)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
