"""GPU parity at the edges of fp16's range: the kernels compute on fp16 operands, and the
layer must still match the fp64 oracle for inputs whose activations, weights or
intermediates fall outside what fp16 holds.

Inputs: bf16 activations x ~ N(0, std^2) with std 300 (h reaches ~1e7, the down outputs
~3e7: both past fp16's 65504), 3e4 (x itself past 65504) and 1e-6 (x below fp16's normal
range); bf16 scales drawn log-uniformly over [1e-5, 1e-1] (many below fp16's normal
range, where a plain fp16 conversion loses bits), with 4- and 8-bit codes; bf16 scales
all near 1e-7 and all near 3e3 (every weight below, or the largest above, fp16's normal
range).  T = 1 runs the one-launch decode kernel, T = 3 the small-batch kernel, T = 40
the grouped GEMMs.  Tolerance as for every parity case.

The grouped path's down pass rescales h blocks of one row that carry different scales;
ordinary inputs rarely produce such rows, so a state word forces a distinct scale on
every block (test_forced_h_rescale), and the result must stay within rounding of the
default run and within tolerance of the oracle.
"""
import numpy as np
import pytest

import oracle
import qsmoe_synth as syn
from gpu_util import W_TOL, check_output, check_routing, report, to_dev, y_to_np

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


def wide_layer(cfg, scale_range=(1e-5, 1e-1)):
    key = (cfg, scale_range)
    if key not in _LAYERS:
        _LAYERS.clear()
        _LAYERS[key] = syn.make_layer(**getattr(syn, cfg), scale_dtype="bf16", scale_range=scale_range)
    return _LAYERS[key]


def oracle_ref(ol, x_np, idx, w, std=1.0):
    """The oracle's output under its own routing, except on tokens whose k-th and
    (k+1)-th logits are too close to order (there the GPU's routing is checked as valid
    and used).  The routing-weight bound holds for logits of order 1; logits scale with
    x, and so does their fp32 rounding: the bound is taken times max(1, std of x)."""
    idx_r, w_r, gap = oracle.route(ol, x_np)
    amb, _ = check_routing(idx, w, idx_r, w_r, gap, w_tol=W_TOL * max(1.0, std))
    use_idx = np.where(amb[:, None], idx, idx_r)
    use_w = np.where(amb[:, None], w.astype(np.float64), w_r)
    return oracle.layer_forward_with_routing(ol, x_np, use_idx, use_w), int(amb.sum())


def run_case(torch, qs, L, x_np, what, std=1.0):
    desc = qs.LayerDesc.from_host(L)
    T = x_np.shape[0]
    ol = oracle.OracleLayer(L)
    for bf16_out in (False, True):
        idx = torch.empty((T, L.top_k), dtype=torch.int32, device="cuda")
        w = torch.empty((T, L.top_k), dtype=torch.float32, device="cuda")
        y = qs.moe_layer_forward(desc, to_dev(x_np, torch), y_dtype=torch.bfloat16 if bf16_out else torch.float32,
                                 topk_idx=idx, topk_w=w)
        torch.cuda.synchronize()
        ref, n_amb = oracle_ref(ol, x_np, idx.cpu().numpy(), w.cpu().numpy(), std)
        assert np.isfinite(ref).all()
        label = f"{what} bf16={bf16_out}"
        rel = check_output(y_to_np(y, torch), ref, bf16_out, label)
        report(label, err_over_rms=rel, ambiguous=n_amb, ref_rms=float(np.sqrt(np.mean(ref ** 2))))


@pytest.mark.parametrize("cfg", ["DECODE", "SKEW"])
@pytest.mark.parametrize("std", [300.0, 3e4, 1e-6])
@pytest.mark.parametrize("T", [1, 3, 40])
def test_range_extremes(torch, qs, cfg, std, T):
    L = wide_layer(cfg)
    x_np = syn.make_x(T, L.hidden, seed=400 + T, std=std)
    run_case(torch, qs, L, x_np, f"range {cfg} x~N(0,{std:g}^2) T={T}", std)


@pytest.mark.parametrize("cfg", ["DECODE", "SKEW"])
@pytest.mark.parametrize("scale_range", [(5e-8, 2e-7), (2e3, 5e3)])
@pytest.mark.parametrize("T", [1, 3, 40])
def test_range_of_scales(torch, qs, cfg, scale_range, T):
    L = wide_layer(cfg, scale_range)
    x_np = syn.make_x(T, L.hidden, seed=500 + T)
    run_case(torch, qs, L, x_np, f"scales {cfg} s in {scale_range} T={T}")


CTL_HBLOCK_EXACT = 33


@pytest.mark.parametrize("cfg", ["DECODE", "SKEW"])
@pytest.mark.parametrize("std", [1.0, 300.0])
def test_forced_h_rescale(torch, qs, cfg, std):
    """Every h block under its own scale: nearly every down tile rescales in LDS.  The
    rescaled h equals the default h except for values the default flushes below 2^-14;
    those shift the fp32 down sums by ~1e-5 and can flip the fp16 rounding of a slot
    value, so the output stays within one fp16 unit of the largest value of the default
    run, and within tolerance of the oracle."""
    L = wide_layer(cfg)
    desc = qs.LayerDesc.from_host(L)
    T = 96
    x_np = syn.make_x(T, L.hidden, seed=600, std=std)
    x = to_dev(x_np, torch)
    ws = qs.new_workspace(desc, T)
    y0 = qs.moe_layer_forward(desc, x, workspace=ws)
    torch.cuda.synchronize()
    ws[:1 << 20].view(torch.int32)[CTL_HBLOCK_EXACT] = 1
    torch.cuda.synchronize()
    idx = torch.empty((T, L.top_k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, L.top_k), dtype=torch.float32, device="cuda")
    y1 = qs.moe_layer_forward(desc, x, workspace=ws, topk_idx=idx, topk_w=w)
    torch.cuda.synchronize()
    assert qs.moe_workspace_status(ws).cpu().numpy().view(np.uint32)[0] == 0
    y0n, y1n = y_to_np(y0, torch), y_to_np(y1, torch)
    rms = float(np.sqrt(np.mean(y0n.astype(np.float64) ** 2)))
    d = float(np.max(np.abs(y1n.astype(np.float64) - y0n)))
    report(f"forced h rescale {cfg} std={std:g}", max_diff_over_rms=d / rms, identical=bool(d == 0.0))
    assert d <= 2.0 ** -10 * float(np.max(np.abs(y0n))), d / rms
    ref, _ = oracle_ref(oracle.OracleLayer(L), x_np, idx.cpu().numpy(), w.cpu().numpy(), std)
    check_output(y1n, ref, False, f"forced h rescale {cfg} std={std:g}")
