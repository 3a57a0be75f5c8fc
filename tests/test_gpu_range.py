"""GPU parity at the edges of fp16's range: the kernels compute on fp16 operands, and the
layer must still match the fp64 oracle for inputs whose activations, weights or
intermediates fall outside what fp16 holds.

Inputs: bf16 activations x ~ N(0, std^2) with std 300 (h reaches ~1e7, the down outputs
~3e7: both past fp16's 65504), 3e4 (x itself past 65504) and 1e-6 (x below fp16's normal
range); bf16 scales drawn log-uniformly over [1e-5, 1e-1] (many below fp16's normal
range, where a plain fp16 conversion loses bits), with 4- and 8-bit codes.  Tolerance as
for every parity case.
"""
import numpy as np
import pytest

import oracle
import qsmoe_synth as syn
from gpu_util import check_output, check_routing, report, to_dev, y_to_np

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


def wide_layer(cfg):
    if cfg not in _LAYERS:
        _LAYERS.clear()
        _LAYERS[cfg] = syn.make_layer(**getattr(syn, cfg), scale_dtype="bf16", scale_range=(1e-5, 1e-1))
    return _LAYERS[cfg]


@pytest.mark.parametrize("cfg", ["DECODE", "SKEW"])
@pytest.mark.parametrize("std", [300.0, 3e4, 1e-6])
@pytest.mark.parametrize("T", [1])
def test_range_extremes(torch, qs, cfg, std, T):
    L = wide_layer(cfg)
    desc = qs.LayerDesc.from_host(L)
    x_np = syn.make_x(T, L.hidden, seed=400 + T, std=std)
    ol = oracle.OracleLayer(L)
    idx_r, w_r, gap = oracle.route(ol, x_np)
    for bf16_out in (False, True):
        idx = torch.empty((T, L.top_k), dtype=torch.int32, device="cuda")
        w = torch.empty((T, L.top_k), dtype=torch.float32, device="cuda")
        y = qs.moe_layer_forward(desc, to_dev(x_np, torch), y_dtype=torch.bfloat16 if bf16_out else torch.float32,
                                 topk_idx=idx, topk_w=w)
        torch.cuda.synchronize()
        idx, w = idx.cpu().numpy(), w.cpu().numpy()
        amb, wmax = check_routing(idx, w, idx_r, w_r, gap)
        use_idx = np.where(amb[:, None], idx, idx_r)
        use_w = np.where(amb[:, None], w.astype(np.float64), w_r)
        ref = oracle.layer_forward_with_routing(ol, x_np, use_idx, use_w)
        assert np.isfinite(ref).all()
        what = f"range {cfg} x~N(0,{std:g}^2) T={T} bf16={bf16_out}"
        rel = check_output(y_to_np(y, torch), ref, bf16_out, what)
        report(what, err_over_rms=rel, ambiguous=int(amb.sum()), ref_rms=float(np.sqrt(np.mean(ref ** 2))))
