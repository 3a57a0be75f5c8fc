"""GPU test of moe_layer_forward_static, the entry point that allocates nothing (its
workspace is the library's static per-GPU array): through the C ABI, on calls in a row of
falling size -- a grouped-path batch, then a single token, then a small batch, then a
prompt longer than the array holds unchunked -- each equal bit for bit to
moe_layer_forward with a workspace of its own.  No torch allocation happens around the
calls (outputs are passed in)."""
import numpy as np
import pytest

import qsmoe_synth as syn
from gpu_util import to_dev

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


def test_static_entry_matches_workspace_entry(torch, qs):
    L = syn.make_layer(**syn.DECODE)
    desc = qs.LayerDesc.from_host(L)
    for T in (700, 1, 3, 2000):
        x = to_dev(syn.make_x(T, L.hidden, seed=300 + T), torch)
        ref_y = torch.empty((T, L.hidden), dtype=torch.bfloat16, device="cuda")
        ref_i = torch.empty((T, L.top_k), dtype=torch.int32, device="cuda")
        ref_w = torch.empty((T, L.top_k), dtype=torch.float32, device="cuda")
        qs.moe_layer_forward(desc, x, y=ref_y, topk_idx=ref_i, topk_w=ref_w,
                             workspace=qs.new_workspace(desc, T))
        y = torch.full((T, L.hidden), 7.0, dtype=torch.bfloat16, device="cuda")
        idx = torch.full((T, L.top_k), -1, dtype=torch.int32, device="cuda")
        w = torch.full((T, L.top_k), -1.0, dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        before = torch.cuda.memory_allocated()
        st = qs.lib().moe_layer_forward_static(desc.ptr, x.data_ptr(), T, y.data_ptr(), qs.MOE_BF16,
                                               idx.data_ptr(), w.data_ptr(),
                                               torch.cuda.current_stream().cuda_stream)
        assert st == qs.MOE_OK, qs.status_string(st)
        assert torch.cuda.memory_allocated() == before
        torch.cuda.synchronize()
        assert torch.equal(y, ref_y), T
        assert torch.equal(idx, ref_i) and torch.equal(w, ref_w), T
        assert np.isfinite(y.float().cpu().numpy()).all()
