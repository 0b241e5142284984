"""The allocation-free router entry against lbv_moe_route (GPU).

lbv_moe_route_noalloc keeps the router's scratch (the W_r planes and the
few-token logits) in a fixed per-GPU array of the library instead of a
caller workspace.  Two calls in a row, the second on fewer tokens (and on the
few-token path, so that both parts of the scratch are used), must give the
ids and weights that lbv_moe_route gives, bitwise: the same kernels run on the
same data.
"""
import numpy as np
import pytest
import torch

import routed_moe_dit_amd as lbv
import synth
from gpu_util import cfg_for, dev, note

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    lbv.load()
    yield


def routes(wl, x, rw, b, mask):
    cfg = cfg_for(wl)
    T = x.shape[0]
    ids = torch.full((T, wl.top_k), -7, dtype=torch.int32, device="cuda")
    w = torch.full((T, wl.top_k), -7.0, dtype=torch.float32, device="cuda")
    ids2, w2 = ids.clone(), w.clone()
    ws = torch.empty(max(lbv.lbv_moe_route_workspace_size(cfg), 16), dtype=torch.uint8,
                     device="cuda")
    lbv.lbv_moe_route(cfg, x, rw, b, mask, ids, w, ws)
    lbv.lbv_moe_route_noalloc(cfg, x, rw, b, mask, ids2, w2)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), w.cpu().numpy(), ids2.cpu().numpy(), w2.cpu().numpy()


def test_route_noalloc_matches_route_on_two_calls():
    wl = synth.WORKLOADS[3].replace(T=5000)
    inp = synth.make_inputs(wl)
    x = dev(inp["x"], "bf16")
    rw, b = dev(inp["router_w"], "f32"), dev(inp["e_bias"], "f32")
    for T in (5000, 777):                       # one-pass router, then the few-token path
        note("route_noalloc T=%d" % T)
        mask = torch.ones(T, dtype=torch.uint8, device="cuda")
        mask[T - 13:] = 0
        i1, w1, i2, w2 = routes(wl, x[:T].contiguous(), rw, b, mask)
        assert (i1[:T - 13] >= 0).all() and (i1[T - 13:] == -1).all()
        assert np.array_equal(i1, i2) and np.array_equal(w1.view(np.uint32), w2.view(np.uint32))


def test_route_noalloc_other_configs():
    """64 experts (its own plane layout) and the fp32 path (no scratch)."""
    for wl in (synth.Workload("e64", T=3000, hidden=1024, num_experts=64, n_group=4,
                              topk_group=2, top_k=6, intermediate=128, n_shared=1, dtype="bf16",
                              seed=21, wr_std=1024 ** -0.5, b_std=0.1),
               synth.WORKLOADS[0]):
        note("route_noalloc %s" % wl.name)
        inp = synth.make_inputs(wl)
        x = dev(inp["x"], wl.dtype)
        i1, w1, i2, w2 = routes(wl, x, dev(inp["router_w"], "f32"), dev(inp["e_bias"], "f32"),
                                None)
        assert np.array_equal(i1, i2) and np.array_equal(w1.view(np.uint32), w2.view(np.uint32))
