"""Parity of the block with fp8 weights and fp8 activations
(lbv_moe_forward_w8a8) with the CPU oracle, through the C ABI.

The x rows are quantized by the same bit-exact quantizer as the weights; act
is rounded to bf16 and cut into MX blocks of 32 on both sides, the oracle
from its fp64 act and the GPU from its fp32 act, so a code can differ only
where the two act values round to different bf16 numbers.  The reference is
oracle.w8a8_experts on the oracle's dequantized weights, at the GPU's
routing where that is a valid near-tie choice (the routing itself is checked
as for the bf16 block).  Bar: relative Frobenius error 5e-3 and max-abs 3e-2,
every token (full size: sampled tokens).
"""
import numpy as np
import pytest
import torch

import oracle
import routed_moe_dit_amd as lbv
import synth
from gpu_util import cfg_for, compare_routing, host, metrics, note, upload
from test_gpu_fp8 import oracle_dequantized
from test_gpu_parity import W, var

pytestmark = pytest.mark.gpu
TOL = dict(rel_frob=5e-3, max_abs=3e-2)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    lbv.load()
    yield


def forward_w8a8(wl, d, wq=None):
    cfg = cfg_for(wl)
    if wq is None:
        wq = lbv.quantize_fp8_weights(d["w13"], d["w2"], d["shared_w13"], d["shared_w2"])
    T = d["x"].shape[0]
    out = torch.empty_like(d["x"])
    ids = torch.empty(T, wl.top_k, dtype=torch.int32, device="cuda")
    w = torch.empty(T, wl.top_k, dtype=torch.float32, device="cuda")
    ws = torch.empty(lbv.lbv_moe_workspace_size(cfg, T), dtype=torch.uint8, device="cuda")
    lbv.lbv_moe_forward_w8a8(cfg, d["x"], d["mask"], d["router_w"], d["e_bias"], wq, out, ids, w,
                             ws)
    torch.cuda.synchronize()
    return out, ids, w


def check_w8a8(wl, inp, dq, out, ids, w, rows=None):
    """Every listed token: the routing as for the bf16 block, the output
    against oracle.w8a8_experts at the oracle's choice (the GPU's where it
    made another near-equal one)."""
    rows = np.arange(wl.T) if rows is None else np.asarray(rows)
    mask = None if inp["mask"] is None else inp["mask"][rows]
    x = inp["x"][rows]
    o = oracle.route(wl, x, inp["router_w"], inp["e_bias"], mask, want_scores=True)
    g_ids = ids.cpu().numpy()[rows]
    same, near = compare_routing(wl, g_ids, w.cpu().numpy()[rows], o, inp["e_bias"], mask)
    ref_ids, ref_w = o["ids"].copy(), o["w"].copy()
    diff = np.nonzero(~same)[0]
    if diff.size:
        alt = oracle.moe_forward_ids(wl, x[diff], inp["router_w"], g_ids[diff], inp["w13"],
                                     inp["w2"], inp["shared_w13"], inp["shared_w2"])
        ref_ids[diff], ref_w[diff] = g_ids[diff], alt["w"]
    want = oracle.w8a8_experts(wl, x, ref_ids, ref_w, dq["w13"], dq["w2"], dq["shared_w13"],
                               dq["shared_w2"])
    m = metrics(host(out)[rows], want)
    print("w8a8 forward %s: %d tokens, %s; near-tie %d, other near-equal choice %d" % (
        wl.name, len(rows), m, near.sum(), diff.size))
    assert m["finite"]
    assert m["rel_frob"] <= TOL["rel_frob"] and m["max_abs"] <= TOL["max_abs"], m
    return m


CASES = [
    W[1],
    W[2],
    var("ns0", n_shared=0, T=97),
    var("ns2", n_shared=2, T=64),
    var("T1", T=1),
    var("E128_K12_ns2", num_experts=128, top_k=12, n_shared=2, T=300, hidden=256),
    var("I1024", T=300, hidden=256, intermediate=1024),
    # odd k-tile counts (17 along H, 5 along I: a zero-filled stage), with
    # 64-row (35 rows per segment) and 128-row tiles (70 rows)
    var("odd_H2176_I640", num_experts=128, top_k=8, T=500, hidden=2176, intermediate=640),
    var("odd_H2176_I640_T1000", num_experts=128, top_k=8, T=1000, hidden=2176, intermediate=640),
    # many 192-row tiles per expert at the LingBot dims
    var("E128_T6000_full_dims", num_experts=128, top_k=8, T=6000, hidden=2048, intermediate=768),
]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("wl", CASES, ids=lambda w: w.name)
def test_forward_w8a8_parity(wl):
    note("forward w8a8 %s" % wl.name)
    inp = synth.make_inputs(wl)
    d = upload(wl, inp)
    out, ids, w = forward_w8a8(wl, d)
    check_w8a8(wl, inp, oracle_dequantized(inp), out, ids, w)


@pytest.mark.timeout(900)
def test_forward_w8a8_parity_full_size():
    """38,000 tokens: every 97th token (392) against the oracle; also reports
    how far fp8 activations move the output from the fp8-weight block (a
    property of the format, not a parity figure)."""
    wl = W[3]
    note("forward w8a8 full %s" % wl.name)
    inp = synth.make_inputs(wl)
    d = upload(wl, inp)
    wq = lbv.quantize_fp8_weights(d["w13"], d["w2"], d["shared_w13"], d["shared_w2"])
    out, ids, w = forward_w8a8(wl, d, wq)
    out8 = torch.empty_like(out)
    cfg = cfg_for(wl)
    ws = torch.empty(lbv.lbv_moe_workspace_size(cfg, wl.T), dtype=torch.uint8, device="cuda")
    lbv.lbv_moe_forward_fp8(cfg, d["x"], d["mask"], d["router_w"], d["e_bias"], wq, out8,
                            torch.empty_like(ids), torch.empty_like(w), ws)
    torch.cuda.synchronize()
    del d, ws
    rows = np.arange(0, wl.T, 97)
    check_w8a8(wl, inp, oracle_dequantized(inp), out, ids, w, rows)
    print("w8a8 vs fp8-weight block, every token: %s" % metrics(host(out), host(out8)))


def test_forward_w8a8_in_hip_graph_replays_bitwise():
    """lbv_moe_forward_w8a8 only enqueues kernels on the caller's stream: each
    replay of a captured call, with a changed input and eager work in
    between, equals the eager call bitwise."""
    wl = W[2]
    note("w8a8 graph capture %s" % wl.name)
    inp = synth.make_inputs(wl)
    d = upload(wl, inp)
    cfg = cfg_for(wl)
    wq = lbv.quantize_fp8_weights(d["w13"], d["w2"], d["shared_w13"], d["shared_w2"])
    T = d["x"].shape[0]
    x = d["x"].clone()
    out = torch.empty_like(x)
    ids = torch.empty(T, wl.top_k, dtype=torch.int32, device="cuda")
    w = torch.empty(T, wl.top_k, dtype=torch.float32, device="cuda")
    ws = torch.empty(lbv.lbv_moe_workspace_size(cfg, T), dtype=torch.uint8, device="cuda")

    def call():
        lbv.lbv_moe_forward_w8a8(cfg, x, d["mask"], d["router_w"], d["e_bias"], wq, out, ids, w,
                                 ws, torch.cuda.current_stream())

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    gen = torch.Generator(device="cpu").manual_seed(7)
    for rep in range(3):
        if rep:
            x.copy_(d["x"][torch.randperm(T, generator=gen).cuda()])
        torch.cuda.synchronize()
        call()
        torch.cuda.synchronize()
        ref = (out.clone(), ids.clone(), w.clone())
        out.zero_()
        ids.zero_()
        w.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref[0]) and torch.equal(ids, ref[1]) and torch.equal(w, ref[2]), rep


def test_forward_w8a8_deterministic_and_isolated():
    """Two calls give the same bits; a sample's outputs do not depend on the
    other samples of the batch (the padded B = 2 workload, sample 1 replaced)."""
    wl = W[2]
    note("w8a8 determinism %s" % wl.name)
    inp = synth.make_inputs(wl)
    d = upload(wl, inp)
    wq = lbv.quantize_fp8_weights(d["w13"], d["w2"], d["shared_w13"], d["shared_w2"])
    a = forward_w8a8(wl, d, wq)
    b = forward_w8a8(wl, d, wq)
    assert all(torch.equal(u, v) for u, v in zip(a, b))
    n0 = wl.samples[0][0]
    d2 = dict(d)
    x2 = d["x"].clone()
    x2[n0:] = x2[n0:].flip(0)
    d2["x"] = x2
    c = forward_w8a8(wl, d2, wq)
    assert torch.equal(c[0][:n0], a[0][:n0]) and torch.equal(c[1][:n0], a[1][:n0])
