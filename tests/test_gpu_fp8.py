"""Parity of the fp8-weight path (e4m3fn codes, one power-of-two scale per
weight row) with the CPU oracle, through the C ABI.

Quantization is integer work: codes and scales must equal the oracle's bit
for bit.  The block with fp8 weights computes what the bf16 block computes
with the dequantized weights decode(q) 2^e (exact in bf16), so its outputs are
held to the bf16 bar against the oracle run on the oracle's own dequantized
weights: relative Frobenius error 5e-3, max-abs 3e-2, every token.
"""
import numpy as np
import pytest
import torch

import oracle
import routed_moe_dit_amd as lbv
import synth
from gpu_util import cfg_for, dev, host, metrics, note, upload
from test_gpu_parity import W, check_forward, var

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    lbv.load()
    yield


def gpu_quantize(w_dev):
    q = torch.empty(w_dev.shape, dtype=torch.uint8, device="cuda")
    sc = torch.empty(w_dev.shape[:-1], dtype=torch.float32, device="cuda")
    lbv.lbv_quantize_fp8_rows(w_dev, q, sc)
    torch.cuda.synchronize()
    return q.cpu().numpy(), sc.cpu().numpy()


def edge_rows(cols, rng):
    """Rows that exercise the exponent choice and the rounding: zeros, a row
    whose maximum is exactly 448 2^k, just above it, every e4m3fn midpoint,
    values in the subnormal range, very large and very small magnitudes."""
    vals = oracle.e4m3_values()[:0x7f]
    rows = []
    rows.append(np.zeros(cols))
    r = rng.uniform(-1, 1, cols) * 448 * 2.0 ** -7
    r[3] = 448 * 2.0 ** -7
    rows.append(r)
    r = rng.uniform(-1, 1, cols) * 448 * 2.0 ** -7
    r[5] = -448 * 2.0 ** -7 * (1 + 2.0 ** -20)
    rows.append(r)
    mids = (vals[:-1] + vals[1:]) / 2
    r = np.resize(np.concatenate([mids, -mids]), cols)
    r[0] = 448.0
    rows.append(r)
    r = rng.uniform(-2.0 ** -6, 2.0 ** -6, cols)
    r[1] = 448.0
    rows.append(r)
    rows.append(rng.standard_normal(cols) * 1e30)
    rows.append(rng.standard_normal(cols) * 1e-30)
    return np.array(rows)


@pytest.mark.parametrize("cols", [16, 80, 768, 2048, 2112, 4096, 4112])
@pytest.mark.parametrize("src", ["bf16", "f32"])
def test_quantize_bit_exact(cols, src):
    note("quantize cols=%d src=%s" % (cols, src))
    rng = np.random.default_rng(cols)
    w = np.concatenate([rng.standard_normal((300, cols)) * 0.02, edge_rows(cols, rng)])
    w = w.astype(np.float32)
    if src == "bf16":
        w = synth.round_to_bf16(w)
    q, sc = gpu_quantize(dev(w, src))
    oq, osc = oracle.quantize_fp8_rows(w)
    assert np.array_equal(sc, osc)
    bad = np.nonzero(q != oq)
    assert bad[0].size == 0, "rows %s cols %s" % (bad[0][:5], bad[1][:5])


def test_quantize_expert_shapes():
    """[E, 2I, H] and [E, H, I] tensors quantize row by row, as their 2-D views."""
    wl = W[1]
    note("quantize expert shapes %s" % wl.name)
    inp = synth.make_inputs(wl)
    for name in ("w13", "w2", "shared_w13", "shared_w2"):
        q, sc = gpu_quantize(dev(inp[name], "bf16"))
        oq, osc = oracle.quantize_fp8_rows(inp[name])
        assert q.shape == inp[name].shape and sc.shape == inp[name].shape[:-1]
        assert np.array_equal(sc, osc) and np.array_equal(q, oq), name


def oracle_dequantized(inp):
    """The inputs with every expert weight replaced by the oracle's own
    dequantized fp8 weight."""
    out = dict(inp)
    for name in ("w13", "w2", "shared_w13", "shared_w2"):
        if inp[name] is not None:
            out[name] = oracle.dequantize_fp8_rows(*oracle.quantize_fp8_rows(inp[name]))
    return out


def forward_fp8(wl, d):
    cfg = cfg_for(wl)
    wq = lbv.quantize_fp8_weights(d["w13"], d["w2"], d["shared_w13"], d["shared_w2"])
    T = d["x"].shape[0]
    out = torch.empty_like(d["x"])
    ids = torch.empty(T, wl.top_k, dtype=torch.int32, device="cuda")
    w = torch.empty(T, wl.top_k, dtype=torch.float32, device="cuda")
    ws = torch.empty(lbv.lbv_moe_workspace_size(cfg, T), dtype=torch.uint8, device="cuda")
    lbv.lbv_moe_forward_fp8(cfg, d["x"], d["mask"], d["router_w"], d["e_bias"], wq, out, ids, w,
                            ws)
    torch.cuda.synchronize()
    return out, ids, w


FP8_CASES = [
    W[1],
    W[2],
    var("ns0", n_shared=0, T=97),
    var("ns2", n_shared=2, T=64),
    var("T1", T=1),
    var("E128_K12_ns2", num_experts=128, top_k=12, n_shared=2, T=300, hidden=256),
    # 128-row tiles (419 rows per segment) and 256-row tiles (558) at the LingBot dims
    var("E128_T6000_full_dims", num_experts=128, top_k=8, T=6000, hidden=2048, intermediate=768),
    var("E128_T8000_full_dims", num_experts=128, top_k=8, T=8000, hidden=2048, intermediate=768),
    # odd k-tile counts and partial n-tiles with 64-, 128- and 256-row tiles
    var("odd_H2112_I704_T200", num_experts=128, top_k=8, T=200, hidden=2112, intermediate=704),
    var("odd_H2112_I704_T500", num_experts=128, top_k=8, T=500, hidden=2112, intermediate=704),
    var("odd_H2112_I704_T8000", num_experts=128, top_k=8, T=8000, hidden=2112, intermediate=704),
]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("wl", FP8_CASES, ids=lambda w: w.name)
def test_forward_fp8_parity(wl):
    note("forward fp8 %s" % wl.name)
    inp = synth.make_inputs(wl)
    d = upload(wl, inp)
    out, ids, w = forward_fp8(wl, d)
    check_forward(wl, oracle_dequantized(inp), out, ids, w)


@pytest.mark.timeout(900)
def test_forward_fp8_parity_full_size():
    """38,000 tokens, every token against the oracle on dequantized weights;
    also reports how far fp8 weights move the output from the bf16-weight
    oracle (a property of the format, not a parity figure)."""
    wl = W[3]
    note("forward fp8 full %s" % wl.name)
    inp = synth.make_inputs(wl)
    d = upload(wl, inp)
    out, ids, w = forward_fp8(wl, d)
    del d
    inq = oracle_dequantized(inp)
    check_forward(wl, inq, out, ids, w)
    rows = np.arange(0, wl.T, 97)
    ref = oracle.moe_forward(wl, inp["x"][rows], inp["router_w"], inp["e_bias"], inp["w13"],
                             inp["w2"], inp["shared_w13"], inp["shared_w2"])
    print("fp8 weights vs bf16-weight oracle on %d sampled tokens: %s" % (
        len(rows), metrics(host(out)[rows], ref["out"])))


def test_forward_fp8_matches_bf16_block_on_dequantized_weights():
    """The fp8 block and the bf16 block given the dequantized weights as bf16
    tensors compute the same products from the same bf16 operands; only the
    order of the fp32 sums may differ (the fp8 kernel walks a k-tile in
    another order), so the outputs agree to within a few bf16 ulps."""
    wl = var("E64_T700", T=700)
    note("fp8 vs bf16 block %s" % wl.name)
    inp = synth.make_inputs(wl)
    d = upload(wl, inp)
    out8, ids8, _ = forward_fp8(wl, d)
    inq = oracle_dequantized(inp)
    dq = upload(wl, inq)
    blk = lbv.MoEBlock(cfg_for(wl), dq["router_w"], dq["e_bias"], dq["w13"], dq["w2"],
                       dq["shared_w13"], dq["shared_w2"])
    out16, ids16, _ = blk(dq["x"], dq["mask"], want_routing=True)
    torch.cuda.synchronize()
    assert torch.equal(ids8, ids16)
    m = metrics(host(out8), host(out16))
    print("fp8 block vs bf16 block on dequantized weights: %s" % m)
    assert m["rel_frob"] <= 5e-3 and m["max_abs"] <= 3e-2


def test_forward_fp8_in_hip_graph_replays_bitwise():
    """lbv_moe_forward_fp8 only enqueues kernels on the caller's stream, so it
    can be captured in a HIP graph: each replay, with a changed input and eager
    work in between, equals the eager call bitwise."""
    wl = W[2]
    note("fp8 graph capture %s" % wl.name)
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
        lbv.lbv_moe_forward_fp8(cfg, x, d["mask"], d["router_w"], d["e_bias"], wq, out, ids, w,
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
    gen = torch.Generator(device="cpu").manual_seed(6)
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
