"""Parity of the steps around the block (RMSNorm + AdaLN in front of it, the
gated residual after it) with the CPU oracle, through the C ABI.

h: every element within half a bf16 ulp of the oracle's unrounded fp64
value, plus the fp32 evaluation error 2^-20 (|x r (1 + scale)| + |shift|)
(the GPU accumulates the sum of squares in fp32, as the pages put it; a value
within that error of a rounding midpoint may round the other way, and where
shift nearly cancels the normalised term that error exceeds h's own ulp), and
at most 1e-3 of the elements rounded differently from the oracle; fp32
storage: the same evaluation-error bound.
FFN output: out - x against the oracle's gate * block(h) on the GPU's own h
(the block's own parity is tested on its own), with the block's tolerance.
"""
import numpy as np
import pytest
import torch

import oracle
import routed_moe_dit_amd as lbv
import synth
from gpu_util import cfg_for, compare_routing, dev, host, metrics, note, upload

pytestmark = pytest.mark.gpu
W = synth.WORKLOADS
BF16_TOL = dict(rel_frob=5e-3, max_abs=3e-2)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    lbv.load()
    yield


def var(name, **kw):
    base = dict(name=name, T=200, hidden=512, num_experts=64, n_group=4, topk_group=2, top_k=6,
                intermediate=128, n_shared=1, dtype="bf16", seed=11, b_std=0.1)
    base.update(kw)
    base.setdefault("wr_std", base["hidden"] ** -0.5)
    return synth.Workload(**base)


CASES = [(W[1], True), (W[1], False), (W[0], True),
         (var("odd_H2112", hidden=2112, T=333), True), (W[2], True)]


def ulp_bf16(v):
    """Spacing of bf16 values at |v| (normal range)."""
    e = np.floor(np.log2(np.maximum(np.abs(v), 2.0 ** -126)))
    return 2.0 ** (e - 7)


def run_adaln(wl, ada, per_token, eps=1e-6):
    cfg = cfg_for(wl)
    x = torch.from_numpy(ada["x"]).cuda()
    temb = torch.from_numpy(ada["temb6"]).cuda()
    table = torch.from_numpy(ada["table"]).cuda()
    h = torch.empty(x.shape, dtype=cfg.torch_dtype, device="cuda")
    lbv.lbv_adaln_rmsnorm(cfg, x, temb, table, eps, h)
    torch.cuda.synchronize()
    return host(h)


@pytest.mark.parametrize("wl,per_token", CASES, ids=lambda v: getattr(v, "name", str(v)))
def test_adaln_rmsnorm_parity(wl, per_token):
    note("adaln %s per_token=%s" % (wl.name, per_token))
    ada = synth.make_adaln_inputs(wl, per_token=per_token)
    got = run_adaln(wl, ada, per_token)
    raw = oracle.adaln_rmsnorm(ada["x"], ada["temb6"], ada["table"], 1e-6, round_bf16=False,
                               per_token=per_token).astype(np.float64)
    # magnitudes of the two terms of h, from the oracle's normalisation alone
    z6 = np.zeros_like(ada["table"])
    xr = oracle.adaln_rmsnorm(ada["x"], z6 if not per_token else np.zeros_like(ada["temb6"]), z6,
                              1e-6, round_bf16=False, per_token=per_token).astype(np.float64)
    t6 = ada["temb6"].astype(np.float64)
    tb = ada["table"].astype(np.float64)
    shift = tb[3][None] + (t6[:, 3] if per_token else t6[3][None])
    scale = tb[4][None] + (t6[:, 4] if per_token else t6[4][None])
    mag = np.abs(xr) * np.abs(1.0 + scale) + np.abs(shift)
    bound = 2.0 ** -20 * mag
    if wl.dtype == "bf16":
        bound = bound + 0.5 * ulp_bf16(raw)
        want = oracle.adaln_rmsnorm(ada["x"], ada["temb6"], ada["table"], 1e-6,
                                    per_token=per_token).astype(np.float64)
        frac = float((got != want).mean())
        print("adaln %s: %d elements, %.2e rounded the other way" % (wl.name, got.size, frac))
        assert frac <= 1e-3
    d = np.abs(got - raw)
    assert (d <= bound).all(), (d - bound).max()


def run_ffn(wl, d, ada, per_token, inplace=False, eps=1e-6):
    cfg = cfg_for(wl)
    x = torch.from_numpy(ada["x"]).cuda()
    temb = torch.from_numpy(ada["temb6"]).cuda()
    table = torch.from_numpy(ada["table"]).cuda()
    out = x if inplace else torch.empty_like(x)
    T = x.shape[0]
    ids = torch.empty(T, wl.top_k, dtype=torch.int32, device="cuda")
    w = torch.empty(T, wl.top_k, dtype=torch.float32, device="cuda")
    ws = torch.empty(lbv.lbv_moe_ffn_adaln_workspace_size(cfg, T), dtype=torch.uint8,
                     device="cuda")
    lbv.lbv_moe_ffn_adaln(cfg, x, d["mask"], temb, table, eps, d["router_w"], d["e_bias"],
                          d["w13"], d["w2"], d["shared_w13"], d["shared_w2"], out, ids, w, ws)
    torch.cuda.synchronize()
    return out, ids, w


@pytest.mark.timeout(900)
@pytest.mark.parametrize("wl,per_token", [(W[1], True), (W[2], False), (W[3], True), (W[0], True)],
                         ids=lambda v: getattr(v, "name", str(v)))
def test_ffn_adaln_parity(wl, per_token):
    """Every token: the block on the GPU's h routed like the oracle's block on
    that h (near ties tau-consistent), and out - x = gate * block(h)."""
    note("ffn_adaln %s per_token=%s" % (wl.name, per_token))
    inp = synth.make_inputs(wl)
    ada = synth.make_adaln_inputs(wl, per_token=per_token)
    d = upload(wl, inp)
    del d["x"]
    h = run_adaln(wl, ada, per_token).astype(np.float32)
    out, ids, w = run_ffn(wl, d, ada, per_token)
    o = oracle.route(wl, h, inp["router_w"], inp["e_bias"], inp["mask"], want_scores=True)
    g_ids = ids.cpu().numpy()
    same, near = compare_routing(wl, g_ids, w.cpu().numpy(), o, inp["e_bias"], inp["mask"])
    blk = oracle.moe_forward(wl, h, inp["router_w"], inp["e_bias"], inp["w13"], inp["w2"],
                             inp["shared_w13"], inp["shared_w2"], inp["mask"])
    moe = blk["out"]
    diff = np.nonzero(~same)[0]
    if diff.size:
        moe[diff] = oracle.moe_forward_ids(wl, h[diff], inp["router_w"], g_ids[diff], inp["w13"],
                                           inp["w2"], inp["shared_w13"], inp["shared_w2"])["out"]
    t6 = ada["temb6"].astype(np.float64)
    gate = ada["table"][5].astype(np.float64)[None] + (t6[:, 5] if per_token else t6[5][None])
    want = gate * moe
    out_h = out.cpu().numpy().astype(np.float64)
    got = out_h - ada["x"].astype(np.float64)
    m = metrics(got, want)
    print("ffn_adaln %s: %d tokens, %s; near-tie %d, other near-equal choice %d" % (
        wl.name, wl.T, m, near.sum(), diff.size))
    assert m["finite"]
    if wl.dtype == "bf16":
        assert m["rel_frob"] <= BF16_TOL["rel_frob"] and m["max_abs"] <= BF16_TOL["max_abs"], m
    else:
        # fp32 throughout: the block's fp32 accumulation error (1e-5 of the
        # update) plus one fp32 rounding of the residual sum
        want_out = ada["x"].astype(np.float64) + want
        bound = 2.0 ** -23 * np.abs(want_out) + 1e-5 * np.abs(want).max()
        assert (np.abs(out_h - want_out) <= bound).all()
    # padding tokens: the shared expert only
    if inp["mask"] is not None:
        assert (g_ids[inp["mask"] == 0] == -1).all()


def test_ffn_adaln_in_place_and_shared_temb():
    """out == x (in place) gives the out-of-place result bitwise; a shared
    temb row equals that row repeated per token."""
    wl = W[1]
    note("ffn_adaln in place")
    inp = synth.make_inputs(wl)
    d = upload(wl, inp)
    ada = synth.make_adaln_inputs(wl, per_token=False)
    o1, i1, w1 = run_ffn(wl, d, ada, False)
    o2, i2, w2 = run_ffn(wl, d, ada, False, inplace=True)
    assert torch.equal(o1, o2) and torch.equal(i1, i2) and torch.equal(w1, w2)
    rep = dict(ada, temb6=np.ascontiguousarray(np.repeat(ada["temb6"][None], wl.T, 0)))
    o3, i3, w3 = run_ffn(wl, d, rep, True)
    assert torch.equal(o1, o3) and torch.equal(i1, i3)
