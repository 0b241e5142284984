"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Bar: expert ids equal as sets on every token whose decision margins exceed
1e-5 (near ties may differ only by a near-equal choice), routing weights within
1e-5 relative, permutation bit-exact, and outputs within relative Frobenius
error 5e-3 and max-abs 3e-2 for bf16 storage (bf16 operands, fp32
accumulation), 1e-5 / 1e-5 for fp32 storage (fp32 everywhere; the error is
fp32 accumulation order over H <= 2048 terms, ~1e-6 relative).
"""
import numpy as np
import pytest
import torch

import oracle
import routed_moe_dit_amd as lbv
import synth
from gpu_util import cfg_for, compare_routing, dev, forward, host, metrics, note, upload

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
BF16_TOL = dict(rel_frob=5e-3, max_abs=3e-2)
F32_TOL = dict(rel_frob=1e-5, max_abs=1e-5)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    lbv.load()          # the HIP library must be present: no fallback exists
    yield


def var(name, **kw):
    base = dict(name=name, T=200, hidden=512, num_experts=64, n_group=4, topk_group=2, top_k=6,
                intermediate=128, n_shared=1, dtype="bf16", seed=11, b_std=0.1)
    base.update(kw)
    base.setdefault("wr_std", base["hidden"] ** -0.5)
    return synth.Workload(**base)


ROUTE_CASES = [
    W[0], W[1], W[2],
    var("E256_ng8_EPL4", num_experts=256, n_group=8, topk_group=4, top_k=8, T=333, hidden=256),
    var("E64_ng2_tg1", num_experts=64, n_group=2, topk_group=1, top_k=6, T=100, hidden=128),
    var("E8_G2_f32", num_experts=8, n_group=4, topk_group=2, top_k=2, T=65, hidden=64,
        dtype="f32"),
    var("E16_plain_T1", num_experts=16, n_group=1, topk_group=1, top_k=5, T=1, hidden=64),
    var("nonorm_negbias", norm_topk_prob=False, b_std=1.0, T=130),
    # above and below the 4096-token switch between the one-pass router and
    # the hidden-split router, for 64 experts and for top_k > 8
    var("E64_T5000", num_experts=64, n_group=4, topk_group=2, top_k=6, T=5000, hidden=256),
    var("E128_K12_T300", num_experts=128, n_group=4, topk_group=2, top_k=12, T=300, hidden=256),
    var("E128_K12_T5000", num_experts=128, n_group=4, topk_group=2, top_k=12, T=5000, hidden=256),
]


def run_route(wl, d):
    cfg = cfg_for(wl)
    T = d["x"].shape[0]
    ids = torch.empty(T, wl.top_k, dtype=torch.int32, device="cuda")
    w = torch.empty(T, wl.top_k, dtype=torch.float32, device="cuda")
    rws = torch.empty(max(lbv.lbv_moe_route_workspace_size(cfg), 16), dtype=torch.uint8,
                      device="cuda")
    lbv.lbv_moe_route(cfg, d["x"], d["router_w"], d["e_bias"], d["mask"], ids, w, rws)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), w.cpu().numpy()


@pytest.mark.parametrize("wl", ROUTE_CASES, ids=lambda w: w.name)
def test_route_parity(wl):
    note("route %s" % wl.name)
    inp = synth.make_inputs(wl)
    d = upload(wl, inp)
    g_ids, g_w = run_route(wl, d)
    o = oracle.route(wl, inp["x"], inp["router_w"], inp["e_bias"], inp["mask"], want_scores=True)
    same, near = compare_routing(wl, g_ids, g_w, o, inp["e_bias"], inp["mask"])
    if inp["mask"] is not None:
        pad = inp["mask"] == 0
        assert (g_ids[pad] == -1).all() and (g_w[pad] == 0).all()
        assert (g_ids[~pad] >= 0).all()
    # every chosen expert lies in a kept group: at most topk_group distinct groups
    G = wl.num_experts // wl.n_group
    for row in g_ids[g_ids[:, 0] >= 0]:
        assert len(set(row.tolist())) == wl.top_k
        assert len({e // G for e in row.tolist()}) <= wl.topk_group
    print("route %s: near-tie tokens %d, mismatched %d" % (wl.name, near.sum(), (~same).sum()))


@pytest.mark.parametrize("wl", [W[3], W[4]], ids=lambda w: w.name)
def test_route_parity_full_size(wl):
    note("route full %s" % wl.name)
    inp = synth.make_inputs(wl)
    d = dict(x=dev(inp["x"], "bf16"), router_w=dev(inp["router_w"], "f32"),
             e_bias=dev(inp["e_bias"], "f32"), mask=None)
    g_ids, g_w = run_route(wl, d)
    o = oracle.route(wl, inp["x"], inp["router_w"], inp["e_bias"], want_scores=True)
    same, near = compare_routing(wl, g_ids, g_w, o, inp["e_bias"])
    print("route %s: near-tie %d of %d, differing (near-equal) sets %d" % (wl.name, near.sum(), wl.T,
                                                                        (~same).sum()))


TIE_CASES = [W[1], var("E64_pairs", num_experts=64, n_group=4, topk_group=2, top_k=6, T=257),
             var("E256_pairs", num_experts=256, n_group=8, topk_group=4, top_k=8, T=333, hidden=256),
             var("E16_pairs_f32", num_experts=16, n_group=4, topk_group=2, top_k=4, T=65, hidden=64,
                 dtype="f32")]


@pytest.mark.parametrize("wl", TIE_CASES, ids=lambda w: w.name)
def test_route_exact_ties_break_to_lower_id(wl):
    """Experts 2m and 2m+1 get the same router row and bias, so their fp32
    logits, scores and selection values are bitwise equal (one expert tile
    computes both from identical operands).  Ties go to the lower id: 2m+1 is
    chosen only together with 2m, and the pair gets equal weights; the oracle
    obeys the same rule, and tokens with clear margins match it."""
    note("route ties %s" % wl.name)
    inp = synth.make_inputs(wl)
    rw, b = inp["router_w"].copy(), inp["e_bias"].copy()
    rw[1::2] = rw[0::2]
    b[1::2] = b[0::2]
    d = upload(wl, inp)
    d["router_w"], d["e_bias"] = dev(rw, "f32"), dev(b, "f32")
    g_ids, g_w = run_route(wl, d)
    o = oracle.route(wl, inp["x"], rw, b, inp["mask"], want_scores=True)
    for ids, ws in ((g_ids, g_w), (o["ids"], o["w"])):
        for row, wrow in zip(ids, ws):
            chosen = dict(zip(row.tolist(), wrow.tolist()))
            for e in chosen:
                if e >= 0 and e % 2 == 1:
                    assert e - 1 in chosen, (row, wl.name)
                    assert chosen[e] == chosen[e - 1]
    same, near = compare_routing(wl, g_ids, g_w, o, b, inp["mask"])
    print("route ties %s: near-tie %d of %d, mismatched %d" % (wl.name, near.sum(), len(g_ids),
                                                             (~same).sum()))


@pytest.mark.parametrize("T,E,K,ns", [(1, 16, 4, 1), (255, 128, 8, 1), (256, 128, 8, 1),
                                      (257, 128, 8, 0), (1000, 64, 6, 2), (2048, 256, 16, 8),
                                      (2049, 128, 8, 1), (38000, 128, 8, 1)])
def test_permute_parity(T, E, K, ns):
    note("permute T=%d E=%d K=%d ns=%d" % (T, E, K, ns))
    wl = var("perm", T=T, num_experts=E, top_k=K, n_shared=ns, n_group=4, topk_group=4)
    rng = np.random.default_rng(T + E)
    # skewed choices like the hot-expert workload, plus unrouted and repeated ids
    p = rng.dirichlet(np.full(E, 0.3))
    ids = np.stack([rng.choice(E, K, replace=False, p=p) for _ in range(T)]).astype(np.int32)
    ids[::5, -1] = -1
    ids[3::13, 1 % K] = ids[3::13, 0]
    cfg = cfg_for(wl)
    ids_d = torch.from_numpy(ids).cuda()
    S, KS = E + ns, K + ns
    off = torch.full((S + 1,), -7, dtype=torch.int32, device="cuda")
    srt = torch.full((T * KS,), -7, dtype=torch.int32, device="cuda")
    inv = torch.full((T * KS,), -7, dtype=torch.int32, device="cuda")
    ws = torch.empty(lbv.lbv_moe_permute_workspace_size(cfg, T), dtype=torch.uint8, device="cuda")
    lbv.lbv_moe_permute(cfg, ids_d, off, srt, inv, ws)
    torch.cuda.synchronize()
    o_off, o_srt, o_inv = oracle.permute(wl, ids)
    R = int(o_off[-1])
    np.testing.assert_array_equal(off.cpu().numpy(), o_off)
    np.testing.assert_array_equal(srt.cpu().numpy()[:R], o_srt[:R])
    np.testing.assert_array_equal(inv.cpu().numpy(), o_inv)




# The bf16 matmuls pick their tile height from the rows per segment on
# average, T (K + ns) / (E + ns): 64 rows below 20, 128 rows below 480, else
# 256 rows.  The cases cover each height at the LingBot dims and with odd dims.
GEMM_CASES = [
    W[0],
    W[1],                                                          # 128-row tiles (56 rows)
    var("ns2_ragged", n_shared=2, T=77),                           # 64-row tiles (9 rows)
    # 54,000 rows, several 128-row tiles per segment (419 rows)
    var("E128_T6000_full_dims", num_experts=128, top_k=8, T=6000, hidden=2048, intermediate=768),
    # 72,000 rows: 256-row tiles (558 rows)
    var("E128_T8000_full_dims", num_experts=128, top_k=8, T=8000, hidden=2048, intermediate=768),
    # an odd number of 64-wide k-tiles on both matmuls (H/64 = 33, I/64 = 11)
    # and partial n-tiles (I/128 = 5.5, H/256 = 8.25), with 256-, 128- and 64-row tiles
    var("odd_H2112_I704_T8000", num_experts=128, top_k=8, T=8000, hidden=2112, intermediate=704),
    var("odd_H2112_I704_T3000", num_experts=128, top_k=8, T=3000, hidden=2112, intermediate=704),
    var("odd_H2112_I704_T500", num_experts=128, top_k=8, T=500, hidden=2112, intermediate=704),
    var("odd_H2112_I704_T200", num_experts=128, top_k=8, T=200, hidden=2112, intermediate=704),
]


def oracle_routing(wl, inp):
    o = oracle.route(wl, inp["x"], inp["router_w"], inp["e_bias"], inp["mask"])
    off, srt, inv = oracle.permute(wl, o["ids"])
    return o, off, srt, inv


@pytest.mark.timeout(600)
@pytest.mark.parametrize("wl", GEMM_CASES, ids=lambda w: w.name)
def test_gemm_w13_silu_parity(wl):
    """Every act row against the oracle's SwiGLU of its (token, expert), on
    the oracle's own routing; rows past the routed count stay untouched."""
    note("gemm_w13 %s" % wl.name)
    inp = synth.make_inputs(wl)
    d = upload(wl, inp)
    o, off, srt, inv = oracle_routing(wl, inp)
    R = int(off[-1])
    KS = wl.top_k + wl.n_shared
    cfg = cfg_for(wl)
    act = torch.zeros(wl.T * KS, wl.intermediate, dtype=d["x"].dtype, device="cuda")
    gws = torch.empty(lbv.lbv_moe_w13_workspace_size(cfg, wl.T), dtype=torch.uint8, device="cuda")
    lbv.lbv_moe_gemm_w13_silu(cfg, d["x"], d["w13"], d["shared_w13"],
                              torch.from_numpy(off).cuda(), torch.from_numpy(srt).cuda(), act, gws)
    torch.cuda.synchronize()
    g = host(act)
    seg = (np.searchsorted(off, np.arange(R), side="right") - 1).astype(np.int32)
    tok = (srt[:R] // KS).astype(np.int32)
    ref = oracle.act_rows(wl, inp["x"], inp["w13"], inp["shared_w13"], tok, seg)
    got = g[:R]
    m = metrics(got, ref)
    print("gemm_w13 %s: %d rows, %s" % (wl.name, R, m))
    if wl.dtype == "bf16":
        # one bf16 rounding of act: |err| <= 2^-8 |act| plus accumulation noise
        bad = np.abs(got - ref) > 2.0 ** -8 * np.abs(ref) + 1e-4 * np.abs(ref).max()
        assert not bad.any(), "rows %s" % np.unique(np.nonzero(bad)[0])[:10]
    else:
        assert m["rel_frob"] <= 1e-5
    assert np.all(g[R:] == 0)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("wl", GEMM_CASES, ids=lambda w: w.name)
def test_gemm_w2_combine_parity(wl):
    """Down projection + combine from given act rows (seeded bf16 values) on
    the oracle's routing: every token against the oracle's down projection and
    weighted combine of the same act vectors."""
    note("gemm_w2_combine %s" % wl.name)
    inp = synth.make_inputs(wl)
    d = upload(wl, inp)
    o, off, srt, inv = oracle_routing(wl, inp)
    R = int(off[-1])
    KS = wl.top_k + wl.n_shared
    act = synth.random_act(wl.T * KS, wl.intermediate, seed=wl.seed + 100)
    act[R:] = 0
    if wl.dtype == "f32":
        act_d = torch.from_numpy(act).cuda()
    else:
        act_d = dev(act, "bf16")
    slot_rows = np.where(inv >= 0, inv, 0)
    act_slots = act[slot_rows].reshape(wl.T, KS, wl.intermediate)
    act_slots[(inv < 0).reshape(wl.T, KS)] = 0
    cfg = cfg_for(wl)
    out = torch.zeros(wl.T, wl.hidden, dtype=d["x"].dtype, device="cuda")
    ws = torch.empty(lbv.lbv_moe_w2_workspace_size(cfg, wl.T), dtype=torch.uint8, device="cuda")
    lbv.lbv_moe_gemm_w2_combine(cfg, act_d, d["w2"], d["shared_w2"],
                                torch.from_numpy(off).cuda(), torch.from_numpy(srt).cuda(),
                                torch.from_numpy(inv).cuda(), torch.from_numpy(o["w"]).cuda(),
                                out, ws)
    torch.cuda.synchronize()
    ref = oracle.down_combine(wl, act_slots, o["ids"], o["w"], inp["w2"], inp["shared_w2"])
    m = metrics(host(out), ref)
    print("gemm_w2_combine %s: %d tokens, %s" % (wl.name, wl.T, m))
    tol = BF16_TOL if wl.dtype == "bf16" else F32_TOL
    assert m["rel_frob"] <= tol["rel_frob"] and m["max_abs"] <= tol["max_abs"], m


FWD_CASES = [
    W[0], W[1],
    var("ns0", n_shared=0, T=97),
    var("ns2", n_shared=2, T=64),
    var("K1", top_k=1, topk_group=1, T=50),
    var("E256_EPL4", num_experts=256, n_group=8, topk_group=4, top_k=8, T=40, hidden=256),
    var("nonorm", norm_topk_prob=False, T=60),
    var("T1", T=1),
    var("f32_ragged", dtype="f32", T=45, hidden=128, intermediate=64),
    var("E128_K12_ns2", num_experts=128, top_k=12, n_shared=2, T=300, hidden=256),
    var("odd_H2112_I704", num_experts=128, top_k=8, T=300, hidden=2112, intermediate=704),
]


def check_forward(wl, inp, out, ids, w, rows=None, tol=None):
    """Every listed token against the oracle: tokens where the GPU chose the
    oracle's expert set against the oracle's output; near-tie tokens where it
    made another near-equal choice (checked by compare_routing) against the
    oracle's output at the GPU's choice.  No token is left out."""
    rows = np.arange(wl.T) if rows is None else np.asarray(rows)
    mask = None if inp["mask"] is None else inp["mask"][rows]
    x = inp["x"][rows]
    ref = oracle.moe_forward(wl, x, inp["router_w"], inp["e_bias"], inp["w13"], inp["w2"],
                             inp["shared_w13"], inp["shared_w2"], mask)
    o = oracle.route(wl, x, inp["router_w"], inp["e_bias"], mask, want_scores=True)
    assert np.array_equal(o["ids"], ref["ids"])
    g_ids = ids.cpu().numpy()[rows]
    same, near = compare_routing(wl, g_ids, w.cpu().numpy()[rows], o, inp["e_bias"], mask)
    want = ref["out"].copy()
    diff = np.nonzero(~same)[0]
    if diff.size:
        alt = oracle.moe_forward_ids(wl, x[diff], inp["router_w"], g_ids[diff], inp["w13"],
                                     inp["w2"], inp["shared_w13"], inp["shared_w2"])
        want[diff] = alt["out"]
    got = host(out)[rows]
    m = metrics(got, want)
    tol = tol or (BF16_TOL if wl.dtype == "bf16" else F32_TOL)
    print("forward %s: %d tokens, %s; near-tie %d, other near-equal choice %d" % (
        wl.name, len(rows), m, near.sum(), diff.size))
    assert m["finite"]
    assert m["rel_frob"] <= tol["rel_frob"], m
    assert m["max_abs"] <= tol["max_abs"], m
    return m


@pytest.mark.parametrize("wl", FWD_CASES, ids=lambda w: w.name)
def test_forward_parity(wl):
    note("forward %s" % wl.name)
    inp = synth.make_inputs(wl)
    d = upload(wl, inp)
    out, ids, w = forward(wl, d)
    check_forward(wl, inp, out, ids, w)


@pytest.mark.timeout(600)
def test_forward_parity_mid_size():
    """8,000 tokens (past the router's 4096-token switch; 558 rows per
    segment, so 256-row matmul tiles): every token against the oracle."""
    wl = var("E128_T8000", num_experts=128, top_k=8, T=8000, hidden=256, intermediate=256)
    note("forward %s" % wl.name)
    inp = synth.make_inputs(wl)
    d = upload(wl, inp)
    out, ids, w = forward(wl, d)
    check_forward(wl, inp, out, ids, w)


@pytest.mark.timeout(600)
def test_forward_parity_padded_batch():
    """CFG batch B=2 with 40 padding tokens: every token against the oracle."""
    wl = W[2]
    note("forward %s" % wl.name)
    inp = synth.make_inputs(wl)
    d = upload(wl, inp)
    out, ids, w = forward(wl, d)
    check_forward(wl, inp, out, ids, w)
    pad = inp["mask"] == 0
    assert (ids.cpu().numpy()[pad] == -1).all()


@pytest.mark.timeout(900)
@pytest.mark.parametrize("wl", [W[3], W[4], W[5]], ids=lambda w: w.name)
def test_forward_parity_full_size(wl):
    """38,000 tokens in one call, every token against the oracle."""
    note("forward full %s" % wl.name)
    inp = synth.make_inputs(wl)
    d = upload(wl, inp)
    out, ids, w = forward(wl, d)
    del d
    check_forward(wl, inp, out, ids, w)
    counts = np.bincount(ids.cpu().numpy().reshape(-1), minlength=wl.num_experts)
    if wl.hot:
        print("hot-expert share of assignments: %.3f" % (counts[list(wl.hot)].sum() / counts.sum()))


def test_sample_isolation_bitwise():
    """A sample's outputs inside the B=2 batch equal those of the sample alone."""
    wl = W[2]
    note("isolation %s" % wl.name)
    inp = synth.make_inputs(wl)
    d = upload(wl, inp)
    out, ids, w = forward(wl, d)
    for lo, hi in ((0, 800), (800, 1600)):
        x1 = d["x"][lo:hi].contiguous()
        m1 = d["mask"][lo:hi].contiguous()
        o1, i1, w1 = forward(wl, d, x=x1, mask=m1)
        assert torch.equal(o1, out[lo:hi]) and torch.equal(i1, ids[lo:hi]) and torch.equal(w1, w[lo:hi])
    perm = torch.randperm(1600, generator=torch.Generator().manual_seed(0)).cuda()
    op, ip, _ = forward(wl, d, x=d["x"][perm].contiguous(), mask=d["mask"][perm].contiguous())
    assert torch.equal(op, out[perm]) and torch.equal(ip, ids[perm])


@pytest.mark.parametrize("E", [128, 64])
def test_routing_independent_of_batch_size(E):
    """5,000 tokens (one-pass router) route bitwise like the same tokens in
    calls of 2,500 and of 1 (few-token router): the two paths form the logits
    in the same order."""
    wl = W[3].replace(T=5000) if E == 128 else var("E64_T5000_iso", num_experts=64, top_k=6,
                                                  T=5000, hidden=2048)
    note("routing vs batch size E=%d" % E)
    inp = synth.make_inputs(wl)
    d = dict(x=dev(inp["x"], "bf16"), router_w=dev(inp["router_w"], "f32"),
             e_bias=dev(inp["e_bias"], "f32"), mask=None)
    ids, w = run_route(wl, d)
    for lo, hi in ((0, 2500), (2500, 5000), (1234, 1235)):
        part = dict(d, x=d["x"][lo:hi].contiguous())
        i2, w2 = run_route(wl, part)
        assert np.array_equal(i2, ids[lo:hi]) and np.array_equal(w2, w[lo:hi]), (lo, hi)


def test_determinism_and_split_calls():
    """Two forwards are bitwise equal, and so is the chain of the four calls."""
    wl = W[1]
    note("determinism %s" % wl.name)
    inp = synth.make_inputs(wl)
    d = upload(wl, inp)
    o1, i1, w1 = forward(wl, d)
    o2, i2, w2 = forward(wl, d)
    assert torch.equal(o1, o2) and torch.equal(i1, i2) and torch.equal(w1, w2)
    cfg = cfg_for(wl)
    T, K, KS, S = wl.T, wl.top_k, wl.top_k + wl.n_shared, wl.num_experts + wl.n_shared
    ids = torch.empty(T, K, dtype=torch.int32, device="cuda")
    w = torch.empty(T, K, dtype=torch.float32, device="cuda")
    rws = torch.empty(lbv.lbv_moe_route_workspace_size(cfg), dtype=torch.uint8, device="cuda")
    lbv.lbv_moe_route(cfg, d["x"], d["router_w"], d["e_bias"], None, ids, w, rws)
    off = torch.empty(S + 1, dtype=torch.int32, device="cuda")
    srt = torch.empty(T * KS, dtype=torch.int32, device="cuda")
    inv = torch.empty(T * KS, dtype=torch.int32, device="cuda")
    pws = torch.empty(lbv.lbv_moe_permute_workspace_size(cfg, T), dtype=torch.uint8, device="cuda")
    lbv.lbv_moe_permute(cfg, ids, off, srt, inv, pws)
    act = torch.empty(T * KS, wl.intermediate, dtype=torch.bfloat16, device="cuda")
    gws = torch.empty(lbv.lbv_moe_w13_workspace_size(cfg, T), dtype=torch.uint8, device="cuda")
    lbv.lbv_moe_gemm_w13_silu(cfg, d["x"], d["w13"], d["shared_w13"], off, srt, act, gws)
    out = torch.empty(T, wl.hidden, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(lbv.lbv_moe_w2_workspace_size(cfg, T), dtype=torch.uint8, device="cuda")
    lbv.lbv_moe_gemm_w2_combine(cfg, act, d["w2"], d["shared_w2"], off, srt, inv, w, out, ws)
    torch.cuda.synchronize()
    assert torch.equal(out, o1) and torch.equal(ids, i1) and torch.equal(w, w1)


def test_bias_selects_but_does_not_weigh():
    """Expert 3 forced into every set by its bias; weights stay functions of the
    raw scores: equal bitwise wherever the slot order did not change."""
    wl = var("bias", T=256)
    note("bias invariant")
    inp = synth.make_inputs(wl)
    d = upload(wl, inp)
    i1, w1 = run_route(wl, d)
    d2 = dict(d)
    b2 = inp["e_bias"].copy()
    b2[3] += 10.0
    d2["e_bias"] = torch.from_numpy(b2).cuda()
    i2, w2 = run_route(wl, d2)
    assert (i2 == 3).any(1).all()
    sameorder = (i1 == i2).all(1)
    assert np.array_equal(w1[sameorder], w2[sameorder])
    o2 = oracle.route(wl, inp["x"], inp["router_w"], b2, want_scores=True)
    compare_routing(wl, i2, w2, o2, b2)


def test_scaling_applied_once():
    """Identical routed experts, no shared expert: out = 2.5 f(x) (not 6.25 f(x))."""
    wl = var("scale", T=32, n_shared=0)
    note("scaling once")
    inp = synth.make_inputs(wl)
    inp["w13"][:] = inp["w13"][:1]
    inp["w2"][:] = inp["w2"][:1]
    d = upload(wl, inp)
    out, ids, w = forward(wl, d)
    f = np.stack([oracle.expert_out(wl, inp["x"][t], inp["w13"], inp["w2"], 0) for t in range(32)])
    m = metrics(host(out), 2.5 * f)
    assert m["rel_frob"] <= 5e-3, m


def test_all_padding_gives_shared_only():
    wl = var("allpad", T=70)
    note("all padding")
    inp = synth.make_inputs(wl)
    inp["mask"] = np.zeros(70, np.uint8)
    d = upload(wl, inp)
    out, ids, w = forward(wl, d)
    assert (ids.cpu().numpy() == -1).all() and (w.cpu().numpy() == 0).all()
    check_forward(wl, inp, out, ids, w)


def test_zero_tokens_is_noop():
    """T == 0: every call succeeds and enqueues nothing."""
    wl = var("zero", T=4)
    note("zero tokens")
    inp = synth.make_inputs(wl)
    d = upload(wl, inp)
    cfg = cfg_for(wl)
    x = d["x"][:0]
    out = torch.empty_like(x)
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    lbv.lbv_moe_forward(cfg, x, None, d["router_w"], d["e_bias"], d["w13"], d["w2"],
                        d["shared_w13"], d["shared_w2"], out, None, None, ws)
    ids = torch.empty(0, wl.top_k, dtype=torch.int32, device="cuda")
    w = torch.empty(0, wl.top_k, dtype=torch.float32, device="cuda")
    lbv.lbv_moe_route(cfg, x, d["router_w"], d["e_bias"], None, ids, w, ws)
    torch.cuda.synchronize()


def test_forward_in_hip_graph_replays_bitwise():
    """lbv_moe_forward only enqueues kernels on the caller's stream (no
    allocation, no memset, no host sync), so it can be captured in a HIP
    graph.  Each replay, with other eager work and synchronisations in between
    and a changed input, equals the eager call on the same input bitwise."""
    wl = W[2]
    note("graph capture %s" % wl.name)
    inp = synth.make_inputs(wl)
    d = upload(wl, inp)
    cfg = cfg_for(wl)
    T = d["x"].shape[0]
    x = d["x"].clone()
    out = torch.empty_like(x)
    ids = torch.empty(T, wl.top_k, dtype=torch.int32, device="cuda")
    w = torch.empty(T, wl.top_k, dtype=torch.float32, device="cuda")
    ws = torch.empty(lbv.lbv_moe_workspace_size(cfg, T), dtype=torch.uint8, device="cuda")

    def call():
        lbv.lbv_moe_forward(cfg, x, d["mask"], d["router_w"], d["e_bias"], d["w13"], d["w2"],
                            d["shared_w13"], d["shared_w2"], out, ids, w, ws,
                            torch.cuda.current_stream())

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()                                    # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    gen = torch.Generator(device="cpu").manual_seed(5)
    for rep in range(4):
        if rep:
            # a new input in place, then eager reference work on other buffers
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
