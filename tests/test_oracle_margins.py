"""Pins of the oracle's decision margins and of its given-choice entry points.

The margins decide which tokens count as tie-free (ids must then match
exactly), so their magnitude and their rank are pinned here against values
fixed by hand and against brute-force enumeration.  Sources: prhub summary of
sglang PR #32341, section 实现拆解 step 1 and risk 4 under 风险与影响 (group
score = sum of the two best biased scores, group-limited top-k); vLLM-Omni
LingBot-Video article, section MoE 实现的源码级要点 (selection on scores plus
bias, weights from the raw scores).

m_grp = g_(topk_group) - g_(topk_group + 1) over the group scores sorted
descending; m_sel = c_(K) - c_(K + 1) over the kept groups' experts.  The best
group subset minus the second-best one is exactly m_grp (swap the weakest kept
group for the strongest dropped one), and likewise for K-subsets and m_sel.
"""
import itertools

import numpy as np
import pytest
from scipy.special import expit

import oracle
import synth


def tiny(**kw):
    base = dict(name="t", T=8, hidden=64, num_experts=16, n_group=4, topk_group=2, top_k=3,
                intermediate=32, n_shared=1, dtype="f32", seed=0, wr_std=64 ** -0.5, b_std=0.1)
    base.update(kw)
    return synth.Workload(**base)


# Selection values c = 0.5 + b (x = 0 and W_r = 0 give every logit 0 and every
# score exactly 0.5); every value is a multiple of 2^-5, so all sums are exact.
C_HAND = np.array([
    0.9375, 0.75, 0.5, 0.25,          # group 0: top-2 sum 1.6875
    0.875, 0.59375, 0.4375, 0.125,    # group 1: 1.46875
    0.8125, 0.5625, 0.3125, 0.0625,   # group 2: 1.375
    0.6875, 0.5, 0.4375, 0.1875,      # group 3: 1.1875
], np.float32)


def hand_route(wl, c):
    H = wl.hidden
    x = np.zeros((1, H), np.float32)
    wr = np.zeros((wl.num_experts, H), np.float32)
    b = (c - np.float32(0.5)).astype(np.float32)
    assert np.array_equal(b + np.float32(0.5), c)
    return oracle.route(wl, x, wr, b)


def test_margins_closed_form():
    """Group scores sorted: 1.6875, 1.46875, 1.375, 1.1875; with 2 groups kept
    m_grp = 1.46875 - 1.375 = 0.09375 (the neighbouring gaps are 0.21875 and
    0.1875, a factor-of-4 error gives 0.375).  Kept groups 0 and 1, their
    experts sorted: 0.9375, 0.875, 0.75, 0.59375, 0.5, ...; with K = 3
    m_sel = 0.75 - 0.59375 = 0.15625 (neighbouring gaps 0.125 and 0.09375; over
    all experts instead of the kept groups' it would be 0.75 - 0.8125 < 0)."""
    wl = tiny()
    r = hand_route(wl, C_HAND)
    assert sorted(r["ids"][0].tolist()) == [0, 1, 4]
    assert r["m_grp"][0] == 0.09375
    assert r["m_sel"][0] == 0.15625
    # the same values for other K and topk_group
    r = hand_route(tiny(top_k=5), C_HAND)             # c_(5) - c_(6) = 0.5 - 0.4375
    assert r["m_sel"][0] == 0.0625 and r["m_grp"][0] == 0.09375
    r = hand_route(tiny(topk_group=3, top_k=2), C_HAND)
    assert r["m_grp"][0] == 1.375 - 1.1875             # g_(3) - g_(4)
    assert r["m_sel"][0] == 0.875 - 0.8125             # third best over groups 0, 1, 2
    r = hand_route(tiny(topk_group=1, top_k=4), C_HAND)
    assert r["m_grp"][0] == 1.6875 - 1.46875
    assert r["m_sel"][0] == np.inf                     # all 4 experts of the group chosen


def test_margins_infinite_without_alternatives_and_zero_on_ties():
    r = hand_route(tiny(topk_group=4, top_k=2), C_HAND)
    assert r["m_grp"][0] == np.inf                     # every group kept
    assert r["m_sel"][0] == 0.875 - 0.8125 and r["ids"][0].tolist() == [0, 4]
    c = C_HAND.copy()
    c[8], c[9] = np.float32(0.875), np.float32(0.59375)   # group 2 now sums to 1.46875, as group 1
    r = hand_route(tiny(), c)
    assert r["m_grp"][0] == 0.0                        # an exact group tie
    assert sorted(r["ids"][0].tolist()) == [0, 1, 4]   # the lower group index wins


def brute_force_margins(c, E, n_group, topk_group, K):
    """Best minus second-best group subset (sum of pair-best group scores), and
    best minus second-best K-subset of the best group subset's experts."""
    G = E // n_group
    g = []
    for j in range(n_group):
        best = None
        for a, b in itertools.combinations(range(j * G, (j + 1) * G), 2):
            v = np.float32(np.float32(c[a]) + np.float32(c[b]))
            best = v if best is None or v > best else best
        g.append(float(best))
    subs = sorted((sum(g[j] for j in sub), sub)
                  for sub in itertools.combinations(range(n_group), topk_group))
    subs = sorted(subs, key=lambda p: -p[0])
    m_grp = subs[0][0] - subs[1][0] if len(subs) > 1 else np.inf
    experts = [e for j in subs[0][1] for e in range(j * G, (j + 1) * G)]
    sums = sorted((sum(float(c[e]) for e in sub)
                   for sub in itertools.combinations(experts, K)), reverse=True)
    m_sel = sums[0] - sums[1] if len(sums) > 1 else np.inf
    return m_grp, m_sel


@pytest.mark.parametrize("E,ng,tg,K", [(16, 4, 2, 3), (16, 4, 2, 4), (16, 4, 1, 2),
                                       (16, 2, 1, 5), (8, 4, 2, 3), (16, 4, 3, 4)])
def test_margins_brute_force_gap(E, ng, tg, K):
    """The oracle's margins equal the subset gaps found by enumeration (sums of
    fp32 values in fp64 are exact here), so a scaled, shifted-by-one-rank or
    wrong-set margin fails."""
    wl = tiny(num_experts=E, n_group=ng, topk_group=tg, top_k=K, T=40, seed=E + 10 * K + tg)
    inp = synth.make_inputs(wl)
    r = oracle.route(wl, inp["x"], inp["router_w"], inp["e_bias"], want_scores=True)
    c = (r["s"] + inp["e_bias"][None, :]).astype(np.float32)
    for t in range(wl.T):
        mg, ms = brute_force_margins(c[t], E, ng, tg, K)
        assert r["m_grp"][t] == pytest.approx(mg, rel=0, abs=1e-12), t
        if r["m_grp"][t] > 0:      # the kept set is unique, so is the expert margin
            assert r["m_sel"][t] == pytest.approx(ms, rel=0, abs=1e-12), t


# ---------------------------------------------------------------------------
# Given-choice entry points against float64 library matmuls
# ---------------------------------------------------------------------------

def mlp(w13, w2, x, width):
    g, u = w13[:width] @ x, w13[width:] @ x
    return w2 @ (g * expit(g) * u)


@pytest.mark.parametrize("norm", [True, False])
def test_forward_ids_library(norm):
    """Arbitrary given ids (not the top-k, with empty slots): weights are the
    raw sigmoid scores at those ids (fp32, slot-order sum, one scaling), the
    output the weighted expert sum plus the shared expert."""
    wl = tiny(T=12, hidden=64, intermediate=32, n_shared=2, top_k=4, norm_topk_prob=norm)
    inp = synth.make_inputs(wl)
    rng = np.random.default_rng(4)
    ids = np.stack([rng.choice(16, 4, replace=False) for _ in range(wl.T)]).astype(np.int32)
    ids[::3, 1] = -1
    res = oracle.moe_forward_ids(wl, inp["x"], inp["router_w"], ids, inp["w13"], inp["w2"],
                                 inp["shared_w13"], inp["shared_w2"])
    r = oracle.route(wl, inp["x"], inp["router_w"], inp["e_bias"], want_scores=True)
    x = inp["x"].astype(np.float64)
    for t in range(wl.T):
        s = r["s"][t]
        tot = np.float32(0)
        for e in ids[t]:
            if e >= 0:
                tot = np.float32(tot + s[e])
        want_w = []
        for e in ids[t]:
            v = np.float32(0) if e < 0 else (np.float32(s[e] / tot) if norm else s[e])
            want_w.append(np.float32(v * np.float32(2.5)) if e >= 0 else np.float32(0))
        assert np.array_equal(res["w"][t], np.array(want_w, np.float32))
        want = mlp(inp["shared_w13"].astype(np.float64), inp["shared_w2"].astype(np.float64),
                   x[t], 64)
        for k, e in enumerate(ids[t]):
            if e >= 0:
                want = want + float(res["w"][t, k]) * mlp(inp["w13"][e].astype(np.float64),
                                                           inp["w2"][e].astype(np.float64),
                                                           x[t], 32)
        np.testing.assert_allclose(res["out"][t], want, rtol=1e-10, atol=1e-13)


def test_forward_ids_at_own_choice_equals_forward():
    wl = tiny(T=20, hidden=64, intermediate=32)
    inp = synth.make_inputs(wl)
    f = oracle.moe_forward(wl, inp["x"], inp["router_w"], inp["e_bias"], inp["w13"], inp["w2"],
                           inp["shared_w13"], inp["shared_w2"])
    g = oracle.moe_forward_ids(wl, inp["x"], inp["router_w"], f["ids"], inp["w13"], inp["w2"],
                               inp["shared_w13"], inp["shared_w2"])
    assert np.array_equal(f["w"], g["w"])
    assert np.array_equal(f["out"], g["out"])


@pytest.mark.parametrize("ns", [1, 2])
def test_act_rows_library(ns):
    """Routed rows use w13[e] (gate rows first, then up rows); shared slice j
    uses gate rows jI.. and up rows I_s + jI.. of the shared gate/up matrix."""
    wl = tiny(T=10, hidden=64, intermediate=16, n_shared=ns)
    inp = synth.make_inputs(wl)
    rng = np.random.default_rng(1)
    tok = rng.integers(0, wl.T, 40).astype(np.int32)
    seg = rng.integers(0, wl.num_experts + ns, 40).astype(np.int32)
    act = oracle.act_rows(wl, inp["x"], inp["w13"], inp["shared_w13"], tok, seg)
    I, Is = 16, 16 * ns
    x = inp["x"].astype(np.float64)
    sw = inp["shared_w13"].astype(np.float64)
    for r in range(40):
        if seg[r] < wl.num_experts:
            W = inp["w13"][seg[r]].astype(np.float64)
            g, u = W[:I] @ x[tok[r]], W[I:] @ x[tok[r]]
        else:
            j = seg[r] - wl.num_experts
            g = sw[j * I:(j + 1) * I] @ x[tok[r]]
            u = sw[Is + j * I:Is + (j + 1) * I] @ x[tok[r]]
        np.testing.assert_allclose(act[r], g * expit(g) * u, rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("ns", [0, 1, 2])
def test_down_combine_library(ns):
    wl = tiny(T=9, hidden=64, intermediate=16, n_shared=ns, top_k=3)
    inp = synth.make_inputs(wl)
    rng = np.random.default_rng(2)
    KS = 3 + ns
    act = rng.standard_normal((9, KS, 16)).astype(np.float32)
    ids = np.stack([rng.choice(16, 3, replace=False) for _ in range(9)]).astype(np.int32)
    ids[4, 2] = -1
    w = rng.uniform(0.1, 1.0, (9, 3)).astype(np.float32)
    out = oracle.down_combine(wl, act, ids, w, inp["w2"], inp["shared_w2"])
    for t in range(9):
        want = np.zeros(64)
        for k in range(3):
            if ids[t, k] >= 0:
                want += float(w[t, k]) * (inp["w2"][ids[t, k]].astype(np.float64) @ act[t, k])
        for j in range(ns):
            want += inp["shared_w2"][:, j * 16:(j + 1) * 16].astype(np.float64) @ act[t, 3 + j]
        np.testing.assert_allclose(out[t], want, rtol=1e-12, atol=1e-14)
