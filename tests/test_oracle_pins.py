"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test names the mistake it is meant to catch.  Sources: prhub summary of
sglang PR #32341 (section 实现拆解 step 1, the moe.py excerpt, risk 4 under
风险与影响) and the vLLM-Omni LingBot-Video article (section
MoE 实现的源码级要点).
"""
import itertools
import json
import os

import numpy as np
import pytest
from scipy.special import expit

import oracle
import synth

HERE = os.path.dirname(os.path.abspath(__file__))


def tiny(**kw):
    base = dict(name="t", T=32, hidden=64, num_experts=16, n_group=4, topk_group=2, top_k=4,
                intermediate=32, n_shared=1, dtype="f32", seed=0, wr_std=64 ** -0.5, b_std=0.1)
    base.update(kw)
    return synth.Workload(**base)


def scores(wl, inp):
    r = oracle.route(wl, inp["x"], inp["router_w"], inp["e_bias"], inp["mask"], want_scores=True)
    c = (r["s"] + inp["e_bias"][None, :]).astype(np.float32)   # fp32 add, as the router does
    return r, c


# ---------------------------------------------------------------------------
# Router logits and sigmoid against library routines
# ---------------------------------------------------------------------------

def test_logits_and_sigmoid_match_library():
    """Catches a wrong sign in the sigmoid, a transposed router weight, a
    dropped term of the dot product."""
    wl = tiny(T=64, hidden=256)
    inp = synth.make_inputs(wl)
    r, _ = scores(wl, inp)
    z64 = inp["x"].astype(np.float64) @ inp["router_w"].astype(np.float64).T
    bound = 256 * 2.0 ** -24 * (np.abs(inp["x"]).astype(np.float64) @ np.abs(inp["router_w"]).T)
    assert np.all(np.abs(r["z"] - z64) <= bound + 1e-30)
    s64 = expit(r["z"].astype(np.float64))
    assert np.max(np.abs(r["s"] - s64) / s64) < 2.0 ** -22


# ---------------------------------------------------------------------------
# Group-limited top-k against brute-force enumeration (no sort / top-k code)
# ---------------------------------------------------------------------------

def brute_force_select(c, E, n_group, topk_group, K):
    G = E // n_group
    # group score: best pair sum inside the group (fp32 add, as on the pages)
    g = []
    for j in range(n_group):
        best = None
        for a, b in itertools.permutations(range(j * G, (j + 1) * G), 2):
            v = np.float32(c[a]) + np.float32(c[b])
            best = v if best is None or v > best else best
        g.append(float(best))
    best_sub, best_val = None, None
    for sub in itertools.combinations(range(n_group), topk_group):
        v = sum(g[j] for j in sub)
        if best_val is None or v > best_val:
            best_sub, best_val = sub, v
    experts = [e for j in best_sub for e in range(j * G, (j + 1) * G)]
    best_set, best_val = None, None
    for sub in itertools.combinations(experts, K):
        v = sum(float(c[e]) for e in sub)
        if best_val is None or v > best_val:
            best_set, best_val = sub, v
    return set(best_set)


CASES = [(16, 4, 2, 4), (16, 4, 1, 3), (16, 2, 1, 4), (16, 4, 4, 4), (8, 2, 1, 2),
         (8, 4, 2, 3), (16, 1, 1, 4), (8, 1, 1, 3), (16, 4, 3, 2), (8, 2, 2, 4)]


@pytest.mark.parametrize("E,ng,tg,K", CASES)
@pytest.mark.parametrize("b_std", [0.1, 1.0])
def test_group_topk_brute_force(E, ng, tg, K, b_std):
    """Catches: group score from the best expert only or from all experts,
    bias left out of selection, experts of dropped groups allowed back in
    (b_std=1.0 makes selection values negative, where masking with 0 would
    differ from exclusion)."""
    wl = tiny(num_experts=E, n_group=ng, topk_group=tg, top_k=K, b_std=b_std,
              seed=100 + E * 7 + ng * 3 + tg + K, T=48)
    inp = synth.make_inputs(wl)
    r, c = scores(wl, inp)
    checked = 0
    for t in range(wl.T):
        if min(r["m_grp"][t], r["m_sel"][t]) < 1e-6:
            continue
        assert set(r["ids"][t].tolist()) == brute_force_select(c[t], E, ng, tg, K), t
        checked += 1
    assert checked >= wl.T // 2
    if b_std == 1.0:
        assert (c < 0).any()


def test_plain_topk_special_case():
    """n_group = topk_group = 1 is plain top-K (textbook: stable argsort)."""
    wl = tiny(num_experts=16, n_group=1, topk_group=1, top_k=5, T=64)
    inp = synth.make_inputs(wl)
    r, c = scores(wl, inp)
    for t in range(wl.T):
        want = np.argsort(-c[t], kind="stable")[:5]
        assert r["ids"][t].tolist() == want.tolist()


def test_ties_go_to_lower_index():
    """Reading of the pages' silence on ties: lower group and expert index win."""
    wl = tiny(num_experts=8, n_group=2, topk_group=1, top_k=2, T=1, hidden=8)
    x = np.zeros((1, 8), np.float32)
    wr = np.zeros((8, 8), np.float32)          # all logits 0, all scores 0.5
    b = np.zeros(8, np.float32)
    r = oracle.route(wl, x, wr, b)
    assert r["ids"][0].tolist() == [0, 1]
    assert r["m_grp"][0] == 0.0 and r["m_sel"][0] == 0.0
    b[5] = 0.25                                 # group 1 now wins; expert 5 first
    r = oracle.route(wl, x, wr, b)
    assert r["ids"][0].tolist() == [5, 4]


# ---------------------------------------------------------------------------
# Bias selects, raw scores weigh; scaling applied exactly once
# ---------------------------------------------------------------------------

def test_bias_shifts_selection_but_not_weights():
    """Catches biased scores used as gate weights."""
    wl = tiny(T=128)
    inp = synth.make_inputs(wl)
    r1, _ = scores(wl, inp)
    b2 = inp["e_bias"].copy()
    b2[3] += 10.0                              # expert 3 forced into every token's set
    r2 = oracle.route(wl, inp["x"], inp["router_w"], b2, want_scores=True)
    assert np.array_equal(r1["s"], r2["s"])    # scores do not depend on the bias
    assert all(3 in row for row in r2["ids"].tolist())
    changed = 0
    for t in range(wl.T):
        s = r2["s"][t].astype(np.float32)
        ids = r2["ids"][t]
        total = np.float32(0)
        for e in ids:
            total = np.float32(total + s[e])
        want = np.array([np.float32(np.float32(s[e] / total) * np.float32(2.5)) for e in ids])
        assert np.array_equal(r2["w"][t], want)
        if set(ids.tolist()) != set(r1["ids"][t].tolist()):
            changed += 1
        elif ids.tolist() == r1["ids"][t].tolist():
            assert np.array_equal(r1["w"][t], r2["w"][t])
        else:   # same set, other slot order: the fp32 sum is taken in another order
            d1 = dict(zip(r1["ids"][t].tolist(), r1["w"][t].tolist()))
            d2 = dict(zip(ids.tolist(), r2["w"][t].tolist()))
            for e in d1:
                assert abs(d1[e] - d2[e]) <= 4e-7 * abs(d1[e])
    assert changed > 0


def test_uniform_bias_shift_changes_nothing():
    wl = tiny(T=128)
    inp = synth.make_inputs(wl)
    r1, _ = scores(wl, inp)
    r2 = oracle.route(wl, inp["x"], inp["router_w"], inp["e_bias"] + np.float32(0.375))
    ok = np.minimum(r1["m_grp"], r1["m_sel"]) > 1e-5
    for t in np.nonzero(ok)[0]:
        assert set(r1["ids"][t]) == set(r2["ids"][t])
        d1 = dict(zip(r1["ids"][t].tolist(), r1["w"][t].tolist()))
        d2 = dict(zip(r2["ids"][t].tolist(), r2["w"][t].tolist()))
        assert d1 == d2


@pytest.mark.parametrize("norm", [True, False])
def test_weight_sum_and_scaling_once(norm):
    """Normalised weights sum to the scaling factor (2.5, not 1 or 6.25);
    without normalisation each weight is 2.5 times its raw score."""
    wl = tiny(T=64, norm_topk_prob=norm)
    inp = synth.make_inputs(wl)
    r, _ = scores(wl, inp)
    if norm:
        assert np.allclose(r["w"].astype(np.float64).sum(1), 2.5, rtol=0, atol=2e-6)
    else:
        for t in range(wl.T):
            s = r["s"][t][r["ids"][t]]
            assert np.array_equal(r["w"][t], (s * np.float32(2.5)).astype(np.float32))


def test_identical_experts_closed_form():
    """All routed experts identical and no shared expert: out = 2.5 f(x)
    exactly up to rounding.  A kernel that scales twice gives 6.25 f(x)."""
    wl = tiny(T=16, n_shared=0)
    inp = synth.make_inputs(wl)
    w13 = np.repeat(inp["w13"][:1], wl.num_experts, axis=0)
    w2 = np.repeat(inp["w2"][:1], wl.num_experts, axis=0)
    res = oracle.moe_forward(wl, inp["x"], inp["router_w"], inp["e_bias"], w13, w2)
    for t in range(wl.T):
        f = oracle.expert_out(wl, inp["x"][t], w13, w2, 0)
        np.testing.assert_allclose(res["out"][t], 2.5 * f, rtol=1e-6, atol=1e-12)


# ---------------------------------------------------------------------------
# Expert MLP: closed forms from unit-vector weights, library matmuls
# ---------------------------------------------------------------------------

def unit_expert(H, I, rng, a_scale=3.0):
    """w13 rows: gate row i = a_i e_{p_i}, up row i = e_{q_i}; w2 row n = e_{r_n}.
    Then y_n = silu(a_{r_n} x_{p_{r_n}}) x_{q_{r_n}} (closed form)."""
    p = rng.integers(0, H, I)
    q = rng.integers(0, H, I)
    r = rng.integers(0, I, H)
    a = rng.uniform(-a_scale, a_scale, I).astype(np.float32)
    w13 = np.zeros((2 * I, H), np.float32)
    w13[np.arange(I), p] = a
    w13[I + np.arange(I), q] = 1.0
    w2 = np.zeros((H, I), np.float32)
    w2[np.arange(H), r] = 1.0
    return w13, w2, (p, q, r, a)


def closed_form_y(x, pqra):
    p, q, r, a = pqra
    u = a[r].astype(np.float64) * x[p[r]]
    return u * expit(u) * x[q[r]]


def test_expert_mlp_closed_form():
    """Catches gate and up swapped (interleaving), SiLU on the wrong half,
    w2 read transposed, a wrong expert index."""
    wl = tiny(hidden=64, intermediate=32, num_experts=4, n_group=2, topk_group=1, top_k=2)
    rng = np.random.default_rng(7)
    w13 = np.zeros((4, 64, 64), np.float32)
    w2 = np.zeros((4, 64, 32), np.float32)
    forms = []
    for e in range(4):
        a, b, f = unit_expert(64, 32, rng)
        w13[e], w2[e] = a, b
        forms.append(f)
    x = rng.standard_normal((8, 64)).astype(np.float32)
    for t in range(8):
        for e in range(4):
            y = oracle.expert_out(wl, x[t], w13, w2, e)
            np.testing.assert_allclose(y, closed_form_y(x[t].astype(np.float64), forms[e]),
                                       rtol=1e-14, atol=1e-300)


def test_expert_mlp_library_matmul():
    wl = tiny(hidden=128, intermediate=64)
    inp = synth.make_inputs(wl)
    x = inp["x"].astype(np.float64)
    for e in (0, 5, 15):
        W = inp["w13"][e].astype(np.float64)
        act_ref = (lambda g, u: g * expit(g) * u)(W[:64] @ x[3], W[64:] @ x[3])
        np.testing.assert_allclose(oracle.expert_act(wl, inp["x"][3], inp["w13"], e), act_ref,
                                   rtol=1e-12, atol=1e-15)
        y_ref = inp["w2"][e].astype(np.float64) @ act_ref
        np.testing.assert_allclose(oracle.expert_out(wl, inp["x"][3], inp["w13"], inp["w2"], e),
                                   y_ref, rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("ns", [1, 2])
def test_shared_expert_closed_form(ns):
    """Routed experts zeroed (w2 = 0): out = shared(x) with weight 1, not 2.5;
    the shared gate/up split at I*n_shared, not at I."""
    H, I = 64, 16
    wl = tiny(hidden=H, intermediate=I, n_shared=ns, T=8)
    inp = synth.make_inputs(wl)
    rng = np.random.default_rng(11)
    sw13, sw2, f = unit_expert(H, I * ns, rng)
    w2 = np.zeros_like(inp["w2"])
    res = oracle.moe_forward(wl, inp["x"], inp["router_w"], inp["e_bias"], inp["w13"], w2,
                             sw13, sw2)
    for t in range(8):
        np.testing.assert_allclose(res["out"][t],
                                   closed_form_y(inp["x"][t].astype(np.float64), f),
                                   rtol=1e-14, atol=1e-300)


def test_full_block_library_matmul():
    """The whole combine against float64 library matmuls at the oracle's ids."""
    wl = tiny(T=24, hidden=64, intermediate=32, n_shared=2)
    inp = synth.make_inputs(wl)
    res = oracle.moe_forward(wl, inp["x"], inp["router_w"], inp["e_bias"], inp["w13"],
                             inp["w2"], inp["shared_w13"], inp["shared_w2"])
    x = inp["x"].astype(np.float64)

    def mlp(w13, w2, xv, width):
        g, u = w13[:width] @ xv, w13[width:] @ xv
        return w2 @ (g * expit(g) * u)

    for t in range(wl.T):
        want = mlp(inp["shared_w13"].astype(np.float64), inp["shared_w2"].astype(np.float64),
                   x[t], 64)
        for k in range(wl.top_k):
            e = res["ids"][t, k]
            want = want + float(res["w"][t, k]) * mlp(inp["w13"][e].astype(np.float64),
                                                       inp["w2"][e].astype(np.float64), x[t], 32)
        np.testing.assert_allclose(res["out"][t], want, rtol=1e-10, atol=1e-13)


# ---------------------------------------------------------------------------
# Padding and per-sample isolation
# ---------------------------------------------------------------------------

def test_padding_gets_shared_only():
    wl = tiny(T=16)
    inp = synth.make_inputs(wl)
    mask = np.ones(16, np.uint8)
    mask[10:] = 0
    res = oracle.moe_forward(wl, inp["x"], inp["router_w"], inp["e_bias"], inp["w13"],
                             inp["w2"], inp["shared_w13"], inp["shared_w2"], mask)
    zero_routed = oracle.moe_forward(wl, inp["x"], inp["router_w"], inp["e_bias"], inp["w13"],
                                     np.zeros_like(inp["w2"]), inp["shared_w13"],
                                     inp["shared_w2"])
    assert (res["ids"][10:] == -1).all() and (res["w"][10:] == 0).all()
    assert (res["ids"][:10] >= 0).all()
    np.testing.assert_array_equal(res["out"][10:], zero_routed["out"][10:])


def test_sample_isolation():
    """Each token's output depends on that token only (B=2 batch vs alone,
    and a permutation of the tokens permutes the outputs)."""
    wl = tiny(T=32)
    inp = synth.make_inputs(wl)
    args = (inp["router_w"], inp["e_bias"], inp["w13"], inp["w2"], inp["shared_w13"],
            inp["shared_w2"])
    both = oracle.moe_forward(wl, inp["x"], *args)
    a = oracle.moe_forward(wl, inp["x"][:16], *args)
    b = oracle.moe_forward(wl, inp["x"][16:], *args)
    np.testing.assert_array_equal(both["out"], np.concatenate([a["out"], b["out"]]))
    perm = np.random.default_rng(0).permutation(32)
    p = oracle.moe_forward(wl, inp["x"][perm], *args)
    np.testing.assert_array_equal(p["out"], both["out"][perm])
    np.testing.assert_array_equal(p["ids"], both["ids"][perm])


def test_margins_predict_stability():
    """Tokens whose margins exceed 1e-5 keep their expert set when the router
    weight is perturbed at the fp32 rounding level."""
    wl = tiny(T=256, hidden=256, num_experts=16)
    inp = synth.make_inputs(wl)
    r1, _ = scores(wl, inp)
    rng = np.random.default_rng(3)
    wr2 = (inp["router_w"] * (1 + 2e-7 * rng.standard_normal(inp["router_w"].shape))).astype(
        np.float32)
    r2 = oracle.route(wl, inp["x"], wr2, inp["e_bias"])
    ok = np.minimum(r1["m_grp"], r1["m_sel"]) > 1e-5
    assert ok.sum() > 200
    for t in np.nonzero(ok)[0]:
        assert set(r1["ids"][t]) == set(r2["ids"][t])
    assert (r1["m_grp"] >= 0).all() and (r1["m_sel"] >= 0).all()


def test_invalid_config_rejected():
    wl = tiny(num_experts=12, n_group=8)      # 8 does not divide 12
    inp = synth.make_inputs(tiny())
    with pytest.raises(ValueError):
        oracle.route(wl, inp["x"][:, :64], inp["router_w"][:12], inp["e_bias"][:12])


# ---------------------------------------------------------------------------
# Constants printed on the pages
# ---------------------------------------------------------------------------

def test_page_constants():
    g = json.load(open(os.path.join(HERE, "golden", "page_constants.json")))
    for wl in synth.WORKLOADS[1:]:
        assert wl.num_experts == g["num_experts"]["value"]
        assert wl.top_k == g["top_k"]["value"]
        assert wl.intermediate == g["moe_intermediate_size"]["value"]
        assert wl.n_group == g["n_group"]["value"]
        assert wl.topk_group == g["topk_group"]["value"]
        assert wl.routed_scaling_factor == g["routed_scaling_factor"]["value"]
        assert wl.n_shared == g["n_shared_experts"]["value"]
        # packed w13 [E, 2I, H] in bf16 is the 768 MiB tensor the review names
        shape = [wl.num_experts, 2 * wl.intermediate, wl.hidden]
        assert shape == g["w13_packed_shape"]["value"]
        assert np.prod(shape) * 2 == g["w13_packed_bytes_bf16"]["value"]
    # parameter count: 48 MoE layers of (128 + 1) experts of 3*H*I plus the router
    # account for all but ~0.2% of the published total (attention adds 4 H^2 per layer)
    wl = synth.WORKLOADS[3]
    H, I, E = wl.hidden, wl.intermediate, wl.num_experts
    per_layer = (E + 1) * 3 * H * I + E * H + E + 4 * H * H
    total = g["checkpoint_params"]["value"]
    assert 0.995 < per_layer * g["num_layers"]["value"] / total < 1.0
    # token counts of the two video shapes
    assert ((9 - 1) // 4 + 1) * (192 // 16) * (320 // 16) == g["video_tokens_9f_192x320"]["value"]
    assert ((81 - 1) // 4 + 1) * (480 // 16) * (480 // 16) == g["video_tokens_81f_480x480"]["value"]
    assert synth.WORKLOADS[1].T == 720 + 80
    assert synth.WORKLOADS[3].T == 2 * (18900 + 100)
