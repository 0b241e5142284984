"""Pins of the oracle's steps around the block: RMSNorm + AdaLN modulation in
front of it and the gated residual after it (prhub summary of sglang PR
#32341, 实现拆解 step 2: AdaLN through scale_shift_table and a token-level
temb6, norms kept in fp32; vLLM-Omni LingBot-Video article, MoE 实现的源码级要点:
RMSNorm accumulates in fp32).  The readings (formula, row order of the
modulation table, no learnable norm weight) are listed with the oracle.
"""
import numpy as np
import pytest

import oracle
import synth


def wl_small(**kw):
    base = dict(name="ada", T=16, hidden=64, num_experts=16, n_group=4, topk_group=2, top_k=4,
                intermediate=32, n_shared=1, dtype="bf16", seed=5, wr_std=64 ** -0.5, b_std=0.1)
    base.update(kw)
    return synth.Workload(**base)


def test_bf16_round_matches_bit_rounding_and_ties():
    """The oracle's rounding from fp64 against round-to-nearest-even on the
    fp32 bit pattern (synth.round_to_bf16) for fp32 values, including exact
    ties; and direct fp64 cases just off a midpoint."""
    rng = np.random.default_rng(0)
    a = (rng.standard_normal(20000) * np.exp(rng.uniform(-20, 20, 20000))).astype(np.float32)
    ties = (np.arange(1, 200, dtype=np.float32) * np.float32(2.0 ** -8) + np.float32(1.0))
    a = np.concatenate([a, ties, -ties]).astype(np.float32)
    want = synth.round_to_bf16(a.copy())
    got = oracle.bf16_round(a.astype(np.float64))
    assert np.array_equal(got, want.astype(np.float64))
    mid = 1.0 + 2.0 ** -8                       # midpoint between 1 and 1 + 2^-7
    assert oracle.bf16_round([mid, mid + 2.0 ** -40, mid - 2.0 ** -40]).tolist() == \
        [1.0, 1.0 + 2.0 ** -7, 1.0]
    mid3 = 1.0 + 3 * 2.0 ** -8                  # ties to the even neighbour 1 + 2^-6
    assert oracle.bf16_round([mid3])[0] == 1.0 + 2.0 ** -6


def zeros6(H):
    return np.zeros((6, H), np.float32)


def test_constant_row_normalises_to_its_sign():
    H = 64
    x = np.stack([np.full(H, c, np.float32) for c in (3.0, -0.25, 1e3)])
    h = oracle.adaln_rmsnorm(x, zeros6(H), zeros6(H), eps=0.0, per_token=False)
    assert h.tolist() == [[1.0] * H, [-1.0] * H, [1.0] * H]


def test_one_hot_row_closed_form():
    """x = c e_j: mean(x^2) = c^2 / H, so h_j = sign(c) sqrt(H) (1 + scale_j) + shift_j
    and h_i = shift_i elsewhere (eps = 0, no rounding)."""
    H = 64
    rng = np.random.default_rng(1)
    table = rng.uniform(-0.5, 0.5, (6, H)).astype(np.float32)
    temb = rng.uniform(-0.5, 0.5, (6, H)).astype(np.float32)
    x = np.zeros((1, H), np.float32)
    x[0, 9] = -2.5
    h = oracle.adaln_rmsnorm(x, temb, table, eps=0.0, round_bf16=False, per_token=False)
    shift = table[3].astype(np.float64) + temb[3]
    scale = table[4].astype(np.float64) + temb[4]
    want = shift.copy()
    want[9] = -np.sqrt(H) * (1 + scale[9]) + shift[9]
    np.testing.assert_allclose(h[0], want.astype(np.float32), rtol=2e-7, atol=0)


def test_scale_minus_one_gives_shift_and_power_of_two_invariance():
    H = 128
    rng = np.random.default_rng(2)
    x = rng.standard_normal((8, H)).astype(np.float32)
    table = zeros6(H)
    table[4] = -1.0                                     # 1 + scale = 0
    temb = rng.standard_normal((8, 6, H)).astype(np.float32)
    temb[:, 4] = 0.0
    h = oracle.adaln_rmsnorm(x, temb, table, eps=1e-6)
    assert np.array_equal(h, synth.round_to_bf16(temb[:, 3].copy()))
    # rmsnorm(2^k x) == rmsnorm(x) exactly when eps = 0
    t2 = rng.standard_normal((8, 6, H)).astype(np.float32)
    a = oracle.adaln_rmsnorm(x, t2, zeros6(H), eps=0.0)
    b = oracle.adaln_rmsnorm(x * np.float32(8.0), t2, zeros6(H), eps=0.0)
    assert np.array_equal(a, b)


def test_eps_enters_under_the_root():
    """x = c 1 with eps: h = c / sqrt(c^2 + eps) (no rounding)."""
    H = 64
    for c, eps in ((1e-3, 1e-6), (0.5, 1e-2)):
        x = np.full((1, H), c, np.float32)
        h = oracle.adaln_rmsnorm(x, zeros6(H), zeros6(H), eps=eps, round_bf16=False,
                                 per_token=False)
        c64 = float(np.float32(c))
        assert h[0, 0] == np.float32(c64 / np.sqrt(c64 * c64 + eps))


def test_token_level_rows_are_used_per_token():
    H = 64
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, H)).astype(np.float32)
    table = rng.standard_normal((6, H)).astype(np.float32)
    temb = rng.standard_normal((6, H)).astype(np.float32)
    shared = oracle.adaln_rmsnorm(x, temb, table, per_token=False)
    per = oracle.adaln_rmsnorm(x, np.repeat(temb[None], 5, 0), table, per_token=True)
    assert np.array_equal(shared, per)
    temb_t = np.repeat(temb[None], 5, 0)
    temb_t[2, 3] += 1.0                                 # token 2's shift only
    per2 = oracle.adaln_rmsnorm(x, temb_t, table, per_token=True)
    assert np.array_equal(np.delete(per2, 2, 0), np.delete(per, 2, 0))
    assert not np.array_equal(per2[2], per[2])
    # rows 0-2 (the attention half) do not enter
    temb_t[:, 0:3] += 5.0
    temb_t[2, 3] -= 1.0
    assert np.array_equal(oracle.adaln_rmsnorm(x, temb_t, table, per_token=True), per)


def test_gated_residual():
    """gate = 0 leaves x exactly; zero expert outputs leave x exactly; the
    residual update is linear in the gate."""
    wl = wl_small()
    inp = synth.make_inputs(wl)
    ada = synth.make_adaln_inputs(wl)
    args = (inp["router_w"], inp["e_bias"], inp["w13"], inp["w2"], inp["shared_w13"],
            inp["shared_w2"])
    t0 = ada["table"].copy()
    e0 = ada["temb6"].copy()
    t0[5] = 0.0
    e0[:, 5] = 0.0
    r = oracle.ffn_adaln(wl, ada["x"], e0, t0, *args)
    assert np.array_equal(r["out"], ada["x"].astype(np.float64))
    z = oracle.ffn_adaln(wl, ada["x"], ada["temb6"], ada["table"], inp["router_w"],
                         inp["e_bias"], inp["w13"], np.zeros_like(inp["w2"]), inp["shared_w13"],
                         np.zeros_like(inp["shared_w2"]))
    assert np.array_equal(z["out"], ada["x"].astype(np.float64))
    r1 = oracle.ffn_adaln(wl, ada["x"], ada["temb6"], ada["table"], *args)
    t2, e2 = ada["table"].copy(), ada["temb6"].copy()
    t2[5] *= 2
    e2[:, 5] *= 2
    r2 = oracle.ffn_adaln(wl, ada["x"], e2, t2, *args)
    x = ada["x"].astype(np.float64)
    np.testing.assert_allclose(r2["out"] - x, 2 * (r1["out"] - x), rtol=1e-12, atol=1e-15)
    # the block sees h, and the router's ids come from h
    blk = oracle.moe_forward(wl, r1["h"], *args)
    assert np.array_equal(blk["ids"], r1["block"]["ids"])


def test_modulation_rows_are_selectable():
    """Rows (shift, scale): (3, 4) in front of the FFN block (the default),
    (0, 1) in front of the attention block.  With eps = 0 a constant row a
    normalises to sign(a), so h = sign(a) (1 + scale) + shift exactly."""
    H = 64
    table = np.repeat((0.1 * (np.arange(6) + 1))[:, None], H, 1).astype(np.float32)
    temb6 = np.zeros((2, 6, H), np.float32)
    x = np.stack([np.full(H, 3.0), np.full(H, -0.5)]).astype(np.float32)
    sgn = np.array([1.0, -1.0])[:, None]
    for rows, (sh, sc) in (((3, 4), (0.4, 0.5)), ((0, 1), (0.1, 0.2))):
        h = oracle.adaln_rmsnorm(x, temb6, table, 0.0, round_bf16=False, rows=rows)
        want = sgn * (1 + np.float64(np.float32(sc))) + np.float64(np.float32(sh))
        assert np.allclose(h, np.broadcast_to(want, (2, H)), rtol=1e-7), rows
    assert np.array_equal(oracle.adaln_rmsnorm(x, temb6, table, 0.0, round_bf16=False),
                          oracle.adaln_rmsnorm(x, temb6, table, 0.0, round_bf16=False,
                                               rows=(3, 4)))
