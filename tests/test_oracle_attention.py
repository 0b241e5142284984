"""Pins of the oracle's attention half (projections, per-head RMSNorm, rotary
embedding with neox style off, masked per-sample softmax attention): closed
forms, invariants and independent library computations.  Source: prhub
summary of sglang PR #32341, the LingBotVideoAttention excerpt under
"关键源码片段" (q/k/v/out projections, norm_q / norm_k over head_dim, rotary
embedding with is_neox_style=False, non-causal attention with the default
scale) and "实现拆解" step 2 (video;text joint attention, padding isolated by
the mask)."""
import numpy as np
import pytest
import scipy.special

import oracle


def rng(seed):
    return np.random.default_rng(seed)


# ---- projections -------------------------------------------------------------

def test_linear_matches_numpy_matmul():
    r = rng(0)
    x = r.standard_normal((7, 48)).astype(np.float32)
    w = r.standard_normal((20, 48)).astype(np.float32)
    b = r.standard_normal(20).astype(np.float32)
    y = oracle.linear(x, w, b)
    ref = x.astype(np.float64) @ w.astype(np.float64).T + b
    assert np.allclose(y, ref, rtol=1e-13, atol=1e-12)
    assert np.allclose(oracle.linear(x, w), ref - b, rtol=1e-13, atol=1e-12)
    # row n of w is output channel n: a unit row picks that input channel
    e = np.zeros((3, 48), np.float32)
    e[0, 5], e[1, 0], e[2, 47] = 1, 1, 1
    assert np.array_equal(oracle.linear(x, e), x[:, [5, 0, 47]].astype(np.float64))


# ---- per-head RMSNorm -----------------------------------------------------------

def test_head_rmsnorm_closed_forms():
    D = 16
    g = np.linspace(0.5, 2.0, D).astype(np.float32)
    for c in (3.0, -0.25):
        u = np.full((2, D), c)
        y = oracle.head_rmsnorm(u, g, 1e-6)
        assert np.allclose(y, c / np.sqrt(c * c + 1e-6) * g.astype(np.float64), rtol=1e-14)
    # scale invariance with eps = 0, and each row normalised on its own
    u = rng(1).standard_normal((5, D))
    y = oracle.head_rmsnorm(u, np.ones(D, np.float32), 0.0)
    y2 = oracle.head_rmsnorm(u * np.array([[1], [10], [0.1], [3], [7]]), np.ones(D, np.float32), 0.0)
    assert np.allclose(y, y2, rtol=1e-13)
    assert np.allclose((y * y).mean(1), 1.0, rtol=1e-13)
    # eps enters under the root with the mean (not the sum) of squares
    u = np.ones((1, D))
    y = oracle.head_rmsnorm(u, np.ones(D, np.float32), 1.0)
    assert np.allclose(y, 1 / np.sqrt(2.0), rtol=1e-14)


# ---- rotary embedding ----------------------------------------------------------

def tables(pos, D, theta=10000.0):
    inv = theta ** (-np.arange(D // 2) * 2.0 / D)
    ang = np.outer(pos, inv)
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32), ang


def test_rope_hand_example_and_identity():
    D = 8
    u = np.zeros((1, 1, D))
    u[0, 0, 0], u[0, 0, 1] = 1.0, 2.0
    cos = np.ones((1, D // 2), np.float32)
    sin = np.zeros((1, D // 2), np.float32)
    assert np.array_equal(oracle.rope(u, cos, sin), u)
    # a quarter turn of pair 0: (a, b) -> (-b, a); pair 1 (channels 2, 3) untouched
    cos[0, 0], sin[0, 0] = 0.0, 1.0
    y = oracle.rope(u, cos, sin)
    assert np.array_equal(y[0, 0, :2], [-2.0, 1.0]) and (y[0, 0, 2:] == 0).all()
    # neox style off: channel D/2 is not pair 0's partner
    u2 = u.copy()
    u2[0, 0, D // 2] = 5.0
    assert np.array_equal(oracle.rope(u2, cos, sin)[0, 0, :2], [-2.0, 1.0])


def test_rope_norms_and_relative_positions():
    D, heads = 32, 3
    r = rng(2)
    u = r.standard_normal((6, heads, D))
    cos, sin, _ = tables(np.arange(6) * 7.0, D)
    y = oracle.rope(u, cos, sin)
    pair = lambda a: a[..., 0::2] ** 2 + a[..., 1::2] ** 2
    assert np.allclose(pair(y), pair(u), rtol=1e-6)
    # q at p and k at p' give a dot product that depends on p - p' only
    q = r.standard_normal((1, 1, D))
    k = r.standard_normal((1, 1, D))
    dots = []
    for p, pk in ((3.0, 1.0), (10.0, 8.0), (102.0, 100.0)):
        cq, sq, _ = tables([p], D)
        ck, sk, _ = tables([pk], D)
        cq, sq, ck, sk = (a.astype(np.float64).astype(np.float32) for a in (cq, sq, ck, sk))
        dots.append(float((oracle.rope(q, cq, sq) * oracle.rope(k, ck, sk)).sum()))
    assert np.allclose(dots, dots[0], rtol=1e-5)


# ---- attention -----------------------------------------------------------------

def qkv(T, heads, D, seed):
    r = rng(seed)
    return tuple(r.standard_normal((T, heads, D)).astype(np.float32) for _ in range(3))


def test_identical_keys_average_the_values():
    T, S, heads, D = 12, 6, 2, 16
    q, k, v = qkv(T, heads, D, 3)
    k[:] = k[0]
    o = oracle.attention(q, k, v, S)
    for b in range(2):
        want = v[b * S:(b + 1) * S].astype(np.float64).mean(0)
        assert np.allclose(o[b * S:(b + 1) * S], want[None], rtol=1e-12, atol=1e-14)


def test_single_key_and_two_key_softmax_scale():
    T, S, heads, D = 8, 8, 1, 16
    q, k, v = qkv(T, heads, D, 4)
    mask = np.zeros(T, np.uint8)
    mask[[0, 5]] = 1
    # one valid token: it is the only key, so its query returns its value exactly
    m1 = np.zeros(T, np.uint8)
    m1[5] = 1
    o = oracle.attention(q, k, v, S, m1)
    assert np.array_equal(o[5], v[5].astype(np.float64)) and (o[np.arange(T) != 5] == 0).all()
    # two keys along channel 0: weights e^{a b_j / sqrt(D)} normalised
    q[:] = 0
    k[:] = 0
    q[:, 0, 0] = 2.0
    k[0, 0, 0], k[5, 0, 0] = 1.0, -0.5
    o = oracle.attention(q, k, v, S, mask)
    s = np.array([2.0 * 1.0, 2.0 * -0.5]) / np.sqrt(D)
    p = np.exp(s - s.max())
    p /= p.sum()
    want = p[0] * v[0].astype(np.float64) + p[1] * v[5].astype(np.float64)
    assert np.allclose(o[0], want, rtol=1e-13)
    assert (o[[1, 2, 3, 4, 6, 7]] == 0).all()          # padding queries give 0


def test_padding_keys_and_other_samples_do_not_matter():
    T, S, heads, D = 20, 10, 2, 8
    q, k, v = qkv(T, heads, D, 5)
    mask = np.ones(T, np.uint8)
    mask[[7, 8, 9, 19]] = 0
    o = oracle.attention(q, k, v, S, mask)
    k2, v2 = k.copy(), v.copy()
    k2[[7, 8, 9]] += 100
    v2[[7, 8, 9]] -= 50
    k2[10:] = 3.0          # the whole second sample changes
    v2[10:] = -1.0
    o2 = oracle.attention(q, k2, v2, S, mask)
    assert np.array_equal(o[:10], o2[:10])
    # permuting the valid keys (with their values) inside a sample changes
    # nothing for any query of it
    k3, v3 = k.copy(), v.copy()
    k3[:7], v3[:7] = k[:7][::-1], v[:7][::-1]
    o3 = oracle.attention(q, k3, v3, S, mask)
    assert np.allclose(o3[:10], o[:10], rtol=1e-12, atol=1e-14)


def test_attention_matches_scipy_softmax():
    T, S, heads, D = 30, 15, 3, 16
    q, k, v = qkv(T, heads, D, 6)
    mask = np.ones(T, np.uint8)
    mask[[3, 14, 29]] = 0
    o = oracle.attention(q, k, v, S, mask)
    for t in range(T):
        for h in range(heads):
            if not mask[t]:
                assert (o[t, h] == 0).all()
                continue
            b = t // S
            js = [j for j in range(b * S, (b + 1) * S) if mask[j]]
            s = k[js, h].astype(np.float64) @ q[t, h].astype(np.float64) / np.sqrt(D)
            want = scipy.special.softmax(s) @ v[js, h].astype(np.float64)
            assert np.allclose(o[t, h], want, rtol=1e-11, atol=1e-13)
    sub = oracle.attention(q, k, v, S, mask, qrows=[29, 0, 16])
    assert np.array_equal(sub, o[[29, 0, 16]])


def test_attention_half_closed_form():
    """q and k projections zero: the head norms give 0, every valid key gets
    the same weight, so the block output is mean(x over the sample's valid
    tokens) W_o^T + b_o (the v block is the identity); padding rows get b_o."""
    T, S, H, heads = 12, 6, 32, 2
    r = rng(7)
    x = r.standard_normal((T, H)).astype(np.float32)
    w_qkv = np.zeros((3 * H, H), np.float32)
    w_qkv[2 * H:] = np.eye(H, dtype=np.float32)
    b_qkv = np.zeros(3 * H, np.float32)
    x = oracle.bf16_round(x).astype(np.float32)
    g = np.ones(H // heads, np.float32)
    cos, sin, _ = tables(np.arange(T) * 1.0, H // heads)
    mask = np.ones(T, np.uint8)
    mask[[4, 5, 11]] = 0
    w_o = oracle.bf16_round(r.standard_normal((H, H)) * 0.1).astype(np.float32)
    b_o = (r.standard_normal(H) * 0.1).astype(np.float32)
    out = oracle.attn_forward(x, w_qkv, b_qkv, g, g, 1e-6, cos, sin, heads, S, mask, w_o, b_o)
    for b in range(2):
        rows = [t for t in range(b * S, (b + 1) * S) if mask[t]]
        mean = oracle.bf16_round(x[rows].astype(np.float64).mean(0))
        want = oracle.bf16_round(mean @ w_o.astype(np.float64).T + b_o)
        for t in range(b * S, (b + 1) * S):
            if mask[t]:
                assert np.allclose(out[t], want, rtol=0, atol=0)
            else:
                assert np.array_equal(out[t], oracle.bf16_round(b_o.astype(np.float64)))
    sub = oracle.attn_forward(x, w_qkv, b_qkv, g, g, 1e-6, cos, sin, heads, S, mask, w_o, b_o,
                              qrows=[7, 0])
    assert np.array_equal(sub, out[[7, 0]])


def test_qkv_blocks_and_norm_weights():
    """Constant q and k projections per head: after the head norm each is
    sign(c) g / sqrt(1 + eps / c^2); with cos = 1, sin = 0 the rotary
    embedding leaves it as is.  q is the first block of the fused projection
    with g_q, k the second with g_k, v the third."""
    T, H, heads = 3, 16, 2
    D = H // heads
    x = np.zeros((T, H), np.float32)
    x[:, 0] = 1.0
    w = np.zeros((3 * H, H), np.float32)
    w[:H, 0], w[H:2 * H, 0], w[2 * H:, 0] = 2.0, -0.5, 0.25
    b = np.zeros(3 * H, np.float32)
    g_q = np.linspace(1, 2, D).astype(np.float32)
    g_k = np.linspace(-1, 3, D).astype(np.float32)
    cos, sin = np.ones((T, D // 2), np.float32), np.zeros((T, D // 2), np.float32)
    q, k, v = oracle.attn_qkv(x, w, b, g_q, g_k, 1e-6, cos, sin, heads)
    for c, g, got in ((2.0, g_q, q), (-0.5, g_k, k)):
        want = oracle.bf16_round(np.sign(c) * g.astype(np.float64) / np.sqrt(1 + 1e-6 / c ** 2))
        assert np.array_equal(got, np.broadcast_to(want, (T, heads, D)).astype(np.float32))
    assert (v == 0.25).all()


def test_attention_half_with_adaln_closed_form():
    """The attention half of a layer: h = AdaLN(x) with rows 0 (shift) and
    1 (scale), the half on h, out = x + gate * block with gate = row 2.  With
    zero q/k projections every valid key weighs the same, so block =
    bf16(bf16(mean of the sample's valid h) W_o^T + b_o) and the output is
    x + (table[2] + temb6[t, 2]) block, in closed form."""
    T, S, H, heads = 12, 6, 32, 2
    r = rng(8)
    x = r.standard_normal((T, H)).astype(np.float32)
    table = (r.standard_normal((6, H)) * 0.3).astype(np.float32)
    temb6 = (r.standard_normal((T, 6, H)) * 0.3).astype(np.float32)
    w_qkv = np.zeros((3 * H, H), np.float32)
    w_qkv[2 * H:] = np.eye(H, dtype=np.float32)
    b_qkv = np.zeros(3 * H, np.float32)
    g = np.ones(H // heads, np.float32)
    cos, sin, _ = tables(np.arange(T) * 1.0, H // heads)
    mask = np.ones(T, np.uint8)
    mask[[5, 11]] = 0
    w_o = oracle.bf16_round(r.standard_normal((H, H)) * 0.1).astype(np.float32)
    b_o = (r.standard_normal(H) * 0.1).astype(np.float32)
    out = oracle.attn_half_adaln(x, temb6, table, 1e-6, w_qkv, b_qkv, g, g, 1e-6, cos, sin, heads,
                                 S, mask, w_o, b_o)
    # h from its own closed form: rmsnorm(x) (1 + scale row 1) + shift row 0, bf16
    xd = x.astype(np.float64)
    rn = xd / np.sqrt((xd * xd).mean(1, keepdims=True) + 1e-6)
    t64 = table.astype(np.float64)
    e64 = temb6.astype(np.float64)
    h = oracle.bf16_round(rn * (1 + t64[1] + e64[:, 1]) + t64[0] + e64[:, 0])
    for b in range(2):
        rows = [t for t in range(b * S, (b + 1) * S) if mask[t]]
        blk = oracle.bf16_round(oracle.bf16_round(h[rows].mean(0)) @ w_o.astype(np.float64).T + b_o)
        for t in range(b * S, (b + 1) * S):
            bt = blk if mask[t] else oracle.bf16_round(b_o.astype(np.float64))
            want = xd[t] + (t64[2] + e64[t, 2]) * bt
            assert np.allclose(out[t], want, rtol=1e-12, atol=1e-12), t
    sub = oracle.attn_half_adaln(x, temb6, table, 1e-6, w_qkv, b_qkv, g, g, 1e-6, cos, sin, heads,
                                 S, mask, w_o, b_o, qrows=[7, 2])
    assert np.array_equal(sub, out[[7, 2]])
