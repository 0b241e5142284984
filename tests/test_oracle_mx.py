"""Pins of the oracle's fp8 activations (MX blocks of 32 values along a row,
one e8m0 power-of-two scale per block, OCP e4m3fn codes) and of the block
with fp8 weights and fp8 activations built on them.  The format facts come
from the OCP Microscaling definition (a block of 32 elements shares one
8-bit exponent scale, byte value b meaning 2^(b - 127)) and the OCP 8-bit
floating point definition (e4m3fn, 448 the largest finite value); the pages
only say FP8 expert backends were left out of the first integration
(vLLM-Omni recipe, Known Limitations)."""
import numpy as np
import pytest

import oracle
import synth

V = oracle.e4m3_values()
FIN = np.array(sorted(set(V[np.isfinite(V)].tolist())))        # the 253 finite values


def nearest_even(t):
    """Brute force over every finite code: the code whose value is nearest t,
    the even one of two at the same distance."""
    codes = np.nonzero(np.isfinite(V))[0]
    d = np.abs(V[codes] - t)
    best = codes[d == d.min()]
    if len(best) > 1:
        vals = V[best]
        best = best[vals == vals[np.argmin(np.abs(vals - t))]] if len(set(vals)) > 1 else best
        even = [c for c in best if c % 2 == 0 and (V[c] != 0 or np.signbit(V[c]) == np.signbit(t))]
        best = even if even else best
    return V[best[0]]


def test_codes_are_nearest_by_brute_force():
    """Every element: decode(q) 2^e is the nearest value of the e4m3fn grid
    scaled by 2^e (ties to the even code), over blocks of many magnitudes."""
    rng = np.random.default_rng(1)
    v = rng.standard_normal((6, 96)) * np.array([1e-3, 0.02, 1.0, 37.0, 3e3, 1e-20])[:, None]
    v[2, 5] = 0.0
    q, e8 = oracle.quantize_mx_rows(v)
    for r in range(v.shape[0]):
        for c in range(v.shape[1]):
            s = 2.0 ** (int(e8[r, c // 32]) - 127)
            assert V[q[r, c]] == nearest_even(v[r, c] / s), (r, c)


def test_block_exponent_is_minimal_and_blocks_are_independent():
    rng = np.random.default_rng(2)
    v = rng.standard_normal((4, 128)) * 10.0 ** rng.uniform(-6, 6, (4, 4)).repeat(32, axis=1)
    q, e8 = oracle.quantize_mx_rows(v)
    for r in range(4):
        for b in range(4):
            amax = np.abs(v[r, 32 * b:32 * b + 32]).max()
            e = int(e8[r, b]) - 127
            assert amax <= 448 * 2.0 ** e and not amax <= 448 * 2.0 ** (e - 1)
    # scaling block 1 of row 0 by 2^10 moves its scale byte by 10 and leaves
    # every code, and every other block's scale, as it was
    w = v.copy()
    w[0, 32:64] *= 1024.0
    q2, e82 = oracle.quantize_mx_rows(w)
    assert np.array_equal(q2, q)
    kb = np.ones((4, 4), bool)
    kb[0, 1] = False
    assert np.array_equal(e82[kb], e8[kb]) and e82[0, 1] == e8[0, 1] + 10


def test_one_block_row_matches_the_weight_row_quantizer():
    """A row of 32 values is one block: the same codes as the (separately
    pinned) fp8 weight-row quantizer and the same power-of-two scale."""
    rng = np.random.default_rng(3)
    w = synth.round_to_bf16((rng.standard_normal((50, 32)) * 10.0 ** rng.uniform(-4, 4, (50, 1)))
                            .astype(np.float32))
    qr, sc = oracle.quantize_fp8_rows(w)
    qm, e8 = oracle.quantize_mx_rows(w.astype(np.float64))
    assert np.array_equal(qm, qr)
    assert np.array_equal(2.0 ** (e8[:, 0].astype(np.float64) - 127), sc.astype(np.float64))


def test_zero_block_and_the_scale_byte_range():
    """An all-zero block has scale byte 127 (2^0) and zero codes; a block
    whose largest magnitude is below 448 2^-127 keeps e = -127 (byte 0), its
    values then quantized on the grid scaled by 2^-127."""
    v = np.zeros((1, 64))
    v[0, 32:] = np.linspace(-1, 1, 32) * 2.0 ** -135
    q, e8 = oracle.quantize_mx_rows(v)
    assert e8[0, 0] == 127 and (q[0, :32] == 0).all()
    assert e8[0, 1] == 0
    for c in range(32, 64):
        assert V[q[0, c]] == nearest_even(v[0, c] * 2.0 ** 127)
    d = oracle.dequantize_mx_rows(q, e8)
    assert (d[0, :32] == 0).all()
    assert np.array_equal(d[0, 32:], V[q[0, 32:]] * 2.0 ** -127)


def test_values_on_the_grid_survive_a_round_trip():
    """decode(c) 2^e with a block holding +-448 2^e quantizes back to c and e."""
    rng = np.random.default_rng(4)
    codes = rng.choice(np.nonzero(np.isfinite(V))[0], (8, 64)).astype(np.uint8)
    codes[:, 0] = 0x7e
    codes[:, 32] = 0xfe
    e = rng.integers(-20, 20, (8, 2))
    v = V[codes] * (2.0 ** e).repeat(32, axis=1)
    q, e8 = oracle.quantize_mx_rows(v)
    # -0 and +0 decode alike: compare values, then codes away from zero
    assert np.array_equal(V[q], V[codes])
    nz = V[codes] != 0
    assert np.array_equal(q[nz], codes[nz])
    assert np.array_equal(e8.astype(int) - 127, e)
    assert np.array_equal(oracle.dequantize_mx_rows(q, e8), v)


def test_act_is_rounded_to_bf16_before_the_blocks():
    """act_to_mx rounds to bf16 first: a value just above an e4m3 midpoint
    whose bf16 rounding lands on the midpoint takes the even neighbour, not
    the upper one that the unrounded value is nearer to."""
    base = np.zeros((1, 32))
    base[0, 0] = 448.0                                   # scale 2^0
    mid = (V[0x39] + V[0x3a]) / 2                        # between 1.125 (odd) and 1.25 (even)
    base[0, 1] = mid * (1 + 2.0 ** -12)                  # within half a bf16 ulp of mid
    q, e8, d = oracle.act_to_mx(base)
    assert e8[0, 0] == 127 and q[0, 1] == 0x3a           # bf16(v) = mid -> even code 0x3a
    q2, _ = oracle.quantize_mx_rows(base)
    assert q2[0, 1] == 0x3a                              # nearest of v itself is 0x3a too
    base[0, 1] = (V[0x38] + V[0x39]) / 2 * (1 + 2.0 ** -12)   # between 1.0 (even) and 1.125 (odd)
    q, _, _ = oracle.act_to_mx(base)
    q2, _ = oracle.quantize_mx_rows(base)
    assert q[0, 1] == 0x38 and q2[0, 1] == 0x39          # bf16 first: tie to even; direct: up


def _tiny():
    wl = synth.Workload("w8a8_tiny", T=23, hidden=64, num_experts=8, n_group=2, topk_group=1,
                        top_k=2, intermediate=64, n_shared=1, dtype="bf16", seed=5, wr_std=0.125,
                        b_std=0.1, samples=((12, 9), (11, 11)))
    inp = synth.make_inputs(wl)
    dq = {k: (None if inp[k] is None else oracle.dequantize_fp8_rows(*oracle.quantize_fp8_rows(inp[k])))
          for k in ("w13", "w2", "shared_w13", "shared_w2")}
    return wl, inp, dq


def test_w8a8_block_is_near_the_fp64_block_on_the_quantized_inputs():
    """Against the same routing evaluated in fp64 on the dequantized x and
    weights (act_rows, then down_combine with act kept in fp32), the only
    further change is act's bf16 and MX roundings: each act value moves by at
    most 2^-9 |a| (bf16) plus half an e4m3 step of its block (2^(E-4) for a
    value in [2^E, 2^(E+1)), 2^(e-10) in the subnormal range), the reference
    act by 2^-24 |a| (fp32), so output n moves by at most the sum over slots
    of |w| sum_i |W2[n, i]| times that.  The change is not zero."""
    wl, inp, dq = _tiny()
    r = oracle.route(wl, inp["x"], inp["router_w"], inp["e_bias"], inp["mask"])
    ids, w = r["ids"], r["w"]
    out8 = oracle.w8a8_experts(wl, inp["x"], ids, w, dq["w13"], dq["w2"], dq["shared_w13"],
                               dq["shared_w2"])
    xd = oracle.dequantize_fp8_rows(*oracle.quantize_fp8_rows(inp["x"]))
    K, E, I, KS = wl.top_k, wl.num_experts, wl.intermediate, wl.top_k + wl.n_shared
    act = np.zeros((wl.T, KS, I))
    bound = np.zeros((wl.T, wl.hidden))
    for t in range(wl.T):
        for k in range(KS):
            e = ids[t, k] if k < K else E + (k - K)
            if e < 0:
                continue
            a = oracle.act_rows(wl, xd[t:t + 1], dq["w13"], dq["shared_w13"], np.array([0]),
                                np.array([e]))[0]
            act[t, k] = a
            up = np.abs(a) * (1 + 2.0 ** -8)               # at least |bf16(a)|
            eb = np.ceil(np.log2(np.maximum(np.abs(up.reshape(-1, 32)).max(axis=1), 1e-300) / 448))
            eb = eb.repeat(32)
            step = np.where(up < 2.0 ** (eb - 6), 2.0 ** (eb - 10),
                            2.0 ** (np.floor(np.log2(np.maximum(up, 1e-300))) - 4))
            da = (2.0 ** -9 + 2.0 ** -24) * np.abs(a) + step
            W2 = dq["w2"][e] if e < E else dq["shared_w2"]
            bound[t] += (abs(w[t, k]) if k < K else 1.0) * (np.abs(W2) @ da)
    ref = oracle.down_combine(wl, act.astype(np.float32), ids, w, dq["w2"], dq["shared_w2"])
    diff = np.abs(out8 - ref)
    assert (diff <= bound * (1 + 1e-9) + 1e-12).all()
    # e4m3 keeps 3 mantissa bits (relative steps up to 2^-3), bf16 keeps 7: the
    # MX rounding dominates, a few percent of the output (2.6% here), far
    # above what the bf16 rounding alone gives (0.16% here)
    rel = np.linalg.norm(out8 - ref) / np.linalg.norm(ref)
    assert 1e-2 < rel < 0.1, rel


def test_w8a8_experts_take_x_through_its_fp8_rows():
    """The x rows are quantized like weight rows, so x and its own dequantized
    fp8 rows give the same expert output bit for bit; x one bf16 step off on
    one token changes that token only."""
    wl, inp, dq = _tiny()
    r = oracle.route(wl, inp["x"], inp["router_w"], inp["e_bias"], inp["mask"])
    args = (r["ids"], r["w"], dq["w13"], dq["w2"], dq["shared_w13"], dq["shared_w2"])
    a = oracle.w8a8_experts(wl, inp["x"], *args)
    xd = oracle.dequantize_fp8_rows(*oracle.quantize_fp8_rows(inp["x"]))
    assert not np.array_equal(xd, inp["x"])
    assert np.array_equal(oracle.w8a8_experts(wl, xd, *args), a)
    x2 = inp["x"].copy()
    x2[4] = synth.round_to_bf16(x2[4] * np.float32(1.37))
    b = oracle.w8a8_experts(wl, x2, *args)
    others = np.arange(wl.T) != 4
    assert np.array_equal(b[others], a[others]) and not np.array_equal(b[4], a[4])


def test_w8a8_padding_token_is_its_shared_expert():
    """A padding token has no routed slots: its output is the shared expert's
    fp8 path alone, the same as with every routed weight set to zero."""
    wl, inp, dq = _tiny()
    res = oracle.moe_forward_w8a8(wl, inp["x"], inp["router_w"], inp["e_bias"], dq["w13"],
                                  dq["w2"], dq["shared_w13"], dq["shared_w2"], inp["mask"])
    pad = np.nonzero(inp["mask"] == 0)[0]
    assert len(pad) == 3 and (res["ids"][pad] == -1).all()
    zero_w = np.zeros_like(res["w"])
    alone = oracle.w8a8_experts(wl, inp["x"], res["ids"], zero_w, dq["w13"], dq["w2"],
                                dq["shared_w13"], dq["shared_w2"])
    assert np.array_equal(res["out"][pad], alone[pad])
    assert not np.array_equal(res["out"][~np.isin(np.arange(wl.T), pad)],
                              alone[~np.isin(np.arange(wl.T), pad)])
