"""Pins of the oracle's FP8 expert weights (OCP e4m3fn codes, one power-of-two
scale per weight row).  The format facts come from the OCP 8-bit floating
point definition (e4m3fn: bias 7, 3 mantissa bits, no infinities, 448 the
largest finite value, 0x7f/0xff NaN); the pages only say FP8 experts were left
out of the first integration (vLLM-Omni recipe, Known Limitations)."""
import itertools

import numpy as np
import pytest

import oracle


def test_known_codes_and_order():
    v = oracle.e4m3_values()
    assert v[0x00] == 0.0 and v[0x80] == 0.0 and np.signbit(v[0x80])
    assert v[0x01] == 2.0 ** -9                    # smallest subnormal
    assert v[0x07] == 7 * 2.0 ** -9                # largest subnormal
    assert v[0x08] == 2.0 ** -6                    # smallest normal
    assert v[0x38] == 1.0 and v[0x39] == 1.125 and v[0x40] == 2.0
    assert v[0x7e] == 448.0 and np.isnan(v[0x7f]) and np.isnan(v[0xff])
    assert v[0xfe] == -448.0
    pos = v[:0x7f]
    assert (np.diff(pos) > 0).all()               # codes 0 .. 0x7e increase
    assert np.array_equal(v[0x80:0xff], -pos[:0x7f])
    # 3 mantissa bits: within each binade the step is 2^(E-3)
    for E in range(-6, 9):
        lo = 2.0 ** E
        grid = pos[(pos >= lo) & (pos < 2 * lo)]
        if E < 8:
            assert np.allclose(np.diff(grid), lo / 8) and len(grid) == 8


def test_rounding_to_nearest_even_and_round_trip():
    v = oracle.e4m3_values()
    fin = np.nonzero(np.isfinite(v))[0]
    vals = np.array(sorted(set(v[fin].tolist())))
    # every finite value quantizes to itself (with scale 1: a row whose max is 448)
    row = np.concatenate([[448.0], vals]).astype(np.float32)
    q, sc = oracle.quantize_fp8_rows(row[None])
    assert sc[0] == 1.0 and np.array_equal(v[q[0]], row.astype(np.float64))
    # midpoints go to the neighbour with the even code; just off a midpoint to the nearer
    mids, above, below = [], [], []
    for a, b in zip(vals[:-1], vals[1:]):
        if a < 0 or b > 448:
            continue
        m = (a + b) / 2
        mids.append(m)
        above.append(b)
        below.append(a)
    row = np.concatenate([[448.0], mids]).astype(np.float32)
    assert np.array_equal(row[1:].astype(np.float64), np.array(mids))   # midpoints are fp32 exact
    q, _ = oracle.quantize_fp8_rows(row[None])
    for i, c in enumerate(q[0, 1:]):
        assert v[c] in (below[i], above[i])        # one of the two neighbours
        assert c % 2 == 0                          # the even code wins the tie
    eps = np.float32(1 + 2 ** -20)
    row = np.concatenate([[448.0], (np.array(mids) * eps)]).astype(np.float32)
    q, _ = oracle.quantize_fp8_rows(row[None])
    assert np.array_equal(v[q[0, 1:]], np.array(above))


def test_power_of_two_scale_choice():
    """e is the smallest integer with max|w| <= 448 2^e."""
    for amax in (448.0, 449.0, 224.0, 224.5, 1.0, 0.02, 3e-5, 1e4):
        row = np.array([[amax, -amax / 3, 0.0]], np.float32)
        q, sc = oracle.quantize_fp8_rows(row)
        e = np.log2(sc[0])
        assert e == int(e)
        assert np.float32(amax) <= 448 * 2.0 ** e and not np.float32(amax) <= 448 * 2.0 ** (e - 1)
    q, sc = oracle.quantize_fp8_rows(np.zeros((2, 5), np.float32))
    assert (sc == 1.0).all() and (q == 0).all()


def test_dequantized_error_bound_and_sign():
    """|decode(q) 2^e - w| <= half a step of the value's binade (2^-4 relative
    for normals, 2^-10 2^e absolute in the subnormal range); signs kept."""
    rng = np.random.default_rng(0)
    w = (rng.standard_normal((64, 256)) * 0.02).astype(np.float32)
    w[3, :10] = 0.0
    q, sc = oracle.quantize_fp8_rows(w)
    d = oracle.dequantize_fp8_rows(q, sc).astype(np.float64)
    w64 = w.astype(np.float64)
    s = sc.astype(np.float64)[:, None]
    bound = np.maximum(np.abs(w64) * 2.0 ** -4, 2.0 ** -10 * s)
    assert (np.abs(d - w64) <= bound).all()
    assert (np.sign(d) * np.sign(w64) >= 0).all()
    assert (np.abs(d) <= 448 * s).all()
    # a smaller exponent would overflow: each row's maximum needs the top binade
    nz = np.abs(w).max(1) > 0
    assert (np.abs(d).max(1)[nz] > 224 * s[nz, 0] * (1 - 2.0 ** -4)).all()


def test_scaled_rows_match_unscaled():
    """Scaling a row by 2^k changes only its exponent: the codes are the same."""
    rng = np.random.default_rng(1)
    w = (rng.standard_normal((8, 64)) * 0.3).astype(np.float32)
    q0, s0 = oracle.quantize_fp8_rows(w)
    for k in (-30, -7, 3, 20):
        q1, s1 = oracle.quantize_fp8_rows(w * np.float32(2.0 ** k))
        assert np.array_equal(q0, q1) and np.array_equal(s1, s0 * np.float32(2.0 ** k))


def test_brute_force_nearest():
    """Against a brute-force search over all finite codes on random inputs."""
    v = oracle.e4m3_values()
    fin = np.isfinite(v)
    codes = np.nonzero(fin)[0]
    vals = v[codes]
    rng = np.random.default_rng(2)
    w = np.concatenate([[448.0], rng.uniform(-448, 448, 2000),
                        rng.uniform(-0.05, 0.05, 500)]).astype(np.float32)
    q, sc = oracle.quantize_fp8_rows(w[None])
    assert sc[0] == 1.0
    for x, c in zip(w.astype(np.float64), q[0]):
        d = np.abs(vals - x)
        best = d.min()
        cand = codes[d == best]
        if len(cand) == 1:
            assert c == cand[0]
        else:  # tie between two neighbours: the even code (for equal values, +0 over -0)
            assert v[c] in vals[d == best] and (c % 2 == 0 or best == abs(x))
