"""The seeded generator: determinism, bf16 exactness, distributions, padding."""
import numpy as np

import synth


def test_deterministic_and_bf16_exact():
    wl = synth.WORKLOADS[1].replace(T=64, num_experts=8)
    a, b = synth.make_inputs(wl), synth.make_inputs(wl)
    assert synth.digest(a) == synth.digest(b)
    for k in ("x", "w13", "w2", "shared_w13", "shared_w2"):
        bits = synth.bf16_bits(a[k])                       # raises unless bf16-exact
        assert np.array_equal(synth.bits_to_f32(bits), a[k])
    assert a["router_w"].dtype == np.float32
    assert abs(a["w13"].std() - 0.02) < 1e-3
    assert abs(a["router_w"].std() - 2048 ** -0.5) < 2e-3


def test_round_to_bf16_ties_even():
    v = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 1.0 + 2 ** -9], np.float32)
    synth.round_to_bf16(v)
    assert v.tolist() == [1.0, 1.0 + 2 ** -6, -1.0, 1.0]


def test_padding_mask_and_hot_experts():
    wl = synth.WORKLOADS[2]
    m = synth.token_mask(wl)
    assert m.sum() == 1560 and (m[1560:] == 0).all() and (m[:1560] == 1).all()
    hw = synth.WORKLOADS[4].replace(T=16, intermediate=8)
    inp = synth.make_inputs(hw)
    assert (inp["x"][:, 0] == 1.0).all()
    col = inp["router_w"][:, 0]
    assert set(np.nonzero(col)[0].tolist()) == set(hw.hot) and (col[list(hw.hot)] == 2.0).all()
