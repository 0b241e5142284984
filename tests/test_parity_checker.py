"""CPU checks of the routing comparison the GPU parity tests use: a near-tie
token may carry another expert set only if that set is a near-equal choice
under the oracle's selection values, and weights must follow the oracle's rule
at the chosen ids."""
import numpy as np
import pytest

import gpu_util
import oracle
import synth


def wl16(**kw):
    base = dict(name="chk", T=1, hidden=64, num_experts=16, n_group=4, topk_group=2, top_k=3,
                intermediate=32, n_shared=1, dtype="f32", seed=0, wr_std=1.0, b_std=0.1)
    base.update(kw)
    return synth.Workload(**base)


C = np.array([0.9375, 0.75, 0.5, 0.25,
              0.875, 0.59375, 0.4375, 0.125,
              0.8125, 0.5625, 0.3125, 0.0625,
              0.6875, 0.5, 0.4375, 0.1875], np.float32)


def oracle_of(wl, c):
    x = np.zeros((1, wl.hidden), np.float32)
    wr = np.zeros((16, wl.hidden), np.float32)
    b = (c - np.float32(0.5)).astype(np.float32)
    return oracle.route(wl, x, wr, b, want_scores=True), b


def weights_for(wl, o, ids):
    s = o["s"][0][ids]
    tot = np.float32(0)
    for v in s:
        tot = np.float32(tot + v)
    return ((s / tot).astype(np.float32) * np.float32(2.5)).astype(np.float32)


def test_same_set_passes():
    wl = wl16()
    o, b = oracle_of(wl, C)
    ids = o["ids"].copy()
    same, near = gpu_util.compare_routing(wl, ids, o["w"], o, b)
    assert same.all() and not near.any()


def test_near_equal_expert_swap_is_accepted():
    """Experts 1 and 5 differ by 2^-20 < tau in c: either one is a valid third pick."""
    wl = wl16()
    c = C.copy()
    c[5] = np.float32(0.75 - 2.0 ** -20)
    o, b = oracle_of(wl, c)
    assert sorted(o["ids"][0].tolist()) == [0, 1, 4]
    alt = np.array([[0, 4, 5]], np.int32)
    same, near = gpu_util.compare_routing(wl, alt, weights_for(wl, o, alt[0])[None], o, b)
    assert near[0] and not same[0]


def test_far_expert_is_rejected_on_a_near_tie_token():
    wl = wl16()
    c = C.copy()
    c[5] = np.float32(0.75 - 2.0 ** -20)
    o, b = oracle_of(wl, c)
    alt = np.array([[0, 4, 6]], np.int32)          # c = 0.4375, far below the cut
    with pytest.raises(AssertionError):
        gpu_util.compare_routing(wl, alt, weights_for(wl, o, alt[0])[None], o, b)


def test_other_set_on_tie_free_token_is_rejected():
    wl = wl16()
    o, b = oracle_of(wl, C)
    alt = np.array([[0, 4, 5]], np.int32)
    with pytest.raises(AssertionError):
        gpu_util.compare_routing(wl, alt, weights_for(wl, o, alt[0])[None], o, b)


def test_near_equal_group_swap_is_accepted_and_wrong_group_rejected():
    """Groups 1 and 2 score within 2^-20: experts of group 2 may replace
    group 1's, but group 3 (far below the cut) may not."""
    wl = wl16()
    c = C.copy()
    c[9] = np.float32(0.59375 + 0.0625 - 2.0 ** -20)   # group 2: 0.8125 + 0.65625 - eps
    o, b = oracle_of(wl, c)
    assert o["m_grp"][0] <= 1e-5
    alt = np.array([[0, 8, 1]], np.int32)            # groups 0 and 2
    gpu_util.compare_routing(wl, alt, weights_for(wl, o, alt[0])[None], o, b)
    bad = np.array([[0, 12, 1]], np.int32)           # group 3
    with pytest.raises(AssertionError):
        gpu_util.compare_routing(wl, bad, weights_for(wl, o, bad[0])[None], o, b)


def test_wrong_weights_are_rejected():
    wl = wl16()
    o, b = oracle_of(wl, C)
    with pytest.raises(AssertionError):
        gpu_util.compare_routing(wl, o["ids"], o["w"] * np.float32(1.0001), o, b)
