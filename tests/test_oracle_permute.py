"""Pin of the oracle's token permutation against a library stable sort and
its invariants (vLLM-Omni LingBot-Video article, "MoE 实现的源码级要点":
token copies reordered by expert, then restored)."""
import numpy as np
import pytest

import oracle
import synth


def wl_of(E=16, K=4, ns=1):
    return synth.Workload("p", T=0, hidden=64, num_experts=E, n_group=4, topk_group=2, top_k=K,
                          intermediate=64, n_shared=ns, dtype="f32", seed=0, wr_std=1, b_std=1)


def library_permute(ids, E, ns):
    T, K = ids.shape
    KS = K + ns
    seg = np.full((T, KS), -1, np.int64)
    for t in range(T):
        seen = set()
        for k in range(K):
            e = int(ids[t, k])
            if 0 <= e < E and e not in seen:
                seg[t, k] = e
            seen.add(e)
        for j in range(ns):
            seg[t, K + j] = E + j
    flat = seg.reshape(-1)
    slots = np.nonzero(flat >= 0)[0]
    order = np.argsort(flat[slots], kind="stable")        # textbook stable sort
    sorted_rows = slots[order]
    counts = np.bincount(flat[slots], minlength=E + ns)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    inv = np.full(T * KS, -1, np.int64)
    inv[sorted_rows] = np.arange(sorted_rows.size)
    return offsets, sorted_rows, inv


@pytest.mark.parametrize("E,K,ns,T", [(16, 4, 1, 100), (16, 4, 0, 37), (8, 3, 2, 64),
                                      (128, 8, 1, 300)])
def test_permute_matches_stable_sort(E, K, ns, T):
    rng = np.random.default_rng(E + K + ns + T)
    ids = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    ids[::7, 0] = -1                   # a padding-like unrouted slot
    ids[::11, K - 1] = ids[::11, 0]    # a repeated id is not routed twice
    wl = wl_of(E, K, ns)
    off, srt, inv = oracle.permute(wl, ids)
    o2, s2, i2 = library_permute(ids, E, ns)
    np.testing.assert_array_equal(off, o2)
    np.testing.assert_array_equal(srt[:off[-1]], s2)
    np.testing.assert_array_equal(inv, i2)
    # invariants: inverse maps, every routed slot exactly once, segments by expert
    R = off[-1]
    assert (np.diff(off) >= 0).all()
    np.testing.assert_array_equal(inv[srt[:R]], np.arange(R))
    KS = K + ns
    for s in range(E + ns):
        for r in range(off[s], off[s + 1]):
            t, k = divmod(int(srt[r]), KS)
            assert (ids[t, k] if k < K else E + k - K) == s
        assert (np.diff(srt[off[s]:off[s + 1]]) > 0).all()
