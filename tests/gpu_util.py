"""Helpers for the GPU parity tests: upload seeded inputs, compare with the oracle."""
import itertools
import sys

import numpy as np
import torch

import routed_moe_dit_amd as lbv
import synth

TAU = 1e-5   # decision margin below which a token counts as a near tie


def note(msg):
    print("[case] " + msg, flush=True)
    sys.stdout.flush()


def cfg_for(wl):
    return lbv.config(hidden=wl.hidden, num_experts=wl.num_experts, top_k=wl.top_k,
                      n_group=wl.n_group, topk_group=wl.topk_group,
                      intermediate=wl.intermediate, n_shared_experts=wl.n_shared,
                      norm_topk_prob=wl.norm_topk_prob,
                      routed_scaling_factor=wl.routed_scaling_factor, dtype=wl.dtype)


def dev(a, dtype):
    """float32 numpy (bf16-exact when dtype == 'bf16') -> device tensor."""
    if a is None:
        return None
    if dtype == "bf16":
        bits = synth.bf16_bits(a).view(np.int16)
        return torch.from_numpy(bits).to("cuda").view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to("cuda")


def upload(wl, inp):
    d = {k: dev(inp[k], wl.dtype) for k in ("x", "w13", "w2", "shared_w13", "shared_w2")}
    d["router_w"] = dev(inp["router_w"], "f32")
    d["e_bias"] = dev(inp["e_bias"], "f32")
    d["mask"] = None if inp["mask"] is None else torch.from_numpy(inp["mask"]).to("cuda")
    return d


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


def forward(wl, d, x=None, mask="default"):
    cfg = cfg_for(wl)
    x = d["x"] if x is None else x
    m = d["mask"] if isinstance(mask, str) else mask
    blk = lbv.MoEBlock(cfg, d["router_w"], d["e_bias"], d["w13"], d["w2"], d["shared_w13"],
                       d["shared_w2"])
    out, ids, w = blk(x, m, want_routing=True)
    torch.cuda.synchronize()
    return out, ids, w


def metrics(gpu, ref):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    d = gpu - ref
    nr = np.linalg.norm(ref)
    return dict(rel_frob=float(np.linalg.norm(d) / nr) if nr > 0 else float(np.linalg.norm(d)),
                max_abs=float(np.abs(d).max()) if d.size else 0.0,
                cosine=float((gpu * ref).sum() / (np.linalg.norm(gpu) * nr + 1e-300)),
                finite=bool(np.isfinite(gpu).all()))


def selection_values(s, e_bias):
    """c = s + bias in fp32 (the router's own add)."""
    return (np.asarray(s, np.float32) + np.asarray(e_bias, np.float32)[None, :]).astype(np.float32)


def group_scores(c, n_group):
    """Sum of the two largest selection values of each group, fp32: [n, n_group]."""
    n, E = c.shape
    top2 = -np.sort(-c.reshape(n, n_group, E // n_group), axis=2)[:, :, :2]
    return (top2[:, :, 0] + top2[:, :, 1]).astype(np.float32)


def tau_consistent(wl, ids, c_row, g_row, tau):
    """True when the expert set `ids` is a valid choice up to tau: its groups
    are among the groups whose score is within tau of the topk_group-th best,
    and for some choice Q of topk_group such groups containing them, every
    chosen expert's c is at least the best unchosen c in Q minus tau."""
    G = wl.num_experts // wl.n_group
    chosen = set(int(e) for e in ids)
    if len(chosen) != wl.top_k or min(chosen) < 0:
        return False
    gcut = np.sort(g_row)[::-1][wl.topk_group - 1]
    near_kept = [j for j in range(wl.n_group) if g_row[j] >= gcut - tau]
    need = sorted({e // G for e in chosen})
    if not set(need) <= set(near_kept) or len(need) > wl.topk_group:
        return False
    others = [j for j in near_kept if j not in need]
    lo = min(float(c_row[e]) for e in chosen)
    for extra in itertools.combinations(others, wl.topk_group - len(need)):
        Q = need + list(extra)
        rest = [float(c_row[e]) for j in Q for e in range(j * G, (j + 1) * G) if e not in chosen]
        if not rest or lo >= max(rest) - tau:
            return True
    return False


def compare_routing(wl, g_ids, g_w, o, e_bias, mask=None, tau=TAU):
    """Checks the GPU routing against the oracle's (o from oracle.route with
    want_scores=True).  Tie-free tokens (both margins above tau): the same expert
    set.  Near-tie tokens: the same set, or another set that is tau-consistent
    with the oracle's selection values.  Every valid token: weights equal to the
    oracle's rule at the GPU's ids within 1e-5 relative.  Padding tokens: ids -1
    and weights 0.  Returns (same-set mask, near-tie mask)."""
    g_ids = np.asarray(g_ids)
    g_w = np.asarray(g_w, np.float64)
    n = g_ids.shape[0]
    valid = np.ones(n, bool) if mask is None else np.asarray(mask) != 0
    assert (g_ids[~valid] == -1).all() and (g_w[~valid] == 0).all()
    near = np.minimum(o["m_grp"], o["m_sel"]) <= tau
    same = (np.sort(g_ids, 1) == np.sort(o["ids"], 1)).all(1)
    bad = ~same & ~near & valid
    assert not bad.any(), "expert sets differ on tie-free tokens %s" % np.nonzero(bad)[0][:10]
    c = selection_values(o["s"], e_bias)
    g = group_scores(c, wl.n_group)
    for t in np.nonzero(~same & valid)[0]:
        assert tau_consistent(wl, g_ids[t], c[t], g[t], tau), \
            "token %d: GPU set %s is not a near-equal choice" % (t, sorted(g_ids[t].tolist()))
    # weights: the oracle's rule applied at the GPU's ids (raw fp32 scores,
    # slot-order sum, one scaling)
    s = np.asarray(o["s"], np.float32)
    vt = np.nonzero(valid)[0]
    sk = np.take_along_axis(s[vt], g_ids[vt].astype(np.int64), 1)
    tot = np.zeros(len(vt), np.float32)
    for k in range(wl.top_k):
        tot = (tot + sk[:, k]).astype(np.float32)
    want = (sk / tot[:, None]).astype(np.float32) if wl.norm_topk_prob else sk
    want = (want * np.float32(wl.routed_scaling_factor)).astype(np.float64)
    err = np.abs(g_w[vt] - want) / np.maximum(np.abs(want), 1e-30)
    assert err.size == 0 or err.max() <= 1e-5, err.max()
    return same, near
