"""Helpers for the GPU parity tests: upload seeded inputs, compare with the oracle."""
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


def compare_routing(g_ids, g_w, o, tau=TAU):
    """Ids must be equal as sets on every token whose decision margins exceed
    tau; weights aligned by id within 1e-5 relative.  Returns (same-set mask,
    near-tie mask)."""
    g_ids = np.asarray(g_ids)
    g_w = np.asarray(g_w, np.float64)
    near = np.minimum(o["m_grp"], o["m_sel"]) <= tau
    og = np.argsort(g_ids, 1, kind="stable")
    oo = np.argsort(o["ids"], 1, kind="stable")
    gi = np.take_along_axis(g_ids, og, 1)
    oi = np.take_along_axis(o["ids"], oo, 1)
    same = (gi == oi).all(1)
    bad = ~same & ~near
    assert not bad.any(), "expert sets differ on tie-free tokens %s" % np.nonzero(bad)[0][:10]
    gw = np.take_along_axis(g_w, og, 1)[same]
    ow = np.take_along_axis(o["w"].astype(np.float64), oo, 1)[same]
    err = np.abs(gw - ow) / np.maximum(np.abs(ow), 1e-30)
    err[ow == 0] = np.abs(gw[ow == 0])
    assert err.size == 0 or err.max() <= 1e-5, err.max()
    return same, near
