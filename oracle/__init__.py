"""CPU oracle for the routed-MoE block: ctypes binding of ``lbv_oracle.c``.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this package.  It shares no code
with the HIP library (``routed_moe_dit_amd``) and never imports it.

What it computes is stated, with the page citations, in ``lbv_oracle.c``.
Every function here is argument marshalling around that C code.

Pins (tests/test_oracle_*.py, CPU only): brute-force enumeration of
group-limited top-k on tiny inputs, the plain top-k special case
(n_group = topk_group = 1), the bias-selects-only invariants, the
no-double-scaling closed form, the expert MLP against closed-form unit-vector
constructions and float64 library matmuls, padding and per-sample isolation.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "lbv_oracle.c")
_LIB = os.path.join(_HERE, "liblbv_oracle.so")


class OrcCfg(ctypes.Structure):
    _fields_ = [
        ("hidden", ctypes.c_int32),
        ("num_experts", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("n_group", ctypes.c_int32),
        ("topk_group", ctypes.c_int32),
        ("intermediate", ctypes.c_int32),
        ("n_shared", ctypes.c_int32),
        ("norm_topk_prob", ctypes.c_int32),
        ("routed_scaling_factor", ctypes.c_float),
    ]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain C, OpenMP over tokens)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-std=c11",
               "-Wall", "-shared", "-fPIC", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        L.orc_route.argtypes = [P, ctypes.c_int64, P, P, P, P, P, P, P, P, P, P]
        L.orc_route.restype = ctypes.c_int
        L.orc_moe_forward.argtypes = [P, ctypes.c_int64, P, P, P, P, P, P, P, P, P, P, P, P, P]
        L.orc_moe_forward.restype = ctypes.c_int
        L.orc_expert_act.argtypes = [P, P, P, ctypes.c_int, P]
        L.orc_expert_act.restype = None
        L.orc_shared_act.argtypes = [P, P, P, P]
        L.orc_shared_act.restype = None
        L.orc_expert_out.argtypes = [P, P, P, P, ctypes.c_int, P]
        L.orc_expert_out.restype = None
        L.orc_moe_forward_ids.argtypes = [P, ctypes.c_int64, P, P, P, P, P, P, P, P, P]
        L.orc_moe_forward_ids.restype = ctypes.c_int
        L.orc_act_rows.argtypes = [P, ctypes.c_int64, P, P, P, P, P, P]
        L.orc_act_rows.restype = None
        L.orc_down_combine.argtypes = [P, ctypes.c_int64, P, P, P, P, P, P]
        L.orc_down_combine.restype = None
        _lib = L
    return _lib


def cfg_of(wl) -> OrcCfg:
    """OrcCfg from anything with the synth.Workload field names."""
    return OrcCfg(wl.hidden, wl.num_experts, wl.top_k, wl.n_group, wl.topk_group,
                  wl.intermediate, wl.n_shared, int(bool(wl.norm_topk_prob)),
                  float(wl.routed_scaling_factor))


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _f32(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float32)


def route(wl, x, router_w, e_bias, mask=None, want_scores=False):
    """Router for every row of x.  Returns dict(ids, w, m_grp, m_sel[, z, s])."""
    x, router_w, e_bias = _f32(x), _f32(router_w), _f32(e_bias)
    n, K, E = x.shape[0], wl.top_k, wl.num_experts
    assert x.shape[1] == wl.hidden and router_w.shape == (E, wl.hidden)
    m = None if mask is None else np.ascontiguousarray(mask, dtype=np.uint8)
    ids = np.empty((n, K), np.int32)
    w = np.empty((n, K), np.float32)
    mg = np.empty(n, np.float64)
    ms = np.empty(n, np.float64)
    z = np.empty((n, E), np.float32) if want_scores else None
    s = np.empty((n, E), np.float32) if want_scores else None
    c = cfg_of(wl)
    rc = lib().orc_route(ctypes.byref(c), n, _p(x), _p(router_w), _p(e_bias), _p(m), _p(ids),
                         _p(w), _p(mg), _p(ms), _p(z), _p(s))
    if rc != 0:
        raise ValueError("oracle: invalid routing configuration")
    out = dict(ids=ids, w=w, m_grp=mg, m_sel=ms)
    if want_scores:
        out.update(z=z, s=s)
    return out


def moe_forward(wl, x, router_w, e_bias, w13, w2, shared_w13=None, shared_w2=None, mask=None):
    """Whole block for every row of x.  Returns dict(out fp64, ids, w, m_grp, m_sel)."""
    x, router_w, e_bias = _f32(x), _f32(router_w), _f32(e_bias)
    w13, w2 = _f32(w13), _f32(w2)
    shared_w13, shared_w2 = _f32(shared_w13), _f32(shared_w2)
    n, K, H = x.shape[0], wl.top_k, wl.hidden
    E, I = wl.num_experts, wl.intermediate
    assert w13.shape == (E, 2 * I, H) and w2.shape == (E, H, I)
    if wl.n_shared > 0:
        Is = I * wl.n_shared
        assert shared_w13.shape == (2 * Is, H) and shared_w2.shape == (H, Is)
    m = None if mask is None else np.ascontiguousarray(mask, dtype=np.uint8)
    out = np.empty((n, H), np.float64)
    ids = np.empty((n, K), np.int32)
    w = np.empty((n, K), np.float32)
    mg = np.empty(n, np.float64)
    ms = np.empty(n, np.float64)
    c = cfg_of(wl)
    rc = lib().orc_moe_forward(ctypes.byref(c), n, _p(x), _p(m), _p(router_w), _p(e_bias),
                               _p(w13), _p(w2), _p(shared_w13), _p(shared_w2), _p(out),
                               _p(ids), _p(w), _p(mg), _p(ms))
    if rc != 0:
        raise ValueError("oracle: invalid routing configuration")
    return dict(out=out, ids=ids, w=w, m_grp=mg, m_sel=ms)


def moe_forward_ids(wl, x, router_w, ids, w13, w2, shared_w13=None, shared_w2=None):
    """Block output for a given expert choice ids [n, K] (entries outside [0, E)
    are empty slots): the oracle's own scores, weights at the given ids.
    Returns dict(out fp64 [n, H], w fp32 [n, K])."""
    x, router_w = _f32(x), _f32(router_w)
    w13, w2 = _f32(w13), _f32(w2)
    shared_w13, shared_w2 = _f32(shared_w13), _f32(shared_w2)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    n, K, H = x.shape[0], wl.top_k, wl.hidden
    assert ids.shape == (n, K)
    assert w13.shape == (wl.num_experts, 2 * wl.intermediate, H)
    out = np.empty((n, H), np.float64)
    w = np.empty((n, K), np.float32)
    c = cfg_of(wl)
    rc = lib().orc_moe_forward_ids(ctypes.byref(c), n, _p(x), _p(router_w), _p(ids), _p(w13),
                                   _p(w2), _p(shared_w13), _p(shared_w2), _p(out), _p(w))
    if rc != 0:
        raise ValueError("oracle: invalid configuration")
    return dict(out=out, w=w)


def act_rows(wl, x, w13, shared_w13, tok, seg):
    """fp64 act [n, I] for (token, segment) pairs; segment E + j is the j-th
    width-I slice of the shared MLP."""
    x, w13, shared_w13 = _f32(x), _f32(w13), _f32(shared_w13)
    tok = np.ascontiguousarray(tok, dtype=np.int32)
    seg = np.ascontiguousarray(seg, dtype=np.int32)
    assert tok.shape == seg.shape and tok.ndim == 1
    assert tok.size == 0 or (tok.min() >= 0 and tok.max() < x.shape[0])
    assert seg.size == 0 or (seg.min() >= 0 and seg.max() < wl.num_experts + wl.n_shared)
    act = np.empty((tok.size, wl.intermediate), np.float64)
    c = cfg_of(wl)
    lib().orc_act_rows(ctypes.byref(c), tok.size, _p(x), _p(w13), _p(shared_w13), _p(tok),
                       _p(seg), _p(act))
    return act


def down_combine(wl, act_slots, ids, w, w2, shared_w2=None):
    """out [n, H] fp64 from given act vectors per slot: act_slots [n, K+ns, I]."""
    act_slots, w2, shared_w2 = _f32(act_slots), _f32(w2), _f32(shared_w2)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    w = _f32(w)
    n, K, KS = ids.shape[0], wl.top_k, wl.top_k + wl.n_shared
    assert act_slots.shape == (n, KS, wl.intermediate) and w.shape == (n, K)
    out = np.empty((n, wl.hidden), np.float64)
    c = cfg_of(wl)
    lib().orc_down_combine(ctypes.byref(c), n, _p(act_slots), _p(ids), _p(w), _p(w2),
                           _p(shared_w2), _p(out))
    return out


def adaln_rmsnorm(x, temb6, table, eps=1e-6, round_bf16=True, per_token=True, rows=(3, 4)):
    """h = rmsnorm(x) * (1 + scale) + shift, shift and scale the rows
    rows = (shift, scale) of table + temb6 ((3, 4) in front of the FFN block,
    (0, 1) in front of the attention block), fp64, rounded to bf16 when
    round_bf16.  x [n, H] fp32; temb6 [n, 6, H] (per_token) or [6, H];
    table [6, H].  Returns fp32 [n, H]."""
    x, temb6, table = _f32(x), _f32(temb6), _f32(table)
    n, H = x.shape
    assert table.shape == (6, H)
    assert temb6.shape == ((n, 6, H) if per_token else (6, H))
    h = np.empty((n, H), np.float32)
    L = lib()
    L.orc_adaln_rmsnorm_rows.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_void_p,
                                         ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                         ctypes.c_double, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_void_p]
    L.orc_adaln_rmsnorm_rows.restype = None
    L.orc_adaln_rmsnorm_rows(H, n, _p(x), _p(temb6), 6 * H if per_token else 0, _p(table),
                             float(eps), int(bool(round_bf16)), int(rows[0]), int(rows[1]), _p(h))
    return h


def bf16_round(values):
    """Nearest bf16 value (ties to even) of each float64 value."""
    v = np.ascontiguousarray(values, dtype=np.float64)
    out = np.empty_like(v)
    L = lib()
    L.orc_bf16_round.argtypes = [ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    L.orc_bf16_round.restype = None
    L.orc_bf16_round(v.size, _p(v), _p(out))
    return out


def ffn_adaln(wl, x, temb6, table, router_w, e_bias, w13, w2, shared_w13=None, shared_w2=None,
              mask=None, eps=1e-6, per_token=True):
    """The FFN half of a DiT layer around the block:
    out = x + gate * block(h), h = bf16(rmsnorm(x) (1 + scale) + shift),
    gate = row 5 of table + temb6, all in fp64 from the fp32 inputs.
    Returns dict(out fp64 [n, H], h fp32, block (the forward dict on h))."""
    h = adaln_rmsnorm(x, temb6, table, eps, round_bf16=wl.dtype == "bf16", per_token=per_token)
    blk = moe_forward(wl, h, router_w, e_bias, w13, w2, shared_w13, shared_w2, mask)
    t6 = np.asarray(temb6, np.float64)
    gate = np.asarray(table, np.float64)[5][None, :] + (t6[:, 5, :] if per_token else t6[5][None, :])
    out = np.asarray(x, np.float64) + gate * blk["out"]
    return dict(out=out, h=h, block=blk)


def quantize_fp8_rows(w):
    """FP8 weight rows: (codes uint8 [..., cols], power-of-two scales fp32 [...])
    of an fp32 array whose last axis is a row."""
    w = _f32(w)
    rows, cols = int(np.prod(w.shape[:-1])), w.shape[-1]
    q = np.empty(w.shape, np.uint8)
    sc = np.empty(w.shape[:-1], np.float32)
    L = lib()
    L.orc_quantize_fp8_rows.argtypes = [ctypes.c_int64, ctypes.c_int64] + [ctypes.c_void_p] * 3
    L.orc_quantize_fp8_rows.restype = None
    L.orc_quantize_fp8_rows(rows, cols, _p(w), _p(q), _p(sc))
    return q, sc


def dequantize_fp8_rows(q, scale):
    """decode(q) * scale, fp32 (exact)."""
    q = np.ascontiguousarray(q, np.uint8)
    scale = _f32(scale)
    rows, cols = int(np.prod(q.shape[:-1])), q.shape[-1]
    assert scale.shape == q.shape[:-1]
    w = np.empty(q.shape, np.float32)
    L = lib()
    L.orc_dequantize_fp8_rows.argtypes = [ctypes.c_int64, ctypes.c_int64] + [ctypes.c_void_p] * 3
    L.orc_dequantize_fp8_rows.restype = None
    L.orc_dequantize_fp8_rows(rows, cols, _p(q), _p(scale), _p(w))
    return w


def e4m3_values():
    """The value of each of the 256 e4m3fn codes (NaN for 0x7f and 0xff)."""
    out = np.empty(256, np.float64)
    L = lib()
    L.orc_e4m3_decode_all.argtypes = [ctypes.c_void_p]
    L.orc_e4m3_decode_all.restype = None
    L.orc_e4m3_decode_all(_p(out))
    return out


def quantize_mx_rows(v):
    """MX blocks of 32 along the last axis of fp64 values v [..., cols]:
    (codes uint8 [..., cols], e8m0 bytes uint8 [..., cols // 32])."""
    v = np.ascontiguousarray(v, np.float64)
    rows, cols = int(np.prod(v.shape[:-1])), v.shape[-1]
    assert cols % 32 == 0
    q = np.empty(v.shape, np.uint8)
    e8 = np.empty(v.shape[:-1] + (cols // 32,), np.uint8)
    L = lib()
    L.orc_quantize_mx_rows.argtypes = [ctypes.c_int64, ctypes.c_int64] + [ctypes.c_void_p] * 3
    L.orc_quantize_mx_rows.restype = None
    L.orc_quantize_mx_rows(rows, cols, _p(v), _p(q), _p(e8))
    return q, e8


def dequantize_mx_rows(q, e8):
    """decode(q) * 2^(e8 - 127) per block of 32, fp64."""
    q = np.ascontiguousarray(q, np.uint8)
    e8 = np.ascontiguousarray(e8, np.uint8)
    rows, cols = int(np.prod(q.shape[:-1])), q.shape[-1]
    assert e8.shape == q.shape[:-1] + (cols // 32,)
    v = np.empty(q.shape, np.float64)
    L = lib()
    L.orc_dequantize_mx_rows.argtypes = [ctypes.c_int64, ctypes.c_int64] + [ctypes.c_void_p] * 3
    L.orc_dequantize_mx_rows.restype = None
    L.orc_dequantize_mx_rows(rows, cols, _p(q), _p(e8), _p(v))
    return v


def act_to_mx(act):
    """The fp8 activations of fp64 act values [..., I]: each value rounded to
    bf16 (the act storage type of the block), then MX blocks of 32.  Returns
    (codes, e8m0 bytes, dequantized values fp64)."""
    q, e8 = quantize_mx_rows(bf16_round(act))
    return q, e8, dequantize_mx_rows(q, e8)


def w8a8_experts(wl, x, ids, w, w13, w2, shared_w13=None, shared_w2=None):
    """Expert part of the block with fp8 weights and fp8 activations, for a
    given routing (ids, w [n, K]; ids outside [0, E) are empty slots): the x
    rows are quantized like weight rows (quantize_fp8_rows) and dequantized,
    each slot's act (act_rows, fp64) goes through act_to_mx, then the down
    projection and combine (down_combine).  w13, w2, shared_w13, shared_w2 are
    the dequantized fp8 weights (dequantize_fp8_rows).  Returns out [n, H]
    fp64."""
    x = _f32(x)
    ids = np.ascontiguousarray(ids, np.int32)
    n, K, NS, E = x.shape[0], wl.top_k, wl.n_shared, wl.num_experts
    KS = K + NS
    xd = dequantize_fp8_rows(*quantize_fp8_rows(x))
    slot_tok = np.repeat(np.arange(n, dtype=np.int32), KS).reshape(n, KS)
    slot_seg = np.concatenate([ids, np.broadcast_to(E + np.arange(NS, dtype=np.int32), (n, NS))],
                              axis=1)
    valid = (slot_seg >= 0) & (slot_seg < E + NS)
    act = act_rows(wl, xd, w13, shared_w13, slot_tok[valid], slot_seg[valid])
    act_slots = np.zeros((n, KS, wl.intermediate), np.float32)
    act_slots[valid] = act_to_mx(act)[2]
    return down_combine(wl, act_slots, ids, w, w2, shared_w2)


def moe_forward_w8a8(wl, x, router_w, e_bias, w13, w2, shared_w13=None, shared_w2=None,
                     mask=None):
    """Whole block with fp8 weights (given dequantized) and fp8 activations:
    the router on x as in moe_forward, then w8a8_experts.  Returns dict(out
    fp64, ids, w, m_grp, m_sel)."""
    r = route(wl, x, router_w, e_bias, mask)
    r["out"] = w8a8_experts(wl, x, r["ids"], r["w"], w13, w2, shared_w13, shared_w2)
    return r


def linear(x, w, b=None):
    """x [T, C] @ w[N, C]^T (+ b[N]) in fp64 (plain loops in C)."""
    x, w, b = _f32(x), _f32(w), _f32(b)
    T, C = x.shape
    N = w.shape[0]
    assert w.shape == (N, C) and (b is None or b.shape == (N,))
    y = np.empty((T, N), np.float64)
    L = lib()
    L.orc_linear.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_int] + [ctypes.c_void_p] * 4
    L.orc_linear.restype = None
    L.orc_linear(T, N, C, _p(x), _p(w), _p(b), _p(y))
    return y


def head_rmsnorm(u, g, eps):
    """u / sqrt(mean(u^2) + eps) * g over the last axis (length D), fp64."""
    u = np.ascontiguousarray(u, np.float64)
    g = _f32(g)
    D = u.shape[-1]
    assert g.shape == (D,)
    y = np.empty_like(u)
    L = lib()
    L.orc_head_rmsnorm.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                   ctypes.c_double, ctypes.c_void_p]
    L.orc_head_rmsnorm.restype = None
    L.orc_head_rmsnorm(u.size // D, D, _p(u), _p(g), float(eps), _p(y))
    return y


def rope(u, cos, sin):
    """Rotary embedding with neox style off on u [T, heads, D]; cos, sin [T, D/2]."""
    u = np.ascontiguousarray(u, np.float64)
    cos, sin = _f32(cos), _f32(sin)
    T, heads, D = u.shape
    assert cos.shape == (T, D // 2) and sin.shape == (T, D // 2)
    y = np.empty_like(u)
    L = lib()
    L.orc_rope.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_int] + [ctypes.c_void_p] * 4
    L.orc_rope.restype = None
    L.orc_rope(T, heads, D, _p(u), _p(cos), _p(sin), _p(y))
    return y


def attention(q, k, v, S, mask=None, qrows=None):
    """Masked, per-sample softmax attention (fp64) of q, k, v [T, heads, D]
    (fp32 values); samples are consecutive runs of S tokens.  Returns
    o [len(qrows) or T, heads, D]."""
    q, k, v = _f32(q), _f32(k), _f32(v)
    T, heads, D = q.shape
    assert k.shape == q.shape and v.shape == q.shape
    m = None if mask is None else np.ascontiguousarray(mask, np.uint8)
    assert m is None or m.shape == (T,)
    rows = None if qrows is None else np.ascontiguousarray(qrows, np.int64)
    nq = T if rows is None else len(rows)
    o = np.empty((nq, heads, D), np.float64)
    L = lib()
    L.orc_attention.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_int] + \
        [ctypes.c_void_p] * 4 + [ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    L.orc_attention.restype = None
    L.orc_attention(T, int(S), heads, D, _p(q), _p(k), _p(v), _p(m), nq, _p(rows), _p(o))
    return o


def attn_qkv(x, w_qkv, b_qkv, g_q, g_k, eps, cos, sin, heads):
    """q, k, v [T, heads, D] as a bf16 model forms them: the fused projection
    rounded to bf16, the q / k head norms rounded to bf16, the rotary
    embedding rounded to bf16 (fp32 values, bf16-exact)."""
    T, H = x.shape
    D = H // heads
    qkv = bf16_round(linear(x, w_qkv, b_qkv)).reshape(T, 3, heads, D)
    qn = bf16_round(head_rmsnorm(qkv[:, 0], g_q, eps))
    kn = bf16_round(head_rmsnorm(qkv[:, 1], g_k, eps))
    q = bf16_round(rope(qn, cos, sin)).astype(np.float32)
    k = bf16_round(rope(kn, cos, sin)).astype(np.float32)
    return q, k, qkv[:, 2].astype(np.float32)


def attn_forward(x, w_qkv, b_qkv, g_q, g_k, eps, cos, sin, heads, S, mask, w_o, b_o, qrows=None):
    """The attention half's block output [len(qrows) or T, H] (fp32 values of
    bf16): projections, head norms, rotary embedding, attention, output
    projection, each rounded to bf16 like the module it stands for."""
    T, H = x.shape
    q, k, v = attn_qkv(x, w_qkv, b_qkv, g_q, g_k, eps, cos, sin, heads)
    o = bf16_round(attention(q, k, v, S, mask, qrows)).reshape(-1, H).astype(np.float32)
    return bf16_round(linear(o, w_o, b_o)).astype(np.float32)


def attn_half_adaln(x, temb6, table, eps, w_qkv, b_qkv, g_q, g_k, qk_eps, cos, sin, heads, S,
                    mask, w_o, b_o, qrows=None):
    """The attention half of a DiT layer: h = AdaLN(x) with rows 0 (shift) and
    1 (scale) of table + temb6 (bf16), the attention half on h (bf16 block
    output), then out = x + gate * block with gate = row 2, fp64.  x [T, H]
    fp32; temb6 [T, 6, H].  Returns [len(qrows) or T, H] float64."""
    T, H = x.shape
    h = adaln_rmsnorm(x, temb6, table, eps, True, True, rows=(0, 1))
    blk = attn_forward(h, w_qkv, b_qkv, g_q, g_k, qk_eps, cos, sin, heads, S, mask, w_o, b_o,
                       qrows=qrows).astype(np.float64)
    rows = np.arange(T) if qrows is None else np.asarray(qrows)
    gate = table[2].astype(np.float64)[None, :] + np.asarray(temb6, np.float64)[rows, 2]
    return x[rows].astype(np.float64) + gate * blk


def expert_act(wl, x_row, w13, e):
    """fp64 act [I] of routed expert e for one token."""
    x_row, w13 = _f32(x_row), _f32(w13)
    act = np.empty(wl.intermediate, np.float64)
    c = cfg_of(wl)
    lib().orc_expert_act(ctypes.byref(c), _p(x_row), _p(w13), int(e), _p(act))
    return act


def shared_act(wl, x_row, shared_w13):
    """fp64 act [I * n_shared] of the shared expert for one token."""
    x_row, shared_w13 = _f32(x_row), _f32(shared_w13)
    act = np.empty(wl.intermediate * wl.n_shared, np.float64)
    c = cfg_of(wl)
    lib().orc_shared_act(ctypes.byref(c), _p(x_row), _p(shared_w13), _p(act))
    return act


def expert_out(wl, x_row, w13, w2, e):
    """fp64 unweighted output [H] of routed expert e for one token."""
    x_row, w13, w2 = _f32(x_row), _f32(w13), _f32(w2)
    y = np.empty(wl.hidden, np.float64)
    c = cfg_of(wl)
    lib().orc_expert_out(ctypes.byref(c), _p(x_row), _p(w13), _p(w2), int(e), _p(y))
    return y


def permute(wl, ids):
    """Stable counting sort of slots by segment.  Returns (offsets, sorted_rows, inv_rows);
    sorted_rows holds -1 past offsets[-1]."""
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    T = ids.shape[0]
    KS = wl.top_k + wl.n_shared
    S = wl.num_experts + wl.n_shared
    offsets = np.zeros(S + 1, np.int32)
    sorted_rows = np.full(T * KS, -1, np.int32)
    inv_rows = np.empty(T * KS, np.int32)
    c = cfg_of(wl)
    L = lib()
    L.orc_permute.argtypes = [ctypes.c_void_p, ctypes.c_int64] + [ctypes.c_void_p] * 4
    L.orc_permute.restype = None
    L.orc_permute(ctypes.byref(c), T, _p(ids), _p(offsets), _p(sorted_rows), _p(inv_rows))
    return offsets, sorted_rows, inv_rows
