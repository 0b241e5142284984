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
