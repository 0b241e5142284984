"""Python binding of liblbv_moe: the routed-MoE feed-forward block of the
LingBot-Video MoE DiT as hand-written HIP kernels for MI355X (gfx950).

Argument marshalling only.  Every step of the block runs in the HIP library
behind the C ABI declared in ``include/lbv_moe.h``; torch supplies device
memory and the current stream.  The functions below have the C names and
take torch tensors (or None for optional pointers).  There is no CPU path:
if the library is missing, loading it raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch  # noqa: F401  (loads the HIP runtime that the library binds to)

__all__ = [
    "LbvError", "MoEConfig", "config", "load", "lbv_abi_version", "lbv_status_string",
    "lbv_moe_check_config", "lbv_moe_workspace_size", "lbv_moe_route_workspace_size",
    "lbv_moe_permute_workspace_size",
    "lbv_moe_w2_workspace_size", "lbv_moe_route", "lbv_moe_permute", "lbv_moe_gemm_w13_silu",
    "lbv_moe_gemm_w2_combine", "lbv_moe_forward", "EXPORTS", "LIB_PATH",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblbv_moe.so")

# status codes of lbv_moe.h
LBV_OK, LBV_ERR_NULL, LBV_ERR_SHAPE, LBV_ERR_UNSUPPORTED = 0, 1, 2, 3
LBV_ERR_ALIAS, LBV_ERR_ALIGN, LBV_ERR_WORKSPACE, LBV_ERR_HIP = 4, 5, 6, 7
LBV_F32, LBV_BF16 = 0, 1
LBV_SCORE_SIGMOID, LBV_SCORE_SOFTMAX = 0, 1

EXPORTS = (
    "lbv_abi_version", "lbv_status_string", "lbv_moe_check_config", "lbv_moe_workspace_size",
    "lbv_moe_route_workspace_size", "lbv_moe_permute_workspace_size", "lbv_moe_w2_workspace_size", "lbv_moe_route",
    "lbv_moe_permute", "lbv_moe_gemm_w13_silu", "lbv_moe_gemm_w2_combine", "lbv_moe_forward",
)


class MoEConfig(ctypes.Structure):
    """Mirror of lbv_moe_config."""

    _fields_ = [
        ("hidden", ctypes.c_int32),
        ("num_experts", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("n_group", ctypes.c_int32),
        ("topk_group", ctypes.c_int32),
        ("intermediate", ctypes.c_int32),
        ("n_shared_experts", ctypes.c_int32),
        ("norm_topk_prob", ctypes.c_int32),
        ("routed_scaling_factor", ctypes.c_float),
        ("score_func", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
    ]

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == LBV_BF16 else torch.float32


def config(hidden=2048, num_experts=128, top_k=8, n_group=4, topk_group=2, intermediate=768,
           n_shared_experts=1, norm_topk_prob=True, routed_scaling_factor=2.5, dtype="bf16",
           score_func="sigmoid") -> MoEConfig:
    """Build a config; the defaults are the LingBot-Video MoE 30B layer."""
    dt = {"bf16": LBV_BF16, "f32": LBV_F32}[dtype]
    sf = {"sigmoid": LBV_SCORE_SIGMOID, "softmax": LBV_SCORE_SOFTMAX}[score_func]
    return MoEConfig(hidden, num_experts, top_k, n_group, topk_group, intermediate,
                     n_shared_experts, int(bool(norm_topk_prob)), float(routed_scaling_factor),
                     sf, dt)


class LbvError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s: %s (status %d)" % (where, lbv_status_string(status), status))


_lib = None


def load():
    """Load liblbv_moe.so (built by ``routed_moe_dit_amd.build``); raises if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("liblbv_moe.so is not built; run `python -m routed_moe_dit_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P, I64, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
    C = ctypes.POINTER(MoEConfig)
    st = ctypes.c_int
    L.lbv_abi_version.argtypes, L.lbv_abi_version.restype = [], ctypes.c_int32
    L.lbv_status_string.argtypes, L.lbv_status_string.restype = [st], ctypes.c_char_p
    L.lbv_moe_check_config.argtypes, L.lbv_moe_check_config.restype = [C], st
    for n in ("lbv_moe_workspace_size", "lbv_moe_permute_workspace_size",
              "lbv_moe_w2_workspace_size"):
        getattr(L, n).argtypes = [C, I64, ctypes.POINTER(SZ)]
        getattr(L, n).restype = st
    L.lbv_moe_route_workspace_size.argtypes = [C, ctypes.POINTER(SZ)]
    L.lbv_moe_route_workspace_size.restype = st
    L.lbv_moe_route.argtypes = [C, I64, P, P, P, P, P, P, P, SZ, P]
    L.lbv_moe_route.restype = st
    L.lbv_moe_permute.argtypes = [C, I64, P, P, P, P, P, SZ, P]
    L.lbv_moe_permute.restype = st
    L.lbv_moe_gemm_w13_silu.argtypes = [C, I64, P, P, P, P, P, P, P]
    L.lbv_moe_gemm_w13_silu.restype = st
    L.lbv_moe_gemm_w2_combine.argtypes = [C, I64, P, P, P, P, P, P, P, P, P, SZ, P]
    L.lbv_moe_gemm_w2_combine.restype = st
    L.lbv_moe_forward.argtypes = [C, I64, P, P, P, P, P, P, P, P, P, P, P, P, SZ, P]
    L.lbv_moe_forward.restype = st
    _lib = L
    return L


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------

def _ptr(t: Optional[torch.Tensor], name: str, dtype=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor or None" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be a device tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _check(status: int, where: str):
    if status != LBV_OK:
        raise LbvError(status, where)


def lbv_abi_version() -> int:
    return load().lbv_abi_version()


def lbv_status_string(status: int) -> str:
    return load().lbv_status_string(status).decode()


def lbv_moe_check_config(cfg: MoEConfig) -> int:
    return load().lbv_moe_check_config(ctypes.byref(cfg))


def _size(fn, cfg, T):
    n = ctypes.c_size_t(0)
    _check(getattr(load(), fn)(ctypes.byref(cfg), int(T), ctypes.byref(n)), fn)
    return n.value


def lbv_moe_workspace_size(cfg: MoEConfig, T: int) -> int:
    return _size("lbv_moe_workspace_size", cfg, T)


def lbv_moe_route_workspace_size(cfg: MoEConfig) -> int:
    n = ctypes.c_size_t(0)
    _check(load().lbv_moe_route_workspace_size(ctypes.byref(cfg), ctypes.byref(n)),
           "lbv_moe_route_workspace_size")
    return n.value


def lbv_moe_permute_workspace_size(cfg: MoEConfig, T: int) -> int:
    return _size("lbv_moe_permute_workspace_size", cfg, T)


def lbv_moe_w2_workspace_size(cfg: MoEConfig, T: int) -> int:
    return _size("lbv_moe_w2_workspace_size", cfg, T)


def lbv_moe_route(cfg, x, router_w, e_bias, mask, topk_ids, topk_w, ws=None, stream=None):
    dt = cfg.torch_dtype
    _check(load().lbv_moe_route(
        ctypes.byref(cfg), x.shape[0], _ptr(x, "x", dt), _ptr(router_w, "router_w", torch.float32),
        _ptr(e_bias, "e_bias", torch.float32), _ptr(mask, "mask", torch.uint8),
        _ptr(topk_ids, "topk_ids", torch.int32), _ptr(topk_w, "topk_w", torch.float32),
        _ptr(ws, "ws"), 0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)),
        "lbv_moe_route")


def lbv_moe_permute(cfg, topk_ids, offsets, sorted_rows, inv_rows, ws, stream=None):
    _check(load().lbv_moe_permute(
        ctypes.byref(cfg), topk_ids.shape[0], _ptr(topk_ids, "topk_ids", torch.int32),
        _ptr(offsets, "offsets", torch.int32), _ptr(sorted_rows, "sorted_rows", torch.int32),
        _ptr(inv_rows, "inv_rows", torch.int32), _ptr(ws, "ws"),
        ws.numel() * ws.element_size(), _stream(stream)), "lbv_moe_permute")


def lbv_moe_gemm_w13_silu(cfg, x, w13, shared_w13, offsets, sorted_rows, act, stream=None):
    dt = cfg.torch_dtype
    _check(load().lbv_moe_gemm_w13_silu(
        ctypes.byref(cfg), x.shape[0], _ptr(x, "x", dt), _ptr(w13, "w13", dt),
        _ptr(shared_w13, "shared_w13", dt), _ptr(offsets, "offsets", torch.int32),
        _ptr(sorted_rows, "sorted_rows", torch.int32), _ptr(act, "act", dt), _stream(stream)),
        "lbv_moe_gemm_w13_silu")


def lbv_moe_gemm_w2_combine(cfg, act, w2, shared_w2, offsets, sorted_rows, inv_rows, topk_w,
                            out, ws, stream=None):
    dt = cfg.torch_dtype
    _check(load().lbv_moe_gemm_w2_combine(
        ctypes.byref(cfg), out.shape[0], _ptr(act, "act", dt), _ptr(w2, "w2", dt),
        _ptr(shared_w2, "shared_w2", dt), _ptr(offsets, "offsets", torch.int32),
        _ptr(sorted_rows, "sorted_rows", torch.int32), _ptr(inv_rows, "inv_rows", torch.int32),
        _ptr(topk_w, "topk_w", torch.float32), _ptr(out, "out", dt), _ptr(ws, "ws"),
        ws.numel() * ws.element_size(), _stream(stream)), "lbv_moe_gemm_w2_combine")


def lbv_moe_forward(cfg, x, mask, router_w, e_bias, w13, w2, shared_w13, shared_w2, out,
                    topk_ids_out, topk_w_out, ws, stream=None):
    dt = cfg.torch_dtype
    _check(load().lbv_moe_forward(
        ctypes.byref(cfg), x.shape[0], _ptr(x, "x", dt), _ptr(mask, "mask", torch.uint8),
        _ptr(router_w, "router_w", torch.float32), _ptr(e_bias, "e_bias", torch.float32),
        _ptr(w13, "w13", dt), _ptr(w2, "w2", dt), _ptr(shared_w13, "shared_w13", dt),
        _ptr(shared_w2, "shared_w2", dt), _ptr(out, "out", dt),
        _ptr(topk_ids_out, "topk_ids_out", torch.int32),
        _ptr(topk_w_out, "topk_w_out", torch.float32), _ptr(ws, "ws"),
        ws.numel() * ws.element_size(), _stream(stream)), "lbv_moe_forward")


class MoEBlock:
    """Holds device weights and a workspace; ``__call__`` runs lbv_moe_forward.

    Weights: router_w [E,H] fp32, e_bias [E] fp32, w13 [E,2I,H], w2 [E,H,I],
    shared_w13 [2 I_s,H], shared_w2 [H,I_s] in the config's dtype.
    """

    def __init__(self, cfg: MoEConfig, router_w, e_bias, w13, w2, shared_w13=None,
                 shared_w2=None):
        self.cfg = cfg
        self.router_w, self.e_bias = router_w, e_bias
        self.w13, self.w2 = w13, w2
        self.shared_w13, self.shared_w2 = shared_w13, shared_w2
        self._ws = None

    def workspace(self, T: int) -> torch.Tensor:
        need = lbv_moe_workspace_size(self.cfg, T)
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(max(need, 256), dtype=torch.uint8, device=self.w13.device)
        return self._ws

    def __call__(self, x, mask=None, out=None, want_routing=False, stream=None):
        T = x.shape[0]
        if out is None:
            out = torch.empty_like(x)
        ids = w = None
        if want_routing:
            ids = torch.empty(T, self.cfg.top_k, dtype=torch.int32, device=x.device)
            w = torch.empty(T, self.cfg.top_k, dtype=torch.float32, device=x.device)
        lbv_moe_forward(self.cfg, x, mask, self.router_w, self.e_bias, self.w13, self.w2,
                        self.shared_w13, self.shared_w2, out, ids, w, self.workspace(T), stream)
        return (out, ids, w) if want_routing else out
