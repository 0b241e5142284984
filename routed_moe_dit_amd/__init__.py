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
    "lbv_moe_permute_workspace_size", "lbv_moe_w13_workspace_size",
    "lbv_moe_w2_workspace_size", "lbv_moe_route", "lbv_moe_route_noalloc", "lbv_moe_permute",
    "lbv_moe_gemm_w13_silu",
    "lbv_moe_gemm_w2_combine", "lbv_moe_forward", "lbv_adaln_rmsnorm",
    "lbv_moe_ffn_adaln_workspace_size", "lbv_moe_ffn_adaln", "Fp8Weights",
    "lbv_quantize_fp8_rows", "quantize_fp8_weights", "lbv_moe_forward_fp8",
    "lbv_moe_forward_w8a8", "AttnConfig",
    "attn_config", "attn_sp", "lbv_attn_workspace_size", "lbv_linear_bf16", "lbv_attn_qk_prep",
    "lbv_attn_core", "lbv_attn_forward", "lbv_attn_half_adaln_workspace_size",
    "lbv_attn_half_adaln", "EXPORTS", "LIB_PATH",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblbv_moe.so")

# status codes of lbv_moe.h
LBV_OK, LBV_ERR_NULL, LBV_ERR_SHAPE, LBV_ERR_UNSUPPORTED = 0, 1, 2, 3
LBV_ERR_ALIAS, LBV_ERR_ALIGN, LBV_ERR_WORKSPACE, LBV_ERR_HIP = 4, 5, 6, 7
LBV_ERR_SCRATCH = 8
LBV_F32, LBV_BF16 = 0, 1
LBV_SCORE_SIGMOID, LBV_SCORE_SOFTMAX = 0, 1

EXPORTS = (
    "lbv_abi_version", "lbv_status_string", "lbv_moe_check_config", "lbv_moe_workspace_size",
    "lbv_moe_route_workspace_size", "lbv_moe_permute_workspace_size", "lbv_moe_w13_workspace_size",
    "lbv_moe_w2_workspace_size", "lbv_moe_route", "lbv_moe_route_noalloc",
    "lbv_moe_permute", "lbv_moe_gemm_w13_silu", "lbv_moe_gemm_w2_combine", "lbv_moe_forward",
    "lbv_adaln_rmsnorm", "lbv_moe_ffn_adaln_workspace_size", "lbv_moe_ffn_adaln",
    "lbv_quantize_fp8_rows", "lbv_moe_forward_fp8", "lbv_moe_forward_w8a8",
    "lbv_attn_workspace_size", "lbv_linear_bf16",
    "lbv_attn_qk_prep", "lbv_attn_core", "lbv_attn_forward", "lbv_attn_half_adaln_workspace_size",
    "lbv_attn_half_adaln",
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


class AttnConfig(ctypes.Structure):
    """Mirror of lbv_attn_config."""

    _fields_ = [("hidden", ctypes.c_int32), ("num_heads", ctypes.c_int32), ("eps", ctypes.c_float)]

    @property
    def head_dim(self):
        return self.hidden // self.num_heads


def attn_config(hidden=2048, num_heads=16, eps=1e-6) -> AttnConfig:
    return AttnConfig(hidden, num_heads, float(eps))


def attn_sp(S: int) -> int:
    """Key positions per channel row of vt: S rounded up to 64."""
    return (S + 63) // 64 * 64


class _Fp8WeightsC(ctypes.Structure):
    """Mirror of lbv_moe_fp8_weights."""

    _fields_ = [(n, ctypes.c_void_p) for n in (
        "w13", "w13_scale", "w2", "w2_scale", "shared_w13", "shared_w13_scale", "shared_w2",
        "shared_w2_scale")]


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
              "lbv_moe_w13_workspace_size", "lbv_moe_w2_workspace_size"):
        getattr(L, n).argtypes = [C, I64, ctypes.POINTER(SZ)]
        getattr(L, n).restype = st
    L.lbv_moe_route_workspace_size.argtypes = [C, ctypes.POINTER(SZ)]
    L.lbv_moe_route_workspace_size.restype = st
    L.lbv_moe_route.argtypes = [C, I64, P, P, P, P, P, P, P, SZ, P]
    L.lbv_moe_route.restype = st
    L.lbv_moe_route_noalloc.argtypes = [C, I64, P, P, P, P, P, P, P]
    L.lbv_moe_route_noalloc.restype = st
    L.lbv_moe_permute.argtypes = [C, I64, P, P, P, P, P, SZ, P]
    L.lbv_moe_permute.restype = st
    L.lbv_moe_gemm_w13_silu.argtypes = [C, I64, P, P, P, P, P, P, P, SZ, P]
    L.lbv_moe_gemm_w13_silu.restype = st
    L.lbv_moe_gemm_w2_combine.argtypes = [C, I64, P, P, P, P, P, P, P, P, P, SZ, P]
    L.lbv_moe_gemm_w2_combine.restype = st
    L.lbv_moe_forward.argtypes = [C, I64, P, P, P, P, P, P, P, P, P, P, P, P, SZ, P]
    L.lbv_moe_forward.restype = st
    F = ctypes.c_float
    L.lbv_adaln_rmsnorm.argtypes = [C, I64, P, P, I64, P, F, P, P]
    L.lbv_adaln_rmsnorm.restype = st
    L.lbv_moe_ffn_adaln_workspace_size.argtypes = [C, I64, ctypes.POINTER(SZ)]
    L.lbv_moe_ffn_adaln_workspace_size.restype = st
    L.lbv_moe_ffn_adaln.argtypes = [C, I64, P, P, P, I64, P, F, P, P, P, P, P, P, P, P, P, P, SZ, P]
    L.lbv_moe_ffn_adaln.restype = st
    L.lbv_quantize_fp8_rows.argtypes = [P, ctypes.c_int32, I64, I64, P, P, P]
    L.lbv_quantize_fp8_rows.restype = st
    for n in ("lbv_moe_forward_fp8", "lbv_moe_forward_w8a8"):
        getattr(L, n).argtypes = [C, I64, P, P, P, P, ctypes.POINTER(_Fp8WeightsC), P, P, P, P, SZ, P]
        getattr(L, n).restype = st
    A = ctypes.POINTER(AttnConfig)
    L.lbv_attn_workspace_size.argtypes = [A, I64, I64, ctypes.POINTER(SZ)]
    L.lbv_attn_workspace_size.restype = st
    L.lbv_linear_bf16.argtypes = [I64, ctypes.c_int32, ctypes.c_int32, P, P, P, P, P, SZ, P]
    L.lbv_linear_bf16.restype = st
    L.lbv_attn_qk_prep.argtypes = [A, I64, I64, P, P, P, P, P, P, P, P, P]
    L.lbv_attn_qk_prep.restype = st
    L.lbv_attn_core.argtypes = [A, I64, I64, P, P, P, P, P, P]
    L.lbv_attn_core.restype = st
    L.lbv_attn_forward.argtypes = [A, I64, I64, P, P, P, P, P, P, P, P, P, P, P, P, SZ, P]
    L.lbv_attn_forward.restype = st
    L.lbv_attn_half_adaln_workspace_size.argtypes = [A, I64, I64, ctypes.POINTER(SZ)]
    L.lbv_attn_half_adaln_workspace_size.restype = st
    L.lbv_attn_half_adaln.argtypes = [A, I64, I64, P, P, P, I64, P, F, P, P, P, P, P, P, P, P, P,
                                      P, SZ, P]
    L.lbv_attn_half_adaln.restype = st
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


def _dims(cfg: MoEConfig):
    H, E, K, I, ns = (cfg.hidden, cfg.num_experts, cfg.top_k, cfg.intermediate,
                      cfg.n_shared_experts)
    return H, E, K, I, ns, K + ns, E + ns


def _shape(t, name, *shape):
    """Checks t.shape against `shape` (None entries are free); None tensors pass."""
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor or None" % name)
    got = tuple(t.shape)
    if len(got) != len(shape) or any(w is not None and g != w for g, w in zip(got, shape)):
        raise ValueError("%s has shape %s, expected %s" % (
            name, list(got), ["*" if w is None else w for w in shape]))


def _numel_at_least(t, name, n):
    if t is not None and t.numel() < n:
        raise ValueError("%s holds %d elements, needs at least %d" % (name, t.numel(), n))


def _need(t, name):
    if t is None:
        raise ValueError("%s is required" % name)


def _same_device(*ts):
    devs = {t.device for t in ts if isinstance(t, torch.Tensor)}
    if len(devs) > 1:
        raise ValueError("all tensors must be on one device, got %s" % sorted(map(str, devs)))


def _shared_shapes(cfg, shared_w13, shared_w2):
    H, E, K, I, ns, KS, S = _dims(cfg)
    if ns > 0:
        _shape(shared_w13, "shared_w13", 2 * I * ns, H)
        _shape(shared_w2, "shared_w2", H, I * ns)
    elif shared_w13 is not None or shared_w2 is not None:
        raise ValueError("shared weights given but n_shared_experts == 0")


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


def lbv_moe_w13_workspace_size(cfg: MoEConfig, T: int) -> int:
    return _size("lbv_moe_w13_workspace_size", cfg, T)


def lbv_moe_w2_workspace_size(cfg: MoEConfig, T: int) -> int:
    return _size("lbv_moe_w2_workspace_size", cfg, T)


def lbv_moe_route(cfg, x, router_w, e_bias, mask, topk_ids, topk_w, ws=None, stream=None):
    dt = cfg.torch_dtype
    H, E, K, I, ns, KS, S = _dims(cfg)
    _shape(x, "x", None, H)
    T = x.shape[0]
    _shape(router_w, "router_w", E, H)
    _shape(e_bias, "e_bias", E)
    _shape(mask, "mask", T)
    _shape(topk_ids, "topk_ids", T, K)
    _shape(topk_w, "topk_w", T, K)
    _same_device(x, router_w, e_bias, mask, topk_ids, topk_w, ws)
    _check(load().lbv_moe_route(
        ctypes.byref(cfg), T, _ptr(x, "x", dt), _ptr(router_w, "router_w", torch.float32),
        _ptr(e_bias, "e_bias", torch.float32), _ptr(mask, "mask", torch.uint8),
        _ptr(topk_ids, "topk_ids", torch.int32), _ptr(topk_w, "topk_w", torch.float32),
        _ptr(ws, "ws"), 0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)),
        "lbv_moe_route")


def lbv_moe_route_noalloc(cfg, x, router_w, e_bias, mask, topk_ids, topk_w, stream=None):
    """lbv_moe_route with the library's fixed per-GPU scratch instead of a
    workspace (allocates nothing; overlapping calls on one GPU race)."""
    dt = cfg.torch_dtype
    H, E, K, I, ns, KS, S = _dims(cfg)
    _shape(x, "x", None, H)
    T = x.shape[0]
    _shape(router_w, "router_w", E, H)
    _shape(e_bias, "e_bias", E)
    _shape(mask, "mask", T)
    _shape(topk_ids, "topk_ids", T, K)
    _shape(topk_w, "topk_w", T, K)
    _same_device(x, router_w, e_bias, mask, topk_ids, topk_w)
    _check(load().lbv_moe_route_noalloc(
        ctypes.byref(cfg), T, _ptr(x, "x", dt), _ptr(router_w, "router_w", torch.float32),
        _ptr(e_bias, "e_bias", torch.float32), _ptr(mask, "mask", torch.uint8),
        _ptr(topk_ids, "topk_ids", torch.int32), _ptr(topk_w, "topk_w", torch.float32),
        _stream(stream)), "lbv_moe_route_noalloc")


def lbv_moe_permute(cfg, topk_ids, offsets, sorted_rows, inv_rows, ws, stream=None):
    H, E, K, I, ns, KS, S = _dims(cfg)
    _shape(topk_ids, "topk_ids", None, K)
    T = topk_ids.shape[0]
    _numel_at_least(offsets, "offsets", S + 1)
    _numel_at_least(sorted_rows, "sorted_rows", T * KS)
    _numel_at_least(inv_rows, "inv_rows", T * KS)
    _need(ws, "ws")
    _same_device(topk_ids, offsets, sorted_rows, inv_rows, ws)
    _check(load().lbv_moe_permute(
        ctypes.byref(cfg), T, _ptr(topk_ids, "topk_ids", torch.int32),
        _ptr(offsets, "offsets", torch.int32), _ptr(sorted_rows, "sorted_rows", torch.int32),
        _ptr(inv_rows, "inv_rows", torch.int32), _ptr(ws, "ws"),
        ws.numel() * ws.element_size(), _stream(stream)), "lbv_moe_permute")


def lbv_moe_gemm_w13_silu(cfg, x, w13, shared_w13, offsets, sorted_rows, act, ws, stream=None):
    dt = cfg.torch_dtype
    H, E, K, I, ns, KS, S = _dims(cfg)
    _shape(x, "x", None, H)
    T = x.shape[0]
    _shape(w13, "w13", E, 2 * I, H)
    _shared_shapes(cfg, shared_w13, None)
    _numel_at_least(offsets, "offsets", S + 1)
    _numel_at_least(sorted_rows, "sorted_rows", T * KS)
    _shape(act, "act", None, I)
    _numel_at_least(act, "act", T * KS * I)
    _need(ws, "ws")
    _same_device(x, w13, shared_w13, offsets, sorted_rows, act, ws)
    _check(load().lbv_moe_gemm_w13_silu(
        ctypes.byref(cfg), T, _ptr(x, "x", dt), _ptr(w13, "w13", dt),
        _ptr(shared_w13, "shared_w13", dt), _ptr(offsets, "offsets", torch.int32),
        _ptr(sorted_rows, "sorted_rows", torch.int32), _ptr(act, "act", dt), _ptr(ws, "ws"),
        ws.numel() * ws.element_size(), _stream(stream)), "lbv_moe_gemm_w13_silu")


def lbv_moe_gemm_w2_combine(cfg, act, w2, shared_w2, offsets, sorted_rows, inv_rows, topk_w,
                            out, ws, stream=None):
    dt = cfg.torch_dtype
    H, E, K, I, ns, KS, S = _dims(cfg)
    _shape(out, "out", None, H)
    T = out.shape[0]
    _shape(act, "act", None, I)
    _numel_at_least(act, "act", T * KS * I)
    _shape(w2, "w2", E, H, I)
    _shared_shapes(cfg, None, shared_w2)
    _numel_at_least(offsets, "offsets", S + 1)
    _numel_at_least(sorted_rows, "sorted_rows", T * KS)
    _numel_at_least(inv_rows, "inv_rows", T * KS)
    _shape(topk_w, "topk_w", T, K)
    _need(ws, "ws")
    _same_device(act, w2, shared_w2, offsets, sorted_rows, inv_rows, topk_w, out, ws)
    _check(load().lbv_moe_gemm_w2_combine(
        ctypes.byref(cfg), T, _ptr(act, "act", dt), _ptr(w2, "w2", dt),
        _ptr(shared_w2, "shared_w2", dt), _ptr(offsets, "offsets", torch.int32),
        _ptr(sorted_rows, "sorted_rows", torch.int32), _ptr(inv_rows, "inv_rows", torch.int32),
        _ptr(topk_w, "topk_w", torch.float32), _ptr(out, "out", dt), _ptr(ws, "ws"),
        ws.numel() * ws.element_size(), _stream(stream)), "lbv_moe_gemm_w2_combine")


def lbv_moe_forward(cfg, x, mask, router_w, e_bias, w13, w2, shared_w13, shared_w2, out,
                    topk_ids_out, topk_w_out, ws, stream=None):
    dt = cfg.torch_dtype
    H, E, K, I, ns, KS, S = _dims(cfg)
    _shape(x, "x", None, H)
    T = x.shape[0]
    _shape(mask, "mask", T)
    _shape(router_w, "router_w", E, H)
    _shape(e_bias, "e_bias", E)
    _shape(w13, "w13", E, 2 * I, H)
    _shape(w2, "w2", E, H, I)
    _shared_shapes(cfg, shared_w13, shared_w2)
    _shape(out, "out", T, H)
    _shape(topk_ids_out, "topk_ids_out", T, K)
    _shape(topk_w_out, "topk_w_out", T, K)
    _need(ws, "ws")
    _same_device(x, mask, router_w, e_bias, w13, w2, shared_w13, shared_w2, out, topk_ids_out,
                 topk_w_out, ws)
    _check(load().lbv_moe_forward(
        ctypes.byref(cfg), T, _ptr(x, "x", dt), _ptr(mask, "mask", torch.uint8),
        _ptr(router_w, "router_w", torch.float32), _ptr(e_bias, "e_bias", torch.float32),
        _ptr(w13, "w13", dt), _ptr(w2, "w2", dt), _ptr(shared_w13, "shared_w13", dt),
        _ptr(shared_w2, "shared_w2", dt), _ptr(out, "out", dt),
        _ptr(topk_ids_out, "topk_ids_out", torch.int32),
        _ptr(topk_w_out, "topk_w_out", torch.float32), _ptr(ws, "ws"),
        ws.numel() * ws.element_size(), _stream(stream)), "lbv_moe_forward")


def _temb_rows(temb6, T, H):
    """(pointer tensor, row stride in elements) of a token-level [T, 6, H] or a
    shared [6, H] time embedding."""
    if temb6 is None:
        raise ValueError("temb6 is required")
    if tuple(temb6.shape) == (T, 6, H):
        return 6 * H
    if tuple(temb6.shape) == (6, H):
        return 0
    raise ValueError("temb6 has shape %s, expected [%d, 6, %d] or [6, %d]" % (
        list(temb6.shape), T, H, H))


def lbv_adaln_rmsnorm(cfg, x, temb6, table, eps, h, stream=None):
    """h = rmsnorm(x) * (1 + scale) + shift (rows 4 and 3 of table + temb6)."""
    dt = cfg.torch_dtype
    H = cfg.hidden
    _shape(x, "x", None, H)
    T = x.shape[0]
    stride = _temb_rows(temb6, T, H)
    _shape(table, "table", 6, H)
    _shape(h, "h", T, H)
    _same_device(x, temb6, table, h)
    _check(load().lbv_adaln_rmsnorm(
        ctypes.byref(cfg), T, _ptr(x, "x", torch.float32), _ptr(temb6, "temb6", torch.float32),
        stride, _ptr(table, "table", torch.float32), float(eps), _ptr(h, "h", dt),
        _stream(stream)), "lbv_adaln_rmsnorm")


def lbv_moe_ffn_adaln_workspace_size(cfg: MoEConfig, T: int) -> int:
    return _size("lbv_moe_ffn_adaln_workspace_size", cfg, T)


def lbv_moe_ffn_adaln(cfg, x, mask, temb6, table, eps, router_w, e_bias, w13, w2, shared_w13,
                      shared_w2, out, topk_ids_out, topk_w_out, ws, stream=None):
    """The FFN half of a DiT layer: out = x + gate * block(AdaLN(x)), fp32
    residual stream (out may be x)."""
    dt = cfg.torch_dtype
    H, E, K, I, ns, KS, S = _dims(cfg)
    _shape(x, "x", None, H)
    T = x.shape[0]
    stride = _temb_rows(temb6, T, H)
    _shape(table, "table", 6, H)
    _shape(mask, "mask", T)
    _shape(router_w, "router_w", E, H)
    _shape(e_bias, "e_bias", E)
    _shape(w13, "w13", E, 2 * I, H)
    _shape(w2, "w2", E, H, I)
    _shared_shapes(cfg, shared_w13, shared_w2)
    _shape(out, "out", T, H)
    _shape(topk_ids_out, "topk_ids_out", T, K)
    _shape(topk_w_out, "topk_w_out", T, K)
    _need(ws, "ws")
    _same_device(x, mask, temb6, table, router_w, e_bias, w13, w2, shared_w13, shared_w2, out,
                 topk_ids_out, topk_w_out, ws)
    _check(load().lbv_moe_ffn_adaln(
        ctypes.byref(cfg), T, _ptr(x, "x", torch.float32), _ptr(mask, "mask", torch.uint8),
        _ptr(temb6, "temb6", torch.float32), stride, _ptr(table, "table", torch.float32),
        float(eps), _ptr(router_w, "router_w", torch.float32),
        _ptr(e_bias, "e_bias", torch.float32), _ptr(w13, "w13", dt), _ptr(w2, "w2", dt),
        _ptr(shared_w13, "shared_w13", dt), _ptr(shared_w2, "shared_w2", dt),
        _ptr(out, "out", torch.float32), _ptr(topk_ids_out, "topk_ids_out", torch.int32),
        _ptr(topk_w_out, "topk_w_out", torch.float32), _ptr(ws, "ws"),
        ws.numel() * ws.element_size(), _stream(stream)), "lbv_moe_ffn_adaln")


def lbv_quantize_fp8_rows(w, q, scale, stream=None):
    """q [..., cols] uint8 e4m3fn codes and scale [...] fp32 powers of two of
    the rows of w [..., cols] (bf16 or fp32)."""
    if w.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("w must be bfloat16 or float32, got %s" % w.dtype)
    if w.dim() < 1:
        raise ValueError("w must have at least one dimension")
    _shape(q, "q", *w.shape)
    _shape(scale, "scale", *w.shape[:-1])
    _same_device(w, q, scale)
    cols = w.shape[-1]
    rows = w.numel() // cols if cols else 0
    _check(load().lbv_quantize_fp8_rows(
        _ptr(w, "w"), LBV_BF16 if w.dtype == torch.bfloat16 else LBV_F32, rows, cols,
        _ptr(q, "q", torch.uint8), _ptr(scale, "scale", torch.float32), _stream(stream)),
        "lbv_quantize_fp8_rows")


class Fp8Weights:
    """FP8 expert weights of one layer: codes (uint8) and row scales (fp32)
    of w13 [E,2I,H], w2 [E,H,I], shared_w13 [2 I_s,H], shared_w2 [H,I_s]."""

    def __init__(self, w13, w13_scale, w2, w2_scale, shared_w13=None, shared_w13_scale=None,
                 shared_w2=None, shared_w2_scale=None):
        self.w13, self.w13_scale = w13, w13_scale
        self.w2, self.w2_scale = w2, w2_scale
        self.shared_w13, self.shared_w13_scale = shared_w13, shared_w13_scale
        self.shared_w2, self.shared_w2_scale = shared_w2, shared_w2_scale

    def tensors(self):
        return (self.w13, self.w13_scale, self.w2, self.w2_scale, self.shared_w13,
                self.shared_w13_scale, self.shared_w2, self.shared_w2_scale)


def quantize_fp8_weights(w13, w2, shared_w13=None, shared_w2=None, stream=None) -> Fp8Weights:
    """Fp8Weights of bf16 / fp32 expert weights (device tensors), quantized on
    the device by lbv_quantize_fp8_rows."""
    out = []
    for w in (w13, w2, shared_w13, shared_w2):
        if w is None:
            out += [None, None]
            continue
        q = torch.empty(w.shape, dtype=torch.uint8, device=w.device)
        sc = torch.empty(w.shape[:-1], dtype=torch.float32, device=w.device)
        lbv_quantize_fp8_rows(w, q, sc, stream)
        out += [q, sc]
    return Fp8Weights(*out)


def lbv_moe_forward_fp8(cfg, x, mask, router_w, e_bias, wq: Fp8Weights, out, topk_ids_out,
                        topk_w_out, ws, stream=None):
    """lbv_moe_forward with fp8 expert weights (bf16 activations)."""
    _forward_fp8_weights("lbv_moe_forward_fp8", cfg, x, mask, router_w, e_bias, wq, out,
                         topk_ids_out, topk_w_out, ws, stream)


def lbv_moe_forward_w8a8(cfg, x, mask, router_w, e_bias, wq: Fp8Weights, out, topk_ids_out,
                         topk_w_out, ws, stream=None):
    """lbv_moe_forward with fp8 expert weights and fp8 activations."""
    _forward_fp8_weights("lbv_moe_forward_w8a8", cfg, x, mask, router_w, e_bias, wq, out,
                         topk_ids_out, topk_w_out, ws, stream)


def _forward_fp8_weights(fn, cfg, x, mask, router_w, e_bias, wq, out, topk_ids_out, topk_w_out,
                         ws, stream):
    H, E, K, I, ns, KS, S = _dims(cfg)
    _shape(x, "x", None, H)
    T = x.shape[0]
    _shape(mask, "mask", T)
    _shape(router_w, "router_w", E, H)
    _shape(e_bias, "e_bias", E)
    _shape(wq.w13, "w13", E, 2 * I, H)
    _shape(wq.w13_scale, "w13_scale", E, 2 * I)
    _shape(wq.w2, "w2", E, H, I)
    _shape(wq.w2_scale, "w2_scale", E, H)
    if ns > 0:
        _shape(wq.shared_w13, "shared_w13", 2 * I * ns, H)
        _shape(wq.shared_w13_scale, "shared_w13_scale", 2 * I * ns)
        _shape(wq.shared_w2, "shared_w2", H, I * ns)
        _shape(wq.shared_w2_scale, "shared_w2_scale", H)
    elif any(t is not None for t in wq.tensors()[4:]):
        raise ValueError("shared weights given but n_shared_experts == 0")
    _shape(out, "out", T, H)
    _shape(topk_ids_out, "topk_ids_out", T, K)
    _shape(topk_w_out, "topk_w_out", T, K)
    _need(ws, "ws")
    _same_device(x, mask, router_w, e_bias, out, topk_ids_out, topk_w_out, ws, *wq.tensors())
    names = ("w13", "w13_scale", "w2", "w2_scale", "shared_w13", "shared_w13_scale", "shared_w2",
             "shared_w2_scale")
    ptrs = [_ptr(t, n, torch.float32 if n.endswith("scale") else torch.uint8)
            for t, n in zip(wq.tensors(), names)]
    cw = _Fp8WeightsC(*ptrs)
    dt = cfg.torch_dtype
    _check(getattr(load(), fn)(
        ctypes.byref(cfg), T, _ptr(x, "x", dt), _ptr(mask, "mask", torch.uint8),
        _ptr(router_w, "router_w", torch.float32), _ptr(e_bias, "e_bias", torch.float32),
        ctypes.byref(cw), _ptr(out, "out", dt), _ptr(topk_ids_out, "topk_ids_out", torch.int32),
        _ptr(topk_w_out, "topk_w_out", torch.float32), _ptr(ws, "ws"),
        ws.numel() * ws.element_size(), _stream(stream)), fn)


def lbv_attn_workspace_size(cfg: AttnConfig, B: int, S: int) -> int:
    n = ctypes.c_size_t(0)
    _check(load().lbv_attn_workspace_size(ctypes.byref(cfg), B, S, ctypes.byref(n)),
           "lbv_attn_workspace_size")
    return n.value


LINEAR_WS_BYTES = 512


def lbv_linear_bf16(x, w, bias, y, ws, stream=None):
    """y [T, N] = x [T, K] w[N, K]^T (+ bias [N] fp32), bf16."""
    _shape(x, "x", None, None)
    T, K = x.shape
    _shape(w, "w", None, K)
    N = w.shape[0]
    _shape(bias, "bias", N)
    _shape(y, "y", T, N)
    _need(ws, "ws")
    _numel_at_least(ws, "ws", LINEAR_WS_BYTES)
    _same_device(x, w, bias, y, ws)
    _check(load().lbv_linear_bf16(
        T, N, K, _ptr(x, "x", torch.bfloat16), _ptr(w, "w", torch.bfloat16),
        _ptr(bias, "bias", torch.float32), _ptr(y, "y", torch.bfloat16), _ptr(ws, "ws"),
        ws.numel() * ws.element_size(), _stream(stream)), "lbv_linear_bf16")


def _attn_shapes(cfg, B, S, **ts):
    H, D = cfg.hidden, cfg.head_dim
    T = B * S
    want = dict(x=(T, H), qkv=(T, 3 * H), q=(T, H), k=(T, H), o=(T, H), out=(T, H),
                vt=(B, cfg.num_heads, D, attn_sp(S)), mask=(T,), g_q=(D,), g_k=(D,),
                cos=(T, D // 2), sin=(T, D // 2), w_qkv=(3 * H, H), b_qkv=(3 * H,), w_o=(H, H),
                b_o=(H,))
    for name, t in ts.items():
        _shape(t, name, *want[name])


def lbv_attn_qk_prep(cfg, B, S, qkv, g_q, g_k, cos, sin, q, k, vt, stream=None):
    _attn_shapes(cfg, B, S, qkv=qkv, g_q=g_q, g_k=g_k, cos=cos, sin=sin, q=q, k=k, vt=vt)
    _same_device(qkv, g_q, g_k, cos, sin, q, k, vt)
    bf, f = torch.bfloat16, torch.float32
    _check(load().lbv_attn_qk_prep(
        ctypes.byref(cfg), B, S, _ptr(qkv, "qkv", bf), _ptr(g_q, "g_q", f), _ptr(g_k, "g_k", f),
        _ptr(cos, "cos", f), _ptr(sin, "sin", f), _ptr(q, "q", bf), _ptr(k, "k", bf),
        _ptr(vt, "vt", bf), _stream(stream)), "lbv_attn_qk_prep")


def lbv_attn_core(cfg, B, S, q, k, vt, mask, o, stream=None):
    _attn_shapes(cfg, B, S, q=q, k=k, vt=vt, mask=mask, o=o)
    _same_device(q, k, vt, mask, o)
    bf = torch.bfloat16
    _check(load().lbv_attn_core(
        ctypes.byref(cfg), B, S, _ptr(q, "q", bf), _ptr(k, "k", bf), _ptr(vt, "vt", bf),
        _ptr(mask, "mask", torch.uint8), _ptr(o, "o", bf), _stream(stream)), "lbv_attn_core")


def lbv_attn_forward(cfg, B, S, x, mask, w_qkv, b_qkv, g_q, g_k, cos, sin, w_o, b_o, out, ws,
                     stream=None):
    _attn_shapes(cfg, B, S, x=x, mask=mask, w_qkv=w_qkv, b_qkv=b_qkv, g_q=g_q, g_k=g_k, cos=cos,
                 sin=sin, w_o=w_o, b_o=b_o, out=out)
    _need(ws, "ws")
    _same_device(x, mask, w_qkv, b_qkv, g_q, g_k, cos, sin, w_o, b_o, out, ws)
    bf, f = torch.bfloat16, torch.float32
    _check(load().lbv_attn_forward(
        ctypes.byref(cfg), B, S, _ptr(x, "x", bf), _ptr(mask, "mask", torch.uint8),
        _ptr(w_qkv, "w_qkv", bf), _ptr(b_qkv, "b_qkv", f), _ptr(g_q, "g_q", f),
        _ptr(g_k, "g_k", f), _ptr(cos, "cos", f), _ptr(sin, "sin", f), _ptr(w_o, "w_o", bf),
        _ptr(b_o, "b_o", f), _ptr(out, "out", bf), _ptr(ws, "ws"),
        ws.numel() * ws.element_size(), _stream(stream)), "lbv_attn_forward")


def lbv_attn_half_adaln_workspace_size(cfg: AttnConfig, B: int, S: int) -> int:
    n = ctypes.c_size_t(0)
    _check(load().lbv_attn_half_adaln_workspace_size(ctypes.byref(cfg), B, S, ctypes.byref(n)),
           "lbv_attn_half_adaln_workspace_size")
    return n.value


def lbv_attn_half_adaln(cfg, B, S, x, mask, temb6, table, eps, w_qkv, b_qkv, g_q, g_k, cos, sin,
                        w_o, b_o, out, ws, stream=None):
    """The attention half with AdaLN (rows 0, 1) and the gated residual
    (row 2): x, out [B S, H] fp32; temb6 [B S, 6, H] or [6, H] (shared)."""
    H = cfg.hidden
    T = B * S
    _attn_shapes(cfg, B, S, mask=mask, w_qkv=w_qkv, b_qkv=b_qkv, g_q=g_q, g_k=g_k, cos=cos,
                 sin=sin, w_o=w_o, b_o=b_o)
    _shape(x, "x", T, H)
    _shape(out, "out", T, H)
    _shape(table, "table", 6, H)
    stride = _temb_rows(temb6, T, H)
    _need(ws, "ws")
    _same_device(x, mask, temb6, table, w_qkv, b_qkv, g_q, g_k, cos, sin, w_o, b_o, out, ws)
    bf, f = torch.bfloat16, torch.float32
    _check(load().lbv_attn_half_adaln(
        ctypes.byref(cfg), B, S, _ptr(x, "x", f), _ptr(mask, "mask", torch.uint8),
        _ptr(temb6, "temb6", f), stride, _ptr(table, "table", f), float(eps),
        _ptr(w_qkv, "w_qkv", bf), _ptr(b_qkv, "b_qkv", f), _ptr(g_q, "g_q", f),
        _ptr(g_k, "g_k", f), _ptr(cos, "cos", f), _ptr(sin, "sin", f), _ptr(w_o, "w_o", bf),
        _ptr(b_o, "b_o", f), _ptr(out, "out", f), _ptr(ws, "ws"), ws.numel() * ws.element_size(),
        _stream(stream)), "lbv_attn_half_adaln")


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
