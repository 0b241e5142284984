"""C ABI checks that need no GPU: the library loads, exports every function
that include/lbv_moe.h declares, and rejects bad arguments before launching
anything (every call here fails validation or has T == 0, so no kernel runs)."""
import ctypes
import os
import re

import pytest

import routed_moe_dit_amd as lbv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    src = open(os.path.join(ROOT, "include", "lbv_moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    return sorted(set(re.findall(r"\b(lbv_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    names = header_functions()
    assert len(names) == 12, names
    assert set(names) == set(lbv.EXPORTS)
    L = ctypes.CDLL(lbv.LIB_PATH)
    for n in names:
        assert getattr(L, n) is not None


def test_version_and_status_strings():
    assert lbv.lbv_abi_version() == 1
    texts = {lbv.lbv_status_string(s) for s in range(8)}
    assert len(texts) == 8
    assert lbv.lbv_status_string(99) == "unknown status"


BAD = [
    (dict(hidden=100), lbv.LBV_ERR_SHAPE),
    (dict(intermediate=96), lbv.LBV_ERR_SHAPE),
    (dict(num_experts=130), lbv.LBV_ERR_SHAPE),            # 4 does not divide 130
    (dict(topk_group=5), lbv.LBV_ERR_SHAPE),
    (dict(top_k=65), lbv.LBV_ERR_SHAPE),                   # more than 2 groups of 32
    (dict(top_k=0), lbv.LBV_ERR_SHAPE),
    (dict(n_shared_experts=-1), lbv.LBV_ERR_SHAPE),
    (dict(routed_scaling_factor=float("nan")), lbv.LBV_ERR_SHAPE),
    (dict(score_func="softmax"), lbv.LBV_ERR_UNSUPPORTED),
    (dict(num_experts=512, n_group=4), lbv.LBV_ERR_UNSUPPORTED),
    (dict(top_k=17, topk_group=4), lbv.LBV_ERR_UNSUPPORTED),
    (dict(n_shared_experts=9), lbv.LBV_ERR_UNSUPPORTED),
    (dict(num_experts=128, n_group=64, topk_group=2, top_k=2), lbv.LBV_ERR_UNSUPPORTED),
    (dict(num_experts=96, n_group=4), lbv.LBV_ERR_UNSUPPORTED),  # 24 / 2 lanes not 2^k
]


@pytest.mark.parametrize("kw,status", BAD)
def test_config_validation(kw, status):
    assert lbv.lbv_moe_check_config(lbv.config(**kw)) == status


def test_valid_configs():
    for kw in (dict(), dict(dtype="f32"), dict(num_experts=16, n_group=4, top_k=4, hidden=256,
                                               intermediate=128),
               dict(num_experts=256, n_group=8, topk_group=4, top_k=8),
               dict(num_experts=8, n_group=4, topk_group=2, top_k=2), dict(n_shared_experts=0),
               dict(norm_topk_prob=False)):
        assert lbv.lbv_moe_check_config(lbv.config(**kw)) == lbv.LBV_OK, kw
    c = lbv.config()
    c.norm_topk_prob = 2
    assert lbv.lbv_moe_check_config(c) == lbv.LBV_ERR_SHAPE
    c = lbv.config()
    c.dtype = 7
    assert lbv.lbv_moe_check_config(c) == lbv.LBV_ERR_UNSUPPORTED


def test_workspace_sizes():
    c = lbv.config()
    s0 = lbv.lbv_moe_workspace_size(c, 0)
    s1 = lbv.lbv_moe_workspace_size(c, 800)
    s3 = lbv.lbv_moe_workspace_size(c, 38000)
    assert s0 < s1 < s3
    # dominated by the bf16 expert outputs T (K + 1) H and act T (K + 1) I
    assert s3 >= 38000 * 9 * (2048 + 768) * 2
    assert lbv.lbv_moe_w2_workspace_size(c, 38000) >= 38000 * 9 * 2048 * 2
    assert lbv.lbv_moe_permute_workspace_size(c, 38000) >= 149 * 128 * 4
    with pytest.raises(lbv.LbvError) as e:
        lbv.lbv_moe_workspace_size(c, -1)
    assert e.value.status == lbv.LBV_ERR_SHAPE
    with pytest.raises(lbv.LbvError):
        lbv.lbv_moe_workspace_size(c, 2 ** 31 // 9 + 1)    # row ids would overflow int32


def test_bf16_offset_limits():
    # bf16 matmuls address x and each packed gate/up weight with 32-bit byte offsets
    c = lbv.config()
    T4g = (1 << 32) // (2048 * 2)                          # x of exactly 4 GiB
    assert lbv.lbv_moe_permute_workspace_size(c, T4g - 1) > 0
    with pytest.raises(lbv.LbvError) as e:
        lbv.lbv_moe_permute_workspace_size(c, T4g)
    assert e.value.status == lbv.LBV_ERR_SHAPE
    assert lbv.lbv_moe_permute_workspace_size(lbv.config(dtype="f32"), T4g) > 0
    big = dict(hidden=1 << 15, intermediate=1 << 15)     # w13 of one expert: 4 GiB in bf16
    assert lbv.lbv_moe_check_config(lbv.config(**big)) == lbv.LBV_ERR_SHAPE
    assert lbv.lbv_moe_check_config(lbv.config(dtype="f32", **big)) == lbv.LBV_OK
    # row offsets are formed with 24-bit multiplies: T, hidden and gate/up rows below 2^24
    small_h = lbv.config(hidden=64, intermediate=64, num_experts=8, n_group=2, topk_group=1, top_k=2)
    assert lbv.lbv_moe_permute_workspace_size(small_h, (1 << 24) - 1) > 0
    with pytest.raises(lbv.LbvError) as e:
        lbv.lbv_moe_permute_workspace_size(small_h, 1 << 24)
    assert e.value.status == lbv.LBV_ERR_SHAPE
    wide = dict(hidden=1 << 15, intermediate=1 << 14, n_shared_experts=2)   # shared_w13 4 GiB
    assert lbv.lbv_moe_check_config(lbv.config(**wide)) == lbv.LBV_ERR_SHAPE
    assert lbv.lbv_moe_check_config(lbv.config(**dict(wide, n_shared_experts=1))) == lbv.LBV_OK


def raw():
    return lbv.load()


A = 0x100000        # aligned fake device addresses: never dereferenced, no launch happens
B = 0x200000
Cc = 0x300000
BIG = 1 << 40


def test_route_validation_paths():
    c = lbv.config()
    L = raw()
    need = lbv.lbv_moe_route_workspace_size(c)
    # three bf16 planes of W_r, then partial logits of the few-token path
    # (4 hidden-dimension parts x 4096 tokens x 128 experts, fp32)
    assert need == 3 * 128 * 2048 * 2 + 4 * 4096 * 128 * 4

    def r(T, x, wr, b, ids, w, ws=Cc, nbytes=need):
        return L.lbv_moe_route(ctypes.byref(c), T, x, wr, b, None, ids, w, ws, nbytes, None)

    assert r(4, None, A, B, Cc, Cc) == lbv.LBV_ERR_NULL
    assert r(4, A, A, B, Cc, Cc, ws=None) == lbv.LBV_ERR_NULL
    assert r(4, A + 2, A, B, Cc, Cc) == lbv.LBV_ERR_ALIGN
    assert r(4, A, A + 4, B, Cc, Cc) == lbv.LBV_ERR_ALIGN
    assert r(4, A, A, B, Cc, Cc, nbytes=need - 1) == lbv.LBV_ERR_WORKSPACE
    assert r(-1, A, A, B, Cc, Cc) == lbv.LBV_ERR_SHAPE
    assert r(0, A, A, B, Cc, Cc) == lbv.LBV_OK                # T == 0 is a no-op
    assert L.lbv_moe_route(None, 4, A, A, B, None, Cc, Cc, Cc, need, None) == lbv.LBV_ERR_NULL
    # the fp32 path needs no scratch
    assert lbv.lbv_moe_route_workspace_size(lbv.config(dtype="f32")) == 0


def test_forward_validation_paths():
    c = lbv.config()
    L = raw()

    def f(T, x, out, ws, ws_bytes, sh=A, cfg=c):
        return L.lbv_moe_forward(ctypes.byref(cfg), T, x, None, A, B, A, A, sh, sh, out, None, None,
                                 ws, ws_bytes, None)

    need = lbv.lbv_moe_workspace_size(c, 16)
    assert f(16, A, None, Cc, need) == lbv.LBV_ERR_NULL
    assert f(16, A, Cc, Cc, need, sh=None) == lbv.LBV_ERR_NULL   # shared expert configured
    assert f(16, A, A + 2048 * 2 * 4, Cc, need) == lbv.LBV_ERR_ALIAS
    assert f(16, A, A, Cc, need) == lbv.LBV_ERR_ALIAS
    assert f(16, A, Cc, Cc + 8, need) == lbv.LBV_ERR_ALIGN
    assert f(16, A, Cc, Cc, need - 1) == lbv.LBV_ERR_WORKSPACE
    assert f(0, A, Cc, Cc, 0) == lbv.LBV_OK
    c0 = lbv.config(n_shared_experts=0)
    assert f(0, A, Cc, Cc, 0, sh=None, cfg=c0) == lbv.LBV_OK


def test_split_call_validation_paths():
    c = lbv.config()
    L = raw()
    P = ctypes.c_void_p
    assert L.lbv_moe_permute(ctypes.byref(c), 8, A, None, B, B, Cc, BIG, None) == lbv.LBV_ERR_NULL
    assert L.lbv_moe_permute(ctypes.byref(c), 8, A, B, B, B, Cc, 0, None) == lbv.LBV_ERR_WORKSPACE
    assert L.lbv_moe_permute(ctypes.byref(c), 0, None, None, None, None, None, 0, None) == lbv.LBV_OK
    assert L.lbv_moe_gemm_w13_silu(ctypes.byref(c), 8, A, B, None, B, B, Cc, None) == \
        lbv.LBV_ERR_NULL
    assert L.lbv_moe_gemm_w13_silu(ctypes.byref(c), 8, A, B + 2, A, B, B, Cc, None) == \
        lbv.LBV_ERR_ALIGN
    assert L.lbv_moe_gemm_w2_combine(ctypes.byref(c), 8, A, B, A, B, B, B, B, Cc, Cc, 0, None) == \
        lbv.LBV_ERR_WORKSPACE
    assert L.lbv_moe_gemm_w2_combine(ctypes.byref(c), 8, A, B, A, B, B, B, B, Cc, None, BIG,
                                     None) == lbv.LBV_ERR_NULL
    del P


def test_binding_rejects_host_tensors():
    import torch
    c = lbv.config(hidden=64, intermediate=64, num_experts=8, n_group=2, topk_group=1, top_k=2)
    x = torch.zeros(4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        lbv.lbv_moe_route(c, x, torch.zeros(8, 64), torch.zeros(8), None,
                          torch.zeros(4, 2, dtype=torch.int32), torch.zeros(4, 2))
