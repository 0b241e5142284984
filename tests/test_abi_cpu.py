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
    assert len(names) == 27, names
    assert set(names) == set(lbv.EXPORTS)
    L = ctypes.CDLL(lbv.LIB_PATH)
    for n in names:
        assert getattr(L, n) is not None


def test_version_and_status_strings():
    assert lbv.lbv_abi_version() == 6
    texts = {lbv.lbv_status_string(s) for s in range(9)}
    assert len(texts) == 9
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
    # the down matmul addresses a segment's act rows (up to T) with 32-bit offsets
    tall = lbv.config(hidden=64, intermediate=1 << 14, num_experts=8, n_group=2, topk_group=1,
                      top_k=2)
    Tact = (1 << 32) // ((1 << 14) * 2)
    assert lbv.lbv_moe_permute_workspace_size(tall, Tact - 1) > 0
    with pytest.raises(lbv.LbvError) as e:
        lbv.lbv_moe_permute_workspace_size(tall, Tact)
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
    # three bf16 planes of W_r, then the logits of the few-token path
    # (4096 tokens x 128 experts, fp32)
    assert need == 3 * 128 * 2048 * 2 + 4096 * 128 * 4

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
    gw = lbv.lbv_moe_w13_workspace_size(c, 8)
    assert gw == 256
    assert L.lbv_moe_gemm_w13_silu(ctypes.byref(c), 8, A, B, None, B, B, Cc, Cc, gw, None) == \
        lbv.LBV_ERR_NULL
    assert L.lbv_moe_gemm_w13_silu(ctypes.byref(c), 8, A, B, A, B, B, Cc, None, gw, None) == \
        lbv.LBV_ERR_NULL
    assert L.lbv_moe_gemm_w13_silu(ctypes.byref(c), 8, A, B + 2, A, B, B, Cc, Cc, gw, None) == \
        lbv.LBV_ERR_ALIGN
    assert L.lbv_moe_gemm_w13_silu(ctypes.byref(c), 8, A, B, A, B, B, Cc, Cc, gw - 1, None) == \
        lbv.LBV_ERR_WORKSPACE
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


def small_cfg(**kw):
    base = dict(hidden=64, intermediate=64, num_experts=8, n_group=2, topk_group=1, top_k=2,
                n_shared_experts=1)
    base.update(kw)
    return lbv.config(**base)


def host_block(c, T=4):
    """Host tensors with the shapes the calls expect (the binding checks shapes
    before it looks at devices, so wrong shapes are reported on the CPU)."""
    import torch
    H, E, K, I, ns = c.hidden, c.num_experts, c.top_k, c.intermediate, c.n_shared_experts
    KS, S = K + ns, E + ns
    return dict(x=torch.zeros(T, H, dtype=torch.bfloat16), router_w=torch.zeros(E, H),
                e_bias=torch.zeros(E), mask=torch.ones(T, dtype=torch.uint8),
                w13=torch.zeros(E, 2 * I, H, dtype=torch.bfloat16),
                w2=torch.zeros(E, H, I, dtype=torch.bfloat16),
                shared_w13=torch.zeros(2 * I * ns, H, dtype=torch.bfloat16),
                shared_w2=torch.zeros(H, I * ns, dtype=torch.bfloat16),
                out=torch.zeros(T, H, dtype=torch.bfloat16),
                ids=torch.zeros(T, K, dtype=torch.int32), w=torch.zeros(T, K),
                off=torch.zeros(S + 1, dtype=torch.int32),
                srt=torch.zeros(T * KS, dtype=torch.int32),
                inv=torch.zeros(T * KS, dtype=torch.int32),
                act=torch.zeros(T * KS, I, dtype=torch.bfloat16),
                ws=torch.zeros(1 << 16, dtype=torch.uint8))


def call(name, c, b):
    if name == "forward":
        lbv.lbv_moe_forward(c, b["x"], b["mask"], b["router_w"], b["e_bias"], b["w13"], b["w2"],
                            b["shared_w13"], b["shared_w2"], b["out"], b["ids"], b["w"], b["ws"])
    elif name == "route":
        lbv.lbv_moe_route(c, b["x"], b["router_w"], b["e_bias"], b["mask"], b["ids"], b["w"],
                          b["ws"])
    elif name == "permute":
        lbv.lbv_moe_permute(c, b["ids"], b["off"], b["srt"], b["inv"], b["ws"])
    elif name == "w13":
        lbv.lbv_moe_gemm_w13_silu(c, b["x"], b["w13"], b["shared_w13"], b["off"], b["srt"],
                                  b["act"], b["ws"])
    else:
        lbv.lbv_moe_gemm_w2_combine(c, b["act"], b["w2"], b["shared_w2"], b["off"], b["srt"],
                                    b["inv"], b["w"], b["out"], b["ws"])


WRONG = [
    ("forward", "x", (4, 128)), ("forward", "mask", (5,)), ("forward", "router_w", (8, 32)),
    ("forward", "e_bias", (7,)), ("forward", "w13", (8, 64, 64)), ("forward", "w2", (8, 64, 32)),
    ("forward", "shared_w13", (64, 64)), ("forward", "shared_w2", (64, 128)),
    ("forward", "out", (3, 64)), ("forward", "ids", (4, 3)), ("forward", "w", (4, 1)),
    ("route", "x", (4, 32)), ("route", "ids", (5, 2)), ("route", "w", (4, 3)),
    ("route", "router_w", (9, 64)), ("route", "mask", (3,)),
    ("permute", "ids", (4, 3)), ("permute", "off", (9,)), ("permute", "srt", (11,)),
    ("permute", "inv", (11,)),
    ("w13", "w13", (8, 128, 32)), ("w13", "shared_w13", (128, 32)), ("w13", "act", (11, 64)),
    ("w13", "act", (12, 32)), ("w13", "srt", (11,)), ("w13", "off", (9,)),
    ("w2", "w2", (8, 32, 64)), ("w2", "shared_w2", (32, 64)), ("w2", "w", (5, 2)),
    ("w2", "out", (4, 32)), ("w2", "act", (11, 64)), ("w2", "inv", (11,)),
]


@pytest.mark.parametrize("name,key,shape", WRONG)
def test_binding_rejects_wrong_shapes(name, key, shape):
    """A mis-shaped tensor is refused before any pointer reaches the library."""
    import torch
    c = small_cfg()
    b = host_block(c)
    b[key] = torch.zeros(*shape, dtype=b[key].dtype)
    with pytest.raises(ValueError) as e:
        call(name, c, b)
    assert "shape" in str(e.value) or "elements" in str(e.value)


@pytest.mark.parametrize("name", ["forward", "route", "permute", "w13", "w2"])
def test_binding_right_shapes_reach_the_device_check(name):
    """With every shape right, the only complaint left is that the tensors are
    on the host."""
    c = small_cfg()
    with pytest.raises(ValueError) as e:
        call(name, c, host_block(c))
    assert "device tensor" in str(e.value)


def test_binding_rejects_shared_weights_without_shared_expert():
    c = small_cfg(n_shared_experts=0)
    b = host_block(small_cfg())
    b["srt"] = b["srt"][:8]
    b["inv"] = b["inv"][:8]
    b["act"] = b["act"][:8]
    with pytest.raises(ValueError) as e:
        call("w13", c, b)
    assert "n_shared_experts" in str(e.value)


def test_route_noalloc_validation_paths():
    """The allocation-free router rejects before touching the device: missing
    pointers, misalignment, and a router scratch beyond its fixed 8 MiB."""
    c = lbv.config()
    L = raw()

    def r(cfg, T, x=A, wr=A, b=B, ids=Cc, w=Cc):
        return L.lbv_moe_route_noalloc(ctypes.byref(cfg), T, x, wr, b, None, ids, w, None)

    assert r(c, 0) == lbv.LBV_OK
    assert r(c, 4, x=None) == lbv.LBV_ERR_NULL
    assert r(c, 4, w=None) == lbv.LBV_ERR_NULL
    assert r(c, 4, x=A + 2) == lbv.LBV_ERR_ALIGN
    # 3 x 128 x 16384 bf16 planes = 12 MiB > 8 MiB
    big = lbv.config(hidden=16384)
    assert lbv.lbv_moe_route_workspace_size(big) > (8 << 20)
    assert r(big, 4) == lbv.LBV_ERR_SCRATCH
    # the LingBot shape fits: 1.5 MiB of planes + 2 MiB of logits
    assert lbv.lbv_moe_route_workspace_size(c) <= (8 << 20)


def test_adaln_validation_paths():
    """AdaLN entries reject before any launch: NULLs, misaligned rows, a
    negative or non-finite eps, partial overlap of out and x (out == x is
    allowed), a short workspace."""
    c = lbv.config()
    L = raw()
    H = 2048
    assert L.lbv_adaln_rmsnorm(ctypes.byref(c), 0, None, None, 0, None, 1e-6, None, None) == \
        lbv.LBV_OK
    assert L.lbv_adaln_rmsnorm(ctypes.byref(c), 4, A, None, 0, B, 1e-6, Cc, None) == \
        lbv.LBV_ERR_NULL
    assert L.lbv_adaln_rmsnorm(ctypes.byref(c), 4, A, A, 6 * H + 2, B, 1e-6, Cc, None) == \
        lbv.LBV_ERR_ALIGN
    assert L.lbv_adaln_rmsnorm(ctypes.byref(c), 4, A, A, 0, B, -1.0, Cc, None) == \
        lbv.LBV_ERR_SHAPE
    assert L.lbv_adaln_rmsnorm(ctypes.byref(c), 4, A, A, 0, B, float("nan"), Cc, None) == \
        lbv.LBV_ERR_SHAPE
    assert L.lbv_adaln_rmsnorm(ctypes.byref(c), 4, A, A, 0, B, 1e-6, A + 64, None) == \
        lbv.LBV_ERR_ALIAS
    need = lbv.lbv_moe_ffn_adaln_workspace_size(c, 16)
    assert need == lbv.lbv_moe_workspace_size(c, 16) + 16 * H * 2

    def f(out, ws_bytes=need, x=A):
        return L.lbv_moe_ffn_adaln(ctypes.byref(c), 16, x, None, B, 0, B, 1e-6, B, B, B, B, B, B,
                                   out, None, None, BIG, ws_bytes, None)
    assert f(A + 4096) == lbv.LBV_ERR_ALIAS            # out overlaps x, not equal
    assert f(Cc, ws_bytes=need - 1) == lbv.LBV_ERR_WORKSPACE
    assert f(Cc + 8) == lbv.LBV_ERR_ALIGN


def test_fp8_validation_paths():
    """The fp8 entries reject before any launch: dtype, shapes, NULLs,
    alignment, overlap, the fp32 config, a short workspace."""
    L = raw()
    q = L.lbv_quantize_fp8_rows
    assert q(A, 2, 4, 64, B, Cc, None) == lbv.LBV_ERR_UNSUPPORTED        # dtype
    assert q(A, lbv.LBV_BF16, 4, 24, B, Cc, None) == lbv.LBV_ERR_SHAPE    # cols % 16
    assert q(A, lbv.LBV_BF16, 4, 0, B, Cc, None) == lbv.LBV_ERR_SHAPE
    assert q(A, lbv.LBV_BF16, -1, 64, B, Cc, None) == lbv.LBV_ERR_SHAPE
    assert q(A, lbv.LBV_BF16, 1 << 32, 16, B, Cc, None) == lbv.LBV_ERR_SHAPE   # grid bound
    assert q(None, lbv.LBV_BF16, 0, 64, None, None, None) == lbv.LBV_OK   # no rows
    assert q(A, lbv.LBV_BF16, 4, 64, None, Cc, None) == lbv.LBV_ERR_NULL
    assert q(A, lbv.LBV_BF16, 4, 64, B + 8, Cc, None) == lbv.LBV_ERR_ALIGN
    assert q(A, lbv.LBV_BF16, 4, 64, B, Cc + 2, None) == lbv.LBV_ERR_ALIGN
    assert q(A, lbv.LBV_F32, 4, 64, A + 512, Cc, None) == lbv.LBV_ERR_ALIAS   # q inside w
    assert q(A, lbv.LBV_F32, 4, 64, B, B + 128, None) == lbv.LBV_ERR_ALIAS    # scale inside q

    c = lbv.config()
    W = lbv._Fp8WeightsC(A, B, A, B, A, B, A, B)
    need = lbv.lbv_moe_workspace_size(c, 16)

    def f(T, out=Cc, ws=BIG, ws_bytes=need, cfg=c, w=W):
        return L.lbv_moe_forward_fp8(ctypes.byref(cfg), T, A, None, A, B,
                                     ctypes.byref(w) if w is not None else None, out, None, None,
                                     ws, ws_bytes, None)
    assert f(16, cfg=lbv.config(dtype="f32")) == lbv.LBV_ERR_UNSUPPORTED
    assert f(0) == lbv.LBV_OK
    assert f(16, w=None) == lbv.LBV_ERR_NULL
    assert f(16, w=lbv._Fp8WeightsC(A, B, A, None, A, B, A, B)) == lbv.LBV_ERR_NULL
    assert f(16, w=lbv._Fp8WeightsC(A, B, A, B, None, B, A, B)) == lbv.LBV_ERR_NULL  # shared expert
    assert f(16, w=lbv._Fp8WeightsC(A + 8, B, A, B, A, B, A, B)) == lbv.LBV_ERR_ALIGN
    assert f(16, w=lbv._Fp8WeightsC(A, B + 2, A, B, A, B, A, B)) == lbv.LBV_ERR_ALIGN
    assert f(16, out=A) == lbv.LBV_ERR_ALIAS
    assert f(16, ws_bytes=need - 1) == lbv.LBV_ERR_WORKSPACE
    c0 = lbv.config(n_shared_experts=0)
    assert f(0, cfg=c0, w=lbv._Fp8WeightsC(A, B, A, B, None, None, None, None)) == lbv.LBV_OK


def test_w8a8_validation_paths():
    """lbv_moe_forward_w8a8 rejects before any launch: the fp32 config, H or I
    not multiples of 128, I above 1024 (act's block scales take 32 bytes per
    row), NULLs, alignment, overlap, a short workspace (the same size as
    lbv_moe_forward's)."""
    L = raw()
    c = lbv.config()
    W = lbv._Fp8WeightsC(A, B, A, B, A, B, A, B)
    need = lbv.lbv_moe_workspace_size(c, 16)

    def f(T, out=Cc, ws=BIG, ws_bytes=need, cfg=c, w=W):
        return L.lbv_moe_forward_w8a8(ctypes.byref(cfg), T, A, None, A, B,
                                      ctypes.byref(w) if w is not None else None, out, None, None,
                                      ws, ws_bytes, None)
    assert f(16, cfg=lbv.config(dtype="f32")) == lbv.LBV_ERR_UNSUPPORTED
    assert f(16, cfg=lbv.config(hidden=2112)) == lbv.LBV_ERR_SHAPE
    assert f(16, cfg=lbv.config(intermediate=704)) == lbv.LBV_ERR_SHAPE
    assert f(16, cfg=lbv.config(intermediate=1152)) == lbv.LBV_ERR_SHAPE
    assert f(16, cfg=lbv.config(intermediate=64)) == lbv.LBV_ERR_SHAPE
    assert f(0, cfg=lbv.config(intermediate=64)) == lbv.LBV_ERR_SHAPE    # shape first
    assert f(0) == lbv.LBV_OK
    assert f(16, w=None) == lbv.LBV_ERR_NULL
    assert f(16, w=lbv._Fp8WeightsC(A, None, A, B, A, B, A, B)) == lbv.LBV_ERR_NULL
    assert f(16, w=lbv._Fp8WeightsC(A, B, A, B, A, B, A, None)) == lbv.LBV_ERR_NULL  # shared expert
    assert f(16, w=lbv._Fp8WeightsC(A, B, A + 8, B, A, B, A, B)) == lbv.LBV_ERR_ALIGN
    assert f(16, w=lbv._Fp8WeightsC(A, B, A, B + 2, A, B, A, B)) == lbv.LBV_ERR_ALIGN
    assert f(16, out=A) == lbv.LBV_ERR_ALIAS
    assert f(16, ws_bytes=need - 1) == lbv.LBV_ERR_WORKSPACE
    assert f(16, cfg=lbv.config(intermediate=1024), ws_bytes=lbv.lbv_moe_workspace_size(
        lbv.config(intermediate=1024), 16) - 1) == lbv.LBV_ERR_WORKSPACE   # I = 1024 is allowed


def test_fp8_binding_shape_checks():
    import torch
    w = torch.zeros(4, 64)
    with pytest.raises(ValueError, match="q has shape"):
        lbv.lbv_quantize_fp8_rows(w, torch.zeros(4, 32, dtype=torch.uint8), torch.zeros(4))
    with pytest.raises(ValueError, match="scale has shape"):
        lbv.lbv_quantize_fp8_rows(w, torch.zeros(4, 64, dtype=torch.uint8), torch.zeros(5))
    with pytest.raises(ValueError, match="bfloat16 or float32"):
        lbv.lbv_quantize_fp8_rows(w.half(), torch.zeros(4, 64, dtype=torch.uint8), torch.zeros(4))
    with pytest.raises(ValueError, match="device tensor"):
        lbv.lbv_quantize_fp8_rows(w, torch.zeros(4, 64, dtype=torch.uint8), torch.zeros(4))


def test_attention_validation_paths():
    """The attention entries reject before any launch."""
    L = raw()
    c = lbv.attn_config()
    need = lbv.lbv_attn_workspace_size(c, 2, 800)
    T, H = 1600, 2048
    # 512 bytes, qkv, q, k, o, and vt with S rounded up to 832 key positions
    assert need == 512 + T * 3 * H * 2 + 3 * T * H * 2 + 2 * H * 832 * 2
    bad = lbv.AttnConfig(2048, 8, 1e-6)                      # head dim 256
    n = ctypes.c_size_t()
    assert L.lbv_attn_workspace_size(ctypes.byref(bad), 1, 8, ctypes.byref(n)) == \
        lbv.LBV_ERR_UNSUPPORTED
    assert L.lbv_attn_workspace_size(ctypes.byref(c), 1, 65537, ctypes.byref(n)) == \
        lbv.LBV_ERR_SHAPE
    neg = lbv.AttnConfig(2048, 16, -1.0)
    assert L.lbv_attn_workspace_size(ctypes.byref(neg), 1, 8, ctypes.byref(n)) == \
        lbv.LBV_ERR_SHAPE

    def f(B=2, S=800, x=A, out=Cc, ws=BIG, ws_bytes=need, cfg=c):
        return L.lbv_attn_forward(ctypes.byref(cfg), B, S, x, None, B_, None, A, A, A, A, B_, None,
                                  out, ws, ws_bytes, None)
    B_ = B
    assert f(B=0) == lbv.LBV_OK
    assert f(x=None) == lbv.LBV_ERR_NULL
    assert f(out=Cc + 8) == lbv.LBV_ERR_ALIGN
    assert f(ws_bytes=need - 1) == lbv.LBV_ERR_WORKSPACE
    assert f(out=A + 64) == lbv.LBV_ERR_ALIAS
    assert L.lbv_linear_bf16(8, 100, 64, A, B, None, Cc, BIG, 512, None) == lbv.LBV_ERR_SHAPE
    assert L.lbv_linear_bf16(8, 128, 64, A, B, None, Cc, BIG, 511, None) == lbv.LBV_ERR_WORKSPACE
    assert L.lbv_linear_bf16(0, 128, 64, None, None, None, None, None, 0, None) == lbv.LBV_OK
    assert L.lbv_linear_bf16(8, 128, 64, A, B, None, A + 16, BIG, 512, None) == lbv.LBV_ERR_ALIAS
    assert L.lbv_attn_core(ctypes.byref(c), 1, 8, A, B, None, None, Cc, None) == lbv.LBV_ERR_NULL
    assert L.lbv_attn_qk_prep(ctypes.byref(c), 1, 8, A, A, A, A, A, B, Cc, BIG + 8, None) == \
        lbv.LBV_ERR_ALIGN


def test_attention_half_adaln_validation_paths():
    L = raw()
    c = lbv.attn_config()
    T, H = 1600, 2048
    need = lbv.lbv_attn_half_adaln_workspace_size(c, 2, 800)
    assert need == lbv.lbv_attn_workspace_size(c, 2, 800) + 2 * T * H * 2

    def f(x=A, out=Cc, temb_stride=6 * H, eps=1e-6, ws_bytes=need, B_=2):
        return L.lbv_attn_half_adaln(ctypes.byref(c), B_, 800, x, None, B, temb_stride, B, eps, B,
                                     None, A, A, A, A, B, None, out, BIG, ws_bytes, None)
    assert f(B_=0) == lbv.LBV_OK
    assert f(x=None) == lbv.LBV_ERR_NULL
    assert f(temb_stride=6 * H + 2) == lbv.LBV_ERR_ALIGN
    assert f(eps=-1.0) == lbv.LBV_ERR_SHAPE
    assert f(ws_bytes=need - 1) == lbv.LBV_ERR_WORKSPACE
    assert f(out=A + 4096) == lbv.LBV_ERR_ALIAS        # overlaps x without being x
