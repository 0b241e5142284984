"""Parity of the attention half (projections, q/k head norms + rotary
embedding, masked per-sample attention) with the CPU oracle, through the C ABI.

Bars:
* projections: every element within one bf16 rounding of the fp64 product
  (|err| <= 2^-8 |ref| + 1e-3 max|ref|, fp32 accumulation over K terms);
* q / k prep: the oracle rounds twice (norm output, rotation output) like the
  GPU; fp32 evaluation may move a value to the neighbouring bf16 number, so
  every element is within 2 ulps of itself plus 2 ulps of its pair's larger
  norm output (a flipped norm output under cancellation), and at most 1e-3
  of them differ at all;
  vt is pure data movement and must match exactly;
* attention and the whole half: relative Frobenius error 5e-3 and max-abs
  3e-2 of the bf16 outputs (bf16 P in the PV product, fp32 accumulation)
  before their final bf16 rounding, so an element may differ by one more
  bf16 ulp of its magnitude; every token (full size: sampled query rows, all
  keys).  The residual updates of the attention half with its modulation are
  fp32 and held to 3e-2 with no such allowance.
"""
import numpy as np
import pytest
import torch

import oracle
import routed_moe_dit_amd as lbv
import synth
from gpu_util import dev, host, metrics, note

pytestmark = pytest.mark.gpu
TOL = dict(rel_frob=5e-3, max_abs=3e-2)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    lbv.load()
    yield


def u8(a):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a, np.uint8)).cuda()


def f32(a):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()


def bf16(a):
    return dev(np.ascontiguousarray(a, np.float32), "bf16")


def check(got, want, name, rounded=True):
    """rounded: got and want are bf16 roundings of values that the bar holds
    within TOL["max_abs"] of each other; each rounding moves a value by at
    most half a bf16 ulp, so an element may differ by one ulp of its
    magnitude beyond that (one ulp is 2^-5 from |o| = 4 on, above 3e-2)."""
    m = metrics(got, want)
    d = np.abs(np.asarray(got, np.float64) - want)
    if rounded and d.size:
        m["max_abs_beyond_ulp"] = float(
            np.maximum(d - ulp_bf16(np.maximum(np.abs(got), np.abs(want))), 0).max())
    print("%s: %s" % (name, m))
    assert m["finite"]
    assert m["rel_frob"] <= TOL["rel_frob"], m
    assert m.get("max_abs_beyond_ulp", m["max_abs"]) <= TOL["max_abs"], m
    return m


# ---- dense projection -------------------------------------------------------------

@pytest.mark.parametrize("T,N,K,bias", [(1, 128, 64, True), (77, 192, 256, False),
                                        (300, 2048, 2048, True), (3000, 6144, 2048, True),
                                        (38000, 2048, 2048, False)])
def test_linear_parity(T, N, K, bias):
    note("linear T=%d N=%d K=%d bias=%s" % (T, N, K, bias))
    r = np.random.default_rng(T + N)
    x = synth.round_to_bf16(r.standard_normal((T, K), dtype=np.float32))
    w = synth.round_to_bf16((r.standard_normal((N, K)) * K ** -0.5).astype(np.float32))
    b = (r.standard_normal(N) * 0.1).astype(np.float32) if bias else None
    y = torch.zeros(T, N, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(lbv.LINEAR_WS_BYTES, dtype=torch.uint8, device="cuda")
    lbv.lbv_linear_bf16(bf16(x), bf16(w), f32(b), y, ws)
    torch.cuda.synchronize()
    rows = np.arange(T) if T <= 3000 else np.unique(np.r_[0:256, T - 256:T,
                                                         r.integers(0, T, 2000)])
    ref = oracle.linear(x[rows], w, b)
    got = host(y)[rows]
    bad = np.abs(got - ref) > 2.0 ** -8 * np.abs(ref) + 1e-3 * np.abs(ref).max()
    print("linear T=%d N=%d K=%d: %d rows checked, %s" % (T, N, K, len(rows), metrics(got, ref)))
    assert not bad.any(), np.argwhere(bad)[:5]


# ---- q / k prep --------------------------------------------------------------------

def ulp_bf16(a):
    """Distance from |a| to the next bf16 number above it (2^-126 floor)."""
    e = np.floor(np.log2(np.maximum(np.abs(a), 2.0 ** -126)))
    return 2.0 ** (e - 7)


@pytest.mark.parametrize("B,S,heads", [(1, 64, 2), (2, 300, 2), (1, 129, 16), (2, 800, 16)])
def test_qk_prep_parity(B, S, heads):
    note("attn prep B=%d S=%d heads=%d" % (B, S, heads))
    H, D = heads * 128, 128
    T = B * S
    r = np.random.default_rng(S + heads)
    qkv = synth.round_to_bf16((r.standard_normal((T, 3 * H)) * 0.7).astype(np.float32))
    g_q = (1 + 0.1 * r.standard_normal(D)).astype(np.float32)
    g_k = (1 + 0.1 * r.standard_normal(D)).astype(np.float32)
    ang = r.uniform(-30, 30, (T, D // 2))
    cos, sin = np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)
    cfg = lbv.attn_config(hidden=H, num_heads=heads, eps=1e-6)
    q = torch.zeros(T, H, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(T, H, dtype=torch.bfloat16, device="cuda")
    Sp = lbv.attn_sp(S)
    vt = torch.full((B, heads, D, Sp), 7.0, dtype=torch.bfloat16, device="cuda")
    lbv.lbv_attn_qk_prep(cfg, B, S, bf16(qkv), f32(g_q), f32(g_k), f32(cos), f32(sin), q, k, vt)
    torch.cuda.synchronize()
    blocks = qkv.reshape(T, 3, heads, D)
    for name, got, blk, g in (("q", q, 0, g_q), ("k", k, 1, g_k)):
        n = oracle.bf16_round(oracle.head_rmsnorm(blocks[:, blk], g, 1e-6))
        want = oracle.bf16_round(oracle.rope(n, cos, sin)).reshape(T, H)
        # a norm output on the other side of a rounding boundary moves the
        # rotated pair by up to an ulp of the pair's larger member, which can
        # be many ulps of a rotated value near zero (cancellation)
        pair = np.maximum(np.abs(n[..., 0::2]), np.abs(n[..., 1::2])).repeat(2, -1).reshape(T, H)
        gv = host(got)
        diff = np.abs(gv - want)
        frac = (diff > 0).mean()
        print("prep %s: %.2e of elements differ, max %.1f ulp" % (
            name, frac, (diff / ulp_bf16(want)).max()))
        assert (diff <= 2 * ulp_bf16(want) + 2 * ulp_bf16(pair)).all()
        assert frac <= 1e-3
    # vt: v transposed per head, positions with bits 2 and 3 of the key swapped,
    # zeros past S
    v = blocks[:, 2].reshape(B, S, heads, D)
    p = np.arange(Sp)
    key = (p & ~12) | ((p & 4) << 1) | ((p & 8) >> 1)
    want = np.zeros((B, heads, D, Sp), np.float32)
    ok = key < S
    want[..., ok] = v[:, key[ok]].transpose(0, 2, 3, 1)
    assert np.array_equal(host(vt), want)


# ---- attention core ----------------------------------------------------------------

def vt_of(v, B, S, heads):
    """Host layout of vt for a given v [B S, heads, D] (test input preparation)."""
    D = v.shape[-1]
    Sp = lbv.attn_sp(S)
    p = np.arange(Sp)
    key = (p & ~12) | ((p & 4) << 1) | ((p & 8) >> 1)
    out = np.zeros((B, heads, D, Sp), np.float32)
    ok = key < S
    out[..., ok] = v.reshape(B, S, heads, D)[:, key[ok]].transpose(0, 2, 3, 1)
    return out


CORE_CASES = [
    # (B, S, heads, mask kind, q/k scale)
    (1, 1, 2, None, 1.0),
    (1, 63, 2, None, 2.0),
    (1, 64, 2, None, 2.0),
    (2, 65, 2, "tail", 2.0),
    (2, 300, 2, "random", 3.0),
    (1, 257, 16, None, 1.0),
    (2, 800, 16, "tail", 2.0),
    (1, 4000, 2, "random", 2.0),
    (2, 130, 2, "one_key", 2.0),
    (2, 96, 2, "empty_sample", 2.0),
]


def core_mask(kind, B, S, r):
    if kind is None:
        return None
    m = np.ones(B * S, np.uint8)
    if kind == "tail":
        m[B * S - S // 10 - 1:] = 0
    elif kind == "random":
        m[r.random(B * S) < 0.2] = 0
    elif kind == "one_key":
        m[:S] = 0
        m[S // 2] = 1
    elif kind == "empty_sample":
        m[S:] = 0
    return m


@pytest.mark.parametrize("B,S,heads,kind,scale", CORE_CASES,
                         ids=lambda v: str(v))
def test_attention_core_parity(B, S, heads, kind, scale):
    note("attn core B=%d S=%d heads=%d mask=%s" % (B, S, heads, kind))
    D = 128
    H, T = heads * D, B * S
    r = np.random.default_rng(B * 1000 + S + heads)
    q, k, v = (synth.round_to_bf16((r.standard_normal((T, heads, D)) * s).astype(np.float32))
               for s in (scale, scale, 1.0))
    mask = core_mask(kind, B, S, r)
    cfg = lbv.attn_config(hidden=H, num_heads=heads)
    o = torch.full((T, H), 3.0, dtype=torch.bfloat16, device="cuda")
    lbv.lbv_attn_core(cfg, B, S, bf16(q.reshape(T, H)), bf16(k.reshape(T, H)),
                      bf16(vt_of(v, B, S, heads)), u8(mask), o)
    torch.cuda.synchronize()
    want = oracle.bf16_round(oracle.attention(q, k, v, S, mask)).reshape(T, H)
    got = host(o)
    check(got, want, "attn core B=%d S=%d heads=%d mask=%s" % (B, S, heads, kind))
    if mask is not None:
        assert (got[mask == 0] == 0).all()


# ---- the whole attention half --------------------------------------------------------

def small_attn(name, B, S, heads, valid, seed):
    return synth.AttnWorkload(name, B=B, S=S, grid=(2, 3, 5), text=7, valid=valid,
                              hidden=heads * 128, heads=heads, seed=seed)


FWD_CASES = [
    small_attn("a_B1_S40", 1, 40, 2, (40,), 31),
    small_attn("a_B2_S100_pad", 2, 100, 2, (100, 61), 32),
    synth.ATTN_WORKLOADS[0],
    synth.ATTN_WORKLOADS[1],
]


def run_forward(aw, inp):
    cfg = lbv.attn_config(hidden=aw.hidden, num_heads=aw.heads, eps=1e-6)
    T, H = aw.T, aw.hidden
    out = torch.zeros(T, H, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(lbv.lbv_attn_workspace_size(cfg, aw.B, aw.S), dtype=torch.uint8,
                     device="cuda")
    lbv.lbv_attn_forward(cfg, aw.B, aw.S, bf16(inp["x"]), u8(inp["mask"]), bf16(inp["w_qkv"]),
                         f32(inp["b_qkv"]), f32(inp["g_q"]), f32(inp["g_k"]), f32(inp["cos"]),
                         f32(inp["sin"]), bf16(inp["w_o"]), f32(inp["b_o"]), out, ws)
    torch.cuda.synchronize()
    return host(out)


def oracle_forward(aw, inp, rows=None):
    return oracle.attn_forward(inp["x"], inp["w_qkv"], inp["b_qkv"], inp["g_q"], inp["g_k"], 1e-6,
                               inp["cos"], inp["sin"], aw.heads, aw.S, inp["mask"], inp["w_o"],
                               inp["b_o"], qrows=rows)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("aw", FWD_CASES, ids=lambda a: a.name)
def test_attn_forward_parity(aw):
    note("attn forward %s" % aw.name)
    inp = synth.make_attn_inputs(aw)
    got = run_forward(aw, inp)
    check(got, oracle_forward(aw, inp), "attn forward %s (every token)" % aw.name)


@pytest.mark.timeout(900)
def test_attn_forward_parity_full_size():
    """2 x 19,000 tokens: every output element of 300 query rows (both
    samples' first and last rows, tile edges, random rows) against the oracle
    with all keys."""
    aw = synth.ATTN_WORKLOADS[2]
    note("attn forward full %s" % aw.name)
    inp = synth.make_attn_inputs(aw)
    got = run_forward(aw, inp)
    r = np.random.default_rng(0)
    S = aw.S
    rows = np.unique(np.r_[0, 1, 255, 256, S - 1, S, S + 255, 2 * S - 1,
                           r.integers(0, aw.T, 292)])
    check(got[rows], oracle_forward(aw, inp, rows), "attn forward full (%d rows)" % len(rows))


def test_attn_samples_isolated_bitwise():
    """Sample 1 of a B = 2 batch gives bitwise the output of sample 1 alone."""
    aw = synth.ATTN_WORKLOADS[1]
    note("attn isolation %s" % aw.name)
    inp = synth.make_attn_inputs(aw)
    got = run_forward(aw, inp)
    one = synth.AttnWorkload("one", B=1, S=aw.S, grid=aw.grid, text=aw.text, valid=aw.valid[1:],
                             hidden=aw.hidden, heads=aw.heads, seed=aw.seed)
    sl = slice(aw.S, 2 * aw.S)
    inp1 = dict(inp)
    for kname in ("x", "cos", "sin"):
        inp1[kname] = np.ascontiguousarray(inp[kname][sl])
    inp1["mask"] = np.ascontiguousarray(inp["mask"][sl])
    got1 = run_forward(one, inp1)
    assert np.array_equal(got[sl], got1)


def test_attn_forward_in_hip_graph_replays_bitwise():
    """lbv_attn_forward only enqueues kernels on the caller's stream (its
    set-up is a kernel, not a memset), so it can be captured in a HIP graph:
    each replay, with a changed input and eager work in between, equals the
    eager call bitwise."""
    aw = synth.ATTN_WORKLOADS[1]
    note("attn graph capture %s" % aw.name)
    inp = synth.make_attn_inputs(aw)
    cfg = lbv.attn_config(hidden=aw.hidden, num_heads=aw.heads, eps=1e-6)
    T, H = aw.T, aw.hidden
    x0 = bf16(inp["x"])
    x = x0.clone()
    dd = {k: f32(inp[k]) for k in ("b_qkv", "g_q", "g_k", "cos", "sin", "b_o")}
    w_qkv, w_o, mask = bf16(inp["w_qkv"]), bf16(inp["w_o"]), u8(inp["mask"])
    out = torch.empty(T, H, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(lbv.lbv_attn_workspace_size(cfg, aw.B, aw.S), dtype=torch.uint8,
                     device="cuda")

    def call():
        lbv.lbv_attn_forward(cfg, aw.B, aw.S, x, mask, w_qkv, dd["b_qkv"], dd["g_q"], dd["g_k"],
                             dd["cos"], dd["sin"], w_o, dd["b_o"], out, ws,
                             torch.cuda.current_stream())

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    gen = torch.Generator(device="cpu").manual_seed(7)
    for rep in range(3):
        if rep:
            x.copy_(x0[torch.randperm(T, generator=gen).cuda()])
        torch.cuda.synchronize()
        call()
        torch.cuda.synchronize()
        ref = out.clone()
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), rep



# ---- the attention half with its AdaLN and gated residual ----------------------------

def run_half_adaln(aw, inp, ada, temb_shared=False):
    cfg = lbv.attn_config(hidden=aw.hidden, num_heads=aw.heads, eps=1e-6)
    T, H = aw.T, aw.hidden
    out = torch.zeros(T, H, dtype=torch.float32, device="cuda")
    ws = torch.empty(lbv.lbv_attn_half_adaln_workspace_size(cfg, aw.B, aw.S), dtype=torch.uint8,
                     device="cuda")
    temb = f32(ada["temb6"][0] if temb_shared else ada["temb6"])
    lbv.lbv_attn_half_adaln(cfg, aw.B, aw.S, f32(ada["x"]), u8(inp["mask"]), temb,
                            f32(ada["table"]), 1e-6, bf16(inp["w_qkv"]), f32(inp["b_qkv"]),
                            f32(inp["g_q"]), f32(inp["g_k"]), f32(inp["cos"]), f32(inp["sin"]),
                            bf16(inp["w_o"]), f32(inp["b_o"]), out, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def oracle_half_adaln(aw, inp, ada, rows=None, temb6=None):
    return oracle.attn_half_adaln(ada["x"], ada["temb6"] if temb6 is None else temb6,
                                  ada["table"], 1e-6, inp["w_qkv"], inp["b_qkv"], inp["g_q"],
                                  inp["g_k"], 1e-6, inp["cos"], inp["sin"], aw.heads, aw.S,
                                  inp["mask"], inp["w_o"], inp["b_o"], qrows=rows)


def check_half(got, want, x, name):
    """The residual is fp32 (x + gate * block): compare the update
    gate * block, whose bf16 block carries the attention half's tolerance."""
    check(got - x, want - x, name, rounded=False)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("aw", FWD_CASES, ids=lambda a: a.name)
def test_attn_half_adaln_parity(aw):
    note("attn half + adaln %s" % aw.name)
    inp = synth.make_attn_inputs(aw)
    ada = synth.make_attn_adaln_inputs(aw)
    got = run_half_adaln(aw, inp, ada)
    x = ada["x"].astype(np.float64)
    check_half(got, oracle_half_adaln(aw, inp, ada), x, "attn half + adaln %s (every token)" % aw.name)


def test_attn_half_adaln_shared_temb_and_in_place():
    """A shared temb6 row (stride 0) and out == x."""
    aw = FWD_CASES[1]
    note("attn half + adaln shared temb, in place %s" % aw.name)
    inp = synth.make_attn_inputs(aw)
    ada = synth.make_attn_adaln_inputs(aw)
    cfg = lbv.attn_config(hidden=aw.hidden, num_heads=aw.heads, eps=1e-6)
    T, H = aw.T, aw.hidden
    xo = f32(ada["x"])
    ws = torch.empty(lbv.lbv_attn_half_adaln_workspace_size(cfg, aw.B, aw.S), dtype=torch.uint8,
                     device="cuda")
    lbv.lbv_attn_half_adaln(cfg, aw.B, aw.S, xo, u8(inp["mask"]), f32(ada["temb6"][0]),
                            f32(ada["table"]), 1e-6, bf16(inp["w_qkv"]), f32(inp["b_qkv"]),
                            f32(inp["g_q"]), f32(inp["g_k"]), f32(inp["cos"]), f32(inp["sin"]),
                            bf16(inp["w_o"]), f32(inp["b_o"]), xo, ws)
    torch.cuda.synchronize()
    shared = np.broadcast_to(ada["temb6"][0], ada["temb6"].shape).copy()
    want = oracle_half_adaln(aw, inp, ada, temb6=shared)
    x = ada["x"].astype(np.float64)
    check_half(xo.cpu().numpy().astype(np.float64), want, x, "attn half + adaln shared/in place")


@pytest.mark.timeout(900)
def test_attn_half_adaln_parity_full_size():
    aw = synth.ATTN_WORKLOADS[2]
    note("attn half + adaln full %s" % aw.name)
    inp = synth.make_attn_inputs(aw)
    ada = synth.make_attn_adaln_inputs(aw)
    got = run_half_adaln(aw, inp, ada)
    r = np.random.default_rng(1)
    rows = np.unique(np.r_[0, aw.S - 1, aw.S, aw.T - 1, r.integers(0, aw.T, 196)])
    x = ada["x"].astype(np.float64)[rows]
    check_half(got[rows], oracle_half_adaln(aw, inp, ada, rows), x,
               "attn half + adaln full (%d rows)" % len(rows))
