"""Seeded sweep of random small configurations through the C ABI, each against
the CPU oracle on every token: the bf16 and fp32 block (experts, groups,
top-k, shared experts, widths, token counts, padding), the block with fp8
weights, the block with fp8 weights and activations, and the attention
kernel (samples, lengths, heads, masks).  Bars as
in the per-step parity tests."""
import numpy as np
import pytest
import torch

import oracle
import routed_moe_dit_amd as lbv
import synth
from gpu_util import forward, note, upload
from test_gpu_attention import bf16, check, u8, vt_of
from test_gpu_fp8 import forward_fp8, oracle_dequantized
from test_gpu_parity import check_forward
from test_gpu_w8a8 import check_w8a8, forward_w8a8

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    lbv.load()
    yield


def random_block(i):
    """A random configuration inside what the library supports."""
    r = np.random.default_rng(1000 + i)
    E = int(r.choice([16, 32, 64, 128, 256]))
    epl = 1
    while 64 * epl < E:
        epl *= 2
    groups = [g for g in (1, 2, 4, 8) if E % g == 0 and (E // g) % epl == 0 and
              ((E // g) // epl) & ((E // g) // epl - 1) == 0 and E // g >= 2]
    n_group = int(r.choice(groups))
    topk_group = int(r.integers(1, n_group + 1))
    K = int(r.integers(1, min(16, topk_group * (E // n_group)) + 1))
    H = int(r.choice([64, 128, 256, 512, 1024]))
    I = int(r.choice([64, 128, 192, 256]))
    T = int(r.choice([1, 7, 64, 65, 300, 1000]))
    ns = int(r.integers(0, 3))
    dtype = "f32" if r.random() < 0.2 else "bf16"
    samples = None
    if T >= 64 and r.random() < 0.4:
        half = T // 2
        samples = ((half, half - int(r.integers(0, half // 2 + 1))),
                   (T - half, T - half - int(r.integers(0, (T - half) // 2 + 1))))
    return synth.Workload(
        "rand%02d_E%d_g%d_%d_K%d_H%d_I%d_T%d_ns%d_%s" % (i, E, n_group, topk_group, K, H, I, T, ns,
                                                        dtype),
        T=T, hidden=H, num_experts=E, n_group=n_group, topk_group=topk_group, top_k=K,
        intermediate=I, n_shared=ns, dtype=dtype, seed=2000 + i, wr_std=H ** -0.5,
        b_std=float(r.choice([0.1, 0.5])), norm_topk_prob=bool(r.random() < 0.8),
        samples=samples)


BLOCKS = [random_block(i) for i in range(24)]


@pytest.mark.parametrize("wl", BLOCKS, ids=lambda w: w.name)
def test_random_block_parity(wl):
    note("sweep forward %s" % wl.name)
    inp = synth.make_inputs(wl)
    d = upload(wl, inp)
    out, ids, w = forward(wl, d)
    check_forward(wl, inp, out, ids, w)


@pytest.mark.parametrize("wl", [w for w in BLOCKS if w.dtype == "bf16"][:8], ids=lambda w: w.name)
def test_random_block_fp8_parity(wl):
    note("sweep fp8 forward %s" % wl.name)
    inp = synth.make_inputs(wl)
    d = upload(wl, inp)
    out, ids, w = forward_fp8(wl, d)
    check_forward(wl, oracle_dequantized(inp), out, ids, w)


A8_BLOCKS = [w for w in BLOCKS if w.dtype == "bf16" and w.hidden % 128 == 0 and
             w.intermediate % 128 == 0]


@pytest.mark.parametrize("wl", A8_BLOCKS, ids=lambda w: w.name)
def test_random_block_w8a8_parity(wl):
    note("sweep w8a8 forward %s" % wl.name)
    inp = synth.make_inputs(wl)
    d = upload(wl, inp)
    out, ids, w = forward_w8a8(wl, d)
    check_w8a8(wl, inp, oracle_dequantized(inp), out, ids, w)


def random_attn(i):
    r = np.random.default_rng(3000 + i)
    B = int(r.integers(1, 4))
    S = int(r.choice([1, 2, 17, 63, 64, 65, 127, 128, 129, 255, 256, 257, 511, 700]))
    heads = int(r.integers(1, 5))
    kind = r.choice(["none", "random", "tail"])
    scale = float(r.choice([0.5, 1.0, 2.0, 3.0]))
    return B, S, heads, str(kind), scale, 4000 + i


ATTN = [random_attn(i) for i in range(12)]


@pytest.mark.parametrize("B,S,heads,kind,scale,seed", ATTN, ids=lambda v: str(v))
def test_random_attention_core_parity(B, S, heads, kind, scale, seed):
    note("sweep attention B=%d S=%d heads=%d mask=%s" % (B, S, heads, kind))
    D = 128
    H, T = heads * D, B * S
    r = np.random.default_rng(seed)
    q, k, v = (synth.round_to_bf16((r.standard_normal((T, heads, D)) * s).astype(np.float32))
               for s in (scale, scale, 1.0))
    mask = None
    if kind == "random":
        mask = (r.random(T) > 0.3).astype(np.uint8)
    elif kind == "tail":
        mask = np.ones(T, np.uint8)
        for b in range(B):
            mask[b * S + S - int(r.integers(0, S // 3 + 1)):(b + 1) * S] = 0
    cfg = lbv.attn_config(hidden=H, num_heads=heads)
    o = torch.full((T, H), 3.0, dtype=torch.bfloat16, device="cuda")
    lbv.lbv_attn_core(cfg, B, S, bf16(q.reshape(T, H)), bf16(k.reshape(T, H)),
                      bf16(vt_of(v, B, S, heads)), u8(mask), o)
    torch.cuda.synchronize()
    want = oracle.bf16_round(oracle.attention(q, k, v, S, mask)).reshape(T, H)
    got = o.float().cpu().numpy().astype(np.float64)
    check(got, want, "sweep attention B=%d S=%d heads=%d mask=%s" % (B, S, heads, kind))
    if mask is not None:
        assert (got[mask == 0] == 0).all()
