"""Seeded synthetic inputs for the routed-MoE feed-forward block.

This module is shared by the tests, the benchmark and the smoke check, and by
both sides of every parity check (the HIP library and the CPU oracle).  It
holds none of the block's arithmetic: it only draws random tensors with the
shapes, value distributions and padding structure of the LingBot-Video video
workloads and rounds the bf16 ones to bf16 storage.

Draw order per workload (one ``numpy.random.default_rng(seed)`` stream):
x, router weight, correction bias, w13, w2, shared w13, shared w2.  Every draw
is ``standard_normal`` in float32 scaled by the tensor's standard deviation.

Shapes (sources: prhub summary of sglang PR #32341, "实现拆解" steps 1 and 3,
and the vLLM-Omni LingBot-Video article, "参数背后的源码级约束"):

* 128 routed experts in 4 groups, 2 groups kept, top-8, expert width 768,
  one shared expert, routed scaling 2.5;
* hidden size 2048, implied by the packed w13 of shape [128, 1536, 2048]
  (768 MiB in bf16) named in the review discussion of the same PR summary;
* token counts from the VAE factors (4 in time, 8 in space) and a 2x2 patch
  (the patch size is an assumption, not on the pages): 9 frames at 192x320 give
  720 video tokens, 81 frames at 480x480 give 18,900; text follows video inside
  a sample and padding sits at the end of a sample; classifier-free guidance
  batches the positive and negative prompt as B=2.
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Optional, Tuple

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "by_name", "make_inputs", "round_to_bf16",
    "bf16_bits", "bits_to_f32", "digest", "token_mask", "random_act", "make_adaln_inputs",
    "AttnWorkload", "ATTN_WORKLOADS", "attn_by_name", "make_attn_inputs", "joint_positions",
    "rope_tables", "make_attn_adaln_inputs",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic layer configuration and its input recipe."""

    name: str
    T: int                      # tokens (batch x sequence, padding included)
    hidden: int                 # H
    num_experts: int            # E
    n_group: int
    topk_group: int
    top_k: int                  # K
    intermediate: int           # I (per routed expert; the shared expert is I * n_shared wide)
    n_shared: int
    dtype: str                  # "f32" or "bf16": storage of x, expert weights and out
    seed: int
    wr_std: float               # router weight std (fp32)
    b_std: float                # e_score_correction_bias std (fp32)
    w_std: float = 0.02         # expert weight std
    x_std: float = 1.0
    routed_scaling_factor: float = 2.5
    norm_topk_prob: bool = True
    # Padded batch: per-sample (sequence length, valid length).  Valid tokens
    # come first inside each sample, padding last.  None = every token valid.
    samples: Optional[Tuple[Tuple[int, int], ...]] = None
    # Hot experts: x[:, 0] is set to 1 and the router weight column 0 to
    # hot_shift on these experts and 0 elsewhere, so their logits rise by
    # exactly hot_shift.
    hot: Optional[Tuple[int, ...]] = None
    hot_shift: float = 2.0

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    @property
    def intermediate_shared(self) -> int:
        return self.intermediate * self.n_shared


_HOT8 = (0, 1, 2, 3, 32, 33, 34, 35)   # 8 experts spread over 2 of the 4 groups
# With the correction bias of std 0.5, the +2.0 logit shift on _HOT8 puts only
# ~26% of assignments on them: the bias is a fixed per-expert offset, and only
# two of them have a bias high enough to win once their sigmoid saturates.
# This set holds, for seed 4 at 38,000 tokens (the bias is drawn after x, so
# its values depend on the token count), the four experts of largest bias in
# each of groups 0 and 1; the same +2.0 shift then puts ~50% on them.
_HOT8_HALF = (7, 18, 28, 31, 33, 34, 38, 39)

WORKLOADS = (
    Workload("tiny_fp32_T64", T=64, hidden=256, num_experts=16, n_group=4, topk_group=2,
             top_k=4, intermediate=128, n_shared=1, dtype="f32", seed=0,
             wr_std=256 ** -0.5, b_std=0.1),
    Workload("smoke_T800", T=800, hidden=2048, num_experts=128, n_group=4, topk_group=2,
             top_k=8, intermediate=768, n_shared=1, dtype="bf16", seed=1,
             wr_std=2048 ** -0.5, b_std=0.1),
    Workload("cfg_B2_T1600_padded", T=1600, hidden=2048, num_experts=128, n_group=4,
             topk_group=2, top_k=8, intermediate=768, n_shared=1, dtype="bf16", seed=2,
             wr_std=2048 ** -0.5, b_std=0.1, samples=((800, 800), (800, 760))),
    Workload("default_gen_T38000", T=38000, hidden=2048, num_experts=128, n_group=4,
             topk_group=2, top_k=8, intermediate=768, n_shared=1, dtype="bf16", seed=3,
             wr_std=2048 ** -0.5, b_std=0.1),
    Workload("hot_expert_T38000", T=38000, hidden=2048, num_experts=128, n_group=4,
             topk_group=2, top_k=8, intermediate=768, n_shared=1, dtype="bf16", seed=4,
             wr_std=2048 ** -0.5, b_std=0.5, hot=_HOT8, hot_shift=2.0),
    Workload("hot_expert_half_T38000", T=38000, hidden=2048, num_experts=128, n_group=4,
             topk_group=2, top_k=8, intermediate=768, n_shared=1, dtype="bf16", seed=4,
             wr_std=2048 ** -0.5, b_std=0.5, hot=_HOT8_HALF, hot_shift=2.0),
)


def by_name(name: str) -> Workload:
    for w in WORKLOADS:
        if w.name == name:
            return w
    raise KeyError(name)


# ---------------------------------------------------------------------------
# bf16 storage helpers (round-to-nearest-even on the float32 bit pattern)
# ---------------------------------------------------------------------------

def round_to_bf16(a: np.ndarray, chunk: int = 1 << 24) -> np.ndarray:
    """Round a finite float32 array to the nearest bf16 value, ties to even,
    in place; returns the same array (its values are now bf16-exact)."""
    assert a.dtype == np.float32 and a.flags.c_contiguous
    u = a.reshape(-1).view(np.uint32)
    for s in range(0, u.size, chunk):
        v = u[s:s + chunk]
        r = (v >> np.uint32(16)) & np.uint32(1)
        r += np.uint32(0x7FFF)
        v += r
        v &= np.uint32(0xFFFF0000)
    return a


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """uint16 bf16 bit patterns of a bf16-exact float32 array."""
    assert a.dtype == np.float32
    u = np.ascontiguousarray(a).view(np.uint32)
    if np.any(u & np.uint32(0xFFFF)):
        raise ValueError("array is not bf16-exact")
    return (u >> np.uint32(16)).astype(np.uint16)


def bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen uint16 bf16 bit patterns to float32 exactly."""
    assert b.dtype == np.uint16
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def token_mask(wl: Workload) -> Optional[np.ndarray]:
    """u8 [T] validity mask (1 = real token, 0 = padding) or None."""
    if wl.samples is None:
        return None
    parts = []
    for seq, valid in wl.samples:
        m = np.zeros(seq, np.uint8)
        m[:valid] = 1
        parts.append(m)
    mask = np.concatenate(parts)
    assert mask.size == wl.T
    return mask


def _draw(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    a = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def make_inputs(wl: Workload, T: Optional[int] = None) -> dict:
    """Draw the workload's tensors.

    Returns float32 arrays (bf16-exact where ``wl.dtype == "bf16"`` for x and
    the expert weights; the router weight and bias are always fp32):
    ``x [T,H]``, ``router_w [E,H]``, ``e_bias [E]``, ``w13 [E,2I,H]``,
    ``w2 [E,H,I]``, ``shared_w13 [2*I*ns,H]``, ``shared_w2 [H,I*ns]`` (both
    None when ns == 0) and ``mask`` (u8 [T] or None).  ``T`` overrides the
    token count (the first T rows of the same recipe are not guaranteed; the
    draw simply uses the smaller shape).
    """
    T = wl.T if T is None else T
    H, E, I, ns = wl.hidden, wl.num_experts, wl.intermediate, wl.n_shared
    rng = np.random.default_rng(wl.seed)
    bf = wl.dtype == "bf16"

    x = _draw(rng, (T, H), wl.x_std)
    router_w = _draw(rng, (E, H), wl.wr_std)
    e_bias = _draw(rng, (E,), wl.b_std)
    w13 = _draw(rng, (E, 2 * I, H), wl.w_std)
    w2 = _draw(rng, (E, H, I), wl.w_std)
    shared_w13 = _draw(rng, (2 * I * ns, H), wl.w_std) if ns > 0 else None
    shared_w2 = _draw(rng, (H, I * ns), wl.w_std) if ns > 0 else None

    if wl.hot is not None:
        x[:, 0] = 1.0
        router_w[:, 0] = 0.0
        router_w[list(wl.hot), 0] = np.float32(wl.hot_shift)

    if bf:
        for a in (x, w13, w2, shared_w13, shared_w2):
            if a is not None:
                round_to_bf16(a)

    mask = token_mask(wl) if T == wl.T else None
    return dict(x=x, router_w=router_w, e_bias=e_bias, w13=w13, w2=w2,
                shared_w13=shared_w13, shared_w2=shared_w2, mask=mask)


def random_act(n: int, width: int, seed: int, std: float = 0.5) -> np.ndarray:
    """A stand-in for gate/up activations (rows of the down projection's input):
    float32 [n, width], N(0, std^2), rounded to bf16 values."""
    a = _draw(np.random.default_rng(seed), (n, width), std)
    return round_to_bf16(a)


def make_adaln_inputs(wl: Workload, T: Optional[int] = None, per_token: bool = True,
                      x_std: float = 1.0, table_std: float = 0.1, temb_std: float = 0.1) -> dict:
    """Inputs of the DiT layer's FFN half around the block (a stream of its
    own, seed + 1000): the fp32 residual stream ``x [T, H]``, the modulation
    table ``table [6, H]`` and the time embedding ``temb6`` ([T, 6, H] when
    per_token, else [6, H]), all float32 N(0, std^2)."""
    T = wl.T if T is None else T
    H = wl.hidden
    rng = np.random.default_rng(wl.seed + 1000)
    x = _draw(rng, (T, H), x_std)
    table = _draw(rng, (6, H), table_std)
    temb6 = _draw(rng, (T, 6, H) if per_token else (6, H), temb_std)
    return dict(x=x, table=table, temb6=temb6)


def digest(inputs: dict) -> dict:
    """SHA-256 (first 16 hex digits) of each input tensor's bytes."""
    out = {}
    for k, v in inputs.items():
        if v is None:
            out[k] = None
        else:
            out[k] = hashlib.sha256(np.ascontiguousarray(v).tobytes()).hexdigest()[:16]
    return out


# ---------------------------------------------------------------------------
# The attention half of a DiT layer (prhub summary of sglang PR #32341,
# LingBotVideoAttention under "关键源码片段"; "实现拆解" step 2: video;text
# joint attention with 3D joint position ids, padding isolated by the mask).
# ---------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class AttnWorkload:
    """B samples of S tokens (padding included); each sample is a video part
    on a latent token grid (frames x rows x columns) followed by text tokens,
    with `valid[b]` real tokens and padding after them."""

    name: str
    B: int
    S: int
    grid: Tuple[int, int, int]
    text: int
    valid: Tuple[int, ...]
    hidden: int
    heads: int
    seed: int
    x_std: float = 1.0
    b_std: float = 0.02
    g_std: float = 0.1
    theta: float = 10000.0

    @property
    def T(self) -> int:
        return self.B * self.S

    @property
    def head_dim(self) -> int:
        return self.hidden // self.heads


ATTN_WORKLOADS = (
    # 9 frames at 192x320: a 3 x 12 x 20 grid (720 tokens) + 80 text tokens
    AttnWorkload("attn_smoke_T800", B=1, S=800, grid=(3, 12, 20), text=80, valid=(800,),
                 hidden=2048, heads=16, seed=21),
    # the classifier-free-guidance pair, 40 padding tokens at the end of sample 2
    AttnWorkload("attn_cfg_B2_T1600", B=2, S=800, grid=(3, 12, 20), text=80, valid=(800, 760),
                 hidden=2048, heads=16, seed=22),
    # 81 frames at 480x480: a 21 x 30 x 30 grid (18,900 tokens) + 100 text, B = 2
    AttnWorkload("attn_default_B2_T38000", B=2, S=19000, grid=(21, 30, 30), text=100,
                 valid=(19000, 19000), hidden=2048, heads=16, seed=23),
)


def attn_by_name(name: str) -> AttnWorkload:
    for w in ATTN_WORKLOADS:
        if w.name == name:
            return w
    raise KeyError(name)


def joint_positions(aw: AttnWorkload) -> np.ndarray:
    """int32 [T, 3] positions (frame, row, column) of every token: video tokens
    in raster order of their grid cell, text token j at (frames + j, 0, 0),
    padding at (0, 0, 0)."""
    F, R, C = aw.grid
    f, r, c = np.meshgrid(np.arange(F), np.arange(R), np.arange(C), indexing="ij")
    video = np.stack([f.ravel(), r.ravel(), c.ravel()], 1)
    text = np.stack([F + np.arange(aw.text), np.zeros(aw.text, int), np.zeros(aw.text, int)], 1)
    sample = np.concatenate([video, text]).astype(np.int32)
    assert len(sample) <= aw.S
    pos = np.zeros((aw.T, 3), np.int32)
    for b in range(aw.B):
        n = min(len(sample), aw.valid[b])
        pos[b * aw.S:b * aw.S + n] = sample[:n]
    return pos


def rope_tables(aw: AttnWorkload) -> Tuple[np.ndarray, np.ndarray]:
    """cos, sin fp32 [T, D/2] for the 3D positions: the D/2 channel pairs are
    split into (time, row, column) blocks of D/2 - 2 (D/6), D/6, D/6 pairs
    (Wan's split), pair j of a block of n turning by pos * theta^(-j / n)."""
    D = aw.head_dim
    nh = D // 6
    n = (D // 2 - 2 * nh, nh, nh)
    pos = joint_positions(aw).astype(np.float64)
    ang = np.concatenate([np.outer(pos[:, a], aw.theta ** (-np.arange(n[a]) / n[a]))
                          for a in range(3)], 1)
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def make_attn_inputs(aw: AttnWorkload) -> dict:
    """The attention half's inputs (one stream, seed aw.seed): ``x [T, H]`` the
    modulated layer input (bf16 values), ``w_qkv [3H, H]`` (q, k, v rows) and
    ``w_o [H, H]`` (bf16 values, std H^-1/2), the biases ``b_qkv [3H]`` and
    ``b_o [H]`` (fp32, std b_std), the q / k norm weights ``g_q, g_k [D]``
    (fp32, 1 + N(0, g_std^2)), the rotary tables ``cos, sin [T, D/2]`` and the
    mask (u8 [T], or None when every token is valid)."""
    T, H, D = aw.T, aw.hidden, aw.head_dim
    rng = np.random.default_rng(aw.seed)
    x = round_to_bf16(_draw(rng, (T, H), aw.x_std))
    w_qkv = round_to_bf16(_draw(rng, (3 * H, H), H ** -0.5))
    b_qkv = _draw(rng, (3 * H,), aw.b_std)
    g_q = 1 + _draw(rng, (D,), aw.g_std)
    g_k = 1 + _draw(rng, (D,), aw.g_std)
    w_o = round_to_bf16(_draw(rng, (H, H), H ** -0.5))
    b_o = _draw(rng, (H,), aw.b_std)
    cos, sin = rope_tables(aw)
    mask = None
    if any(v < aw.S for v in aw.valid):
        mask = np.zeros(T, np.uint8)
        for b, v in enumerate(aw.valid):
            mask[b * aw.S:b * aw.S + v] = 1
    return dict(x=x, w_qkv=w_qkv, b_qkv=b_qkv, g_q=g_q, g_k=g_k, w_o=w_o, b_o=b_o, cos=cos,
                sin=sin, mask=mask)


def make_attn_adaln_inputs(aw: AttnWorkload, x_std: float = 1.0, table_std: float = 0.1,
                           temb_std: float = 0.1) -> dict:
    """The residual stream and modulation around the attention half (a stream
    of its own, seed + 1000): ``x [T, H]``, ``table [6, H]`` and a token-level
    ``temb6 [T, 6, H]``, float32 N(0, std^2)."""
    rng = np.random.default_rng(aw.seed + 1000)
    x = _draw(rng, (aw.T, aw.hidden), x_std)
    table = _draw(rng, (6, aw.hidden), table_std)
    temb6 = _draw(rng, (aw.T, 6, aw.hidden), temb_std)
    return dict(x=x, table=table, temb6=temb6)
