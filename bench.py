"""Benchmark of the routed-MoE block (LingBot-Video MoE layer) on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one lbv_moe_forward (router, permutation, gate/up GEMM with SiLU,
down GEMM, weighted combine) over the workload's tokens, inputs resident in
HBM.  Prints one JSON line:
  * MoE-layer tokens/s over K timed steps (one event before the first step
    and one after each step, so the per-step median / p10 / p90 come from the
    same region);
  * the grouped-GEMM TFLOP/s: the algorithmic FLOPs of both grouped matmuls
    (routed + shared) over the summed time of lbv_moe_gemm_w13_silu and
    lbv_moe_gemm_w2_combine, and its fraction of the bf16 MFMA peak;
  * stage times of the four split calls (events on the launch stream);
  * a roofline object for the dominant kernel, the gate/up GEMM: bound by
    HBM when its algorithmic FLOP per byte is below the machine balance (few
    tokens: the weights stream once), else by the bf16 matrix cores;
  * router and permutation rates, the input digests, and the CPU oracle timed
    on a bounded token sample on the host;
  * beside the headline (each leg on by default, --no-<leg> skips it): the FFN
    half of a DiT layer with its AdaLN (adaln), the block with fp8 weights and
    with fp8 weights and activations (fp8, w8a8), and the attention half of
    the layer on the same token layout (attention_half).
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
FP32_PEAK_TFLOPS = 157.3       # MI355X fp32 vector
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
KERNEL_SOURCES = ("routed_moe_dit_amd/csrc/gemm.hip", "routed_moe_dit_amd/csrc/lbv_pipe.h",
                  "routed_moe_dit_amd/csrc/lbv_internal.h")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="default_gen_T38000")
    p.add_argument("--cpu-sample", type=int, default=12000,
                   help="tokens of the same workload the CPU oracle is timed on")
    p.add_argument("--no-cpu-baseline", action="store_true")
    # the legs beside the headline block (on by default; --no-adaln etc. skip them)
    p.add_argument("--adaln", action=argparse.BooleanOptionalAction, default=True,
                   help="also time the FFN half of a DiT layer around the block "
                        "(lbv_moe_ffn_adaln, token-level temb6) and its AdaLN kernel alone")
    p.add_argument("--fp8", action=argparse.BooleanOptionalAction, default=True,
                   help="also time the block with fp8 (e4m3fn, per-row power-of-two scale) "
                        "expert weights (lbv_moe_forward_fp8), the device quantizer, and the "
                        "block with fp8 weights and fp8 activations (lbv_moe_forward_w8a8)")
    p.add_argument("--attn", action=argparse.BooleanOptionalAction, default=True,
                   help="also time the attention half of the layer (lbv_attn_forward) on the "
                        "attention workload of the same token layout, and its kernels")
    p.add_argument("--copy-calibration", action="store_true",
                   help="after the measurements, run a plain 1 GiB device copy three times, so "
                        "that a hardware-counter run can scale its byte counters")
    return p.parse_args()


def kernel_source_hash():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(workload, kernel):
    """Bytes per launch from a counter summary in profiles/ (a JSON block with
    the kernel, the workload and the hash of the kernel sources it was taken
    on); None when there is none for the current sources."""
    d = os.path.join(ROOT, "profiles")
    want = kernel_source_hash()
    for name in sorted(os.listdir(d)) if os.path.isdir(d) else []:
        if not name.endswith(".md"):
            continue
        text = open(os.path.join(d, name)).read()
        for block in re.findall(r"```json\n(.*?)\n```", text, flags=re.S):
            try:
                rec = json.loads(block)
            except ValueError:
                continue
            if (rec.get("kind") == "traffic" and rec.get("workload") == workload and
                    rec.get("kernel") == kernel and rec.get("source_sha256") == want):
                return float(rec["read_bytes"]) + float(rec["write_bytes"])
    return None


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def pct(a, q):
    return float(np.percentile(np.asarray(a, np.float64), q))


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: this build runs the MoE block on one GPU only; --gpus %d is not "
              "supported (each GPU would run the same block on its own share of tokens with "
              "no exchange)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch

    import routed_moe_dit_amd as lbv
    import synth

    torch.cuda.set_device(0)
    wl = synth.by_name(args.workload)
    t_gen = time.time()
    inp = synth.make_inputs(wl)
    t_gen = time.time() - t_gen
    digests = synth.digest(inp)

    def dev(a, bf):
        if a is None:
            return None
        if bf:
            return torch.from_numpy(synth.bf16_bits(a).view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    bf = wl.dtype == "bf16"
    esz = 2 if bf else 4
    x = dev(inp["x"], bf)
    router_w, e_bias = dev(inp["router_w"], False), dev(inp["e_bias"], False)
    w13, w2 = dev(inp["w13"], bf), dev(inp["w2"], bf)
    sw13, sw2 = dev(inp["shared_w13"], bf), dev(inp["shared_w2"], bf)
    mask = None if inp["mask"] is None else torch.from_numpy(inp["mask"]).cuda()
    cfg = lbv.config(hidden=wl.hidden, num_experts=wl.num_experts, top_k=wl.top_k,
                     n_group=wl.n_group, topk_group=wl.topk_group, intermediate=wl.intermediate,
                     n_shared_experts=wl.n_shared, norm_topk_prob=wl.norm_topk_prob,
                     routed_scaling_factor=wl.routed_scaling_factor, dtype=wl.dtype)
    T, H, I, E, K, NS = wl.T, wl.hidden, wl.intermediate, wl.num_experts, wl.top_k, wl.n_shared
    KS, S = K + NS, E + NS
    out = torch.empty_like(x)
    ids = torch.empty(T, K, dtype=torch.int32, device="cuda")
    wts = torch.empty(T, K, dtype=torch.float32, device="cuda")
    ws = torch.empty(lbv.lbv_moe_workspace_size(cfg, T), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        lbv.lbv_moe_forward(cfg, x, mask, router_w, e_bias, w13, w2, sw13, sw2, out, ids, wts, ws,
                            stream)

    # ---- whole-block throughput: K steps, an event after each ---------------------
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t0 = time.perf_counter()
    evs[0].record(stream)
    for i in range(args.steps):
        step()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = evs[0].elapsed_time(evs[-1]) / args.steps
    per_step = [evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)]

    # ---- per-stage timing with the split calls on the same stream ------------------
    off = torch.empty(S + 1, dtype=torch.int32, device="cuda")
    srt = torch.empty(T * KS, dtype=torch.int32, device="cuda")
    inv = torch.empty(T * KS, dtype=torch.int32, device="cuda")
    pws = torch.empty(lbv.lbv_moe_permute_workspace_size(cfg, T), dtype=torch.uint8,
                      device="cuda")
    act = torch.empty(T * KS, I, dtype=x.dtype, device="cuda")
    yws = torch.empty(lbv.lbv_moe_w2_workspace_size(cfg, T), dtype=torch.uint8, device="cuda")
    gws = torch.empty(lbv.lbv_moe_w13_workspace_size(cfg, T), dtype=torch.uint8, device="cuda")
    rws = torch.empty(max(lbv.lbv_moe_route_workspace_size(cfg), 16), dtype=torch.uint8,
                      device="cuda")
    stages = ["route", "permute", "gemm_w13_silu", "gemm_w2_combine"]

    def split(evs_):
        evs_[0].record(stream)
        lbv.lbv_moe_route(cfg, x, router_w, e_bias, mask, ids, wts, rws, stream)
        evs_[1].record(stream)
        lbv.lbv_moe_permute(cfg, ids, off, srt, inv, pws, stream)
        evs_[2].record(stream)
        lbv.lbv_moe_gemm_w13_silu(cfg, x, w13, sw13, off, srt, act, gws, stream)
        evs_[3].record(stream)
        lbv.lbv_moe_gemm_w2_combine(cfg, act, w2, sw2, off, srt, inv, wts, out, yws, stream)
        evs_[4].record(stream)

    nst = max(5, min(args.steps, 30))
    evsets = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(nst)]
    for _ in range(2):
        split(evsets[0])
    torch.cuda.synchronize()
    for i in range(nst):
        split(evsets[i])
    torch.cuda.synchronize()
    stage_runs = {s: [e[j].elapsed_time(e[j + 1]) for e in evsets] for j, s in enumerate(stages)}
    stage_ms = {s: float(np.mean(v)) for s, v in stage_runs.items()}

    # ---- algorithmic work -----------------------------------------------------------
    ids_h = ids.cpu().numpy()
    R_routed = int((ids_h >= 0).sum())
    Rp = R_routed + T * NS
    flops_w13 = 4.0 * H * I * Rp
    flops_w2 = 2.0 * H * I * Rp
    gemm_flops = flops_w13 + flops_w2
    gemm_ms = stage_ms["gemm_w13_silu"] + stage_ms["gemm_w2_combine"]
    gemm_tflops = gemm_flops / (gemm_ms * 1e-3) / 1e12
    routed_tflops = 6.0 * H * I * R_routed / (gemm_ms * 1e-3) / 1e12
    valid_tokens = T if inp["mask"] is None else int(inp["mask"].sum())
    counts = np.bincount(ids_h[ids_h >= 0].reshape(-1), minlength=E)
    hit = counts > 0
    # gate/up GEMM bytes per launch: the w13 rows of every expert hit, the
    # shared gate/up rows, x read once, act written once
    w13_bytes = (int(hit.sum()) * 2 * I * H + 2 * I * NS * H) * esz
    bytes_w13 = w13_bytes + T * H * esz + Rp * I * esz
    ai_w13 = flops_w13 / bytes_w13
    w13_s = stage_ms["gemm_w13_silu"] * 1e-3
    if ai_w13 < BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9):
        roof = {"bound": "hbm", "achieved": bytes_w13 / w13_s / 1e9, "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "algorithmic_bytes_per_launch": bytes_w13}
    else:
        roof = {"bound": "mfma", "achieved": flops_w13 / w13_s / 1e12, "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "algorithmic_flops_per_launch": flops_w13}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = recorded_traffic(wl.name, "gemm_w13_silu")
    roof["kernel"] = "gemm_w13_silu (lbv_moe_gemm_w13_silu)"
    roof["kernel_ms"] = stage_ms["gemm_w13_silu"]
    roof["arithmetic_intensity_flop_per_byte"] = ai_w13

    route_s = stage_ms["route"] * 1e-3
    route_flops = 2.0 * H * E * T
    perm_bytes = T * K * 4 + 2 * T * KS * 4 + (S + 1) * 4
    weight_bytes = (int(hit.sum()) * 3 * I * H + 3 * I * NS * H) * esz
    block_bytes = weight_bytes + 2 * T * H * esz + 8 * T * K + E * H * 4
    res = {
        "metric": "MoE-layer tokens/s",
        "value": T / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if bf else "f32",
        "data": "synthetic (seeded, shapes of the LingBot-Video video workloads)",
        "config": {"workload": wl.name, "tokens": T, "valid_tokens": valid_tokens, "hidden": H,
                   "num_experts": E, "top_k": K, "n_group": wl.n_group,
                   "topk_group": wl.topk_group, "intermediate": I, "n_shared": NS,
                   "routed_rows": R_routed},
        "step_ms": {"median": pct(per_step, 50), "p10": pct(per_step, 10),
                    "p90": pct(per_step, 90), "n": len(per_step)},
        "grouped_gemm_tflops": gemm_tflops,
        "grouped_gemm_frac_bf16_peak": gemm_tflops / BF16_PEAK_TFLOPS,
        "routed_gemm_tflops": routed_tflops,
        "valid_tokens_per_s": valid_tokens / (ms_per_step * 1e-3),
        "stage_ms": stage_ms,
        "stage_ms_p90": {s: pct(v, 90) for s, v in stage_runs.items()},
        "block_hbm_frac": block_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "router": {"x_read_gbs": T * H * esz / route_s / 1e9,
                   "fp32_equiv_tflops": route_flops / route_s / 1e12,
                   "frac_fp32_peak": route_flops / route_s / 1e12 / FP32_PEAK_TFLOPS},
        "permute": {"bytes": perm_bytes, "gbs": perm_bytes / (stage_ms["permute"] * 1e-3) / 1e9,
                    "frac_hbm": perm_bytes / (stage_ms["permute"] * 1e-3) / 1e9 / HBM_PEAK_GBS},
        "expert_load_max_over_mean": float(counts.max() / max(counts.mean(), 1e-9)),
        "roofline": roof,
        "kernel_source_sha256": kernel_source_hash(),
        "input_sha256": digests,
        "wall_s_timed": wall,
        "input_gen_s": t_gen,
    }
    if wl.hot:
        res["hot_expert_share"] = float(counts[list(wl.hot)].sum() / max(counts.sum(), 1))

    # ---- the FFN half of a DiT layer around the block (AdaLN, gated residual) ------
    if args.adaln:
        ada = synth.make_adaln_inputs(wl, per_token=True)
        xr = torch.from_numpy(ada["x"]).cuda()
        temb = torch.from_numpy(ada["temb6"]).cuda()
        table = torch.from_numpy(ada["table"]).cuda()
        del ada
        fout = torch.empty_like(xr)
        fws = torch.empty(lbv.lbv_moe_ffn_adaln_workspace_size(cfg, T), dtype=torch.uint8,
                          device="cuda")
        hbuf = torch.empty(T, H, dtype=x.dtype, device="cuda")

        def ffn():
            lbv.lbv_moe_ffn_adaln(cfg, xr, mask, temb, table, 1e-6, router_w, e_bias, w13, w2,
                                  sw13, sw2, fout, ids, wts, fws, stream)

        def timed(fn, n):
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
            e = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
            e[0].record(stream)
            for i in range(n):
                fn()
                e[i + 1].record(stream)
            torch.cuda.synchronize()
            return [e[i].elapsed_time(e[i + 1]) for i in range(n)]

        f_ms = timed(ffn, max(10, args.steps // 2))
        a_ms = timed(lambda: lbv.lbv_adaln_rmsnorm(cfg, xr, temb, table, 1e-6, hbuf, stream),
                     max(10, args.steps // 2))
        a_bytes = T * H * 4 + 2 * T * H * 4 + T * H * esz     # x, shift + scale rows, h
        res["adaln"] = {
            "ffn_adaln_ms": float(np.median(f_ms)),
            "ffn_adaln_tokens_per_s": T / (float(np.median(f_ms)) * 1e-3),
            "extra_over_block_ms": float(np.median(f_ms)) - pct(per_step, 50),
            "adaln_kernel_ms": float(np.median(a_ms)),
            "adaln_algorithmic_bytes": a_bytes,
            "adaln_gbs": a_bytes / (float(np.median(a_ms)) * 1e-3) / 1e9,
            "adaln_frac_hbm": a_bytes / (float(np.median(a_ms)) * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "temb6": "token-level [T, 6, H] fp32",
        }
        del temb, fws

    # ---- fp8 expert weights: the same block, weights read as e4m3fn codes ----------
    if args.fp8 and bf:
        qev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        qev[0].record(stream)
        wq = lbv.quantize_fp8_weights(w13, w2, sw13, sw2, stream)
        qev[1].record(stream)
        torch.cuda.synchronize()
        q_ms = qev[0].elapsed_time(qev[1])

        def step8():
            lbv.lbv_moe_forward_fp8(cfg, x, mask, router_w, e_bias, wq, out, ids, wts, ws, stream)

        for _ in range(args.warmup):
            step8()
        torch.cuda.synchronize()
        e8 = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        e8[0].record(stream)
        for i in range(args.steps):
            step8()
            e8[i + 1].record(stream)
        torch.cuda.synchronize()
        ms8 = e8[0].elapsed_time(e8[-1]) / args.steps
        per8 = [e8[i].elapsed_time(e8[i + 1]) for i in range(args.steps)]
        wbytes8 = (int(hit.sum()) * 3 * I * H + 3 * I * NS * H) * (1 + 4.0 / H)
        res["fp8"] = {
            "ms_per_step": ms8,
            "tokens_per_s": T / (ms8 * 1e-3),
            "step_ms_median": pct(per8, 50),
            "speedup_vs_bf16_weights": ms_per_step / ms8,
            "expert_weight_bytes_read": wbytes8,
            "expert_weight_bytes_read_bf16": weight_bytes,
            "quantize_all_weights_ms": q_ms,
            "format": "e4m3fn codes, one power-of-two fp32 scale per weight row; bf16 "
                      "activations, fp32 accumulation",
        }

        # fp8 weights and fp8 activations: both matmuls on the fp8 matrix cores
        if H % 128 == 0 and I % 128 == 0 and I <= 1024:
            def step_a8():
                lbv.lbv_moe_forward_w8a8(cfg, x, mask, router_w, e_bias, wq, out, ids, wts, ws,
                                         stream)

            for _ in range(args.warmup):
                step_a8()
            torch.cuda.synchronize()
            ea = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
            ea[0].record(stream)
            for i in range(args.steps):
                step_a8()
                ea[i + 1].record(stream)
            torch.cuda.synchronize()
            msa = ea[0].elapsed_time(ea[-1]) / args.steps
            pera = [ea[i].elapsed_time(ea[i + 1]) for i in range(args.steps)]
            res["w8a8"] = {
                "ms_per_step": msa,
                "tokens_per_s": T / (msa * 1e-3),
                "step_ms_median": pct(pera, 50),
                "speedup_vs_bf16": ms_per_step / msa,
                "speedup_vs_fp8_weights": ms8 / msa,
                "matmul_flops": gemm_flops,
                "format": "fp8 weights as above; x rows quantized like weight rows (one "
                          "power-of-two scale per token); act rounded to bf16, then MX blocks "
                          "of 32 (e4m3fn codes, e8m0 scale); scaled fp8 MFMA, fp32 "
                          "accumulation",
            }
        del wq

    # ---- the attention half of the layer on the same token layout -----------------
    if args.attn and bf:
        aw = [a for a in synth.ATTN_WORKLOADS if a.T == T]
        if aw:
            aw = aw[0]
            ai = synth.make_attn_inputs(aw)
            acfg = lbv.attn_config(hidden=aw.hidden, num_heads=aw.heads, eps=1e-6)
            ad = {k_: (dev(v_, k_ in ("x", "w_qkv", "w_o")) if v_ is not None and v_.dtype == np.float32
                       else (None if v_ is None else torch.from_numpy(v_).cuda()))
                  for k_, v_ in ai.items()}
            del ai
            B_, S_ = aw.B, aw.S
            aout = torch.empty(T, H, dtype=torch.bfloat16, device="cuda")
            aws = torch.empty(lbv.lbv_attn_workspace_size(acfg, B_, S_), dtype=torch.uint8,
                              device="cuda")
            lws = torch.empty(lbv.LINEAR_WS_BYTES, dtype=torch.uint8, device="cuda")
            qkv = torch.empty(T, 3 * H, dtype=torch.bfloat16, device="cuda")
            aq, ak, ao = (torch.empty(T, H, dtype=torch.bfloat16, device="cuda") for _ in range(3))
            avt = torch.empty(B_, aw.heads, 128, lbv.attn_sp(S_), dtype=torch.bfloat16,
                              device="cuda")

            def half():
                lbv.lbv_attn_forward(acfg, B_, S_, ad["x"], ad["mask"], ad["w_qkv"], ad["b_qkv"],
                                     ad["g_q"], ad["g_k"], ad["cos"], ad["sin"], ad["w_o"],
                                     ad["b_o"], aout, aws, stream)

            def timed_n(fn, n):
                for _ in range(2):
                    fn()
                torch.cuda.synchronize()
                e = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
                e[0].record(stream)
                for i in range(n):
                    fn()
                    e[i + 1].record(stream)
                torch.cuda.synchronize()
                return [e[i].elapsed_time(e[i + 1]) for i in range(n)]

            nrep = max(5, min(args.steps, 20))
            h_ms = timed_n(half, nrep)
            parts = {
                "qkv_proj": lambda: lbv.lbv_linear_bf16(ad["x"], ad["w_qkv"], ad["b_qkv"], qkv, lws,
                                                        stream),
                "qk_prep": lambda: lbv.lbv_attn_qk_prep(acfg, B_, S_, qkv, ad["g_q"], ad["g_k"],
                                                        ad["cos"], ad["sin"], aq, ak, avt, stream),
                "attention": lambda: lbv.lbv_attn_core(acfg, B_, S_, aq, ak, avt, ad["mask"], ao,
                                                       stream),
                "out_proj": lambda: lbv.lbv_linear_bf16(ao, ad["w_o"], ad["b_o"], aout, lws,
                                                        stream),
            }
            part_ms = {k_: float(np.median(timed_n(f_, nrep))) for k_, f_ in parts.items()}
            # the same half with its AdaLN (rows 0, 1) and gated residual (row 2)
            ada = synth.make_attn_adaln_inputs(aw)
            xr = torch.from_numpy(ada["x"]).cuda()
            temb = torch.from_numpy(ada["temb6"]).cuda()
            table = torch.from_numpy(ada["table"]).cuda()
            del ada
            hout = torch.empty_like(xr)
            hws = torch.empty(lbv.lbv_attn_half_adaln_workspace_size(acfg, B_, S_),
                              dtype=torch.uint8, device="cuda")
            ha_ms = timed_n(lambda: lbv.lbv_attn_half_adaln(
                acfg, B_, S_, xr, ad["mask"], temb, table, 1e-6, ad["w_qkv"], ad["b_qkv"],
                ad["g_q"], ad["g_k"], ad["cos"], ad["sin"], ad["w_o"], ad["b_o"], hout, hws,
                stream), nrep)
            del xr, temb, table, hout, hws
            valid = [min(v_, S_) for v_ in aw.valid]
            attn_flops = 4.0 * sum(v_ * v_ for v_ in valid) * H      # QK^T and PV, valid tokens
            a_s = part_ms["attention"] * 1e-3
            res["attention_half"] = {
                "workload": aw.name,
                "ms": float(np.median(h_ms)),
                "tokens_per_s": T / (float(np.median(h_ms)) * 1e-3),
                "with_adaln_and_residual_ms": float(np.median(ha_ms)),
                "stage_ms": part_ms,
                "qkv_proj_tflops": 2.0 * T * 3 * H * H / (part_ms["qkv_proj"] * 1e-3) / 1e12,
                "out_proj_tflops": 2.0 * T * H * H / (part_ms["out_proj"] * 1e-3) / 1e12,
                "roofline": {"kernel": "attn_fwd_kernel (lbv_attn_core)", "bound": "mfma",
                             "achieved": attn_flops / a_s / 1e12, "peak": BF16_PEAK_TFLOPS,
                             "unit": "TFLOP/s", "frac": attn_flops / a_s / 1e12 / BF16_PEAK_TFLOPS,
                             "algorithmic_flops_per_launch": attn_flops, "traffic": None},
                "layout": "B=%d samples of S=%d tokens, %d heads of 128" % (B_, S_, aw.heads),
            }
            del ad, aout, aws, qkv, aq, ak, ao, avt

    # ---- CPU oracle on a bounded sample of the same workload -----------------------
    if not args.no_cpu_baseline:
        import oracle

        n = min(args.cpu_sample, T)
        rows = np.linspace(0, T - 1, n).astype(np.int64)
        m = None if inp["mask"] is None else inp["mask"][rows]
        threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
        tc = time.perf_counter()
        oracle.moe_forward(wl, inp["x"][rows], inp["router_w"], inp["e_bias"], inp["w13"],
                           inp["w2"], inp["shared_w13"], inp["shared_w2"], m)
        dt = time.perf_counter() - tc
        res["cpu_baseline"] = {"value": n / dt, "unit": "tokens/s", "cores": threads,
                               "kind": "oracle", "cpu_model": cpu_model(),
                               "sample": "%d of %d tokens of %s, evenly spaced; %.1f s" %
                                         (n, T, wl.name, dt)}
    print(json.dumps(res), flush=True)

    if args.copy_calibration:
        src = torch.ones(1 << 29, dtype=torch.float16, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()


if __name__ == "__main__":
    main()
