"""Benchmark of the routed-MoE block (LingBot-Video MoE layer) on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one lbv_moe_forward (router, permutation, gate/up GEMM with SiLU,
down GEMM, weighted combine) over the workload's tokens, inputs resident in
HBM.  Prints one JSON line: MoE-layer tokens/s over K timed steps, the
grouped-GEMM TFLOP/s and its fraction of the bf16 MFMA peak, a roofline
object for the dominant kernel (the gate/up GEMM) timed with events around
its own launches on the launch stream, and the CPU oracle timed on a bounded
token sample on the host.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
HBM_PEAK_GBS = 8000.0

# Bytes the gate/up GEMM moves between L2 and memory per launch on
# default_gen_T38000: rocprofv3 FETCH_SIZE and WRITE_SIZE (KiB per dispatch,
# two --pmc runs of `bench.py --copy-calibration`), each scaled by what the same
# counter reads for a plain 1 GiB device copy (FETCH_SIZE x 2.000, WRITE_SIZE
# x 1.000): 3,297,198 KiB x 2 read + 556,954 KiB written.  Re-measure whenever
# the kernel changes (None then).
GEMM_W13_TRAFFIC_BYTES = 7.3228e9


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="default_gen_T38000")
    p.add_argument("--cpu-sample", type=int, default=8192,
                   help="tokens of the same workload the CPU oracle is timed on")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--copy-calibration", action="store_true",
                   help="after the measurements, run a plain 1 GiB device copy three times, so "
                        "that a hardware-counter run can scale its byte counters")
    return p.parse_args()


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

    def dev(a, bf):
        if a is None:
            return None
        if bf:
            return torch.from_numpy(synth.bf16_bits(a).view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    bf = wl.dtype == "bf16"
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

    # ---- whole-block throughput ------------------------------------------------
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = ev0.elapsed_time(ev1) / args.steps

    # ---- per-stage timing with the split calls on the same stream ------------------
    off = torch.empty(S + 1, dtype=torch.int32, device="cuda")
    srt = torch.empty(T * KS, dtype=torch.int32, device="cuda")
    inv = torch.empty(T * KS, dtype=torch.int32, device="cuda")
    pws = torch.empty(lbv.lbv_moe_permute_workspace_size(cfg, T), dtype=torch.uint8,
                      device="cuda")
    act = torch.empty(T * KS, I, dtype=x.dtype, device="cuda")
    yws = torch.empty(lbv.lbv_moe_w2_workspace_size(cfg, T), dtype=torch.uint8, device="cuda")
    rws = torch.empty(max(lbv.lbv_moe_route_workspace_size(cfg), 16), dtype=torch.uint8,
                      device="cuda")
    stages = ["route", "permute", "gemm_w13_silu", "gemm_w2_combine"]

    def split(evs):
        evs[0].record(stream)
        lbv.lbv_moe_route(cfg, x, router_w, e_bias, mask, ids, wts, rws, stream)
        evs[1].record(stream)
        lbv.lbv_moe_permute(cfg, ids, off, srt, inv, pws, stream)
        evs[2].record(stream)
        lbv.lbv_moe_gemm_w13_silu(cfg, x, w13, sw13, off, srt, act, stream)
        evs[3].record(stream)
        lbv.lbv_moe_gemm_w2_combine(cfg, act, w2, sw2, off, srt, inv, wts, out, yws, stream)
        evs[4].record(stream)

    nst = max(5, min(args.steps, 20))
    evsets = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(nst)]
    for _ in range(2):
        split(evsets[0])
    torch.cuda.synchronize()
    for i in range(nst):
        split(evsets[i])
    torch.cuda.synchronize()
    stage_ms = {s: float(np.mean([e[j].elapsed_time(e[j + 1]) for e in evsets]))
                for j, s in enumerate(stages)}

    # ---- algorithmic work ----------------------------------------------------------
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
    w13_tflops = flops_w13 / (stage_ms["gemm_w13_silu"] * 1e-3) / 1e12
    counts = np.bincount(ids_h[ids_h >= 0].reshape(-1), minlength=E)

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
        "config": {"workload": wl.name, "tokens": T, "hidden": H, "num_experts": E,
                   "top_k": K, "n_group": wl.n_group, "topk_group": wl.topk_group,
                   "intermediate": I, "n_shared": NS, "routed_rows": R_routed},
        "grouped_gemm_tflops": gemm_tflops,
        "grouped_gemm_frac_bf16_peak": gemm_tflops / BF16_PEAK_TFLOPS,
        "routed_gemm_tflops": routed_tflops,
        "valid_tokens_per_s": valid_tokens / (ms_per_step * 1e-3),
        "stage_ms": stage_ms,
        "router_x_read_gbs": T * H * (2 if bf else 4) / (stage_ms["route"] * 1e-3) / 1e9,
        "expert_load_max_over_mean": float(counts.max() / max(counts.mean(), 1e-9)),
        "roofline": {
            "kernel": "gemm_w13_silu (lbv_moe_gemm_w13_silu)",
            "bound": "mfma",
            "achieved": w13_tflops,
            "peak": BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": w13_tflops / BF16_PEAK_TFLOPS,
            "traffic": GEMM_W13_TRAFFIC_BYTES,
            "algorithmic_flops_per_launch": flops_w13,
        },
        "wall_s_timed": wall,
        "input_gen_s": t_gen,
    }

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
                               "kind": "oracle",
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
