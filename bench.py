#!/usr/bin/env python3
"""Benchmark of the MoE-layer forward on one MI355X.

One step = the whole hot path (route -> permute -> routed experts' up and
down projections -> shared expert -> combine) over one batch of synthetic
tokens whose inputs are already resident in HBM.  The default workload is the
Step-5-Preview-shaped prefill: 8192 tokens, hidden 4096, 352 routed experts,
top-8, expert and shared intermediate 1536, clipped SwiGLU at 7.0, bf16.

Prints one JSON line with tokens/s, the whole-layer TFLOP/s and bytes/s, the
roofline of the dominant kernel (routed experts' first projection + SwiGLU,
timed with HIP events on the stream it runs on), the oracle timed on the
host cores on a bounded token sample, and the 64-token decode shape's
bandwidth.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

METRIC = "MoE-layer fwd tokens/s + % bf16 MFMA peak (prefill) / % HBM BW (decode)"
HBM_PEAK = 8.0e12          # bytes/s, MI355X HBM3E
BF16_PEAK = 2.5166e15      # dense bf16 MFMA FLOP/s


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="step5_prefill")
    ap.add_argument("--decode-workload", default="step5_decode")
    ap.add_argument("--fp8-workload", default="step5_fp8_prefill", help="'' to skip the FP8 report")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--decode-half-workload", default="step5_decode_half",
                    help="second decode report (hot experts take about half of the selections); '' to skip")
    ap.add_argument("--no-ep-proxy", action="store_true",
                    help="skip the report on one expert-parallel rank's share (44 experts, MFMA-bound)")
    ap.add_argument("--no-balanced", action="store_true", help="skip the static balanced routing report")
    ap.add_argument("--no-block", action="store_true", help="skip the RMSNorm + residual block report")
    ap.add_argument("--no-train", action="store_true", help="skip the forward + backward training report")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target oracle time for the CPU baseline")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB a few times (scales HBM counters) and exit")
    return ap.parse_args()


def layer_flops(wl, touched):
    c = wl.cfg
    T, H, E, k, I, Is = wl.T, c.hidden_size, c.num_experts, c.top_k, c.moe_intermediate_size, c.share_expert_dim
    return 2 * T * E * H + 6 * T * k * H * I + 6 * T * H * Is


def layer_bytes(wl, touched):
    """Algorithmic HBM bytes of one layer forward: the weights of the experts
    the routing touches, the shared expert and router weights, the bias, the
    input once and the fp32 output once."""
    c = wl.cfg
    T, H, E, I, Is = wl.T, c.hidden_size, c.num_experts, c.moe_intermediate_size, c.share_expert_dim
    bpw = 1 if c.expert_dtype == "fp8" else 2
    b = touched * 3 * H * I * bpw + 3 * H * Is * 2 + 2 * E * H + 4 * E + 2 * T * H
    b += (2 if c.out_dtype == "bf16" else 4) * T * H
    return b


def up_kernel_bytes(wl, touched):
    """Algorithmic bytes of the routed experts' first-projection launch: W13
    of every touched expert once, x once, h written once.  (The whole-layer
    call runs the shared expert in launches of its own, and so do the timed
    separate entry points.)"""
    c = wl.cfg
    T, H, k, I = wl.T, c.hidden_size, c.top_k, c.moe_intermediate_size
    if c.expert_dtype == "fp8":
        # codes + block scales of W13; x read once (bf16); h codes + scales written
        return touched * (2 * I * H + (2 * I // 128) * (H // 128) * 4) + T * H * 2 + T * k * (I + I // 128 * 4)
    return touched * 2 * I * H * 2 + T * H * 2 + T * k * I * 2


TRAFFIC_FILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                            "routed_up_bf16_step5_prefill_hbm_counters.md")
KERNEL_SRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "sparse_moe_layer_route_amd", "csrc",
                          "grouped_gemm.hip")


def counter_traffic(wl):
    """HBM bytes per launch of the routed first projection from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary (scaled by a plain copy's
    counts), or None when the summary is for another workload or the kernel
    source has changed since the counters were taken."""
    import hashlib
    import re
    if wl.name != "step5_prefill" or not os.path.exists(TRAFFIC_FILE):
        return None
    text = open(TRAFFIC_FILE).read()
    t = re.search(r"^traffic_bytes_per_launch:\s*(\d+)", text, re.M)
    h = re.search(r"^kernel_source_sha256:\s*([0-9a-f]{64})", text, re.M)
    if not t or not h:
        return None
    if hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest() != h.group(1):
        return None
    return int(t.group(1))


def note(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this MoE-layer forward runs on a single MI355X and has no "
              "multi-GPU path (expert-parallel sharding is a design note only); run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import moe_inputs as mi
    import sparse_moe_layer_route_amd as moe

    dev = "cuda"
    if args.copy_calibration:
        n = args.copy_calibration * 2**20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": 3}), flush=True)
        return
    moe.load()
    wl = mi.WORKLOADS[args.workload]
    cfg, T, k, E, H, I = wl.cfg, wl.T, wl.cfg.top_k, wl.cfg.num_experts, wl.cfg.hidden_size, \
        wl.cfg.moe_intermediate_size
    r = time_layer(args, wl, moe, torch, mi)
    ms_step, up_ms, layer_fwd_ms, touched = r["ms_step"], r["up_ms"], r["layer_forward_ms"], r["touched"]
    tok_s = T / (ms_step * 1e-3)
    fl = layer_flops(wl, touched)
    by = layer_bytes(wl, touched)
    up_bytes = up_kernel_bytes(wl, touched)
    up_achieved = up_bytes / (up_ms * 1e-3)
    res = {
        "metric": METRIC, "value": tok_s, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8_e4m3" if cfg.expert_dtype == "fp8" else "bf16", "data": "synthetic",
        "config": {"workload": wl.name, "tokens": T, "hidden_size": H, "num_experts": E, "top_k": k,
                   "moe_intermediate_size": I, "share_expert_dim": cfg.share_expert_dim,
                   "swiglu_limit": cfg.swiglu_limit, "swiglu_limit_shared": cfg.swiglu_limit_shared,
                   "router_scaling_factor": cfg.router_scaling_factor, "experts_touched": touched,
                   "parallelism": "single GPU"},
        "tflops": fl / (ms_step * 1e-3) / 1e12,
        "mfma_frac": fl / (ms_step * 1e-3) / BF16_PEAK,
        "layer_gbs": by / (ms_step * 1e-3) / 1e9,
        "hbm_frac": by / (ms_step * 1e-3) / HBM_PEAK,
        "layer_roofline_frac": max(fl / BF16_PEAK, by / HBM_PEAK) / (ms_step * 1e-3),
        "layer_forward_ms": layer_fwd_ms,
        "roofline": {"kernel": "first projection + clipped SwiGLU of the routed experts "
                               "(moe_expert_up, gg::kernel<0, true, 256, 256>)",
                     "bound": "hbm", "achieved": up_achieved / 1e9, "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                     "frac": up_achieved / HBM_PEAK, "traffic": counter_traffic(wl), "avg_ms": up_ms,
                     "algorithmic_bytes": up_bytes},
    }

    if args.fp8_workload:
        wf = mi.WORKLOADS[args.fp8_workload]
        rf = time_layer(args, wf, moe, torch, mi)
        ub = up_kernel_bytes(wf, rf["touched"])
        res["fp8"] = {"workload": wf.name, "experts_touched": rf["touched"], "ms_per_step": rf["ms_step"],
                      "tokens_per_s": wf.T / (rf["ms_step"] * 1e-3),
                      "tflops": layer_flops(wf, rf["touched"]) / (rf["ms_step"] * 1e-3) / 1e12,
                      "layer_forward_ms": rf["layer_forward_ms"],
                      "up_ms": rf["up_ms"], "up_gbs": ub / (rf["up_ms"] * 1e-3) / 1e9,
                      "up_hbm_frac": ub / (rf["up_ms"] * 1e-3) / HBM_PEAK}

    if not args.no_balanced:
        note(f"{wl.name} with the static balanced routing")
        rb = time_balanced(args, wl, moe, torch, mi)
        res["balanced_routing"] = {
            "workload": wl.name, "routing": "static balanced (pair t*k+j -> expert (t*k+j) mod E), "
                                            "moe_balanced_ids + moe_layer_forward_routed",
            "experts_touched": rb["touched"], "ms_per_step": rb["ms_step"], "tokens_per_s": T / (rb["ms_step"] * 1e-3),
            "tflops": layer_flops(wl, rb["touched"]) / (rb["ms_step"] * 1e-3) / 1e12,
            "mfma_frac": layer_flops(wl, rb["touched"]) / (rb["ms_step"] * 1e-3) / BF16_PEAK,
            "hbm_frac": layer_bytes(wl, rb["touched"]) / (rb["ms_step"] * 1e-3) / HBM_PEAK}

    if not args.no_block:
        note(f"{wl.name} as a block: RMSNorm in front, fp32 residual add in the combine")
        res["block"] = time_block(args, wl, moe, torch, mi)

    if not args.no_train and cfg.expert_dtype == "bf16":
        note(f"{wl.name} training step: moe_layer_forward_train + moe_layer_backward")
        res["train"] = time_train(args, wl, moe, torch, mi)

    if not args.no_ep_proxy and cfg.expert_dtype == "bf16":
        we = mi.WORKLOADS["ep_rank_proxy"]
        note(f"{we.name}: one expert-parallel rank's share ({we.cfg.num_experts} experts, {we.T} tokens)")
        r = time_layer(args, we, moe, torch, mi)
        fl = layer_flops(we, r["touched"])
        up_fl = 2 * we.T * we.cfg.top_k * we.cfg.hidden_size * 2 * we.cfg.moe_intermediate_size
        res["ep_rank_proxy"] = {
            "workload": we.name, "experts": we.cfg.num_experts, "tokens": we.T, "experts_touched": r["touched"],
            "layer_forward_ms": r["layer_forward_ms"], "tflops": fl / (r["layer_forward_ms"] * 1e-3) / 1e12,
            "mfma_frac": fl / (r["layer_forward_ms"] * 1e-3) / BF16_PEAK,
            "up_ms": r["up_ms"], "up_tflops": up_fl / (r["up_ms"] * 1e-3) / 1e12,
            "up_mfma_frac": up_fl / (r["up_ms"] * 1e-3) / BF16_PEAK}

    if not args.no_decode:
        note(f"decode workload {args.decode_workload}")
        res["decode"] = bench_decode(args, mi.WORKLOADS[args.decode_workload], moe, torch)
        if args.decode_half_workload:
            note(f"decode workload {args.decode_half_workload}")
            res["decode_half"] = bench_decode(args, mi.WORKLOADS[args.decode_half_workload], moe, torch)

    if not args.no_cpu_baseline:
        note("CPU baseline (oracle on a token sample)")
        res["cpu_baseline"] = cpu_baseline(args, wl, mi)

    print(json.dumps(res), flush=True)


def time_layer(args, wl, moe, torch, mi):
    """Warm up, then time args.steps steps, each one moe_layer_forward call
    (the whole layer in one call: routing, permutation, both expert
    projections with the shared expert, combine), bracketed by a
    synchronisation on both sides.  Then, as a second timed region of as many
    steps, the same layer through its separate entry points, with the routed
    experts' first projection bracketed by HIP events on its stream: that
    kernel's average duration for the roofline object."""
    dev = "cuda"
    cfg, T, k, H = wl.cfg, wl.T, wl.cfg.top_k, wl.cfg.hidden_size
    note(f"generating {wl.name} inputs")
    inp = mi.make_inputs(wl, dev, seed=0)
    ws = moe.workspace(cfg, T)
    stream = torch.cuda.current_stream()
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    counts = torch.empty((cfg.num_experts,), dtype=torch.int32, device=dev)
    out = torch.empty((T, H), dtype=torch.float32, device=dev)
    h = torch.empty(moe.moe_hidden_bytes(cfg, T), dtype=torch.uint8, device=dev)
    # the separate entry points with the shared expert in launches of its own,
    # as moe_layer_forward runs it at these sizes (on its side stream), so the
    # routed experts' first projection is the same launch in both regions
    fused = False
    y_rows = torch.empty((T * k + (T if fused else 0), H), dtype=torch.float16, device=dev)
    y_sh = None if fused else torch.empty((T, H), dtype=torch.float32, device=dev)
    s13, s2 = inp.get("w13_scale"), inp.get("w2_scale")
    ws13, ws2 = (inp["ws13"], inp["ws2"]) if fused else (None, None)

    def layer():
        moe.moe_layer_forward(cfg, inp, out=out, ws=ws, stream=stream, expert_counts=counts)

    def stepwise(ev):
        moe.moe_route(cfg, inp["x"], inp["w_router"], inp["router_bias"], ids, w, ws=ws, stream=stream)
        _, offsets, r2p, p2r = moe.moe_permute(cfg, ids, ws=ws, stream=stream)
        ev[0].record(stream)
        moe.moe_expert_up(cfg, inp["x"], offsets, r2p, inp["w13"], s13, h=h, ws=ws, stream=stream, ws13=ws13)
        ev[1].record(stream)
        moe.moe_expert_down(cfg, T, h, offsets, inp["w2"], s2, y_rows=y_rows, ws=ws, stream=stream, ws2=ws2)
        if fused:
            moe.moe_combine(cfg, y_rows, p2r, w, shared_rows=y_rows[T * k:], out=out, stream=stream)
        else:
            moe.moe_shared_ffn(cfg, inp["x"], inp["ws13"], inp["ws2"], y_shared=y_sh, ws=ws, stream=stream)
            moe.moe_combine(cfg, y_rows, p2r, w, y_sh, out=out, stream=stream)

    note(f"{wl.name}: warmup {args.warmup} + timed {args.steps} steps")
    warm_ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    for _ in range(args.warmup):
        layer()
        stepwise(warm_ev)
    torch.cuda.synchronize()
    touched = int((counts > 0).sum().item())

    lw = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    lw[0].record(stream)
    for _ in range(args.steps):
        layer()
    lw[1].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    layer_fwd_ms = lw[0].elapsed_time(lw[1]) / args.steps

    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
    for i in range(args.steps):
        stepwise(events[i])
    torch.cuda.synchronize()
    up_ms = sum(a.elapsed_time(b) for a, b in events) / args.steps
    del inp, ws, h, y_rows, y_sh, out
    torch.cuda.empty_cache()
    return {"ms_step": ms_step, "up_ms": up_ms, "layer_forward_ms": layer_fwd_ms, "touched": touched}


def time_balanced(args, wl, moe, torch, mi):
    """The layer with the static balanced routing (the routing the Step-5
    full-depth benchmark runs): each step writes the balanced ids and runs
    moe_layer_forward_routed; steps bracketed by HIP events on the stream."""
    cfg, T, H, E = wl.cfg, wl.T, wl.cfg.hidden_size, wl.cfg.num_experts
    inp = mi.make_inputs(wl, "cuda", seed=0)
    ws = moe.workspace(cfg, T)
    stream = torch.cuda.current_stream()
    ids = torch.empty((T, cfg.top_k), dtype=torch.int32, device="cuda")
    out = torch.empty((T, H), dtype=torch.float32, device="cuda")
    counts = torch.empty((E,), dtype=torch.int32, device="cuda")

    def step():
        moe.moe_balanced_ids(cfg, T, ids, stream=stream)
        moe.moe_layer_forward_routed(cfg, inp, ids, out=out, ws=ws, expert_counts=counts, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    touched = int((counts > 0).sum().item())
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(stream)
    for _ in range(args.steps):
        step()
    ev[1].record(stream)
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / args.steps
    del inp, ws, out
    torch.cuda.empty_cache()
    return {"ms_step": ms, "touched": touched}


def time_block(args, wl, moe, torch, mi):
    """moe_block_forward (zero-centred RMSNorm, the layer, fp32 residual add
    in the combine) and the RMSNorm kernel alone, each over args.steps
    launches bracketed by HIP events on the stream."""
    cfg, T, H = wl.cfg, wl.T, wl.cfg.hidden_size
    inp = dict(mi.make_inputs(wl, "cuda", seed=0), **mi.block_inputs(wl, "cuda", seed=0))
    ws = moe.workspace(cfg, T)
    stream = torch.cuda.current_stream()
    out = torch.empty((T, H), dtype=torch.float32, device="cuda")
    x = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    for _ in range(args.warmup):
        moe.moe_block_forward(cfg, inp, resid_out=out, ws=ws, stream=stream)
        moe.moe_rmsnorm(cfg, inp["resid"], inp["norm_weight"], inp["eps"], x=x, stream=stream)
    torch.cuda.synchronize()
    ev[0].record(stream)
    for _ in range(args.steps):
        moe.moe_block_forward(cfg, inp, resid_out=out, ws=ws, stream=stream)
    ev[1].record(stream)
    ev[2].record(stream)
    for _ in range(args.steps):
        moe.moe_rmsnorm(cfg, inp["resid"], inp["norm_weight"], inp["eps"], x=x, stream=stream)
    ev[3].record(stream)
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / args.steps
    norm_us = ev[2].elapsed_time(ev[3]) * 1e3 / args.steps
    norm_bytes = T * H * 4 + T * H * 2 + H * 4          # fp32 rows in, bf16 rows out, the weight
    del inp, ws, out, x
    torch.cuda.empty_cache()
    return {"workload": wl.name, "ms_per_step": ms, "tokens_per_s": T / (ms * 1e-3), "rmsnorm_us": norm_us,
            "rmsnorm_gbs": norm_bytes / (norm_us * 1e-6) / 1e9,
            "rmsnorm_hbm_frac": norm_bytes / (norm_us * 1e-6) / HBM_PEAK}


def time_train(args, wl, moe, torch, mi):
    """One training step of the layer: moe_layer_forward_train then
    moe_layer_backward (dL/dout given), each bracketed by HIP events."""
    cfg, T, H, E, k, I = (wl.cfg, wl.T, wl.cfg.hidden_size, wl.cfg.num_experts, wl.cfg.top_k,
                          wl.cfg.moe_intermediate_size)
    inp = mi.make_inputs(wl, "cuda", seed=0)
    g = torch.Generator(device="cuda").manual_seed(3)
    dout = torch.randn((T, H), generator=g, device="cuda", dtype=torch.float32)
    stream = torch.cuda.current_stream()
    ws = moe.workspace(cfg, T)
    bws = torch.empty(moe.moe_backward_workspace_size(cfg, T), dtype=torch.uint8, device="cuda")
    saved = torch.empty(moe.moe_saved_bytes(cfg, T), dtype=torch.uint8, device="cuda")
    out = torch.empty((T, H), dtype=torch.float32, device="cuda")
    grads = None
    for _ in range(args.warmup):
        moe.moe_layer_forward_train(cfg, inp, out=out, saved=saved, ws=ws, stream=stream)
        grads = moe.moe_layer_backward(cfg, inp, saved, dout, grads=grads, ws=bws, stream=stream)
    torch.cuda.synchronize()
    P = T * k
    ids = saved[:P * 4].view(torch.int32)
    touched = int(torch.unique(ids).numel())
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for i in range(args.steps):
        ev[i][0].record(stream)
        moe.moe_layer_forward_train(cfg, inp, out=out, saved=saved, ws=ws, stream=stream)
        ev[i][1].record(stream)
        moe.moe_layer_backward(cfg, inp, saved, dout, grads=grads, ws=bws, stream=stream)
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    fwd = sum(a.elapsed_time(b) for a, b, _ in ev) / args.steps
    bwd = sum(b.elapsed_time(c) for _, b, c in ev) / args.steps
    # backward FLOPs: data and weight gradients of both projections, routed
    # rows and the shared expert's (two forward GEMMs' worth each)
    rows = P + (T if cfg.share_expert_dim else 0)
    bwd_flops = 2 * (2 * rows * 3 * I * H)
    # HBM floor of the backward: fp32 weight gradients of every expert written
    # once, the touched experts' bf16 weights read once
    grad_bytes = 4 * (E * 3 * I * H + E * H + (3 * cfg.share_expert_dim * H))
    w_bytes = 2 * (touched * 3 * I * H + 3 * cfg.share_expert_dim * H)
    del inp, ws, bws, saved, out, grads, dout
    torch.cuda.empty_cache()
    return {"workload": wl.name, "forward_train_ms": fwd, "backward_ms": bwd, "step_ms": fwd + bwd,
            "tokens_per_s": T / ((fwd + bwd) * 1e-3), "experts_touched": touched,
            "backward_tflops": bwd_flops / (bwd * 1e-3) / 1e12,
            "backward_mfma_frac": bwd_flops / (bwd * 1e-3) / BF16_PEAK,
            "backward_floor_bytes": grad_bytes + w_bytes,
            "backward_hbm_frac": (grad_bytes + w_bytes) / (bwd * 1e-3) / HBM_PEAK}


def bench_decode(args, wl, moe, torch):
    import moe_inputs as mi
    inp = mi.make_inputs(wl, "cuda", seed=0)
    T, k, E, H = wl.T, wl.cfg.top_k, wl.cfg.num_experts, wl.cfg.hidden_size
    ws = moe.workspace(wl.cfg, T)
    out = torch.empty((T, H), dtype=torch.float32, device="cuda")
    counts = torch.empty((E,), dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    for _ in range(max(args.warmup, 3)):
        moe.moe_layer_forward(wl.cfg, inp, out=out, ws=ws, expert_counts=counts, stream=stream)
    torch.cuda.synchronize()
    touched = int((counts > 0).sum().item())
    n = max(args.steps, 20)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(stream)
    for _ in range(n):
        moe.moe_layer_forward(wl.cfg, inp, out=out, ws=ws, stream=stream)
    ev[1].record(stream)
    torch.cuda.synchronize()
    us = ev[0].elapsed_time(ev[1]) * 1e3 / n
    by = layer_bytes(wl, touched)
    # the same layer call captured once into a HIP graph and replayed, as a
    # decode loop would run it (launch gaps removed; the work is identical)
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        moe.moe_layer_forward(wl.cfg, inp, out=out, ws=ws, stream=side)   # warm-up on the capture stream
        side.synchronize()
        with torch.cuda.graph(g, stream=side):
            moe.moe_layer_forward(wl.cfg, inp, out=out, ws=ws, stream=side)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    ev[0].record(stream)
    for _ in range(n):
        g.replay()
    ev[1].record(stream)
    torch.cuda.synchronize()
    us_graph = ev[0].elapsed_time(ev[1]) * 1e3 / n
    del g, inp, ws
    torch.cuda.empty_cache()
    return {"workload": wl.name, "tokens": T, "experts_touched": touched, "us_per_step": us,
            "tokens_per_s": T / (us * 1e-6), "gbs": by / (us * 1e-6) / 1e9, "hbm_frac": by / (us * 1e-6) / HBM_PEAK,
            "us_per_step_graph": us_graph, "hbm_frac_graph": by / (us_graph * 1e-6) / HBM_PEAK,
            "algorithmic_bytes": by}


def cpu_baseline(args, wl, mi):
    """The oracle, as it stands, on the host cores over a bounded token sample
    of the same workload (rows are independent, so tokens/s scales)."""
    import numpy as np
    from oracle import oracle as orc
    inp = mi.make_inputs(wl, "cuda", seed=0)
    host = {k: v.cpu() for k, v in inp.items()}
    del inp
    rng = np.random.default_rng(0)
    n = 4 * orc.num_threads()          # tokens are spread over the threads: calibrate with all busy
    t0 = time.perf_counter()
    orc.layer(wl.cfg, host, tokens=rng.choice(wl.T, n, replace=False))
    dt = time.perf_counter() - t0
    n2 = int(min(wl.T, max(n, n * args.cpu_seconds / max(dt, 1e-3))))
    toks = rng.choice(wl.T, n2, replace=False)
    t0 = time.perf_counter()
    orc.layer(wl.cfg, host, tokens=toks)
    dt2 = time.perf_counter() - t0
    return {"value": n2 / dt2, "unit": "tokens/s", "cores": orc.num_threads(), "kind": "oracle",
            "sample": f"{n2} of {wl.T} tokens of {wl.name} (seeded), full layer per token, {dt2:.1f} s"}


if __name__ == "__main__":
    main()
