#!/usr/bin/env python3
"""Benchmark of the MoE-layer forward on one MI355X.

One step = the whole hot path (route -> permute -> routed experts' up and
down projections with the shared expert -> combine) over one batch of
synthetic tokens whose inputs are already resident in HBM: one
moe_layer_forward call.  The workload of record is the Step-5-Preview-shaped
prefill: 8192 tokens, hidden 4096, 352 routed experts, top-8, expert and
shared intermediate 1536, clipped SwiGLU at 7.0, bf16.

Prints one JSON line with tokens/s, the whole layer's TFLOP/s and bytes/s,
the roofline of the dominant kernel (the first projection + clipped SwiGLU
of the routed experts, with the shared expert as one more group, as the
layer runs it; timed with HIP events on the stream it runs on), the
attainable peaks measured in the same run (a device copy, a vendor bf16
GEMM), the Step-3.5-Flash prefill, the FP8-expert prefill, the 64-token
decode shapes (the memory-side cache flushed between timed calls, medians),
and the oracle timed on the host cores on a bounded token sample.
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
FP8_PEAK = 5.0332e15       # dense fp8 MFMA FLOP/s


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="step5_prefill")
    ap.add_argument("--step35-workload", default="step35_prefill", help="'' to skip the Step-3.5 prefill report")
    ap.add_argument("--decode-workload", default="step5_decode")
    ap.add_argument("--fp8-workload", default="step5_fp8_prefill", help="'' to skip the FP8 report")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--decode-half-workload", default="step5_decode_half",
                    help="decode with the hot bias calibrated so the hot experts take about half of the "
                         "selections; '' to skip")
    ap.add_argument("--no-ep-proxy", action="store_true",
                    help="skip the report on one expert-parallel rank's share (44 experts, MFMA-bound)")
    ap.add_argument("--no-balanced", action="store_true", help="skip the static balanced routing report")
    ap.add_argument("--no-block", action="store_true", help="skip the RMSNorm + residual block report")
    ap.add_argument("--no-train", action="store_true", help="skip the forward + backward training report")
    ap.add_argument("--no-peaks", action="store_true", help="skip measuring the attainable peaks")
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
    the routing touches (and their FP8 block scales), the shared expert and
    router weights, the bias, the input once and the output once."""
    c = wl.cfg
    T, H, E, I, Is = wl.T, c.hidden_size, c.num_experts, c.moe_intermediate_size, c.share_expert_dim
    bpw = 1 if c.expert_dtype == "fp8" else 2
    b = touched * 3 * H * I * bpw + 3 * H * Is * 2 + 2 * E * H + 4 * E + 2 * T * H
    if c.expert_dtype == "fp8":
        b += touched * ((2 * I // 128) * (H // 128) + (H // 128) * (I // 128)) * 4
    b += (2 if c.out_dtype == "bf16" else 4) * T * H
    return b


def shared_in_launch(cfg):
    """The shared expert runs as one more group of the routed launches (bf16
    experts, shared width equal to the experts')."""
    return cfg.expert_dtype == "bf16" and cfg.share_expert_dim > 0 and cfg.share_expert_dim == \
        cfg.moe_intermediate_size


def up_kernel_bytes(wl, touched):
    """Algorithmic bytes of the first-projection launch the layer makes: the
    first-projection weights of every touched expert once (and the shared
    expert's when it is a group of the launch), the activations once.  Its
    output h is an intermediate the method does not need and is not
    counted."""
    c = wl.cfg
    T, H, I, Is = wl.T, c.hidden_size, c.moe_intermediate_size, c.share_expert_dim
    if c.expert_dtype == "fp8":
        # codes + block scales of W13; x read once as E4M3 codes with one fp32 scale per 128 columns
        return touched * (2 * I * H + (2 * I // 128) * (H // 128) * 4) + T * H + T * (H // 128) * 4
    b = touched * 2 * I * H * 2 + T * H * 2
    if shared_in_launch(c):
        b += 2 * Is * H * 2
    return b


def up_kernel_flops(wl):
    c = wl.cfg
    rows = wl.T * c.top_k + (wl.T if shared_in_launch(c) else 0)
    return 2 * rows * 2 * c.moe_intermediate_size * c.hidden_size


_HERE = os.path.dirname(os.path.abspath(__file__))
# workload -> (counter summary under profiles/, source of the kernel it measures)
TRAFFIC_FILES = {
    "step5_prefill": (os.path.join(_HERE, "profiles", "routed_gemms_bf16_step5_prefill_counters.md"),
                      os.path.join(_HERE, "sparse_moe_layer_route_amd", "csrc", "grouped_gemm.hip")),
    "step5_fp8_prefill": (os.path.join(_HERE, "profiles", "routed_gemms_fp8_step5_prefill_counters.md"),
                          os.path.join(_HERE, "sparse_moe_layer_route_amd", "csrc", "fp8_gemm.hip")),
}


def counter_traffic(wl):
    """HBM bytes per launch of the first projection from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary (scaled by a plain copy's
    counts), or None when there is no summary for the workload or the kernel
    source has changed since the counters were taken."""
    import hashlib
    import re
    if wl.name not in TRAFFIC_FILES:
        return None
    summary, src = TRAFFIC_FILES[wl.name]
    if not os.path.exists(summary):
        return None
    text = open(summary).read()
    t = re.search(r"^traffic_bytes_per_launch:\s*(\d+)", text, re.M)
    h = re.search(r"^kernel_source_sha256:\s*([0-9a-f]{64})", text, re.M)
    if not t or not h:
        return None
    if hashlib.sha256(open(src, "rb").read()).hexdigest() != h.group(1):
        return None
    return int(t.group(1))


def note(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def median(xs):
    s = sorted(xs)
    n = len(s)
    return s[n // 2] if n % 2 else 0.5 * (s[n // 2 - 1] + s[n // 2])


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
    peaks = None if args.no_peaks else measure_peaks(torch)
    wl = mi.WORKLOADS[args.workload]
    cfg, T, k, E, H, I = wl.cfg, wl.T, wl.cfg.top_k, wl.cfg.num_experts, wl.cfg.hidden_size, \
        wl.cfg.moe_intermediate_size
    r = time_layer(args, wl, moe, torch, mi)
    ms_step, touched = r["ms_step"], r["touched"]
    tok_s = T / (ms_step * 1e-3)
    res = {
        "metric": METRIC, "value": tok_s, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8_e4m3" if cfg.expert_dtype == "fp8" else "bf16", "data": "synthetic",
        "config": {"workload": wl.name, "tokens": T, "hidden_size": H, "num_experts": E, "top_k": k,
                   "moe_intermediate_size": I, "share_expert_dim": cfg.share_expert_dim,
                   "swiglu_limit": cfg.swiglu_limit, "swiglu_limit_shared": cfg.swiglu_limit_shared,
                   "router_scaling_factor": cfg.router_scaling_factor, "experts_touched": touched,
                   "parallelism": "single GPU"},
    }
    res.update(layer_report(wl, r, peaks))
    res["roofline"] = up_roofline(wl, r, peaks, counter_traffic(wl))
    if peaks:
        res["attainable_peaks"] = peaks

    if args.step35_workload:
        w35 = mi.WORKLOADS[args.step35_workload]
        note(f"{w35.name}")
        r35 = time_layer(args, w35, moe, torch, mi)
        res["step35_prefill"] = dict(layer_report(w35, r35, peaks), workload=w35.name, experts_touched=r35["touched"],
                                     first_projection=up_roofline(w35, r35, peaks, None))

    if args.fp8_workload:
        wf = mi.WORKLOADS[args.fp8_workload]
        note(f"{wf.name}")
        rf = time_layer(args, wf, moe, torch, mi)
        rep = layer_report(wf, rf, peaks)
        fl = layer_flops(wf, rf["touched"])
        rep["fp8_mfma_frac"] = fl / (rf["ms_step"] * 1e-3) / FP8_PEAK
        res["fp8"] = dict(rep, workload=wf.name, experts_touched=rf["touched"],
                          first_projection=up_roofline(wf, rf, peaks, counter_traffic(wf)))

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
        res["ep_rank_proxy"] = {
            "workload": we.name, "experts": we.cfg.num_experts, "tokens": we.T, "experts_touched": r["touched"],
            "ms_per_step": r["ms_step"], "tflops": fl / (r["ms_step"] * 1e-3) / 1e12,
            "mfma_frac": fl / (r["ms_step"] * 1e-3) / BF16_PEAK,
            "first_projection": up_roofline(we, r, peaks, None)}

    if not args.no_decode:
        note(f"decode workload {args.decode_workload}")
        res["decode"] = bench_decode(args, mi.WORKLOADS[args.decode_workload], moe, torch, peaks)
        if args.decode_half_workload:
            base = mi.WORKLOADS[args.decode_half_workload]
            bias, share = calibrate_hot_bias(base, moe, torch, mi)
            note(f"decode with the hot bias calibrated to {bias:.4f} (hot share {share:.3f})")
            rep = bench_decode(args, mi.workload(args.decode_half_workload, hot_bias=bias), moe, torch, peaks)
            rep.update(hot_bias=bias, hot_share=share)
            res["decode_half"] = rep

    if not args.no_cpu_baseline:
        note("CPU baseline (oracle on a token sample)")
        res["cpu_baseline"] = cpu_baseline(args, wl, mi)

    print(json.dumps(res), flush=True)


def layer_report(wl, r, peaks):
    """Whole-layer rates of a timed layer."""
    fl, by = layer_flops(wl, r["touched"]), layer_bytes(wl, r["touched"])
    s = r["ms_step"] * 1e-3
    fp8 = wl.cfg.expert_dtype == "fp8"
    rep = {"ms_per_step": r["ms_step"], "tokens_per_s": wl.T / s, "tflops": fl / s / 1e12,
           "mfma_frac": fl / s / BF16_PEAK, "layer_gbs": by / s / 1e9, "hbm_frac": by / s / HBM_PEAK,
           "layer_roofline_frac": max(fl / (FP8_PEAK if fp8 else BF16_PEAK), by / HBM_PEAK) / s,
           "layer_forward_ms": r["layer_forward_ms"], "algorithmic_bytes": by, "flops": fl}
    if peaks:
        rep["hbm_frac_attainable"] = by / s / (peaks["hbm_gbs"] * 1e9)
        if not fp8:
            rep["mfma_frac_attainable"] = fl / s / (peaks["bf16_tflops"] * 1e12)
    return rep


def up_roofline(wl, r, peaks, traffic):
    """The first projection's launch as the layer makes it: algorithmic bytes
    per launch / its average duration (HIP events on its stream)."""
    c = wl.cfg
    fp8 = c.expert_dtype == "fp8"
    b = up_kernel_bytes(wl, r["touched"])
    fl = up_kernel_flops(wl)
    s = r["up_ms"] * 1e-3
    kern = ("f8::kernel<0> (FP8 routed experts' first projection + clipped SwiGLU + h quantisation)" if fp8 else
            "gg::kernel<0, true, 256, 256> (routed experts' first projection + clipped SwiGLU"
            + (", shared expert as one more group)" if shared_in_launch(c) else ")"))
    out = {"kernel": kern, "bound": "hbm", "achieved": b / s / 1e9, "peak": HBM_PEAK / 1e9, "unit": "GB/s",
           "frac": b / s / HBM_PEAK, "traffic": traffic, "avg_ms": r["up_ms"], "algorithmic_bytes": b,
           "tflops": fl / s / 1e12, "mfma_frac": fl / s / (FP8_PEAK if fp8 else BF16_PEAK)}
    if peaks:
        out["frac_attainable"] = b / s / (peaks["hbm_gbs"] * 1e9)
    return out


def measure_peaks(torch):
    """Attainable peaks on this chip: HBM as the fastest of a device-to-device
    copy of 2 GiB (bytes read + written per second) and two read-only
    streams over 2 GiB, an int64 sum and a bf16 matrix-vector product (bytes
    read per second), and the vendor library's bf16 GEMM of 8192 x 8192 x
    8192 (hipBLASLt through torch.matmul); medians of 10."""
    note("measuring attainable peaks (device copy, vendor bf16 GEMM)")
    n = 2 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ts = []
    for i in range(13):
        ev[0].record()
        dst.copy_(src)
        ev[1].record()
        torch.cuda.synchronize()
        if i >= 3:
            ts.append(ev[0].elapsed_time(ev[1]) * 1e-3)
    copy = 2 * n / median(ts)
    del dst
    # read-only streams over the same 2 GiB (bytes read per second): an int64
    # sum and a bf16 matrix-vector product (the vendor library's GEMV)
    i64 = src.view(torch.int64)
    mat = src.view(torch.bfloat16).view(32768, 32768)
    vec = torch.ones(32768, device="cuda", dtype=torch.bfloat16)
    reads = []
    for f in (lambda: i64.sum(), lambda: torch.mv(mat, vec)):
        ts = []
        for i in range(13):
            ev[0].record()
            f()
            ev[1].record()
            torch.cuda.synchronize()
            if i >= 3:
                ts.append(ev[0].elapsed_time(ev[1]) * 1e-3)
        reads.append(n / median(ts))
    read = max(reads)
    del src, i64, mat, vec
    hbm = max(copy, read)
    a = torch.randn((8192, 8192), device="cuda", dtype=torch.bfloat16)
    b = torch.randn((8192, 8192), device="cuda", dtype=torch.bfloat16)
    ts = []
    for i in range(13):
        ev[0].record()
        torch.matmul(a, b)
        ev[1].record()
        torch.cuda.synchronize()
        if i >= 3:
            ts.append(ev[0].elapsed_time(ev[1]) * 1e-3)
    gemm = 2 * 8192 ** 3 / median(ts)
    del a, b
    torch.cuda.empty_cache()
    return {"hbm_gbs": hbm / 1e9,
            "hbm_how": "the fastest of a 2 GiB device-to-device copy (read + written bytes), an int64 sum over "
                       "2 GiB and a bf16 matrix-vector product over a 2 GiB matrix (read bytes), medians of 10",
            "hbm_copy_gbs": copy / 1e9, "hbm_read_gbs": read / 1e9,
            "bf16_tflops": gemm / 1e12, "bf16_how": "torch.matmul (hipBLASLt) 8192^3 bf16, median of 10"}


def time_layer(args, wl, moe, torch, mi):
    """Warm up, then time args.steps steps, each one moe_layer_forward call,
    bracketed by a synchronisation on both sides.  Then, as a second timed
    region of as many steps, the same layer through its separate entry points
    (the same launches in the same order), with the first projection
    bracketed by HIP events on its stream: that launch's average duration
    for the roofline object."""
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
    fused = shared_in_launch(cfg)
    y_rows = moe.binding.expert_rows(cfg, T * k + (T if fused else 0), dev)
    y_sh = None if fused or not cfg.share_expert_dim else torch.empty((T, H), dtype=torch.float32, device=dev)
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
        elif y_sh is not None:
            moe.moe_shared_ffn(cfg, inp["x"], inp["ws13"], inp["ws2"], y_shared=y_sh, ws=ws, stream=stream)
            moe.moe_combine(cfg, y_rows, p2r, w, y_sh, out=out, stream=stream)
        else:
            moe.moe_combine(cfg, y_rows, p2r, w, out=out, stream=stream)

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
    in the combine), then its front end both ways: the RMSNorm kernel and
    moe_route as two steps, and moe_rmsnorm_route (one fused pass from 512
    tokens); each over args.steps launches bracketed by HIP events on the
    stream."""
    cfg, T, H = wl.cfg, wl.T, wl.cfg.hidden_size
    inp = dict(mi.make_inputs(wl, "cuda", seed=0), **mi.block_inputs(wl, "cuda", seed=0))
    ws = moe.workspace(cfg, T)
    stream = torch.cuda.current_stream()
    out = torch.empty((T, H), dtype=torch.float32, device="cuda")
    x = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    ids = torch.empty((T, cfg.top_k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, cfg.top_k), dtype=torch.float32, device="cuda")
    norm = lambda: moe.moe_rmsnorm(cfg, inp["resid"], inp["norm_weight"], inp["eps"], x=x, stream=stream)
    route = lambda: moe.moe_route(cfg, x, inp["w_router"], inp["router_bias"], topk_ids=ids, topk_w=w, ws=ws,
                                  stream=stream)
    fused = lambda: moe.moe_rmsnorm_route(cfg, inp["resid"], inp["norm_weight"], inp["eps"], inp["w_router"],
                                          inp["router_bias"], x=x, topk_ids=ids, topk_w=w, ws=ws, stream=stream)
    block = lambda: moe.moe_block_forward(cfg, inp, resid_out=out, ws=ws, stream=stream)
    regions = [block, norm, route, fused]
    for _ in range(args.warmup):
        for f in regions:
            f()
    torch.cuda.synchronize()
    us = []
    for f in regions:
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        for _ in range(args.steps):
            f()
        ev[1].record(stream)
        torch.cuda.synchronize()
        us.append(ev[0].elapsed_time(ev[1]) * 1e3 / args.steps)
    block_us, norm_us, route_us, fused_us = us
    ms = block_us * 1e-3
    norm_bytes = T * H * 4 + T * H * 2 + H * 4          # fp32 rows in, bf16 rows out, the weight
    del inp, ws, out, x, ids, w
    torch.cuda.empty_cache()
    return {"workload": wl.name, "ms_per_step": ms, "tokens_per_s": T / (ms * 1e-3), "rmsnorm_us": norm_us,
            "rmsnorm_gbs": norm_bytes / (norm_us * 1e-6) / 1e9,
            "rmsnorm_hbm_frac": norm_bytes / (norm_us * 1e-6) / HBM_PEAK,
            "route_us": route_us, "norm_route_two_steps_us": norm_us + route_us,
            "norm_route_fused_us": fused_us}


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


def hot_share(wl, moe, torch, inp):
    """Share of the (token, slot) selections that go to the hot experts."""
    ids, _ = moe.moe_route(wl.cfg, inp["x"], inp["w_router"], inp["router_bias"])
    hot = torch.zeros(wl.cfg.num_experts, dtype=torch.bool, device="cuda")
    hot[inp["hot_experts"]] = True
    return float(hot[ids.long()].float().mean().item())


def calibrate_hot_bias(wl, moe, torch, mi, target=0.5, tol=0.02):
    """Bisection on the hot experts' bias until they take target +- tol of
    the decode batch's selections (the routing itself runs on the GPU)."""
    inp = mi.make_inputs(wl, "cuda", seed=0)
    base = inp["router_bias"].clone()
    base[inp["hot_experts"]] -= wl.hot_bias
    lo, hi = 0.0, 1.0
    bias, share = hi, 1.0
    for _ in range(30):
        bias = 0.5 * (lo + hi)
        inp["router_bias"] = base.clone()
        inp["router_bias"][inp["hot_experts"]] += bias
        share = hot_share(wl, moe, torch, inp)
        if abs(share - target) <= tol:
            break
        if share < target:
            lo = bias
        else:
            hi = bias
    del inp
    torch.cuda.empty_cache()
    return bias, share


def bench_decode(args, wl, moe, torch, peaks):
    """The decode layer call, one at a time: before each timed call an
    untimed read of a 1 GiB buffer fills the 256 MiB memory-side cache with
    clean lines of other data (as the previous layer's weight reads would),
    so the call streams its expert weights from HBM; the median of the
    per-call HIP-event times.  The same for the call captured once in a HIP
    graph and replayed.  Also reported: the median after a 1 GiB write
    instead, which leaves the cache full of dirty lines whose write-back to
    HBM then runs inside the timed call."""
    import moe_inputs as mi
    inp = mi.make_inputs(wl, "cuda", seed=0)
    T, k, E, H = wl.T, wl.cfg.top_k, wl.cfg.num_experts, wl.cfg.hidden_size
    ws = moe.workspace(wl.cfg, T)
    out = torch.empty((T, H), dtype=torch.float32, device="cuda")
    counts = torch.empty((E,), dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    flush_sum = torch.empty((), dtype=torch.float32, device="cuda")
    for _ in range(max(args.warmup, 3)):
        moe.moe_layer_forward(wl.cfg, inp, out=out, ws=ws, expert_counts=counts, stream=stream)
    torch.cuda.synchronize()
    touched = int((counts > 0).sum().item())
    n = max(args.steps, 20)

    def timed(fn, dirty=False):
        ts = []
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        for _ in range(n):
            if dirty:
                flush.fill_(1.0)
            else:
                torch.sum(flush, dim=0, out=flush_sum)
            ev[0].record(stream)
            fn()
            ev[1].record(stream)
            torch.cuda.synchronize()
            ts.append(ev[0].elapsed_time(ev[1]) * 1e3)
        return median(ts)

    us = timed(lambda: moe.moe_layer_forward(wl.cfg, inp, out=out, ws=ws, stream=stream))
    us_dirty = timed(lambda: moe.moe_layer_forward(wl.cfg, inp, out=out, ws=ws, stream=stream), dirty=True)
    by = layer_bytes(wl, touched)
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
    us_graph = timed(g.replay)
    del g, inp, ws, flush, flush_sum
    torch.cuda.empty_cache()
    rep = {"workload": wl.name, "tokens": T, "experts_touched": touched, "us_per_step": us,
           "tokens_per_s": T / (us * 1e-6), "gbs": by / (us * 1e-6) / 1e9, "hbm_frac": by / (us * 1e-6) / HBM_PEAK,
           "us_per_step_graph": us_graph, "hbm_frac_graph": by / (us_graph * 1e-6) / HBM_PEAK,
           "us_per_step_after_write_flush": us_dirty,
           "algorithmic_bytes": by,
           "timing": "median of %d calls, 1 GiB of other data read before each (untimed)" % n}
    if peaks:
        rep["hbm_frac_attainable"] = by / (us * 1e-6) / (peaks["hbm_gbs"] * 1e9)
    return rep


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
