"""Benchmark of the NVFP4 MoE hot path on one MI355X.

A step is one whole MoE layer forward over one batch: route + permute -> up/gate grouped
GEMM with fused SwiGLU -> down grouped GEMM -> weighted unpermute-reduce, all through the
C ABI. Default workload: the decode MoE layer with 256 experts, top-8, 512 tokens
(~16 rows per expert), hidden 6144, expert FFN 2048, NVFP4 weights, bf16 activations
(W4A16) -- the workload behind the pages' "0.8-55 TFLOPS at per-expert M=16-64" ("The 2x
Gap", section "The Investigation So Far").

Prints ONE JSON line: throughput (algorithmic TFLOP/s of the layer, from the wall clock
around steps that carry no instrumentation), the dominant kernel's HBM roofline
(weight+scale+activation bytes per launch / launch time from HIP events recorded on the
kernels' stream in an instrumented pass of as many steps), and the oracle's CPU rate on a
bounded sample of the same workload.

The line also carries the workload's token sweep (each token count's layer step replayed
from a HIP graph after a 1 GiB read that evicts the Infinity Cache: median and p10/p90 of
the replays) and the box's measured ceilings (a plain read of 4 GiB through torch, and a
large bf16 torch.mm), each fraction given against both the spec peak and the measured one.

Usage: python bench.py [--steps K] [--warmup W] [--tokens T] [--workload NAME]
       [--format nvfp4|mxfp4] [--no-cpu-baseline] [--no-sweep] [--no-ceilings]
       [--sweep FILE] [--sweep-tokens T1,T2,...] [--copy-calibration]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0      # dense; the f16 MFMA runs at the same rate
FP4_PEAK_TFLOPS = 10100.0
FP8_PEAK_TFLOPS = 5000.0
PAGES_DECODE_TFLOPS = (0.8, 55.0)   # RTX PRO 6000 (SM120), FP4, per-expert M=16-64


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=30)
    p.add_argument("--workload", default="decode")
    p.add_argument("--tokens", type=int, default=None)
    p.add_argument("--format", default="nvfp4", choices=["nvfp4", "mxfp4"],
                   help="mxfp4: the layer with MXFP4 weights, activations and h (W4A4 on the scaled "
                        "FP4 matrix cores)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--combine", type=int, default=0, choices=[0, 1],
                   help="1: the down GEMM and the weighted reduce as one call (the combine entry points)")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--sweep", default=None, help="also write per-T results of the workload's sweep to FILE")
    p.add_argument("--sweep-tokens", default=None,
                   help="comma-separated token counts that replace the workload's sweep points")
    p.add_argument("--no-sweep", action="store_true",
                   help="leave out the cold token sweep that the default line carries")
    p.add_argument("--no-ceilings", action="store_true",
                   help="leave out the measured HBM-read and bf16 torch.mm ceilings")
    p.add_argument("--copy-calibration", action="store_true",
                   help="run a plain 1 GiB device copy (for scaling HBM counters) and exit")
    return p.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: the expert- and tensor-parallel sharding of the layer "
              "over several GPUs is not implemented; use --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    from nvfp4_block_scaled_moe_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    from nvfp4_block_scaled_moe_amd import inputs, layer, ops

    dev = "cuda"
    if args.copy_calibration:
        a = torch.empty(1 << 28, dtype=torch.float32, device=dev)   # 1 GiB
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": a.numel() * 4, "copy_calibration_bytes_written": b.numel() * 4}))
        return

    wl = inputs.WORKLOADS[args.workload]
    T = args.tokens or wl.T
    mode = ops.W4A16 if wl.mode == "w4a16" else ops.W4A4
    mx = args.format == "mxfp4"
    if mx:
        mode = MXFP4
    t0 = time.time()
    w = None if wl.name == "dense" else (layer.quantize_experts_mxfp4(wl, dev) if mx else layer.quantize_experts(wl, dev))
    x = inputs.activations_bf16(wl, T).to(dev)
    lg = inputs.router_logits(wl, T).to(dev)
    torch.cuda.synchronize()
    setup_s = time.time() - t0
    print(f"[bench] setup {setup_s:.1f}s: {wl.name} T={T} E={wl.E} k={wl.k} H={wl.H} F={wl.F} "
          f"mode={'mxfp4' if mx else wl.mode}",
          file=sys.stderr, flush=True)

    if wl.name == "dense":
        print(json.dumps(dense_line(torch, ops, inputs, wl, args, T)), flush=True)
        return
    res = measure(torch, ops, layer, wl, w, x, lg, T, mode, args.steps, args.warmup, combine=bool(args.combine))
    ceil = None if args.no_ceilings else ceilings(torch)
    line = dict(
        metric="MoE NVFP4 grouped-GEMM TFLOPS + weight GB/s vs tokens/expert, % roofline",
        value=round(res["tflops"], 2), unit="TFLOP/s", n_gpus=1, steps=args.steps, warmup=args.warmup,
        ms_per_step=round(res["ms_per_step"], 4), higher_is_better=True, scaling="weak",
        vs_baseline=(round(res["tflops"] / PAGES_DECODE_TFLOPS[1], 2)
                     if (wl.name == "decode" and T == 512) else None),
        dtype="fp4" if mx else "f16", data="synthetic",
        config=dict(workload=describe(wl, T, mx), tokens=T, experts=wl.E, top_k=wl.k, hidden=wl.H,
                    ffn=wl.F, mode="MXFP4 W4A4" if mx else wl.mode.upper(),
                    tokens_per_expert=round(T * wl.k / wl.E, 3), touched_experts=res["touched"],
                    compute=("MXFP4 weights and activations on v_mfma_scale_f32_16x16x128_f8f6f4 (UE8M0 "
                             "scales applied by the matrix cores), fp32 accumulation" if mx else
                             "NVFP4 weights decoded exactly to f16, v_mfma_f32_16x16x32_f16, fp32 accumulation")),
        weight_GBps=round(res["weight_gbs"], 1),
        weight_hbm_frac=round(res["weight_gbs"] / HBM_PEAK_GBS, 4),
        step_us=res["step_us"], stage_us=res["stage_us"], up_gemm_path=res["up_path"],
        roofline=res.get("roofline"),
        baseline_context=("pages: 0.8-55 TFLOPS for FP4 MoE GEMMs at per-expert M=16-64 (256 experts, "
                          "top-8, 512 concurrent) on RTX PRO 6000 Blackwell SM120; vs_baseline divides by 55"),
    )
    if line["roofline"] is not None:
        line["roofline"]["traffic"] = measured_traffic(wl, T, mx)
    if ceil is not None:
        line["measured_ceilings"] = ceil
        rf = line["roofline"]
        if rf is not None and rf["unit"] == "GB/s":
            rf["frac_of_measured_read"] = round(rf["achieved"] / ceil["hbm_read_GBps"], 4)
        elif rf is not None and rf.get("peak") == BF16_PEAK_TFLOPS:
            rf["frac_of_measured_bf16_mm"] = round(rf["achieved"] / ceil["bf16_mm_TFLOPs"], 4)
        elif rf is not None and rf.get("peak") == FP4_PEAK_TFLOPS and ceil.get("mxfp4_scaled_mm_TFLOPs"):
            rf["frac_of_measured_mxfp4_mm"] = round(rf["achieved"] / ceil["mxfp4_scaled_mm_TFLOPs"], 4)
        line["weight_frac_of_measured_read"] = round(res["weight_gbs"] / ceil["hbm_read_GBps"], 4)
    points = [int(t) for t in args.sweep_tokens.split(",")] if args.sweep_tokens else wl.sweep
    if points and not args.no_sweep:
        line["token_sweep_cold"] = token_sweep(torch, ops, layer, inputs, wl, w, mode, dev, args, points,
                                               ceil["hbm_read_GBps"] if ceil else None)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(torch, wl, w, x, lg, T, mode, args.cpu_seconds)
    else:
        line["cpu_baseline"] = None
    if args.sweep:
        rows = []
        for Ts in points or (T,):
            xs = inputs.activations_bf16(wl, Ts).to(dev)
            ls = inputs.router_logits(wl, Ts).to(dev)
            r = measure(torch, ops, layer, wl, w, xs, ls, Ts, mode, max(5, args.steps // 2), 2, graph=True,
                        combine=bool(args.combine))
            rows.append(dict(tokens=Ts, tokens_per_expert=Ts * wl.k / wl.E, **{k: v for k, v in r.items()}))
            print(f"[bench] sweep T={Ts}: {r['tflops']:.1f} TFLOP/s, weights {r['weight_gbs']:.0f} GB/s, "
                  f"cold {r['cold_ms_per_step']:.4f} ms ({r['cold_weight_gbs']:.0f} GB/s)",
                  file=sys.stderr, flush=True)
        with open(args.sweep, "w") as f:
            json.dump(dict(workload=wl.name, rows=rows), f, indent=1)
    print(json.dumps(line), flush=True)


def kernel_source_sha(src_name):
    """sha256 prefix over a kernel file and the headers it includes (the epilogue lives in
    gemm_common.h), as recorded in the committed traffic summaries."""
    import hashlib
    h = hashlib.sha256()
    for name in (src_name, "gemm_common.h", "common.h", "kernels.h"):
        with open(os.path.join(ROOT, "nvfp4_block_scaled_moe_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(wl, T, mx=False):
    """HBM bytes per up/gate launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE summary
    (copy-calibrated), or None when none covers this workload or the kernel source has
    changed since the counters were taken."""
    import hashlib
    import re
    known = {("decode", 512, False): ("gemm_stream_decode512_traffic.md", "gemm_stream.hip"),
             ("prefill", 8192, False): ("gemm_large_prefill8192_traffic.md", "gemm_large.hip"),
             ("prefill", 8192, True): ("gemm_mx_prefill8192_traffic.md", "gemm_mx.hip")}
    if (wl.name, T, mx) not in known:
        return None
    prof_name, src_name = known[(wl.name, T, mx)]
    prof = os.path.join(ROOT, "profiles", prof_name)
    try:
        text = open(prof).read()
        sha = kernel_source_sha(src_name)
    except OSError:
        return None
    m_sha = re.search(r"kernel_source_sha256_prefix:\s*([0-9a-f]+)", text)
    m_b = re.search(r"up_gate_traffic_bytes_per_launch:\s*([0-9]+)", text)
    if not (m_sha and m_b) or m_sha.group(1) != sha:
        return None
    return int(m_b.group(1))


def describe(wl, T, mx=False):
    return (f"{wl.name} MoE layer: {wl.E} experts, top-{wl.k}, {T} tokens, hidden {wl.H}, "
            f"expert FFN {wl.F}, " + ("MXFP4 W4A4" if mx else wl.mode.upper())
            + (", FP8 activations" if wl.act == "fp8" else "")
            + (f", Zipf({wl.zipf}) routing bias" if wl.zipf else ""))


MXFP4 = "mxfp4"   # bench-local tag for the MXFP4 layer (not a library mode)


def layer_work(wl, T, touched, mx=False):
    """Algorithmic flops and the touched experts' weight bytes: packed codes (1/2 B) plus
    E4M3 scales per 16 (1/16 B) for NVFP4, UE8M0 scales per 32 (1/32 B) for MXFP4."""
    S = T * wl.k
    bpw = 17 / 32 if mx else 9 / 16
    flops = 2.0 * S * (2 * wl.F * wl.H + wl.H * wl.F)
    w13 = touched * (2 * wl.F) * wl.H * bpw
    w2 = touched * wl.H * wl.F * bpw
    return flops, w13, w2


def pct(vals, q):
    """q-th percentile (0..100) of a list, linear interpolation."""
    import numpy as np
    return float(np.percentile(np.asarray(vals, dtype=np.float64), q))


def stats_us(vals_us):
    return dict(mean=round(sum(vals_us) / len(vals_us), 2), median=round(pct(vals_us, 50), 2),
                p10=round(pct(vals_us, 10), 2), p90=round(pct(vals_us, 90), 2), n=len(vals_us))


def make_step(torch, ops, wl, w, x, lg, T, mode, paths, combine=False):
    """One layer forward as a closure; ev (7 events or None) brackets the stages (with
    ``combine`` the down stage holds the weighted reduce and the reduce stage is empty)."""
    k = wl.k
    fp8 = wl.act == "fp8"
    S = T * k
    mx = mode == MXFP4

    def step(ev=None):
        mark = (lambda i: ev[i].record()) if ev else (lambda i: None)
        mark(0)
        if mode == ops.W4A16:   # routing + the token rows' preparation (one launch up to 16 tokens)
            rr = ops.moe_dispatch_w4a16(lg, x, k, fp8_act=fp8)
        else:
            xx = ops.act_fp8_e4m3_roundtrip(x) if fp8 else x
            rr = ops.moe_route_permute(lg, k)
        mark(1)
        common = dict(expert_offsets=rr["expert_offsets"], active_experts=rr["active_experts"],
                      n_active=rr["n_active"])
        if mx:
            xq, xs = ops.mxfp4_quantize(xx)
            mark(2)
            hq, hs = ops.moe_grouped_gemm_mxfp4_swiglu_q(xq, xs, w.w13_t, gather_index=rr["sorted_slot"],
                                                         gather_div=k, rows=S, **common)
            mark(3)
            paths["up"] = "mx"
            mark(4)   # h is quantized by the up/gate epilogue
            if combine:
                out = ops.moe_grouped_gemm_mxfp4_combine(hq, hs, w.w2_t, sorted_slot=rr["sorted_slot"],
                                                         slot_to_row=rr["slot_to_row"], topk_w=rr["topk_w"],
                                                         **common)
            else:
                y = ops.moe_grouped_gemm_mxfp4(ops.EPI_NONE, hq, hs, w.w2_t, rows=S, out_dtype=torch.float32,
                                               **common)
        elif mode == ops.W4A16:
            mark(2)
            h = ops.moe_grouped_gemm_nvfp4(ops.W4A16_PREPARED, ops.EPI_SWIGLU, rr["x_prep"], w.w13_t,
                                           gather_index=rr["sorted_slot"], gather_div=k, rows=S, a_rows=T,
                                           out_dtype=torch.bfloat16, **common)
            mark(3)
            paths["up"] = ops.last_dispatch()
            mark(4)
            if combine:
                out = ops.moe_grouped_gemm_nvfp4_combine(ops.W4A16, h, w.w2_t, sorted_slot=rr["sorted_slot"],
                                                         slot_to_row=rr["slot_to_row"], topk_w=rr["topk_w"],
                                                         **common)
            else:
                y = ops.moe_grouped_gemm_nvfp4(ops.W4A16, ops.EPI_NONE, h, w.w2_t,
                                               rows=S, out_dtype=torch.float32, **common)
        else:
            xq, xs, xg = ops.nvfp4_quantize(xx)
            mark(2)
            h, amax = ops.moe_grouped_gemm_nvfp4(ops.W4A4, ops.EPI_SWIGLU, xq, w.w13_t,
                                                 a_scales=xs, a_g=xg, gather_index=rr["sorted_slot"],
                                                 gather_div=k, rows=S, out_dtype=torch.float32,
                                                 want_amax=True, **common)
            mark(3)
            paths["up"] = ops.last_dispatch()
            hq, hs, hg = ops.nvfp4_quantize(h, amax=amax)
            mark(4)
            if combine:
                out = ops.moe_grouped_gemm_nvfp4_combine(ops.W4A4, hq, w.w2_t, sorted_slot=rr["sorted_slot"],
                                                         slot_to_row=rr["slot_to_row"], topk_w=rr["topk_w"],
                                                         a_scales=hs, a_g=hg, **common)
            else:
                y = ops.moe_grouped_gemm_nvfp4(ops.W4A4, ops.EPI_NONE, hq, w.w2_t,
                                               a_scales=hs, a_g=hg, rows=S, out_dtype=torch.float32, **common)
        mark(5)
        if not combine:
            out = ops.moe_unpermute_reduce(y, rr["slot_to_row"], rr["topk_w"])
        mark(6)
        return out
    return step


def graph_times(torch, step, steps, warm_reps, dev):
    """Capture one layer step in a HIP graph; per-replay device time (us) warm (back to back)
    and cold (each replay after a 1 GiB read, outside the timed events, that evicts the 256 MB
    Infinity Cache, which could otherwise hold a small layer's touched weights between replays;
    a read leaves clean lines, so no write-back lands in the replay)."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    g.replay()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(warm_reps)]
    for a, b in ev:
        a.record()
        g.replay()
        b.record()
    torch.cuda.synchronize()
    warm = [a.elapsed_time(b) * 1e3 for a, b in ev]
    scratch = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    sink = torch.empty((), dtype=torch.float32, device=dev)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in ev:
        torch.sum(scratch, dim=0, out=sink)
        a.record()
        g.replay()
        b.record()
    torch.cuda.synchronize()
    cold = [a.elapsed_time(b) * 1e3 for a, b in ev]
    del scratch, sink, g
    return warm, cold


def measure(torch, ops, layer, wl, w, x, lg, T, mode, steps, warmup, graph=False, combine=False):
    """Time `steps` eager layer forwards with nothing else on the stream (the headline rate),
    then two instrumented passes of `steps` forwards each: one HIP event per step boundary
    (per-step device times: median, p10, p90) and seven events per step bracketing every stage
    (stage means; the up/gate call's time for the roofline). Events go on the current stream,
    the stream every library call is launched on; each event record costs the GPU a few
    microseconds (about 3 us each, measured: 7 per decode step added ~22 us), which is why the
    headline pass carries none."""
    k = wl.k
    S = T * k
    r = ops.moe_route_permute(lg, k)
    torch.cuda.synchronize()
    touched = int(r["n_active"].item())
    mx = mode == MXFP4
    flops, w13_bytes, w2_bytes = layer_work(wl, T, touched, mx)
    paths = {}
    step = make_step(torch, ops, wl, w, x, lg, T, mode, paths, combine)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    up_path = paths["up"]
    if graph:
        warm, cold = graph_times(torch, step, steps, max(5, steps // 2), x.device)
        ms = sum(warm) / len(warm) / 1e3
        cold_ms = sum(cold) / len(cold) / 1e3
        stage = None
        step_us = None
    else:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            step()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / steps
        bounds = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        bounds[0].record()
        for i in range(steps):
            step()
            bounds[i + 1].record()
        torch.cuda.synchronize()
        step_us = stats_us([1e3 * bounds[i].elapsed_time(bounds[i + 1]) for i in range(steps)])
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(7)] for _ in range(steps)]
        for i in range(steps):
            step(evs[i])
        torch.cuda.synchronize()
        names = ["route_permute", "quantize_x", "up_gate_swiglu", "quantize_h", "down", "unpermute_reduce"]
        per = {n: [1e3 * e[j].elapsed_time(e[j + 1]) for e in evs] for j, n in enumerate(names)}
        stage = {n: round(sum(v) / len(v), 2) for n, v in per.items()}
        step_us["staged_mean"] = round(sum(1e3 * e[0].elapsed_time(e[6]) for e in evs) / steps, 2)
    act_in = T * wl.H * (2 if mode == ops.W4A16 else (17 / 32 if mx else 9 / 16))
    h_bytes = S * wl.F * (2 if mode == ops.W4A16 else (17 / 32 if mx else 4))
    up_bytes = w13_bytes + act_in + h_bytes
    up_flops = 2.0 * S * 2 * wl.F * wl.H
    res = dict(ms_per_step=ms, tflops=flops / (ms * 1e-3) / 1e12,
               weight_gbs=(w13_bytes + w2_bytes) / (ms * 1e-3) / 1e9, touched=touched, stage_us=stage,
               step_us=step_us,
               **(dict(cold_ms_per_step=cold_ms, cold_weight_gbs=(w13_bytes + w2_bytes) / (cold_ms * 1e-3) / 1e9,
                       cold_us=stats_us(cold))
                  if graph else {}),
               up_path="mx" if mx else ("mfma" if up_path == ops.PATH_MFMA else "stream"))
    if stage:
        up = stats_us(per["up_gate_swiglu"])
        up_us = up["mean"]
        timing = dict(launch_us=up_us, launch_us_median=up["median"], launch_us_p10=up["p10"],
                      launch_us_p90=up["p90"], launches=up["n"])
        if mx:
            ach = up_flops / (up_us * 1e-6) / 1e12
            res["roofline"] = dict(
                bound="mfma", kernel="gemm_mx_kernel (MXFP4 up/gate + SwiGLU, h quantized in the epilogue)",
                achieved=round(ach, 1), peak=FP4_PEAK_TFLOPS, unit="TFLOP/s", frac=round(ach / FP4_PEAK_TFLOPS, 4),
                traffic=None, flops_per_launch=up_flops, **timing,
                timed="HIP events around the moe_grouped_gemm_mxfp4_swiglu_q call: mtile_schedule_kernel + "
                      "gemm_mx_kernel",
                flops_note="2*S*2F*H useful flops (rows of ragged m-tiles padded on the GPU are not counted); "
                           "dense FP4 MFMA peak",
                weight_GBps_up=round(w13_bytes / (up_us * 1e-6) / 1e9, 1))
        elif up_path == ops.PATH_MFMA:
            ach = up_flops / (up_us * 1e-6) / 1e12
            res["roofline"] = dict(
                bound="mfma", kernel="gemm_large_kernel (up/gate + SwiGLU)", achieved=round(ach, 1),
                peak=BF16_PEAK_TFLOPS, unit="TFLOP/s", frac=round(ach / BF16_PEAK_TFLOPS, 4), traffic=None,
                flops_per_launch=up_flops, **timing,
                timed="HIP events around the moe_grouped_gemm_nvfp4 call: " +
                      ("act_prep_fp4_kernel (also builds the m-tile list)" if mode == ops.W4A4 else
                       "mtile_schedule_kernel (rows prepared by moe_dispatch_w4a16)") + " + gemm_large_kernel",
                flops_note="2*S*2F*H useful flops (rows of ragged m-tiles padded on the GPU are not counted); "
                           "f16 MFMA peak (the exact NVFP4 decode runs on v_mfma_f32_16x16x32_f16)")
            if mode == ops.W4A4:
                res["roofline"]["fp4_peak_frac"] = round(ach / FP4_PEAK_TFLOPS, 4)
        else:
            ach = up_bytes / (up_us * 1e-6) / 1e9
            res["roofline"] = dict(
                bound="hbm", kernel="gemm_stream_kernel (up/gate + SwiGLU)", achieved=round(ach, 1),
                peak=HBM_PEAK_GBS, unit="GB/s", frac=round(ach / HBM_PEAK_GBS, 4), traffic=None,
                bytes_per_launch=int(up_bytes), **timing,
                timed="HIP events around the moe_grouped_gemm_nvfp4 call: gemm_stream_kernel" +
                      (" (W4A16 rows prepared by moe_dispatch_w4a16 in the routing stage)" if mode == ops.W4A16
                       else ""),
                bytes_note="W13 packed+scales of touched experts (9/16 B/weight) + activations in + h out")
    return res


def ceilings(torch):
    """The box's measured ceilings: the best of three plain reads of 4 GiB through torch
    (a full float32 sum, float32 row sums, a bf16 matrix-vector product; bytes read / call
    time) and a bf16 torch.mm of 8192 x 8192 x 8192 (hipBLASLt), each timed with HIP events
    over 10 calls after 3 warm-ups."""
    dev = "cuda"
    out = {}

    def timed(fn, reps=10):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / reps     # s per call
    a = torch.ones(1 << 30, dtype=torch.float32, device=dev)          # 4 GiB
    rates = {"sum_f32": a.numel() * 4 / timed(lambda: a.sum()),
             "row_sums_f32_[2^20,1024]": a.numel() * 4 / timed(lambda: a.view(1 << 20, 1024).sum(1))}
    b = a.view(torch.bfloat16).view(65536, 32768)                     # the same 4 GiB as a bf16 matrix
    v = torch.ones(32768, dtype=torch.bfloat16, device=dev)
    rates["gemv_bf16_[65536,32768]"] = b.numel() * 2 / timed(lambda: torch.mv(b, v))
    del a, b, v
    best = max(rates, key=rates.get)
    out["hbm_read_GBps"] = round(rates[best] / 1e9, 1)
    out["hbm_read_kernel"] = f"torch {best} over 4 GiB (best of {', '.join(rates)})"
    out["hbm_read_all_GBps"] = {k: round(v / 1e9, 1) for k, v in rates.items()}
    out["hbm_read_frac_of_spec"] = round(rates[best] / 1e9 / HBM_PEAK_GBS, 4)
    m = 8192
    x = torch.randn((m, m), dtype=torch.bfloat16, device=dev)
    y = torch.randn((m, m), dtype=torch.bfloat16, device=dev)
    t = timed(lambda: torch.mm(x, y))
    out["bf16_mm_TFLOPs"] = round(2.0 * m ** 3 / t / 1e12, 1)
    out["bf16_mm_shape"] = f"torch.mm bf16 {m}x{m}x{m}"
    out["bf16_mm_frac_of_spec"] = round(2.0 * m ** 3 / t / 1e12 / BF16_PEAK_TFLOPS, 4)
    del x, y
    # the vendor library's block-scaled GEMMs of the same shape (torch._scaled_mm -> hipBLASLt)
    for name, fn in vendor_scaled_mm(torch, m, m, m).items():
        try:
            t = timed(fn)
            out[f"{name}_TFLOPs"] = round(2.0 * m ** 3 / t / 1e12, 1)
        except Exception as exc:    # not offered by this torch / hipBLASLt build
            out[f"{name}_TFLOPs"] = None
            out[f"{name}_error"] = f"{type(exc).__name__}: {str(exc)[:120]}"
    out["scaled_mm_shape"] = f"torch._scaled_mm {m}x{m}x{m}, bf16 out"
    torch.cuda.empty_cache()
    return out


def vendor_scaled_mm(torch, M, N, K, a_codes=None, a_scales=None, w_codes=None, w_scales=None):
    """torch._scaled_mm calls (hipBLASLt) computing A[M,K] W[N,K]^T in bf16: MXFP4 (E2M1 codes
    packed two per byte, UE8M0 scales per 32, the quantizer's own row-major layout; random codes
    unless given) and FP8 E4M3 with per-tensor unit scales. Returns name -> callable."""
    dev = "cuda"
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    rnd = lambda shape, lo, hi: torch.randint(lo, hi, shape, dtype=torch.uint8, device=dev, generator=g)
    qa = a_codes if a_codes is not None else rnd((M, K // 2), 0, 256)
    qw = w_codes if w_codes is not None else rnd((N, K // 2), 0, 256)
    sa = a_scales if a_scales is not None else rnd((M, K // 32), 120, 130)
    sw = w_scales if w_scales is not None else rnd((N, K // 32), 120, 130)
    fa = torch.randn((M, K), device=dev, generator=g).to(torch.float8_e4m3fn)
    fw = torch.randn((N, K), device=dev, generator=g).to(torch.float8_e4m3fn)
    one = torch.ones((), device=dev)
    f4 = torch.float4_e2m1fn_x2
    e8 = torch.float8_e8m0fnu
    return {
        "mxfp4_scaled_mm": lambda: torch._scaled_mm(qa.view(f4), qw.view(f4).t(), scale_a=sa.view(e8),
                                                    scale_b=sw.view(e8), out_dtype=torch.bfloat16),
        "fp8_scaled_mm": lambda: torch._scaled_mm(fa, fw.t(), scale_a=one, scale_b=one, out_dtype=torch.bfloat16),
    }


def token_sweep(torch, ops, layer, inputs, wl, w, mode, dev, args, points, read_gbs):
    """The workload's token sweep, each point's layer step replayed from a HIP graph: cold
    (after a 1 GiB read) median and p10/p90 over `steps` replays, warm median; weight bytes
    of the touched experts over the cold median against the 8 TB/s spec (and the measured
    read ceiling)."""
    rows = []
    for Ts in points:
        xs = inputs.activations_bf16(wl, Ts).to(dev)
        ls = inputs.router_logits(wl, Ts).to(dev)
        r = ops.moe_route_permute(ls, wl.k)
        torch.cuda.synchronize()
        touched = int(r["n_active"].item())
        flops, w13b, w2b = layer_work(wl, Ts, touched, mode == MXFP4)
        paths = {}
        step = make_step(torch, ops, wl, w, xs, ls, Ts, mode, paths, bool(args.combine))
        for _ in range(3):
            step()
        torch.cuda.synchronize()
        warm, cold = graph_times(torch, step, args.steps, 20, dev)
        c = stats_us(cold)
        gbs = (w13b + w2b) / (c["median"] * 1e-6) / 1e9
        row = dict(tokens=Ts, tokens_per_expert=round(Ts * wl.k / wl.E, 4), touched_experts=touched,
                   cold_us_median=c["median"], cold_us_p10=c["p10"], cold_us_p90=c["p90"],
                   warm_us_median=round(pct(warm, 50), 2), replays=c["n"],
                   tflops=round(flops / (c["median"] * 1e-6) / 1e12, 2), weight_GBps=round(gbs, 1),
                   weight_hbm_frac=round(gbs / HBM_PEAK_GBS, 4),
                   ideal_us=round((w13b + w2b) / (HBM_PEAK_GBS * 1e9) * 1e6, 2))
        if read_gbs:
            row["weight_frac_of_measured_read"] = round(gbs / read_gbs, 4)
        rows.append(row)
        print(f"[bench] sweep T={Ts}: cold {c['median']:.1f} us (p10 {c['p10']:.1f}, p90 {c['p90']:.1f}), "
              f"weights {gbs:.0f} GB/s ({gbs / HBM_PEAK_GBS:.3f} of 8 TB/s), warm {row['warm_us_median']:.1f} us",
              file=sys.stderr, flush=True)
    return rows


def dense_line(torch, ops, inputs, wl, args, M):
    """The dense NVFP4 GEMM Y[M,N] = A[M,K] W[N,K]^T (E = 1, no SwiGLU) in W4A16 and W4A4,
    beside torch.mm on bf16 copies of the same operands. A is bf16 for W4A16; for W4A4 it is
    quantized to NVFP4 before the timed region (the pages compare the GEMMs alone)."""
    dev = "cuda"
    N, K = wl.F, wl.H
    wt = ops.nvfp4_quantize(inputs.expert_weight_fp32(wl, "dense", 0, dev), tiled=True)
    a = inputs.activations_bf16(wl, M).to(dev)
    aq, as_, ag = ops.nvfp4_quantize(a)
    one = torch.tensor([0, M], dtype=torch.int32, device=dev)
    act = torch.zeros(1, dtype=torch.int32, device=dev)
    na = torch.ones(1, dtype=torch.int32, device=dev)
    wbf = inputs.expert_weight_fp32(wl, "dense", 0, dev).to(torch.bfloat16)
    flops = 2.0 * M * N * K

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / args.steps      # us per call

    common = dict(expert_offsets=one, active_experts=act, n_active=na, out_dtype=torch.bfloat16)
    t16 = timed(lambda: ops.moe_grouped_gemm_nvfp4(ops.W4A16, ops.EPI_NONE, a, wt, **common))
    path16 = ops.last_dispatch()
    t4 = timed(lambda: ops.moe_grouped_gemm_nvfp4(ops.W4A4, ops.EPI_NONE, aq, wt, a_scales=as_,
                                                  a_g=ag, **common))
    tmm = timed(lambda: torch.mm(a, wbf.t()))
    # the MXFP4 variant of the same GEMM (group-32 UE8M0 scales) on the scaled FP4 matrix cores
    wmx_p, wmx_s = ops.mxfp4_quantize(inputs.expert_weight_fp32(wl, "dense", 0, dev))
    wmx = ops.mxfp4_weights_tile(wmx_p.unsqueeze(0), wmx_s.unsqueeze(0))
    amx, amx_s = ops.mxfp4_quantize(a)
    tmx = timed(lambda: ops.moe_grouped_gemm_mxfp4(ops.EPI_NONE, amx, amx_s, wmx, **common))
    # the vendor library on the same MXFP4 operands, and FP8 E4M3 per tensor, same shape
    vendor = {}
    for name, fn in vendor_scaled_mm(torch, M, N, K, amx, amx_s, wmx_p, wmx_s).items():
        try:
            vendor[f"{name}_us"] = round(timed(fn), 2)
        except Exception as exc:
            vendor[f"{name}_us"] = None
            vendor[f"{name}_error"] = f"{type(exc).__name__}: {str(exc)[:120]}"
    # block-scaled FP8 (MXFP8: E4M3 elements, UE8M0 per 32) on the scaled FP8 matrix cores
    w8 = ops.mxfp8_weights_tile(*ops.mxfp8_quantize(inputs.expert_weight_fp32(wl, "dense", 0, dev).unsqueeze(0)))
    a8, a8_s = ops.mxfp8_quantize(a)
    t8 = timed(lambda: ops.moe_grouped_gemm_mxfp8(ops.EPI_NONE, a8, a8_s, w8, **common))
    tf = lambda us: flops / (us * 1e-6) / 1e12
    return dict(
        metric="MoE NVFP4 grouped-GEMM TFLOPS + weight GB/s vs tokens/expert, % roofline",
        value=round(tf(t16), 2), unit="TFLOP/s", n_gpus=1, steps=args.steps, warmup=args.warmup,
        ms_per_step=round(t16 / 1e3, 5), higher_is_better=True, scaling="weak", vs_baseline=None,
        dtype="f16", data="synthetic",
        config=dict(workload=f"dense NVFP4 GEMM M={M} N={N} K={K}, W4A16 (bf16 activations)", M=M, N=N, K=K,
                    path="mfma" if path16 == ops.PATH_MFMA else "stream"),
        w4a4_tflops=round(tf(t4), 2), w4a4_us=round(t4, 2),
        w4a4_f16_peak_frac=round(tf(t4) / BF16_PEAK_TFLOPS, 4), w4a4_fp4_peak_frac=round(tf(t4) / FP4_PEAK_TFLOPS, 4),
        torch_mm_bf16_tflops=round(tf(tmm), 2), torch_mm_bf16_us=round(tmm, 2),
        mxfp4_w4a4_tflops=round(tf(tmx), 2), mxfp4_w4a4_us=round(tmx, 2),
        mxfp4_w4a4_fp4_peak_frac=round(tf(tmx) / FP4_PEAK_TFLOPS, 4),
        mxfp8_w8a8_tflops=round(tf(t8), 2), mxfp8_w8a8_us=round(t8, 2),
        mxfp8_w8a8_fp8_peak_frac=round(tf(t8) / FP8_PEAK_TFLOPS, 4),
        **vendor,
        roofline=dict(bound="mfma", kernel="gemm_large_kernel (dense NVFP4 W4A16)",
                      achieved=round(tf(t16), 1), peak=BF16_PEAK_TFLOPS, unit="TFLOP/s",
                      frac=round(tf(t16) / BF16_PEAK_TFLOPS, 4), traffic=None, launch_us=round(t16, 2),
                      timed="HIP events around 'steps' back-to-back moe_grouped_gemm_nvfp4 calls (every launch "
                            "of the call: activation prep with the m-tile list, GEMM, split-K reduce)"),
        baseline_context="pages: 437 TFLOPS FP4 vs 225 TFLOPS BF16 at M=512 on RTX PRO 6000 (SM120)",
        cpu_baseline=None,
    )


def cpu_baseline(torch, wl, w, x, lg, T, mode, seconds):
    """The oracle (float64 NumPy) on a bounded sample of the same layer: per-expert
    dequantize + up/gate GEMM + SwiGLU + down GEMM for as many active experts as fit in
    about `seconds`, scaled to TFLOP/s of algorithmic work."""
    import numpy as np
    from oracle import moe as omoe
    from oracle import mxfp4 as omx
    from oracle import nvfp4 as onv
    mx = mode == MXFP4
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    lgn = lg.cpu().numpy()
    ids, rw = omoe.route(lgn, wl.k)
    perm = omoe.permute(ids, wl.E)
    xs = x.float().cpu().numpy().astype(np.float64)
    if mx:   # the MXFP4 layer's activations as the GEMM sees them
        xs = omx.dequantize(*omx.quantize(xs.astype(np.float32)))
    tok = perm["sorted_slot"] // wl.k
    offsets = perm["offsets"]
    order = [int(e) for e in perm["active"]]
    done_rows, done_experts, flops = 0, 0, 0.0
    t_total = 0.0
    for e in order:
        if mx:
            q13 = (w.w13_packed[e].cpu().numpy(), w.w13_scales[e].cpu().numpy())
            q2 = (w.w2_packed[e].cpu().numpy(), w.w2_scales[e].cpu().numpy())
            dq = omx.dequantize
        else:
            q13 = (w.w13_packed[e].cpu().numpy(), w.w13_scales[e].cpu().numpy(), w.w13_g[e].item())
            q2 = (w.w2_packed[e].cpu().numpy(), w.w2_scales[e].cpu().numpy(), w.w2_g[e].item())
            dq = onv.dequantize
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        t0 = time.perf_counter()
        A = xs[tok[r0:r1]]
        G = omoe.swiglu(A @ dq(*q13).T)
        h = omx.dequantize(*omx.quantize(G.astype(np.float32))) if mx else omoe.bf16_round(G)
        _ = h @ dq(*q2).T
        t_total += time.perf_counter() - t0
        done_rows += r1 - r0
        done_experts += 1
        flops += 2.0 * (r1 - r0) * 3 * wl.F * wl.H
        if t_total >= seconds:
            break
    return dict(value=round(flops / t_total / 1e12, 6), unit="TFLOP/s", cores=int(threads), kind="oracle",
                sample=f"{done_experts} of {len(order)} active experts ({done_rows} of {T * wl.k} routed rows) "
                       f"of the same layer: float64 dequantize + up/gate + SwiGLU"
                       f"{' + h requantize' if mx else ''} + down, {t_total:.1f} s")


if __name__ == "__main__":
    main()
