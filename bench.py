#!/usr/bin/env python3
"""MoE layer fwd+bwd throughput on one MI355X, with per-kernel roofline and the CPU oracle.

A step is one pass of the whole layer over one synthetic batch: route, permute into the ring,
the forward grouped GEMMs and combine, and the full backward. Inputs are resident in HBM
before timing starts. The default workload is the DeepSeek-V3-shaped routed layer: T=2048
tokens, d=7168, 256 experts, top-8, SwiGLU intermediate 2048, BF16.

Prints one JSON line. `value` is tokens/s over the timed steps (hipEvents between steps on the
layer's stream, nothing between the launches). `roofline` is the dominant kernel's algorithmic
bytes (or flops) per launch divided by its average launch time. Those times come from a second
timed region of as many steps, in which the library records events around each of its launches
on that same stream (`ms_per_step_traced` is that region's step time). `cpu_baseline` times the
float64 CPU oracle on a bounded sample of the same workload, extrapolated to the whole layer,
with per-workload samples beside it. Further lines: the other grid form (persistent), MXFP8
and MXFP4 modes, the local expert slice, the tiny layer (eager and as a HIP graph) and the streaming
macrobatch (serial and overlapped).
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_GBPS = 8000.0         # MI355X HBM3E, GB/s
MFMA_BF16_TFLOPS = 2500.0  # dense bf16 MFMA, TFLOP/s
MFMA_FP8_TFLOPS = 5000.0   # dense fp8 MFMA (the MXFP8 scaled MFMA), TFLOP/s
MFMA_FP4_TFLOPS = 10100.0  # dense fp4 MFMA (the MXFP4 scaled MFMA), TFLOP/s
# fp32 FMA on the vector ALUs without packed-fp32 instructions (the library is built without
# them): 256 CUs x 4 SIMDs x 16 lanes x 2 flop x 2.4 GHz. Packed fp32 would double it (157.3).
VALU_FP32_TFLOPS = 78.6


def algorithmic(cfg, routed=True, accumulate=False, mx=False, mx_wgrad=False, bf16_dw=False,
                fbits=8):
    """Algorithmic bytes and flops per launch of each kernel: what the method must move and
    compute (each tensor read or written once, no padding, no re-reads). M = T*k rows.
    In the MX modes (`mx`) a quantised tensor of n elements is n * fbits / 8 code bytes (fbits
    8 for MXFP8, 4 for MXFP4) plus n/32 scale bytes, and the weights are read in the quantised
    copies. dW1 and dW2 elements are 4 bytes, 2 with `bf16_dw`."""
    T, d, E, k, I = cfg["T"], cfg["d"], cfg["E"], cfg["k"], cfg["I"]
    M = T * k
    nb = (M + 255) // 256
    acc = 2 if accumulate else 1
    wb = 2 if bf16_dw else 4  # bytes per dW1 / dW2 element
    q = lambda n: n * fbits // 8 + n // 32  # bytes of n MX elements with their scales
    b = {}
    if routed:
        b["widen_router"] = (E * d * 2 + E * d * 4, 0)
        b["router_logits"] = (T * d * 2 + E * d * 2 + T * E * 4, 2 * T * d * E)
        b["router_topk"] = (T * E * 4 + T * k * 8, 0)
    b["perm_hist"] = (M * 8 + nb * E * 4, 0)
    b["perm_scan"] = (2 * nb * E * 4 + E * 8, 0)
    b["sched_build"] = (E * 4, 0)
    b["combine"] = (M * d * 2 + T * d * 2 + M * 8, 2 * M * d)
    b["dw_router"] = (M * (I // 128) * 4 + M * 12, 0)
    b["scale_gather"] = (T * d * 2 + M * d * 2 + M * 8, M * d)
    b["bwd_down_wgrad"] = (acc * E * d * I * wb + T * d * 2 + M * I * 2, 2 * M * d * I)
    b["uncombine"] = (M * d * 2 + T * d * 2 + (E * d * 2 if routed else 0) + M * 8, M * d)
    if not mx:
        b["perm_place"] = (T * d * 2 + M * d * 2 + M * 16, 0)
        b["fwd_gateup"] = (E * 2 * I * d * 2 + M * d * 2 + M * 2 * I * 2 + M * I * 2,
                           2 * M * d * 2 * I)
        b["fwd_down"] = (E * d * I * 2 + M * I * 2 + M * d * 2, 2 * M * I * d)
        b["bwd_down_dgrad"] = (E * d * I * 2 + T * d * 2 + M * 2 * I * 2 * 2 + M * I * 2
                               + M * (I // 128) * 4, 2 * M * d * I)
        b["bwd_gate_dgrad"] = (E * 2 * I * d * 2 + M * 2 * I * 2 + M * d * 2, 2 * M * 2 * I * d)
        b["bwd_gate_wgrad"] = (acc * E * 2 * I * d * wb + M * 2 * I * 2 + M * d * 2,
                               2 * M * 2 * I * d)
        if routed:
            b["dwr"] = (M * d * 2 + acc * E * d * 4 + M * 4, 2 * M * d)
    else:
        # one pass per weight: read it once, write both quantised copies
        b["quant_w1"] = (E * 2 * I * d * 2 + 2 * q(E * 2 * I * d), 0)
        b["quant_w2"] = (E * d * I * 2 + 2 * q(E * d * I), 0)
        b["perm_place"] = (T * d * 2 + q(M * d) + M * 16, 0)
        b["fwd_gateup"] = (q(E * 2 * I * d) + q(M * d) + M * 2 * I * 2 + M * I * 2 + q(M * I),
                           2 * M * d * 2 * I)
        b["fwd_down"] = (q(E * d * I) + q(M * I) + M * d * 2, 2 * M * I * d)
        b["quant_dy"] = (T * d * 2 + q(T * d), 0)
        b["bwd_down_dgrad"] = (q(E * d * I) + q(T * d) + M * 2 * I * 2 + M * I * 2
                               + M * 2 * I * 2 + q(M * 2 * I) + M * (I // 128) * 4, 2 * M * d * I)
        b["bwd_gate_dgrad"] = (q(E * 2 * I * d) + q(M * 2 * I) + M * d * 2, 2 * M * 2 * I * d)
        b["bwd_gate_wgrad"] = (acc * E * 2 * I * d * wb + M * 2 * I * 2 + q(M * d),
                               2 * M * 2 * I * d)
        if routed:
            b["dwr"] = (q(M * d) + acc * E * d * 4 + M * 4, 2 * M * d)
        if mx_wgrad:
            # each operand read once in bf16 (Xp as its MXFP8 image) and quantised along the
            # positions; the GEMM reads the quantised copies and writes fp32 dW
            b["bwd_down_wgrad"] = (acc * E * d * I * wb + T * d * 2 + M * I * 2 + q(M * d)
                                   + q(M * I), 2 * M * d * I)
            b["bwd_gate_wgrad"] = (acc * E * 2 * I * d * wb + M * 2 * I * 2 + q(M * d)
                                   + q(M * 2 * I) + q(M * d), 2 * M * 2 * I * d)
    return b


GEMMS = ("fwd_gateup", "fwd_down", "bwd_down_dgrad", "bwd_down_wgrad", "bwd_gate_dgrad",
         "bwd_gate_wgrad")


MX_GEMMS = ("fwd_gateup", "fwd_down", "bwd_down_dgrad", "bwd_gate_dgrad")  # scaled MFMA


def mfma_peak(name, mx, mx_wgrad=False, fbits=8):
    """Dense MFMA peak of a GEMM kernel: fp8 (MXFP8) or fp4 (MXFP4) for the scaled-MFMA GEMMs,
    else bf16 (the weight-gradient GEMMs run bf16 MFMA unless the MXFP8 weight gradients are
    on)."""
    if mx and (name in MX_GEMMS or mx_wgrad):
        return MFMA_FP4_TFLOPS if fbits == 4 else MFMA_FP8_TFLOPS
    return MFMA_BF16_TFLOPS


def kernel_roofline(name, nbytes, flops, us, mx=False, mx_wgrad=False, fbits=8):
    """Achieved rate against the roofline that bounds the kernel."""
    s = us * 1e-6
    if name == "router_logits":
        ach = flops / s / 1e12
        return {"bound": "alu", "achieved": ach, "peak": VALU_FP32_TFLOPS, "unit": "TFLOP/s",
                "frac": ach / VALU_FP32_TFLOPS}
    peak = mfma_peak(name, mx, mx_wgrad, fbits)
    gbps = nbytes / s / 1e9
    if flops and name in GEMMS:
        # a GEMM also carries all three views: % of its MFMA peak, % of HBM peak, and % of the
        # attainable rate min(MFMA peak, HBM peak x flop/B)
        tflops = flops / s / 1e12
        attainable = min(peak, HBM_GBPS * 1e9 * flops / nbytes / 1e12)
        views = {"tflops": tflops, "frac_mfma_peak": tflops / peak, "hbm_gbps": gbps,
                 "frac_hbm": gbps / HBM_GBPS, "attainable_tflops": attainable,
                 "frac_attainable": tflops / attainable}
        if flops / nbytes > peak * 1e12 / (HBM_GBPS * 1e9):
            return {"bound": "mfma", "achieved": tflops, "peak": peak, "unit": "TFLOP/s",
                    "frac": tflops / peak, **views}
        return {"bound": "hbm", "achieved": gbps, "peak": HBM_GBPS, "unit": "GB/s",
                "frac": gbps / HBM_GBPS, **views}
    return {"bound": "hbm", "achieved": gbps, "peak": HBM_GBPS, "unit": "GB/s",
            "frac": gbps / HBM_GBPS}


def measured_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter summary, or None
    when there is none or the kernel's sources changed since the counters were taken."""
    import json as _json
    from mixture_experts_layer_deterministic_amd.profsum import KERNELS, source_hash
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = _json.load(open(path)).get("kernels", {}).get(kernel)
    src = {n: f for _, n, f in KERNELS}.get(kernel)
    if not rec or not src or rec["source_sha"] != source_hash(src):
        return None
    return rec["read_bytes"] + rec["write_bytes"]


def _oracle_threads():
    from threadpoolctl import threadpool_info
    return max([p.get("num_threads", 1) for p in threadpool_info()] + [1])


def _oracle_step(inp, cfg, experts=None):
    """One oracle forward + backward of the workload (expert math limited to `experts`)."""
    import oracle
    import workload
    X = workload.to_numpy(inp["X"])
    dY = workload.to_numpy(inp["dY"])
    W1 = workload.HostExperts(inp["W1"])
    W2 = workload.HostExperts(inp["W2"])
    kw = dict(Wr=workload.to_numpy(inp["Wr"]), k=cfg["k"]) if "Wr" in inp else dict(
        topk_idx=workload.to_numpy(inp["topk_idx"]), topk_w=workload.to_numpy(inp["topk_w"]))
    f = oracle.forward(X, W1, W2, experts=experts, **kw)
    oracle.backward(f, X, W1, W2, dY, Wr=kw.get("Wr"), experts=experts)


def cpu_baseline(inp, cfg, s_small=8, s_large=40):
    """The CPU oracle on a bounded sample of the workload: the full router and bookkeeping plus
    the expert math of the first `s` experts, for two values of s. Its time is linear in the
    expert count (near-uniform load), so the whole-layer time is extrapolated to all E experts.
    `cores` is the BLAS thread count the oracle's matrix products ran on (its element-wise
    numpy steps run on one thread); `os_cpu_count` is what the host reports."""
    E = cfg["E"]
    times = {}
    for s in (s_small, s_large):
        ex = list(range(min(s, E)))
        t0 = time.perf_counter()
        _oracle_step(inp, cfg, experts=ex)
        times[len(ex)] = time.perf_counter() - t0
    (sa, ta), (sb, tb) = sorted(times.items())
    slope = (tb - ta) / max(sb - sa, 1)
    full = ta + slope * (E - sa)
    return {"value": cfg["T"] / full, "unit": "tokens/s", "cores": _oracle_threads(),
            "os_cpu_count": os.cpu_count(), "kind": "oracle",
            "sample": (f"{cfg['name']} seed 0, full router and bookkeeping, expert math of "
                       f"experts 0..{sa - 1} ({ta:.2f} s) and 0..{sb - 1} ({tb:.2f} s) "
                       f"fwd+bwd; whole-layer time extrapolated linearly to {E} experts "
                       f"= {full:.1f} s"),
            "layer_seconds": full}


def cpu_tiny(dev):
    """The oracle on the whole tiny workload (no sampling), on all BLAS threads and on one."""
    import workload
    from threadpoolctl import threadpool_limits
    cfg = workload.config("tiny")
    inp = workload.make_inputs("tiny", seed=0, device=dev)
    out = {}
    for label, limit in (("all_threads", None), ("one_thread", 1)):
        if limit is None:
            t0 = time.perf_counter()
            _oracle_step(inp, cfg)
            dt = time.perf_counter() - t0
            threads = _oracle_threads()
        else:
            with threadpool_limits(limits=limit):
                t0 = time.perf_counter()
                _oracle_step(inp, cfg)
                dt = time.perf_counter() - t0
            threads = 1
        out[label] = {"seconds": round(dt, 3), "tokens_per_s": round(cfg["T"] / dt, 1),
                      "threads": threads}
    return out


def cpu_expert_sample(inp, cfg, rows_total):
    """The oracle on the lightest non-empty expert of a given-routing workload, scaled by rows:
    the whole layer's expert math is linear in the rows (identical expert shapes)."""
    import numpy as np
    import workload
    idx = workload.to_numpy(inp["topk_idx"]).reshape(-1)
    counts = np.bincount(idx, minlength=cfg["E"])
    nz = np.flatnonzero(counts)
    e = int(nz[np.argmin(counts[nz])])
    t0 = time.perf_counter()
    _oracle_step(inp, cfg, experts=[e])
    dt = time.perf_counter() - t0
    full = dt * rows_total / counts[e]
    return {"seconds_sample": round(dt, 3), "sample": f"expert {e} ({counts[e]} rows) fwd+bwd",
            "layer_seconds": round(full, 2), "rows_per_s": round(rows_total / full, 1),
            "threads": _oracle_threads()}


def cpu_stream_sample(inp, cfg):
    """The oracle on one microbatch of the streaming macrobatch, experts 0..15 of its 512,
    scaled to 512 experts and 8 microbatches (near-uniform load)."""
    import workload
    one = dict(inp, X=inp["X"][0], dY=inp["dY"][0])
    t0 = time.perf_counter()
    _oracle_step(one, cfg, experts=list(range(16)))
    dt = time.perf_counter() - t0
    t1 = time.perf_counter()
    _oracle_step(one, cfg, experts=list(range(32)))
    dt2 = time.perf_counter() - t1
    per_mb = dt + (dt2 - dt) / 16 * (cfg["E"] - 16)
    full = per_mb * cfg["microbatches"]
    del workload
    return {"sample": "microbatch 0, router and bookkeeping plus experts 0..15 and 0..31; "
                      "extrapolated linearly to 512 experts and 8 microbatches",
            "seconds_sample": round(dt + dt2, 2), "layer_seconds": round(full, 1),
            "tokens_per_s": round(cfg["T"] * cfg["microbatches"] / full, 1),
            "threads": _oracle_threads()}


def time_steps(step, stream, steps, warmup):
    """Mean, median and minimum ms per step over `steps` steps after `warmup` untimed ones.
    Events sit only between steps, on the layer's stream."""
    import torch
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    t_host = time.perf_counter()
    marks[0].record(stream)
    for i in range(steps):
        step()
        marks[i + 1].record(stream)
    torch.cuda.synchronize()
    t_host = time.perf_counter() - t_host
    per = sorted(marks[i].elapsed_time(marks[i + 1]) for i in range(steps))
    h = len(per) // 2
    median = per[h] if len(per) % 2 else 0.5 * (per[h - 1] + per[h])
    return {"ms": marks[0].elapsed_time(marks[-1]) / steps, "ms_median": median,
            "ms_min": per[0], "t_host": t_host}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="dsv3")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--persistent", action="store_true",
                    help="time the persistent grids as the headline (default: one-shot grids)")
    ap.add_argument("--bf16-dw", action="store_true",
                    help="store dW1 and dW2 as bf16 in the headline run (default: fp32)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-trace", action="store_true", help="skip the per-kernel traced pass")
    ap.add_argument("--no-mxfp8", action="store_true",
                    help="skip the MXFP8-mode run on the same inputs")
    ap.add_argument("--no-mxfp4", action="store_true",
                    help="skip the MXFP4-mode run on the same inputs")
    ap.add_argument("--no-expert-slice", action="store_true",
                    help="skip the local expert-slice (local_zipf) run")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the persistent, tiny and streaming-macrobatch lines")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="first run one plain device copy of this many MiB, a known-size "
                         "reference for HBM byte counters")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one MI355X: the library has no multi-GPU path "
              "(no collectives, no sharding); run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import mixture_experts_layer_deterministic_amd as m
    import workload
    from mixture_experts_layer_deterministic_amd.layer import MoeLayer

    if not os.path.exists(m.LIB_PATH):
        from mixture_experts_layer_deterministic_amd import build
        build.build(verbose=False)

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = workload.config(args.workload)
    if cfg.get("microbatches"):
        # the streaming macrobatch alone (it is also the `stream` line of the default run), so
        # that a profiler's trace holds its kernels only
        print("[bench] streaming macrobatch alone", file=sys.stderr, flush=True)
        out, _ = run_stream(workload, dev, torch.cuda.current_stream(), args)
        print(json.dumps({"metric": "streaming macrobatch fwd+bwd tokens/s",
                          "value": out["serial"]["tokens_per_s"], "unit": "tokens/s",
                          "n_gpus": 1, "higher_is_better": True, "dtype": "bf16",
                          "data": "synthetic", "config": {"workload": "stream"}, "stream": out}),
              flush=True)
        return
    print(f"[bench] generating {args.workload} inputs (seed {args.seed})", file=sys.stderr,
          flush=True)
    inp = workload.make_inputs(args.workload, seed=args.seed, device=dev)
    T, d, E, k, I = cfg["T"], cfg["d"], cfg["E"], cfg["k"], cfg["I"]
    routed = "Wr" in inp
    mx = cfg["precision"] in ("mxfp8", "mxfp4")
    fbits = 4 if cfg["precision"] == "mxfp4" else 8
    stream = torch.cuda.current_stream()

    if args.calib_copy_mib:
        n = args.calib_copy_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    main_run = run_layer(m, MoeLayer, inp, cfg, stream, args, mx=mx,
                         persistent=args.persistent, bf16_dw=args.bf16_dw, fbits=fbits)
    ms, kernels = main_run["ms"], main_run["kernels"]
    tokens_per_s = T / (ms * 1e-3)

    dominant = max(kernels, key=lambda n: kernels[n]["us"]) if kernels else None
    roof = None
    if dominant:
        kd = kernels[dominant]
        roof = {"kernel": dominant, "bound": kd["bound"], "achieved": kd["achieved"],
                "peak": kd["peak"], "unit": kd["unit"], "frac": kd["frac"],
                # the committed counter records are of the fp32-dW layer
                "traffic": None if args.bf16_dw else measured_traffic(args.workload, dominant),
                "alg_bytes": kd["alg_bytes"], "us_per_step": kd["us"],
                "launches_per_step": kd["launches_per_step"]}
    pc = {}
    for n in ("perm_place", "combine", "scale_gather", "uncombine"):
        if n in kernels:
            pc[n] = {"GB/s": kernels[n].get("achieved"), "frac_hbm": kernels[n].get("frac")}

    extra = {}
    if not args.no_extra and args.workload == "dsv3" and not mx:
        # the same layer on the persistent grids (or on one-shot grids when those are headline)
        print("[bench] the other grid form on the same inputs", file=sys.stderr, flush=True)
        r = run_layer(m, MoeLayer, inp, cfg, stream, args, mx=False,
                      persistent=not args.persistent, trace=False)
        extra["other_grid"] = {"persistent": not args.persistent,
                               "tokens_per_s": round(T / (r["ms"] * 1e-3), 1),
                               "ms_per_step": round(r["ms"], 4),
                               "ms_per_step_median": round(r["ms_median"], 4)}
        torch.cuda.empty_cache()

    # The same layer in MXFP8 mode on the same inputs: the second precision the metric names.
    mx_line = None
    if not mx and not args.no_mxfp8 and routed:
        print("[bench] MXFP8 mode on the same inputs", file=sys.stderr, flush=True)
        torch.cuda.empty_cache()
        r = run_layer(m, MoeLayer, inp, cfg, stream, args, mx=True)
        mx_line = {"tokens_per_s": round(T / (r["ms"] * 1e-3), 1),
                   "ms_per_step": round(r["ms"], 4),
                   "weight_quantize_ms": round(r["quant_ms"], 4),
                   "layer_ms_without_weight_quantize": round(r["ms"] - r["quant_ms"], 4),
                   "grouped_gemm": r["gemm"], "kernels": r["kernels"]}
        torch.cuda.empty_cache()

    # and in MXFP4 mode (E2M1 elements, the same scales and axes)
    mx4_line = None
    if not mx and not args.no_mxfp4 and routed and I % 256 == 0:
        print("[bench] MXFP4 mode on the same inputs", file=sys.stderr, flush=True)
        r = run_layer(m, MoeLayer, inp, cfg, stream, args, mx=True, fbits=4)
        mx4_line = {"tokens_per_s": round(T / (r["ms"] * 1e-3), 1),
                    "ms_per_step": round(r["ms"], 4),
                    "weight_quantize_ms": round(r["quant_ms"], 4),
                    "layer_ms_without_weight_quantize": round(r["ms"] - r["quant_ms"], 4),
                    "grouped_gemm": r["gemm"], "kernels": r["kernels"]}
        torch.cuda.empty_cache()

    # The weight gradients stored as bf16 (the alternative to fp32 main gradients): the same
    # sums rounded once, with half the dW bytes, in both precisions.
    bf16_dw_line = None
    if not args.no_extra and args.workload == "dsv3" and not mx:
        print("[bench] bf16 weight gradients on the same inputs", file=sys.stderr, flush=True)
        bf16_dw_line = {}
        for tag, is_mx in (("bf16", False), ("mxfp8", True)):
            if is_mx and (args.no_mxfp8 or not routed):
                continue
            torch.cuda.empty_cache()
            r = run_layer(m, MoeLayer, inp, cfg, stream, args, mx=is_mx, bf16_dw=True)
            bf16_dw_line[tag] = {
                "tokens_per_s": round(T / (r["ms"] * 1e-3), 1), "ms_per_step": round(r["ms"], 4),
                "ms_per_step_median": round(r["ms_median"], 4),
                "grouped_gemm": r["gemm"],
                "kernels": {g: r["kernels"][g] for g in GEMMS if g in r["kernels"]}}
            if is_mx:
                bf16_dw_line[tag]["weight_quantize_ms"] = round(r["quant_ms"], 4)
                bf16_dw_line[tag]["layer_ms_without_weight_quantize"] = round(
                    r["ms"] - r["quant_ms"], 4)
        torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline and not mx:
        print("[bench] timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        cpu = cpu_baseline(inp, cfg)
    del inp
    torch.cuda.empty_cache()

    # The local expert slice (16,384 received rows over 8 experts, Zipf-skewed): there the
    # grouped GEMMs are MFMA-bound, so it is where their fraction of the MFMA peak means something.
    slice_line = None
    if args.workload == "dsv3" and not args.no_expert_slice:
        print("[bench] local expert slice (local_zipf)", file=sys.stderr, flush=True)
        cz = workload.config("local_zipf")
        iz = workload.make_inputs("local_zipf", seed=args.seed, device=dev)
        r = run_layer(m, MoeLayer, iz, cz, stream, args, mx=False)
        slice_line = {"workload": "local_zipf", "rows": cz["T"] * cz["k"], "E": cz["E"],
                      "ms_per_step": round(r["ms"], 4),
                      "rows_per_s": round(cz["T"] * cz["k"] / (r["ms"] * 1e-3), 1),
                      "grouped_gemm": r["gemm"],
                      "gemm_us": {g: r["kernels"][g]["us"] for g in GEMMS if g in r["kernels"]},
                      "kernels": r["kernels"]}
        if not args.no_mxfp8:
            # MXFP8 on the same slice: its GEMMs against the fp8 MFMA peak where they are
            # MFMA-bound rather than weight-streaming
            print("[bench] local expert slice in MXFP8 mode", file=sys.stderr, flush=True)
            rz = run_layer(m, MoeLayer, iz, cz, stream, args, mx=True)
            slice_line["mxfp8"] = {
                "ms_per_step": round(rz["ms"], 4),
                "weight_quantize_ms": round(rz["quant_ms"], 4),
                "layer_ms_without_weight_quantize": round(rz["ms"] - rz["quant_ms"], 4),
                "grouped_gemm": rz["gemm"],
                "gemm_us": {g: rz["kernels"][g]["us"] for g in GEMMS if g in rz["kernels"]}}
            # and with the weight gradients in MXFP8 too
            print("[bench] local expert slice, MXFP8 with MXFP8 weight gradients",
                  file=sys.stderr, flush=True)
            rw = run_layer(m, MoeLayer, iz, cz, stream, args, mx=True, mx_wgrad=True)
            slice_line["mxfp8_wgrad"] = {
                "ms_per_step": round(rw["ms"], 4),
                "layer_ms_without_weight_quantize": round(rw["ms"] - rw["quant_ms"], 4),
                "grouped_gemm": rw["gemm"],
                "gemm_us": {g: rw["kernels"][g]["us"] for g in GEMMS if g in rw["kernels"]},
                "wgrad_parts_us": {g: rw["kernels"][g].get("parts_us")
                                   for g in ("bwd_down_wgrad", "bwd_gate_wgrad")
                                   if g in rw["kernels"]}}
        if not args.no_mxfp4 and cz["I"] % 256 == 0:
            print("[bench] local expert slice in MXFP4 mode", file=sys.stderr, flush=True)
            r4 = run_layer(m, MoeLayer, iz, cz, stream, args, mx=True, fbits=4)
            slice_line["mxfp4"] = {
                "ms_per_step": round(r4["ms"], 4),
                "weight_quantize_ms": round(r4["quant_ms"], 4),
                "layer_ms_without_weight_quantize": round(r4["ms"] - r4["quant_ms"], 4),
                "grouped_gemm": r4["gemm"],
                "gemm_us": {g: r4["kernels"][g]["us"] for g in GEMMS if g in r4["kernels"]}}
        if cpu is not None:
            cpu.setdefault("per_config", {})["local_zipf"] = cpu_expert_sample(
                iz, cz, cz["T"] * cz["k"])
        del iz
        torch.cuda.empty_cache()

    if not args.no_extra and args.workload == "dsv3":
        print("[bench] tiny layer", file=sys.stderr, flush=True)
        extra["tiny"] = run_tiny(m, MoeLayer, workload, dev, stream, args)
        print("[bench] streaming macrobatch", file=sys.stderr, flush=True)
        extra["stream"], ist = run_stream(workload, dev, stream, args)
        if cpu is not None:
            cpu.setdefault("per_config", {})["stream"] = cpu_stream_sample(
                ist, workload.config("stream"))
            cpu["per_config"]["tiny"] = cpu_tiny(dev)
        del ist
        torch.cuda.empty_cache()

    # practical HBM ceiling: one plain 2 GiB device copy (read + write), best of 3. Skipped in
    # counter runs, where the only device copy must be the calibration copy.
    n = 2 << 30
    hbm_copy = None
    if not args.calib_copy_mib:
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        best = None
        for _ in range(3):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            dst.copy_(src)
            b.record(stream)
            torch.cuda.synchronize()
            t = a.elapsed_time(b)
            best = t if best is None else min(best, t)
        hbm_copy = round(2 * n / (best * 1e-3) / 1e9, 1)
        del src, dst

    line = {
        "metric": "MoE layer fwd+bwd tokens/s",
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "ms_per_step_median": round(main_run["ms_median"], 4),
        "ms_per_step_min": round(main_run["ms_min"], 4),
        "ms_per_step_traced": (round(main_run["ms_traced"], 4)
                               if main_run.get("ms_traced") else None),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("mxfp4-e2m1/bf16" if fbits == 4 else "mxfp8-e4m3/bf16") if mx else "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "T": T, "d": d, "E": E, "k": k, "I": I,
                   "precision": cfg["precision"], "weight_grad_dtype": "bf16" if args.bf16_dw else "fp32",
                   "persistent": bool(args.persistent), "seed": args.seed},
        "roofline": roof,
        "cpu_baseline": cpu,
        "grouped_gemm": main_run["gemm"],
        "permute_combine": pc,
        "mxfp8": mx_line,
        "mxfp4": mx4_line,
        "bf16_dw": bf16_dw_line,
        "expert_slice": slice_line,
        **extra,
        "hbm_copy": {"GB/s": hbm_copy, "bytes": 2 * n, "what": "one plain device copy, read + write"},
        "kernels": kernels,
        "host_seconds_timed": round(main_run["t_host"], 4),
    }
    print(json.dumps(line))


def run_tiny(m, MoeLayer, workload, dev, stream, args):
    """The tiny layer (T=256, d=256, 8 experts, top-2): launch-bound. Eager steps, then the
    same step captured once into a HIP graph and replayed (one host launch per step)."""
    import torch
    cfg = workload.config("tiny")
    inp = workload.make_inputs("tiny", seed=args.seed, device=dev)
    L = MoeLayer(cfg["T"], cfg["d"], cfg["E"], cfg["k"], cfg["I"], device=dev)
    X, Wr, W1, W2, dY = (inp[n] for n in ("X", "Wr", "W1", "W2", "dY"))
    eager = time_steps(lambda: L.step(X, Wr, W1, W2, dY, stream=stream), stream,
                       max(args.steps, 50), args.warmup)
    out = {"T": cfg["T"], "eager": {"tokens_per_s": round(cfg["T"] / (eager["ms"] * 1e-3), 1),
                                    "ms_per_step": round(eager["ms"], 4),
                                    "ms_per_step_median": round(eager["ms_median"], 4),
                                    "host_ms_per_step": round(eager["t_host"] * 1e3
                                                              / max(args.steps, 50), 4)}}
    # the forward as one launch (moe_forward_fused), then the same backward
    fused = time_steps(lambda: L.step(X, Wr, W1, W2, dY, stream=stream, fused=True), stream,
                       max(args.steps, 50), args.warmup)
    out["fused_forward"] = {"tokens_per_s": round(cfg["T"] / (fused["ms"] * 1e-3), 1),
                            "ms_per_step": round(fused["ms"], 4),
                            "ms_per_step_median": round(fused["ms_median"], 4)}
    out["forward_only_ms"] = forward_only(L, X, Wr, W1, W2, stream, args)
    try:
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(side):
            L.step(X, Wr, W1, W2, dY)  # warm the side stream
            torch.cuda.synchronize()
            with torch.cuda.graph(g, stream=side):
                L.step(X, Wr, W1, W2, dY)
        torch.cuda.synchronize()
        graph = time_steps(g.replay, torch.cuda.current_stream(), max(args.steps, 50),
                           args.warmup)
        out["graph"] = {"tokens_per_s": round(cfg["T"] / (graph["ms"] * 1e-3), 1),
                        "ms_per_step": round(graph["ms"], 4),
                        "ms_per_step_median": round(graph["ms_median"], 4)}
        del g
    except RuntimeError as e:  # report, keep the rest of the bench line
        out["graph"] = {"error": str(e)[:200]}
    del L, inp
    return out


def forward_only(L, X, Wr, W1, W2, stream, args):
    """The forward alone: route + permute + forward as separate launches, and as one."""
    sep = time_steps(lambda: (L.route(X, Wr, stream), L.permute(X, 0, stream),
                              L.forward(W1, W2, 0, stream=stream)), stream,
                     max(args.steps, 50), args.warmup)
    one = time_steps(lambda: L.forward_fused(X, Wr, W1, W2, 0, stream=stream), stream,
                     max(args.steps, 50), args.warmup)
    return {"separate": round(sep["ms"], 4), "fused": round(one["ms"], 4)}


def run_stream(workload, dev, stream, args):
    """The streaming macrobatch: 8 microbatches of 2368 tokens through one 512 MiB ring (2
    slots), forward 0..7, backward 7..0 with the overwritten slots replayed. Tokens/s counts the
    8 x 2368 tokens of a macrobatch, replay included; serial, then with the next microbatch's
    routing and permutation on a second stream, and with each microbatch's forward as one
    launch."""
    from mixture_experts_layer_deterministic_amd.layer import Macrobatch
    cfg = workload.config("stream")
    inp = workload.make_inputs("stream", seed=args.seed, device=dev)
    n = cfg["microbatches"]
    tokens = n * cfg["T"]
    out = {"microbatches": n, "T": cfg["T"], "tokens": tokens, "ring_bytes": cfg["ring_bytes"]}
    # one microbatch's forward alone, as separate launches and as one
    from mixture_experts_layer_deterministic_amd.layer import MoeLayer
    Lm = MoeLayer(cfg["T"], cfg["d"], cfg["E"], cfg["k"], cfg["I"], device=dev)
    out["microbatch_forward_only_ms"] = forward_only(Lm, inp["X"][0], inp["Wr"], inp["W1"],
                                                     inp["W2"], stream, args)
    del Lm
    for mode in ("serial", "overlap", "fused_forward"):
        mb = Macrobatch(cfg["T"], cfg["d"], cfg["E"], cfg["k"], cfg["I"], n, cfg["ring_bytes"],
                        device=dev, overlap=mode == "overlap", fused=mode == "fused_forward")
        out["ring_slots"] = mb.S
        r = time_steps(lambda: mb.run(inp["X"], inp["Wr"], inp["W1"], inp["W2"], inp["dY"],
                                      stream), stream, max(3, args.steps // 4), 1)
        out[mode] = {
            "tokens_per_s": round(tokens / (r["ms"] * 1e-3), 1),
            "ms_per_macrobatch": round(r["ms"], 3),
            "ms_per_macrobatch_median": round(r["ms_median"], 3)}
        del mb
    return out, inp


def run_layer(m, MoeLayer, inp, cfg, stream, args, mx, persistent=False, trace=True,
              mx_wgrad=False, bf16_dw=False, fbits=8):
    """Warm up and time `args.steps` layer steps without any per-launch event, then (unless
    `trace` is off) time as many again with the library's per-launch events on the layer's
    stream, for the per-kernel times. In the MX modes (`mx`; fbits 8 MXFP8, 4 MXFP4) each step
    first quantises the weights."""
    import torch
    T, d, E, k, I = cfg["T"], cfg["d"], cfg["E"], cfg["k"], cfg["I"]
    dev = inp["X"].device
    routed = "Wr" in inp
    prec = (m.MOE_PREC_MXFP4 if fbits == 4 else m.MOE_PREC_MXFP8) if mx else m.MOE_PREC_BF16
    L = MoeLayer(T, d, E, k, I, device=dev, persistent=persistent, precision=prec,
                 mx_wgrad=mx_wgrad, bf16_dw=bf16_dw)
    wr = inp.get("Wr")
    if not routed:
        L.set_routing(inp["topk_idx"], inp["topk_w"])
    X, W1, W2, dY = inp["X"], inp["W1"], inp["W2"], inp["dY"]

    def step():
        if mx:
            L.quantize_weights(W1, W2, stream)
        L.step(X, wr, W1, W2, dY, stream=stream)

    tag = ("mxfp4" if fbits == 4 else "mxfp8") if mx else "bf16"
    print(f"[bench] {tag}{' persistent' if persistent else ''}"
          f"{' bf16-dW' if bf16_dw else ''}: "
          f"warmup and {args.steps} untraced steps", file=sys.stderr, flush=True)
    res = time_steps(step, stream, args.steps, args.warmup)

    # launches per step (traced once, untimed)
    probe = [torch.cuda.Event(enable_timing=True) for _ in range(128)]
    for e in probe:
        e.record(stream)
    torch.cuda.synchronize()
    keep = m.moe_trace_begin([e.cuda_event for e in probe])
    step()
    per_step = m.moe_trace_end()
    torch.cuda.synchronize()
    del keep

    kernels = {}
    alg = algorithmic(cfg, routed=routed, mx=mx, mx_wgrad=mx_wgrad, bf16_dw=bf16_dw, fbits=fbits)
    if trace and not args.no_trace:
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * per_step * args.steps)]
        for e in ev:
            e.record(stream)
        torch.cuda.synchronize()
        names = (ctypes.c_char_p * (per_step * args.steps))()
        print(f"[bench] {args.steps} traced steps ({per_step} launches each)", file=sys.stderr,
              flush=True)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        keep = m.moe_trace_begin([e.cuda_event for e in ev], names)
        a.record(stream)
        for _ in range(args.steps):
            step()
        b.record(stream)
        torch.cuda.synchronize()
        m.moe_trace_end()
        res["ms_traced"] = a.elapsed_time(b) / args.steps
        tot = {}
        cnt = {}
        for i in range(per_step * args.steps):
            n = names[i].decode()
            tot[n] = tot.get(n, 0.0) + ev[2 * i].elapsed_time(ev[2 * i + 1]) * 1e3
            cnt[n] = cnt.get(n, 0) + 1
        # A step's work of one kind may take several launches (the GEMMs run their 256-row
        # blocks and their remainders as two, "<name>_big" and "<name>"; in the MX modes the
        # gate wgrad also expands the big experts' Xp rows, "<name>_expand"): a kernel's `us`
        # is its time per step, summed over them, and `parts` splits it.
        parts = {}
        for n in list(tot):
            base = n
            for suffix in ("_big", "_expand", "_qL", "_qR"):
                if n.endswith(suffix):
                    base = n[:-len(suffix)]
            parts.setdefault(base, {})[n] = tot[n] / args.steps
        for n, pt in parts.items():
            us = sum(pt.values())
            launches = sum(cnt[p] for p in pt) // args.steps
            nbytes, flops = alg.get(n, (0, 0))
            r = kernel_roofline(n, nbytes, flops, us, mx, mx_wgrad, fbits) if nbytes else {}
            kernels[n] = {"us": round(us, 2), "launches_per_step": launches,
                          "alg_bytes": nbytes, "alg_flops": flops,
                          **{kk: (round(v, 4) if isinstance(v, float) else v)
                             for kk, v in r.items()}}
            if len(pt) > 1:
                kernels[n]["parts_us"] = {p: round(v, 2) for p, v in pt.items()}
        del keep
    quant_ms = sum(kernels[n]["us"] for n in kernels if n.startswith("quant_w")) / 1e3
    gemm = None
    gemm_us = sum(kernels[g]["us"] for g in GEMMS if g in kernels)
    if gemm_us:
        flops = sum(alg[g][1] for g in GEMMS)
        nbytes = sum(alg[g][0] for g in GEMMS)
        # the time-weighted MFMA peak of the six GEMMs at their own dtypes
        peak = sum(kernels[g]["us"] * mfma_peak(g, mx, mx_wgrad, fbits) for g in GEMMS
                   if g in kernels) / gemm_us
        tf = flops / (gemm_us * 1e-6) / 1e12
        attainable = sum(
            kernels[g]["us"] * min(mfma_peak(g, mx, mx_wgrad, fbits),
                                   HBM_GBPS * 1e9 * alg[g][1] / alg[g][0] / 1e12)
            for g in GEMMS if g in kernels) / gemm_us
        gemm = {"tflops": round(tf, 2), "mfma_peak_tflops": round(peak, 1),
                "frac_mfma_peak": round(tf / peak, 4),
                "attainable_tflops": round(attainable, 2),
                "frac_attainable": round(tf / attainable, 4),
                "alg_bytes": nbytes, "hbm_gbps": round(nbytes / (gemm_us * 1e-6) / 1e9, 1),
                "share_of_step": round(gemm_us / 1e3 / res.get("ms_traced", res["ms"]), 4)}
    del L
    return dict(res, kernels=kernels, gemm=gemm, quant_ms=quant_ms)


if __name__ == "__main__":
    main()
