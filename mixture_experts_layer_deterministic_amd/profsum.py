"""Summaries of rocprofv3 output for the MoE layer's kernels.

Usage, after one kernel-trace run and two counter runs (FETCH_SIZE, then WRITE_SIZE) of bench.py:
    python -m mixture_experts_layer_deterministic_amd.profsum \
        --stats DIR/run_kernel_stats.csv --fetch DIR/run_counter_collection.csv \
        --write DIR/run_counter_collection.csv --calib-mib 1024 \
        --workload dsv3 --command "..." --out profiles/NAME.md --traffic profiles/traffic_dsv3.json

It writes a short markdown table (per-kernel launches, average duration, HBM bytes per launch)
and a JSON record of the HBM bytes per launch of every kernel. Each kernel's entry in the JSON
record carries a hash of the source files it is built from. bench.py reports a kernel's traffic
only while that hash still matches the sources, so counters taken on older code never appear.

HBM bytes come from the TCC counters FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each scaled by
what the same counter reads for one plain device copy of known size in the same run: the copy
reads and writes exactly calib-mib MiB.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")

# rocprofv3 kernel-name pattern -> (bench name, the sources it is built from besides the
# common headers)
R = ("router.hip", "router.h")
P = ("permute.hip", "permute.h")
G = ("gemm.hip", "gemm_tiles.h")
W = ("wgrad.hip",)
M = ("mx.hip",)
C = ("elementwise.hip", "combine.h")
KERNELS = [
    (r"widen_router_kernel", "widen_router", R),
    (r"router_logits_kernel", "router_logits", R),
    (r"router_topk_kernel", "router_topk", R),
    (r"perm_hist_kernel", "perm_hist", P),
    (r"perm_scan_kernel", "perm_scan", P),
    (r"perm_place_kernel", "perm_place", P),
    (r"wgrad_sched_kernel", "wgrad_sched", W),
    (r"expand_big_rows_kernel", "bwd_gate_wgrad_expand", W),
    (r"sched_build_kernel", "sched_build", G),
    (r"dma_kernel<moe::DmaGateUp>", "fwd_gateup_big", G),
    (r"dma_kernel<moe::DmaDown>", "fwd_down_big", G),
    (r"dma_kernel<moe::DmaGateDgrad>", "bwd_gate_dgrad_big", G),
    (r"dma_kernel<moe::DmaDownDgrad>", "bwd_down_dgrad_big", G),
    (r"gg_kernel<moe::FwdGateUp", "fwd_gateup", G),
    (r"gg_kernel<moe::FwdDown", "fwd_down", G),
    (r"gg_kernel<moe::BwdDownDgrad", "bwd_down_dgrad", G),
    (r"gg_kernel<moe::BwdGateDgrad", "bwd_gate_dgrad", G),
    (r"gg_kernel<moe::MxFwdGateUp", "fwd_gateup", G),
    (r"gg_kernel<moe::MxFwdDown", "fwd_down", G),
    (r"gg_kernel<moe::MxBwdDownDgrad", "bwd_down_dgrad", G),
    (r"gg_kernel<moe::MxBwdGateDgrad", "bwd_gate_dgrad", G),
    (r"dmx_kernel<moe::DmxGateUp>", "fwd_gateup_big", G),
    (r"dmx_kernel<moe::DmxDown>", "fwd_down_big", G),
    (r"dmx_kernel<moe::DmxGateDgrad>", "bwd_gate_dgrad_big", G),
    (r"dmx_kernel<moe::DmxDownDgrad>", "bwd_down_dgrad_big", G),
    (r"DmaWgrad<(true|false), false, (true|false)>", "bwd_down_wgrad_big", W),
    (r"DmaWgrad<(true|false), true, (true|false)>", "bwd_gate_wgrad_big", W),
    (r"wgrad_kernel<(true|false), false", "bwd_down_wgrad", W),
    (r"wgrad_kernel<(true|false), true", "bwd_gate_wgrad", W),
    (r"moe::combine_kernel", "combine", C),
    (r"dw_router_kernel", "dw_router", C),
    (r"uncombine_kernel", "uncombine", C),
    (r"dwr_kernel", "dwr", C),
    (r"scale_gather_kernel", "scale_gather", M),
    (r"quant_rows_kernel", "quant_rows", M),
    (r"quant_weight_kernel", "quant_weight", M),
    (r"fused_forward_kernel", "fused_forward",
     ("fused.hip", "router.h", "permute.h", "gemm_tiles.h", "combine.h")),
]
COMMON_SOURCES = ("common.h", "dma.h", "kernels.h")


def bench_name(raw: str):
    """(bench name, source file) of a rocprofv3 kernel name, or None for other kernels."""
    if "moe::" not in raw:
        return None
    for pat, name, src in KERNELS:
        if re.search(pat, raw):
            return name, src
    return None


def _code_only(text: str) -> str:
    """The source without its comments and with whitespace runs collapsed: a change to a
    comment does not change the code the counters were taken on."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_hash(srcs) -> str:
    h = hashlib.sha256()
    for f in (*srcs, *COMMON_SOURCES):
        with open(os.path.join(CSRC, f), encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def _counter_per_kernel(path, calib_bytes):
    rows = sorted(csv.DictReader(open(path)), key=lambda r: int(r["Dispatch_Id"]))
    # the calibration copy is the largest device copy before the layer's first kernel (input
    # set-up may add small copies after it)
    first = next((i for i, r in enumerate(rows) if bench_name(r["Kernel_Name"])), len(rows))
    copies = [float(r["Counter_Value"]) for r in rows[:first] if "copyBuffer" in r["Kernel_Name"]]
    if not copies:
        raise SystemExit(f"{path}: no calibration copy found")
    scale = calib_bytes / (max(copies) * 1024.0)  # bytes per counted byte
    out = {}
    for r in rows:
        bn = bench_name(r["Kernel_Name"])
        if bn:
            out.setdefault(bn[0], []).append(float(r["Counter_Value"]) * 1024.0 * scale)
    return {k: sum(v) / len(v) for k, v in out.items()}, scale


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--stats", required=True)
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--calib-mib", type=int, default=1024)
    ap.add_argument("--workload", required=True)
    ap.add_argument("--command", required=True)
    ap.add_argument("--out", required=True)
    ap.add_argument("--traffic")
    ap.add_argument("--bench-log", help="bench.py output of the profiled run: its JSON line's "
                                        "roofline kernel is quoted next to the trace")
    args = ap.parse_args()

    stats = {}
    srcs = {}
    for r in csv.DictReader(open(args.stats)):
        bn = bench_name(r["Name"])
        if not bn:
            continue
        name, src = bn
        srcs[name] = src
        s = stats.setdefault(name, [0, 0.0])
        s[0] += int(r["Calls"])
        s[1] += float(r["TotalDurationNs"])
    total = sum(v[1] for v in stats.values())
    fetch = write = None
    if args.fetch and args.write:
        fetch, fs = _counter_per_kernel(args.fetch, args.calib_mib << 20)
        write, ws = _counter_per_kernel(args.write, args.calib_mib << 20)

    lines = [f"# rocprofv3 kernel summary: {args.workload}", "",
             f"Command: `{args.command}`", ""]
    if args.bench_log:
        import json as _json
        line = [ln for ln in open(args.bench_log) if ln.startswith("{")][-1]
        b = _json.loads(line)
        r = b["roofline"]
        per = r["us_per_step"] / max(r["launches_per_step"], 1)
        lines += [f"The bench line of the same run: roofline kernel `{r['kernel']}`, "
                  f"{r['us_per_step']:.1f} us per step over {r['launches_per_step']} launch(es) "
                  f"(HIP events on the layer's stream), {b['ms_per_step']:.2f} ms per step under "
                  f"the profiler; the trace's average for `{r['kernel']}` is below.", ""]
        del per
    if fetch is not None:
        lines += [f"HBM bytes: FETCH_SIZE x {fs:.3f} and WRITE_SIZE x {ws:.3f}, the factors that "
                  f"map a plain {args.calib_mib} MiB device copy onto its true size.", ""]
    lines += ["| kernel | launches | avg us | share of layer time | HBM read GB/launch | "
              "HBM write GB/launch |", "|---|---|---|---|---|---|"]
    for name, (calls, dur) in sorted(stats.items(), key=lambda kv: -kv[1][1]):
        fr = f"{fetch[name] / 1e9:.3f}" if fetch and name in fetch else "-"
        wr = f"{write[name] / 1e9:.3f}" if write and name in write else "-"
        lines.append(f"| {name} | {calls} | {dur / calls / 1e3:.1f} | {dur / total:.1%} | {fr} | {wr} |")
    with open(args.out, "w") as f:
        f.write("\n".join(lines) + "\n")
    if args.traffic and fetch is not None:
        rec = {"workload": args.workload, "command": args.command, "kernels": {}}
        for name in sorted(set(fetch) & set(write)):
            rec["kernels"][name] = {"read_bytes": round(fetch[name]), "write_bytes": round(write[name]),
                                    "source_sha": source_hash(srcs.get(name) or
                                                              dict((n, s) for _, n, s in KERNELS)[name])}
        with open(args.traffic, "w") as f:
            json.dump(rec, f, indent=1)
            f.write("\n")
    print("\n".join(lines))


if __name__ == "__main__":
    main()
