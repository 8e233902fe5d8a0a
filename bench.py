#!/usr/bin/env python3
"""Throughput benchmark of the GMA forward (bidirectional and causal) on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input of each bf16
workload: the bidirectional forward at B=8, H=8, N=4096 (d_r=64, d_v=64, K=64), the causal
forward at B=8, H=12, N=2048 (d_r=64, d_v=64, K=32, chunk 64), the long-context
bidirectional forward at B=4, H=4, N=65536 (d_r=32, d_v=64, K=128) and the long causal
forward at B=2, H=16, N=32768 (d_r=64, d_v=128, K=256), all bf16 I/O with fp32
accumulation.  Inputs are resident in HBM before timing starts and
rotate over several independent input sets (more bytes than the 256 MB Infinity Cache)
so that every step reads from HBM.

Output: one JSON line with the whole-step throughput (tokens/s), each workload's kernel
against its roofline (HBM or bf16 MFMA, whichever bounds it at peak; per-kernel times from
the library's hipEvent hooks, taken in a second pass over the same steps, one workload at a
time), the step's dominant kernel as `roofline`, and the oracle timed on the host cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--sets S] [--no-cpu-baseline]
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

METRIC = "GMA forward tokens/s (bidir & causal) + achieved HBM GB/s / MFMA % of peak"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16
DEFAULT_STEP = ["bidir_b8h8_n4096", "causal_b8h12_n2048", "bidir_long_n65536", "causal_long_n32768"]


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--sets", type=int, default=3, help="independent input sets rotated over the steps")
    ap.add_argument("--workloads", default=",".join(DEFAULT_STEP),
                    help="comma-separated workload names that make up one step")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--traffic-probe", choices=["copy", "step"], default=None,
                    help="run only a workload for rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE: a plain device copy of "
                         "known size (calibration) or three steps of the benchmark")
    ap.add_argument("--traffic-summarize", metavar="DIR", default=None,
                    help="turn the counter CSVs of the four probe runs under DIR into profiles/traffic.json")
    ap.add_argument("--trace-summarize", metavar="DIR", default=None,
                    help="summarise the library kernels of a rocprofv3 --kernel-trace --stats run of this script "
                         "(CSV output under DIR) into --trace-out")
    ap.add_argument("--trace-out", metavar="FILE", default=None)
    ap.add_argument("--trace-command", default=None, help="the command that produced DIR, recorded in the summary")
    ap.add_argument("--memory-sweep", action="store_true",
                    help="peak device memory of the bidirectional forward at the long-context dims (B=4, H=4, d_r=32, "
                         "d_v=64, K=128, bf16) for N = 4096 .. 65536, with a linear fit; JSON to stdout (and --trace-out)")
    ap.add_argument("--hip-trace-summarize", metavar="DIR", default=None,
                    help="count the HIP API calls made while the library runs, from a rocprofv3 --hip-trace "
                         "--kernel-trace run of --traffic-probe step (CSV output under DIR), into --trace-out")
    ap.add_argument("--counters-summarize", metavar="DIR", default=None,
                    help="summarise rocprofv3 --pmc runs of --traffic-probe step (one subdirectory per pass under DIR) "
                         "into utilisation figures per library kernel, written to --trace-out")
    return ap.parse_args()


COPY_BYTES = 1 << 29  # 512 MiB: larger than the 256 MiB Infinity Cache, so the copy streams HBM


def traffic_json(workloads: str) -> str:
    """Where the calibrated HBM traffic of a workload set is kept (one file per set)."""
    if workloads == ",".join(DEFAULT_STEP):
        return os.path.join(ROOT, "profiles", "traffic.json")
    return os.path.join(ROOT, "profiles", "traffic_%s.json" % workloads.replace(",", "+"))


def kernel_source_hash() -> str:
    """sha256 over every kernel source; a measured traffic figure is valid only for this hash."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "gaussian_mixture_sequence_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def traffic_probe(mode: str, args) -> int:
    import torch
    if mode == "copy":
        # an elementwise kernel (16-byte vector loads and stores, like the library's kernels)
        # that reads and writes COPY_BYTES each; a device-to-device copy goes through a blit
        # kernel whose FETCH_SIZE reads half its bytes, so it is not used for calibration
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        return 0
    args.steps, args.warmup, args.no_cpu_baseline = 3, 0, True
    return main(args, probe_only=True)


def traffic_summarize(d: str, workloads: str) -> int:
    """Per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of the copy and of the step kernels, from the CSVs
    of four runs under d: copy_fetch, copy_write, step_fetch, step_write."""
    import csv
    import glob
    import re

    def per_kernel(run, counter):
        out = {}
        for f in glob.glob(os.path.join(d, run, "*_counter_collection.csv")):
            for row in csv.DictReader(open(f)):
                if row["Counter_Name"] != counter:
                    continue
                name = re.sub(r"\(.*", "", row["Kernel_Name"].replace("(anonymous namespace)::", "")).replace("void ", "")
                out.setdefault(name, {}).setdefault(row["Dispatch_Id"], 0.0)
                out[name][row["Dispatch_Id"]] += float(row["Counter_Value"])
        return {k: sum(v.values()) / len(v) * 1024.0 for k, v in out.items()}  # bytes per dispatch

    cf, cw = per_kernel("copy_fetch", "FETCH_SIZE"), per_kernel("copy_write", "WRITE_SIZE")
    copy_name = max(cf, key=cf.get)  # the copy kernel dominates its run
    f_fetch, f_write = COPY_BYTES / cf[copy_name], COPY_BYTES / cw[copy_name]
    sf, sw = per_kernel("step_fetch", "FETCH_SIZE"), per_kernel("step_write", "WRITE_SIZE")
    kernels = {}
    for k in sorted(set(sf) | set(sw)):
        if not k.startswith("gma::"):
            continue
        fb, wb = sf.get(k, 0.0) * f_fetch, sw.get(k, 0.0) * f_write
        kernels[k] = {"fetch_bytes": round(fb), "write_bytes": round(wb), "hbm_bytes": round(fb + wb)}
    res = {"source_sha256": kernel_source_hash(), "workloads": workloads, "copy_kernel": copy_name,
           "copy_bytes": COPY_BYTES,
           "fetch_factor": round(f_fetch, 4), "write_factor": round(f_write, 4), "kernels": kernels,
           "commands": ["rocprofv3 --pmc FETCH_SIZE --output-format csv -d DIR/copy_fetch -o copy_fetch -- "
                        "python bench.py --traffic-probe copy",
                        "rocprofv3 --pmc WRITE_SIZE --output-format csv -d DIR/copy_write -o copy_write -- "
                        "python bench.py --traffic-probe copy",
                        "rocprofv3 --pmc FETCH_SIZE --output-format csv -d DIR/step_fetch -o step_fetch -- "
                        "python bench.py --traffic-probe step",
                        "rocprofv3 --pmc WRITE_SIZE --output-format csv -d DIR/step_write -o step_write -- "
                        "python bench.py --traffic-probe step",
                        "python bench.py --traffic-summarize DIR"]}
    if workloads != ",".join(DEFAULT_STEP):
        res["commands"] = [c.replace("--traffic-probe step", "--traffic-probe step --workloads " + workloads)
                           .replace("--traffic-summarize DIR", "--traffic-summarize DIR --workloads " + workloads)
                           for c in res["commands"]]
    path = traffic_json(workloads)
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as f:
        json.dump(res, f, indent=1)
    print(json.dumps(res, indent=1))
    return 0


def trace_summarize(d: str, out: str, workloads: str, command: str) -> int:
    """Per-kernel launch statistics (microseconds, from rocprofv3 kernel timestamps) of the library's
    kernels in a kernel-trace run under d, cross-checked against rocprofv3's own stats file."""
    import csv
    import glob
    import re
    import statistics
    durs = {}
    for f in glob.glob(os.path.join(d, "**", "*_kernel_trace.csv"), recursive=True):
        for row in csv.DictReader(open(f)):
            name = re.sub(r"\(.*", "", row["Kernel_Name"].replace("(anonymous namespace)::", "")).replace("void ", "")
            if name.startswith("gma::"):
                durs.setdefault(name, []).append((int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) / 1000.0)
    stats = {}
    for f in glob.glob(os.path.join(d, "**", "*_kernel_stats.csv"), recursive=True):
        for row in csv.DictReader(open(f)):
            name = re.sub(r"\(.*", "", row["Name"].replace("(anonymous namespace)::", "")).replace("void ", "")
            if name.startswith("gma::"):
                stats[name] = float(row["AverageNs"]) / 1000.0
    if not durs:
        print("no library kernels in %s" % d, file=sys.stderr)
        return 1
    total = sum(sum(v) for v in durs.values())
    lines = ["# Kernel trace summary: %s (bf16 unless the kernel name says otherwise)" % workloads,
             "# command (run from the repository root on one MI355X):", "#   " + (command or "?"),
             "# durations in microseconds from rocprofv3 kernel timestamps; library kernels only",
             "%-44s %6s %9s %9s %9s %9s %7s" % ("kernel", "calls", "avg_us", "median_us", "min_us", "max_us", "pct")]
    for name, v in sorted(durs.items(), key=lambda kv: -sum(kv[1])):
        lines.append("%-44s %6d %9.2f %9.2f %9.2f %9.2f %7.2f" % (
            name, len(v), statistics.mean(v), statistics.median(v), min(v), max(v), 100.0 * sum(v) / total))
    lines.append("# stats.csv averages (us): " + ", ".join("%s %.2f" % kv for kv in sorted(stats.items())))
    os.makedirs(os.path.dirname(os.path.abspath(out)), exist_ok=True)
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))
    return 0


def counters_summarize(d: str, out: str, workloads: str, command: str) -> int:
    """SQ counters per library kernel (mean per dispatch, summed over the device) and the
    derived figures rocprofv3 defines: MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE per XCD
    x 1024 SIMDs); VALU busy = SQ_ACTIVE_INST_VALU / 256 CUs / GRBM_GUI_ACTIVE per XCD; LDS bank
    conflict = SQ_LDS_BANK_CONFLICT / 256 / GRBM_GUI_ACTIVE per XCD; wait and issue fractions of
    SQ_WAVE_CYCLES."""
    import csv
    import glob
    import re
    vals = {}
    for f in glob.glob(os.path.join(d, "**", "*_counter_collection.csv"), recursive=True):
        per = {}
        for row in csv.DictReader(open(f)):
            name = re.sub(r"\(.*", "", row["Kernel_Name"].replace("(anonymous namespace)::", "")).replace("void ", "")
            if not name.startswith("gma::"):
                continue
            key = (name, row["Counter_Name"], row["Dispatch_Id"])
            per[key] = per.get(key, 0.0) + float(row["Counter_Value"])
        for (name, ctr, _), v in per.items():
            vals.setdefault(name, {}).setdefault(ctr, []).append(v)
    if not vals:
        print("no library kernels in %s" % d, file=sys.stderr)
        return 1
    lines = ["# SQ counter summary: %s" % workloads, "# commands (run from the repository root on one MI355X):"]
    lines += ["#   " + c for c in (command or "?").split(" ;; ")]
    for name, ctrs in sorted(vals.items()):
        m = {c: sum(v) / len(v) for c, v in ctrs.items()}
        lines.append("%s" % name)
        for c in sorted(m):
            lines.append("  %-28s %16.0f" % (c, m[c]))
        g = m.get("GRBM_GUI_ACTIVE", 0.0) / 8.0  # per XCD
        if g > 0:
            if "SQ_VALU_MFMA_BUSY_CYCLES" in m:
                lines.append("  %-28s %15.1f%%" % ("MFMA busy", 100.0 * m["SQ_VALU_MFMA_BUSY_CYCLES"] / (g * 1024)))
            if "SQ_ACTIVE_INST_VALU" in m:
                lines.append("  %-28s %15.1f%%" % ("VALU busy", 100.0 * m["SQ_ACTIVE_INST_VALU"] / 256 / g))
            if "SQ_LDS_BANK_CONFLICT" in m:
                lines.append("  %-28s %15.1f%%" % ("LDS bank-conflict stall", 100.0 * m["SQ_LDS_BANK_CONFLICT"] / 256 / g))
        if m.get("SQ_WAVE_CYCLES"):
            for c, label in (("SQ_WAIT_ANY", "waiting on a counter"), ("SQ_WAIT_INST_ANY", "waiting for issue"),
                             ("SQ_ACTIVE_INST_ANY", "issuing")):
                if c in m:
                    lines.append("  %-28s %15.1f%%" % (label + " (of wave time)", 100.0 * m[c] / m["SQ_WAVE_CYCLES"]))
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))
    return 0


def memory_sweep(out: str) -> int:
    """Device memory of one forward at the long-context dims for growing N: what the caller
    allocates (inputs, output and the library's workspace; torch.cuda.memory_allocated) and the
    peak while the call runs (torch.cuda.max_memory_allocated, which stays at the former: the
    library allocates nothing).  A least-squares line in N fits it; the quadratic term of a second
    fit is reported relative to the largest value (Sec. 5.1: memory grows linearly in N)."""
    import numpy as np
    import torch
    from gaussian_mixture_sequence_amd import binding as gb
    from gaussian_mixture_sequence_amd.inputs import WORKLOADS, make_inputs
    gb.load()
    res = {"command": "python bench.py --memory-sweep", "variants": {}}
    for causal in (False, True):
        base = WORKLOADS["bidir_long_n65536"].with_(causal=causal)
        rows = []
        for n in (4096, 8192, 16384, 32768, 49152, 65536):
            w = base.with_(N=n)
            torch.cuda.empty_cache()
            torch.cuda.synchronize()
            before = torch.cuda.memory_allocated()
            d = {k: v.cuda() for k, v in make_inputs(w).items()}
            op = gb.GMA_OP_CAUSAL if causal else gb.GMA_OP_BIDIR
            ws_bytes = gb.gma_workspace_size(op, w.B, w.H, w.N, w.d_r, w.d_v, w.K, gb.GMA_BF16, w.chunk if causal else 0)
            ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")
            o = torch.empty(w.B, w.H, w.N, w.d_v, dtype=torch.bfloat16, device="cuda")
            torch.cuda.synchronize()
            held = torch.cuda.memory_allocated()
            torch.cuda.reset_peak_memory_stats()
            if causal:
                gb.gma_forward_causal(d["xq"], d["xk"], d["v"], d["mu"], d["sigma2"], d["pi"], w.eps, chunk=w.chunk,
                                      out=o, workspace=ws)
            else:
                gb.gma_forward_bidir(d["xq"], d["xk"], d["v"], d["mu"], d["sigma2"], d["pi"], w.eps, out=o, workspace=ws)
            torch.cuda.synchronize()
            peak = torch.cuda.max_memory_allocated()
            rows.append({"N": n, "call_bytes": int(held - before), "peak_during_call_minus_held": int(peak - held),
                         "workspace_bytes": int(ws_bytes),
                         "gamma_fp32_bytes_if_materialised": int(2 * w.B * w.H * n * w.K * 4)})
            del d, ws, o
        ns = np.array([r["N"] for r in rows], float)
        pk = np.array([r["call_bytes"] for r in rows], float)
        b, a = np.polyfit(ns, pk, 1)
        q = np.polyfit(ns, pk, 2)
        res["variants"]["causal" if causal else "bidirectional"] = {
            "workload": "%s forward, B=4 H=4 d_r=32 d_v=64 K=128 bf16" % ("causal" if causal else "bidirectional"),
            "rows": rows,
            "linear_fit": {"bytes_per_position": b, "intercept_bytes": a,
                           "max_abs_residual_rel": float(np.abs(pk - (a + b * ns)).max() / pk.max())},
            "quadratic_term_rel": float(abs(q[0]) * ns.max() ** 2 / pk.max())}
    text = json.dumps(res, indent=1)
    print(text)
    if out:
        with open(out, "w") as f:
            f.write(text + "\n")
    return 0


def hip_trace_summarize(d: str, out: str, command: str) -> int:
    """HIP API calls from the first library kernel launch on, by function name, from the CSVs of a
    rocprofv3 --hip-trace --kernel-trace run of `--traffic-probe step` (every buffer is allocated
    before that launch).  Allocation calls in that window would be the library's."""
    import csv
    import glob
    kt = [r for f in glob.glob(os.path.join(d, "**", "*_kernel_trace.csv"), recursive=True) for r in csv.DictReader(open(f))]
    api = [r for f in glob.glob(os.path.join(d, "**", "*_hip_api_trace.csv"), recursive=True) for r in csv.DictReader(open(f))]
    gma = [r for r in kt if "gma::" in r["Kernel_Name"]]
    if not gma or not api:
        print("no library kernels or no HIP API records under %s" % d, file=sys.stderr)
        return 1
    first_corr = min(int(r["Correlation_Id"]) for r in gma)
    start = min(int(r["Start_Timestamp"]) for r in api if int(r["Correlation_Id"]) == first_corr)
    counts = {}
    for r in api:
        if int(r["Start_Timestamp"]) >= start:
            counts[r["Function"]] = counts.get(r["Function"], 0) + 1
    alloc = {k: v for k, v in counts.items() if "alloc" in k.lower() or "free" in k.lower()}
    lines = ["# HIP API calls from the first library kernel launch on (%d library kernel dispatches)" % len(gma),
             "# command (run from the repository root on one MI355X):", "#   " + (command or "?"),
             "allocation or free calls in the window: %d %s" % (sum(alloc.values()), json.dumps(alloc))]
    lines += ["%-40s %8d" % kv for kv in sorted(counts.items(), key=lambda kv: -kv[1])]
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))
    return 0


def measured_traffic(kernel_symbol_prefix: str, workloads: str):
    """HBM bytes per launch of the kernel, from the workload set's traffic record when that record
    was taken on the current kernel sources."""
    try:
        with open(traffic_json(workloads)) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != kernel_source_hash():
        return None
    for k, v in t.get("kernels", {}).items():
        if k.startswith(kernel_symbol_prefix):
            return v["hbm_bytes"]
    return None


def alg_bytes_per_token_head(w, kernel: str) -> float:
    """Algorithmic HBM bytes per (token, head) that a kernel must move (per query row for
    cross-attention, with the context rows' share folded in)."""
    e = 2 if w.dtype == "bf16" else 4
    if w.cross:  # X_K and V of N_k context rows in; X_Q of N_q rows in and O out
        return e * (w.d_r + w.d_v) * (w.n_ctx + w.N) / max(w.N, 1)
    if w.decode:  # one position: X_Q, X_K, V in, O out, and the fp32 memory read and written
        return e * (2 * w.d_r + 2 * w.d_v) + 2 * 4 * w.K * (w.d_v + 1)
    if w.diagnostics:  # the routing vectors in; the outputs (per token, not per head) are negligible
        return e * w.d_r
    if w.responsibilities:  # the routing vectors in, Gamma out, both in the I/O dtype
        return e * (w.d_r + w.K)
    if w.backward:  # the register-tiled passes keep the responsibilities (fp32, K per row) between passes
        g = 4 * w.K
        T = 64  # positions per tile of the causal K-blocked passes (C: T fp32 per row)
        # the K-blocked passes cache both sides' responsibilities; the block passes read them back
        if kernel.endswith("_kb_write") or kernel.endswith("_kb_aggregate"):
            return e * (w.d_r + w.d_v) + g              # X_K and V in, Gamma_K out
        if kernel.endswith("_kb_query_gamma"):
            return e * w.d_r + g                        # X_Q in, Gamma_Q out
        if kernel.endswith("_bwd_kb_query_rows"):
            return e * (w.d_r + w.d_v) + g + 8          # X_Q and dO in, Gamma_Q and (D, a') out
        if kernel.endswith("_bwdc_kb_query_rows"):
            return 2 * e * w.d_v + 2 * g + 8 + 4 * T    # V and dO in, both Gammas in, (D, a') and C out
        if kernel.endswith("_bwd_kb_key_rows"):
            return 2 * e * w.d_v + g + 4                # V in, dV out, Gamma_K in, w out
        if kernel.endswith("_bwdc_kb_key_rows"):
            return 3 * e * w.d_v + g + 4 + 4 * T        # V and dO in, dV out, Gamma_K and C in, w out
        if kernel.endswith("_bwd_kb_query") or kernel.endswith("_bwd_kb_key"):
            return e * (2 * w.d_r + w.d_v) + g          # X and dO (or V) in, dX out, Gamma in
        if kernel.endswith("_bwdc_kb_query") or kernel.endswith("_bwdc_kb_key"):
            return e * (2 * w.d_r + 2 * w.d_v) + 2 * g  # X, V and dO in, dX out, both Gammas in
        if kernel.endswith("_bwdc_aggregate"):
            return e * (w.d_r + w.d_v) + g          # X_K and V in, Gamma_K out
        if kernel.endswith("_bwdc_query"):
            return e * (2 * w.d_r + 2 * w.d_v) + 2 * g  # X_Q, V, dO in, dX_Q out, Gamma_K in, Gamma_Q out
        if kernel.endswith("_bwdc_key"):
            return e * (2 * w.d_r + 3 * w.d_v) + 2 * g  # X_K, V, dO in, dX_K, dV out, Gamma_K and Gamma_Q in
        if kernel.endswith("_bwd_write"):
            return e * (w.d_r + w.d_v) + g          # X_K and V in, Gamma_K out
        if kernel.endswith("_bwd_query"):
            return e * (2 * w.d_r + w.d_v)          # X_Q and dO in, dX_Q out
        if kernel.endswith("_bwd_key"):
            return e * (2 * w.d_r + 2 * w.d_v) + g  # X_K and V in, dX_K and dV out, Gamma_K in
        if kernel == "step":
            return e * (4 * w.d_r + 3 * w.d_v)  # X_Q, X_K, V, dO in; dX_Q, dX_K, dV out
        return 0.0
    if kernel.endswith("_write") or kernel.endswith("_causal_aggregate"):
        return e * (w.d_r + w.d_v)          # X_K and V in
    if kernel.endswith("_read"):
        return e * (w.d_r + w.d_v)          # X_Q in, O out
    if kernel.endswith("_scan") or kernel.endswith("_bidir") or kernel.endswith("_causal"):
        return e * (2 * w.d_r + 2 * w.d_v)  # X_Q, X_K, V in, O out (whole forward in one launch)
    return 0.0


# fp32 vector peak without packed-fp32 instructions (the library is built with them disabled):
# 256 CUs x 4 SIMDs x 16 lanes x 2 flops per FMA x 2.4 GHz
F32_VALU_PEAK_TFLOPS = 78.6


def alg_flops_per_token_head(w, kernel: str) -> float:
    """Algorithmic fp32 flops per (row, head) of the backward passes (an FMA counts 2): per (k, d)
    the direct-form score 3 (difference, then a fused square-scale-add), dX 4 and the three moments
    5; per (k, c) each product with the memory 2; per k the softmax 3, Eq. 18 4, D / Z terms 2 each.
    A pass that reads responsibilities another pass computed does no score work for them."""
    if not w.backward:
        return 0.0
    K, dr, dv = w.K, w.d_r, w.d_v
    T = 64  # positions per tile of the causal passes: the masked in-tile products cost T/2 per row
    # the K-blocked passes: row passes form the responsibilities and the per-row sums, block
    # passes (one component block each) the score gradient, moments and dX shares
    if kernel.endswith("_kb_write") or kernel.endswith("_kb_aggregate"):
        return 3 * K * dr + 2 * K * dv + 4 * K
    if kernel.endswith("_kb_query_gamma"):
        return 3 * K * dr + 3 * K
    if kernel.endswith("_bwd_kb_query_rows"):     # scores, N_i and D_i, a'_i
        return 3 * K * dr + 2 * K * dv + 6 * K + 2 * dv
    if kernel.endswith("_bwdc_kb_query_rows"):    # C, N_i and D_i, C V, a'_i, what the row sends
        return 4 * K * dv + T * K + T * dv + 4 * K + 2 * dv
    if kernel.endswith("_bwd_kb_key_rows"):       # dV_j and w_j
        return 2 * K * dv + 2 * K + 2 * dv
    if kernel.endswith("_bwdc_kb_key_rows"):      # dV_j and w_j with the in-tile queries
        return 2 * K * dv + T * dv + 2 * K + T + 2 * dv
    if kernel.endswith("_bwd_kb_query"):          # g, ds, moments, dX, the memory gradient
        return 9 * K * dr + 4 * K * dv + 5 * K
    if kernel.endswith("_bwd_kb_key"):
        return 9 * K * dr + 2 * K * dv + 4 * K
    if kernel.endswith("_bwdc_kb_query") or kernel.endswith("_bwdc_kb_key"):  # A, g, ds, moments, dX
        return 9 * K * dr + 2 * K * dv + T * K + T * dv + 4 * K
    if kernel.endswith("_bwdc_aggregate"):
        return 3 * K * dr + 2 * K * dv + 4 * K
    if kernel.endswith("_bwdc_query"):  # the bidirectional query pass and the memory update
        return 12 * K * dr + 8 * K * dv + 12 * K + 2 * dv + 2 * T * K + 2 * T * dv
    if kernel.endswith("_bwdc_key"):    # the bidirectional key pass without scores, the suffix update
        return 9 * K * dr + 6 * K * dv + 5 * K + 2 * T * K + 2 * T * dv
    if kernel.endswith("_bwd_write"):
        return 3 * K * dr + 2 * K * dv + 4 * K
    if kernel.endswith("_bwd_query"):
        return 12 * K * dr + 6 * K * dv + 12 * K + 2 * dv
    if kernel.endswith("_bwd_key"):  # Gamma_K comes from the write pass
        return 9 * K * dr + 4 * K * dv + 5 * K
    return 0.0


def alg_mfma_flops_per_token_head(w, kernel: str) -> float:
    """Algorithmic flops per (token, head) of a bf16 forward kernel: the score contractions of both
    sides, 2 x 2 K d_r MACs (Sec. 3.4, Eq. 12's 2 N K d_r term), the write and the read,
    2 x K (d_v + 1) MACs, and for the chunked causal form the in-chunk products, C (K + d_v + 1)
    MACs for a chunk of C positions (an FMA counts 2 flops)."""
    if w.backward or w.diagnostics or w.dtype != "bf16":
        return 0.0
    K, dr, dv = w.K, w.d_r, w.d_v
    if w.responsibilities:  # one side's score contraction
        return 4 * K * dr if kernel.endswith("_resp") else 0.0
    full = 8 * K * dr + 4 * K * (dv + 1)
    if kernel.endswith("_write") or kernel.endswith("_causal_aggregate"):
        return 4 * K * dr + 2 * K * (dv + 1)
    if kernel.endswith("_read"):
        return 4 * K * dr + 2 * K * (dv + 1)
    if kernel.endswith("_causal") or kernel.endswith("_scan"):
        return full + 2 * w.chunk * (K + dv + 1)
    if kernel.endswith("_bidir") or kernel.endswith("_cross"):
        return full
    return 0.0


def component_tiles(K: int) -> int:
    """32-component tiles the bf16 kernels are compiled for (K padded to 1, 2, 4 or 8 tiles)."""
    t = (K + 31) // 32
    return 1 if t <= 1 else 2 if t <= 2 else 4 if t <= 4 else 8


def kernel_symbol(w, name: str) -> str:
    """The demangled symbol (up to its argument list) of the kernel a bench name stands for."""
    if w.dtype == "bf16" and not w.backward and not w.diagnostics and not w.decode:
        kt, vt = component_tiles(w.K), w.d_v // 32
        if name.endswith("_bidir") or name.endswith("_cross"):
            return "gma::bf::bidir_kernel<%d, %d, %d>" % (w.d_r, kt, vt)
        if name.endswith("_write") or name.endswith("_read"):  # the phases as their own launches
            return "gma::bf::%s_kernel<%d, %d, %d>" % (name.rsplit("_", 1)[1], w.d_r, kt, vt)
        if name.endswith("_combine"):
            return "gma::bf::combine_kernel"
        if name.endswith("_causal"):
            if kt == 8 and w.d_r <= 64:  # the third argument is the kernel's wave count
                return "gma::bf::wide_causal_kernel<%d, %d, " % (w.d_r, vt)
            if kt <= 4 and w.d_r * kt <= 256:
                return "gma::bf::causal_kernel<%d, %d, %d, %d>" % (w.d_r, kt, vt, max(32, w.chunk))
    return KERNEL_SYMBOL.get(name, "?")


def kernel_roofline(w, name: str, entry: dict, workloads: str, steps: int):
    """A kernel's algorithmic rate against its roofline: the bf16 forwards against HBM and bf16
    MFMA peaks (bound = whichever would take longer at peak), the fp32 backward passes against the
    fp32 vector peak."""
    avg_us = entry["avg_us"]
    sym = kernel_symbol(w, name)
    base = {"kernel": "%s/%s" % (w.name, name), "symbol": sym, "avg_us": avg_us,
            "launches_per_step": entry["launches"] / max(steps, 1),
            "traffic": measured_traffic(sym, workloads)}
    if "alg_TFLOPs" in entry:  # the fp32 backward: bound by vector ALU issue
        ach = entry["alg_TFLOPs"]
        return dict(base, bound="alu", achieved=ach, peak=F32_VALU_PEAK_TFLOPS, unit="TFLOP/s",
                    frac=round(ach / F32_VALU_PEAK_TFLOPS, 4), alg_flops_per_launch=entry["alg_flops_per_launch"],
                    alg_bytes_per_launch=entry.get("alg_bytes_per_launch"))
    if "alg_GBps" not in entry:
        return None
    hbm_frac = entry["alg_GBps"] / HBM_PEAK_GBPS
    r = dict(base, alg_bytes_per_launch=entry["alg_bytes_per_launch"], hbm_frac=round(hbm_frac, 4))
    t_hbm = entry["alg_bytes_per_launch"] / (HBM_PEAK_GBPS * 1e9)
    t_mfma = entry.get("alg_mfma_flops_per_launch", 0) / (BF16_MFMA_PEAK_TFLOPS * 1e12)
    if "alg_mfma_TFLOPs" in entry:
        r["alg_mfma_flops_per_launch"] = entry["alg_mfma_flops_per_launch"]
        r["mfma_frac"] = round(entry["alg_mfma_TFLOPs"] / BF16_MFMA_PEAK_TFLOPS, 4)
    if t_mfma > t_hbm:
        ach = entry["alg_mfma_TFLOPs"]
        r.update(bound="mfma", achieved=ach, peak=BF16_MFMA_PEAK_TFLOPS, unit="TFLOP/s",
                 frac=round(ach / BF16_MFMA_PEAK_TFLOPS, 4))
    else:
        ach = entry["alg_GBps"]
        r.update(bound="hbm", achieved=ach, peak=HBM_PEAK_GBPS, unit="GB/s", frac=round(hbm_frac, 4))
    return r


def cpu_baseline(ws_list) -> dict:
    """The oracle (fp64 C with OpenMP over (batch, head) problems) on a bounded sample of every
    workload of the step: the first batch entries of each workload, as many whole sequences as
    there are threads (all heads of a sequence at once), timed on the host cores; then, on one
    thread, the first 2048 positions of one (batch, head) problem of each workload.  The method
    is linear in the sequence length, so a workload's rate is its sample's token rate, and the
    step's is its tokens over the summed estimated times of its workloads."""
    import oracle
    from gaussian_mixture_sequence_amd.inputs import make_inputs
    if any(w.backward for w in ws_list):
        cpu_inputs = [(w, {k: oracle._f64(v) for k, v in make_inputs(w).items()}) for w in ws_list if w.backward]
        return cpu_backward_sample(cpu_inputs)
    threads = oracle.num_threads()

    def run(w, inp, b1, h1, n1):
        sl = {k: (v[:b1, :h1, :n1].contiguous() if k in ("xq", "xk", "v") else v[:h1].contiguous())
              for k, v in inp.items()}
        if w.diagnostics:
            t0 = time.perf_counter()
            oracle.diagnostics.diagnostics(sl["xq"], sl["mu"], sl["sigma2"], sl["pi"])
            return time.perf_counter() - t0
        if w.responsibilities:
            t0 = time.perf_counter()
            oracle.responsibilities(sl["xq"], sl["mu"], sl["sigma2"], sl["pi"])
            return time.perf_counter() - t0
        fn = oracle.forward_causal if w.causal else oracle.forward_cross if w.cross else oracle.forward_bidir
        t0 = time.perf_counter()
        fn(sl["xq"], sl["xk"], sl["v"], sl["mu"], sl["sigma2"], sl["pi"], w.eps)
        return time.perf_counter() - t0

    samples, est_s, est_1_s = [], 0.0, 0.0
    for w in ws_list:
        inp = make_inputs(w)
        bs = max(1, min(w.B, threads // max(w.H, 1)))
        dt = run(w, inp, bs, w.H, w.N)
        rate = bs * w.N / dt  # tokens (all heads) per second
        est_s += w.B * w.N / rate
        samples.append("%s: %d sequence(s) x %d heads x %d positions in %.2f s" % (w.name, bs, w.H, w.N, dt))
    oracle.set_num_threads(1)
    try:
        for w in ws_list:
            inp = make_inputs(w)
            n1 = min(w.N, 2048)
            dt = run(w, inp, 1, 1, n1)
            est_1_s += w.B * w.N * w.H / (n1 / dt)  # one head-row per position per second
    finally:
        oracle.set_num_threads(threads)
    tokens = sum(w.B * w.N for w in ws_list)
    return {"value": round(tokens / est_s, 1), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "; ".join(samples) + "; fp64 C oracle, OpenMP over (batch, head); step time estimated "
                      "from each workload's sample rate",
            "single_thread": {"value": round(tokens / est_1_s, 1), "unit": "tokens/s", "cores": 1,
                              "sample": "first 2048 positions of (batch 0, head 0) of each workload, one thread"}}


KERNEL_SYMBOL = {"bf16_scan": "gma::bf::scan_kernel", "bf16_bidir": "gma::bf::bidir_kernel",
                 "bf16_cross": "gma::bf::bidir_kernel", "bf16_resp": "gma::bf::resp_kernel",
                 "bf16_decode": "gma::dec::decode_kernel", "bf16_diag": "gma::diag::diag_fused_kernel",
                 "f32_bwd_query": "gma::f32_bwd_tiled_kernel<1, ", "f32_bwd_key": "gma::f32_bwd_tiled_kernel<2, ",
                 "f32_bwdc_query": "gma::f32_bwd_tiled_kernel<3, ", "f32_bwdc_key": "gma::f32_bwd_tiled_kernel<4, ",
                 "f32_bwd_kb_query": "gma::f32_bwd_kb_block_kernel<true, ",
                 "f32_bwd_kb_key": "gma::f32_bwd_kb_block_kernel<false, ",
                 "f32_bwdc_kb_query": "gma::f32_bwdc_kb_block_kernel<true, ",
                 "f32_bwdc_kb_key": "gma::f32_bwdc_kb_block_kernel<false, ",
                 "bf16_causal": "gma::bf::causal_kernel", "bf16_causal_aggregate": "gma::bf::write_kernel<64, 1"}


def cpu_backward_sample(cpu_inputs):
    """The oracle's backward (numpy fp64) on successive (batch, head) problems of the workload until
    about 10 s have been timed; a problem of N positions is N / H tokens of the whole workload."""
    import oracle.backward
    w, d = cpu_inputs[0]
    done = 0
    tc = time.perf_counter()
    while True:
        b, h = divmod(done % (w.B * w.H), w.H)
        sl = {k: (v[b:b + 1, h:h + 1] if k in ("xq", "xk", "v", "d_o") else v[h:h + 1]) for k, v in d.items()}
        fn = oracle.backward.backward_causal if w.causal else oracle.backward.backward_bidir
        fn(sl["xq"], sl["xk"], sl["v"], sl["mu"], sl["sigma2"], sl["pi"], w.eps, sl["d_o"])
        done += 1
        cpu_s = time.perf_counter() - tc
        if cpu_s >= 10.0:
            break
    try:  # numpy's BLAS pool runs the matrix products; everything else is one thread
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except ImportError:
        threads = 1
    return {"value": round(done * w.N / w.H / cpu_s, 1), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "%d (batch, head) problems of %d positions (the first of the workload's %d, in order), "
                      "numpy fp64 backward oracle (BLAS pool for the matrix products); %.2f s wall; a problem is N / H = %g tokens"
                      % (done, w.N, w.B * w.H, cpu_s, w.N / w.H)}


def main(args=None, probe_only=False) -> int:
    args = args or parse()
    if args.traffic_summarize:
        return traffic_summarize(args.traffic_summarize, args.workloads)
    if args.trace_summarize:
        return trace_summarize(args.trace_summarize, args.trace_out, args.workloads, args.trace_command)
    if args.memory_sweep:
        return memory_sweep(args.trace_out)
    if args.hip_trace_summarize:
        return hip_trace_summarize(args.hip_trace_summarize, args.trace_out, args.trace_command)
    if args.counters_summarize:
        return counters_summarize(args.counters_summarize, args.trace_out, args.workloads, args.trace_command)
    if args.traffic_probe and not probe_only:
        return traffic_probe(args.traffic_probe, args)
    if args.gpus != 1:
        print("bench.py: this implementation runs on a single GPU; --gpus %d is not supported "
              "(multi-GPU sharding is a design note only)" % args.gpus, file=sys.stderr)
        return 2
    import numpy as np
    import torch

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    from gaussian_mixture_sequence_amd import binding as gb
    from gaussian_mixture_sequence_amd.inputs import WORKLOADS, make_inputs

    gb.load()  # raises if libgma.so is missing: there is no fallback path
    names = [n for n in args.workloads.split(",") if n]
    ws_list = [WORKLOADS[n] for n in names]
    dev = torch.device("cuda:0")

    # ---- inputs resident in HBM: `sets` independent input sets per workload
    sets = []   # sets[s][i] = dict of device tensors for workload i
    for s in range(args.sets):
        row = []
        for w in ws_list:
            inp = make_inputs(w, seed=w.seed + 1000 * s)
            d = {k: v.to(dev) for k, v in inp.items()}
            if w.decode:  # one contiguous [B,H,1,.] slice per position, and two memories to alternate
                for k in ("xq", "xk", "v"):
                    d[k + "_t"] = [d[k][:, :, t:t + 1].contiguous() for t in range(w.N)]
                d["state"] = [torch.zeros(w.B, w.H, w.K, w.d_v + 1, dtype=torch.float32, device=dev)
                              for _ in range(2)]
            row.append(d)
        sets.append(row)
    outs, wss = [], []
    for i, w in enumerate(ws_list):
        dt = sets[0][i]["xq"].dtype
        if w.backward:
            d0 = sets[0][i]
            outs.append([{"dXQ": torch.empty_like(d0["xq"]), "dXK": torch.empty_like(d0["xk"]),
                          "dV": torch.empty_like(d0["v"]), "dmu": torch.empty_like(d0["mu"]),
                          "dsigma2": torch.empty_like(d0["sigma2"]), "dpi": torch.empty_like(d0["pi"])}
                         for _ in range(args.sets)])
        elif w.responsibilities:
            outs.append([torch.empty(w.B, w.H, w.N, w.K, dtype=dt, device=dev) for _ in range(args.sets)])
        else:
            outs.append([torch.empty(w.B, w.H, 1 if w.decode else w.N, w.d_v, dtype=dt, device=dev)
                         for _ in range(args.sets)])
        op = gb.GMA_OP_CAUSAL if w.causal else gb.GMA_OP_BIDIR
        io = gb.GMA_BF16 if w.dtype == "bf16" else gb.GMA_F32
        if w.cross:
            nbytes = gb.gma_cross_workspace_size(w.B, w.H, w.N, w.n_ctx, w.d_r, w.d_v, w.K, io)
        elif w.diagnostics:
            nbytes = gb.gma_workspace_size(gb.GMA_OP_DIAGNOSTICS, w.B, w.H, w.N, w.d_r, 0, w.K, io)
        elif w.responsibilities:
            nbytes = gb.gma_workspace_size(gb.GMA_OP_RESPONSIBILITIES, w.B, w.H, w.N, w.d_r, 1, w.K, io)
        elif w.backward:
            nbytes = gb.gma_workspace_size(gb.GMA_OP_BACKWARD_CAUSAL if w.causal else gb.GMA_OP_BACKWARD_BIDIR,
                                           w.B, w.H, w.N, w.d_r, w.d_v, w.K, io)
        else:
            nbytes = gb.gma_workspace_size(op, w.B, w.H, 1 if w.decode else w.N, w.d_r, w.d_v, w.K, io, w.chunk)
        wss.append(torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev))
    stream = torch.cuda.current_stream()

    def step(k: int) -> None:
        for i in range(len(ws_list)):
            step_one(k, i)

    def step_one(k: int, i: int) -> None:
        s = k % args.sets
        w = ws_list[i]
        if True:
            d = sets[s][i]
            if w.diagnostics:
                gb.gma_responsibility_diagnostics(d["xq"], d["mu"], d["sigma2"], d["pi"], workspace=wss[i],
                                                  stream=stream)
            elif w.responsibilities:
                gb.gma_responsibilities(d["xq"], d["mu"], d["sigma2"], d["pi"], out=outs[i][s], workspace=wss[i],
                                        stream=stream)
            elif w.backward and w.causal:
                gb.gma_backward_causal(d["xq"], d["xk"], d["v"], d["mu"], d["sigma2"], d["pi"], d["d_o"], w.eps,
                                       out=outs[i][s], workspace=wss[i], stream=stream)
            elif w.backward:
                gb.gma_backward_bidir(d["xq"], d["xk"], d["v"], d["mu"], d["sigma2"], d["pi"], d["d_o"], w.eps,
                                      out=outs[i][s], workspace=wss[i], stream=stream)
            elif w.decode:
                t = (k // args.sets) % w.N
                gb.gma_forward_causal_state(d["xq_t"][t], d["xk_t"][t], d["v_t"][t], d["mu"], d["sigma2"], d["pi"],
                                            w.eps, chunk=w.chunk, state_in=d["state"][t % 2],
                                            state_out=d["state"][(t + 1) % 2], out=outs[i][s], workspace=wss[i],
                                            stream=stream)
            elif w.causal:
                gb.gma_forward_causal(d["xq"], d["xk"], d["v"], d["mu"], d["sigma2"], d["pi"], w.eps,
                                      chunk=w.chunk, out=outs[i][s], workspace=wss[i], stream=stream)
            elif w.cross:
                gb.gma_forward_cross(d["xq"], d["xk"], d["v"], d["mu"], d["sigma2"], d["pi"], w.eps,
                                     out=outs[i][s], workspace=wss[i], stream=stream)
            else:
                gb.gma_forward_bidir(d["xq"], d["xk"], d["v"], d["mu"], d["sigma2"], d["pi"], w.eps,
                                     out=outs[i][s], workspace=wss[i], stream=stream)

    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    if probe_only:  # counters of exactly `steps` steps, nothing else launched
        for k in range(args.steps):
            step(k)
        torch.cuda.synchronize()
        return 0

    # ---- timed region: exactly `steps` steps between two synchronisations
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for k in range(args.steps):
        step(k)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    dev_ms = ev0.elapsed_time(ev1)
    tokens_per_step = sum(w.B * (1 if w.decode else w.N) for w in ws_list)
    value = tokens_per_step * args.steps / wall

    # ---- per-kernel durations: the same steps again, one workload at a time, with the library's
    # hipEvent hooks (events recorded on the launch stream around every library launch)
    per_wl = []
    prof_ms = 0.0
    for i in range(len(ws_list)):
        gb.gma_profiling(True)
        torch.cuda.synchronize()
        tp0 = time.perf_counter()
        for k in range(args.steps):
            step_one(k, i)
        torch.cuda.synchronize()
        prof_ms += 1000.0 * (time.perf_counter() - tp0)
        per_wl.append(gb.gma_profiling_collect())
        gb.gma_profiling(False)

    kernels, rooflines = {}, []
    for w, kstats in zip(ws_list, per_wl):
        for name, (launches, total_ms) in kstats.items():
            avg_us = 1000.0 * total_ms / max(launches, 1)
            entry = {"launches": launches, "avg_us": round(avg_us, 3)}
            per_launch = alg_bytes_per_token_head(w, name) * w.B * w.H * (1 if w.decode else w.N)
            if per_launch:
                entry["alg_bytes_per_launch"] = int(per_launch)
                entry["alg_GBps"] = round(per_launch / (avg_us * 1e-6) / 1e9, 1)
            flops = alg_flops_per_token_head(w, name) * w.B * w.H * w.N
            if flops:
                entry["alg_flops_per_launch"] = int(flops)
                entry["alg_TFLOPs"] = round(flops / (avg_us * 1e-6) / 1e12, 2)
            mflops = alg_mfma_flops_per_token_head(w, name) * w.B * w.H * (1 if w.decode else w.N)
            if mflops:
                entry["alg_mfma_flops_per_launch"] = int(mflops)
                entry["alg_mfma_TFLOPs"] = round(mflops / (avg_us * 1e-6) / 1e12, 2)
            kernels["%s/%s" % (w.name, name)] = entry
        if kstats:  # the workload's dominant kernel against its roofline
            name = max(kstats.items(), key=lambda kv: kv[1][1])[0]
            r = kernel_roofline(w, name, kernels["%s/%s" % (w.name, name)], args.workloads, args.steps)
            if r:
                rooflines.append(r)
    # the step's dominant kernel (largest share of the step's time)
    roofline = None
    if rooflines:
        roofline = max(rooflines, key=lambda r: r["avg_us"] * r["launches_per_step"])

    # ---- sanity: outputs finite
    for i in range(len(ws_list)):
        o = outs[i][0]
        if not all(torch.isfinite(t.float()).all() for t in (o.values() if isinstance(o, dict) else [o])):
            print("bench.py: non-finite output in %s" % names[i], file=sys.stderr)
            return 1

    step_bytes = sum(w.B * w.H * (1 if w.decode else w.N) *
                     alg_bytes_per_token_head(w, "step" if w.backward else "bf16_scan") for w in ws_list)
    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(1000.0 * wall / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if any(w.dtype == "bf16" for w in ws_list) else "f32",
        "data": "synthetic (seeded; mu~N(0,mu_std), sigma2=softplus(N(0,1))+1e-3, pi=softmax(N(0,1)), "
                "X_Q,X_K,V~N(0,1); %d rotating input sets)" % args.sets,
        "config": {
            "workload": " + ".join("%s (%s B=%d H=%d %s d_r=%d d_v=%d K=%d%s)" % (
                w.name, ("responsibilities" if w.responsibilities else "diagnostics" if w.diagnostics else
                         "causal" if w.causal else "cross" if w.cross else "bidir") + (" backward" if w.backward else ""),
                w.B, w.H,
                "N_q=%d N_k=%d" % (w.N, w.n_ctx) if w.cross else "N=%d" % w.N, w.d_r, w.d_v, w.K,
                ", chunk=%d" % w.chunk if w.causal and not w.backward else "") for w in ws_list),
            "tokens_per_step": tokens_per_step,
            "eps": 1e-6,
        },
        "device_ms_per_step": round(dev_ms / args.steps, 4),
        "step_alg_hbm_GBps": round(step_bytes / (wall / args.steps) / 1e9, 1),
        "step_alg_hbm_frac": round(step_bytes / (wall / args.steps) / 1e9 / HBM_PEAK_GBPS, 4),
        "roofline": roofline,
        "rooflines": rooflines,
        "kernels": kernels,
        "profiled_ms_per_step": round(prof_ms / args.steps, 4),
    }

    # ---- the oracle on the host cores, same workloads (first input set), fp64
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(ws_list)
    print(json.dumps(result))
    return 0


if __name__ == "__main__":
    sys.exit(main())
