#!/usr/bin/env python3
"""Turn rocprofv3 CSV output of bench.py runs into the short text summaries
kept under profiles/ (and the per-launch HBM traffic figure bench.py reports).

    python bench_profiles.py --workload gqa_causal_bf16 \
        --trace DIR --trace-cmd "..." --bench-json FILE \
        [--fetch DIR --write DIR --pmc-cmd "..."]

--trace: directory of a `rocprofv3 --kernel-trace --stats --output-format csv`
run of bench.py; the summary lists every kernel's statistics and the mean
duration of the attention kernel over the timed launches (the last --steps
dispatches), next to the bench line printed by the same run.

--counters: directory of a `rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES
SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_INSTS_MFMA SQ_INSTS_VALU
SQ_INSTS_LDS GRBM_GUI_ACTIVE` run; the summary gives MFMA busy % (MFMA busy
cycles over 1024 SIMDs x the GPU-active cycles of one XCD), the LDS
bank-conflict share of LDS-active cycles and instruction counts per wave.

--fetch / --write: directories of `rocprofv3 --pmc FETCH_SIZE` and
`--pmc WRITE_SIZE` runs of bench.py with --copy-calibration-mib M.  The
counters are in KiB per dispatch.  The plain device copy of M MiB that the
same runs launch reads and writes exactly M MiB, so
factor = M*1024 / (counter reading of the copy) converts each counter to
bytes; the attention kernel's per-launch HBM bytes are
fetch*factor_f + write*factor_w, averaged over its dispatches.
"""
from __future__ import annotations

import argparse
import csv
import json
import os
import statistics
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# The library's kernels of each pass (rocprofv3 prints some names mangled,
# some demangled); a pass's "step" is one launch of each of its kernels.
KERNELS = {
    "fwd": ("attn_fwd16p_kernel", "attn_fwd_kernel"),
    "bwd": ("delta_kernel", "dkdv_kernel", "dq_kernel"),
    "decode": ("decode_kernel", "decode_merge_kernel"),
}
MODE = "fwd"


def short_name(mangled: str) -> str:
    for names in KERNELS.values():
        for key in names:
            if key in mangled:
                return key
    return mangled[:60]


def is_attn(name: str) -> bool:
    return "mi_attn" in name and short_name(name) in KERNELS[MODE]


def read_csv(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def trace_summary(args) -> str:
    stats = read_csv(os.path.join(args.trace, "run_kernel_stats.csv"))
    trace = read_csv(os.path.join(args.trace, "run_kernel_trace.csv"))
    attn = [r for r in trace if is_attn(r["Kernel_Name"])]
    kinds = sorted({short_name(r["Kernel_Name"]) for r in attn}, key=KERNELS[MODE].index)
    per_kind = {k: [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in attn
                    if short_name(r["Kernel_Name"]) == k] for k in kinds}
    # timed launches: the last --steps of each kernel; a step's time is their sum
    timed_k = {k: v[-args.steps:] for k, v in per_kind.items()}
    timed = [sum(x) for x in zip(*timed_k.values())]
    durs = [d for v in per_kind.values() for d in v]
    bench = None
    if args.bench_json and os.path.exists(args.bench_json):
        with open(args.bench_json) as f:
            for line in f:
                if line.startswith("{"):
                    bench = json.loads(line)
    r0 = attn[0] if attn else {}
    lines = [f"# rocprofv3 kernel trace: {' + '.join(kinds)}, workload {args.workload}", "",
             "Command (run from the repository root on one MI355X):", "",
             "```", args.trace_cmd, "```", "",
             "## Kernel statistics (all dispatches, as rocprofv3 --stats prints them)", "",
             "| kernel | calls | total ms | average us | min us | max us |",
             "|---|---|---|---|---|---|"]
    for s in stats:
        lines.append(f"| {short_name(s['Name'])} | {s['Calls']} | "
                     f"{int(s['TotalDurationNs']) / 1e6:.3f} | {float(s['AverageNs']) / 1e3:.1f} | "
                     f"{int(s['MinNs']) / 1e3:.1f} | {int(s['MaxNs']) / 1e3:.1f} |")
    lines += ["", "## Kernels of the pass", ""]
    for k in kinds:
        rk = next(r for r in attn if short_name(r["Kernel_Name"]) == k)
        tk = timed_k[k]
        lines += [f"- {k}: grid {rk.get('Grid_Size_X')}x{rk.get('Grid_Size_Y')} work-items, "
                  f"workgroup {rk.get('Workgroup_Size_X')}, LDS {rk.get('LDS_Block_Size')} B, "
                  f"scratch {rk.get('Scratch_Size')} B, arch VGPR {rk.get('VGPR_Count')}, "
                  f"AGPR {rk.get('Accum_VGPR_Count')}, SGPR {rk.get('SGPR_Count')}; "
                  f"{len(per_kind[k])} dispatches; mean over the {len(tk)} timed ones "
                  f"{statistics.mean(tk):.1f} us (median {statistics.median(tk):.1f}, "
                  f"min {min(tk):.1f}, max {max(tk):.1f})"]
    lines += [f"- one step (one launch of each): mean {statistics.mean(timed):.1f} us over "
              f"{len(timed)} timed steps (median {statistics.median(timed):.1f})"]
    if bench:
        rf = bench["roofline"]
        lines += [f"- the same run's bench line: kernel_ms {rf['kernel_ms']} (HIP events around "
                  f"each launch), value {bench['value']} {bench['unit']}, roofline achieved "
                  f"{rf['achieved']} of {rf['peak']} {rf['unit']} (frac {rf['frac']})",
                  f"- trace mean / event mean = "
                  f"{statistics.mean(timed) / (rf['kernel_ms'] * 1e3):.3f}"]
    return "\n".join(lines) + "\n"


def counter_values(d, name):
    """Per kernel of the pass: its readings of counter `name` (one per
    dispatch); and the calibration copies' readings."""
    rows = read_csv(os.path.join(d, "run_counter_collection.csv"))
    attn = {}
    for r in rows:
        if is_attn(r["Kernel_Name"]) and r["Counter_Name"] == name:
            attn.setdefault(short_name(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
    copy = [float(r["Counter_Value"]) for r in rows
            if "copyBuffer" in r["Kernel_Name"] and r["Counter_Name"] == name]
    return attn, copy


def counters_summary(args) -> str:
    rows = read_csv(os.path.join(args.counters, "run_counter_collection.csv"))
    dominant = KERNELS[MODE][1] if MODE == "bwd" else None  # dkdv: the slowest kernel
    by = {}
    for r in rows:
        if not is_attn(r["Kernel_Name"]):
            continue
        if dominant and short_name(r["Kernel_Name"]) != dominant:
            continue
        if MODE == "decode" and short_name(r["Kernel_Name"]) != "decode_kernel":
            continue
        d = by.setdefault(int(r["Dispatch_Id"]), {"kname": r["Kernel_Name"], "grid": int(r["Grid_Size"]),
                                                  "wg": int(r["Workgroup_Size"]),
                                                  "ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
        d[r["Counter_Name"]] = float(r["Counter_Value"])
    ds = list(by.values())
    mean = lambda k: statistics.mean(d[k] for d in ds)
    n_simd, n_xcd = 1024, 8
    gui = mean("GRBM_GUI_ACTIVE") / n_xcd  # the counter sums the XCDs
    busy = mean("SQ_VALU_MFMA_BUSY_CYCLES") / (n_simd * gui)
    waves = ds[0]["grid"] / 64
    conf = mean("SQ_LDS_BANK_CONFLICT") / mean("SQ_LDS_IDX_ACTIVE")
    ns = statistics.mean(d["ns"] for d in ds)
    lines = [f"# Counters: {short_name(ds[0]['kname'])}, workload {args.workload}", "",
             "Command (run from the repository root on one MI355X):", "", "```", args.counters_cmd, "```", "",
             f"- dispatches: {len(ds)}, mean duration {ns / 1e3:.1f} us, GPU-active {gui:.4g} cycles per XCD"
             + (f" (shader clock {gui / ns:.2f} GHz)" if ns > 1e5 else
                " (too short for a clock estimate: the GPU-active window is mostly launch)"),
             f"- MFMA busy: {100 * busy:.1f}% (SQ_VALU_MFMA_BUSY_CYCLES {mean('SQ_VALU_MFMA_BUSY_CYCLES'):.4g} "
             f"over {n_simd} SIMDs x {gui:.4g} cycles)",
             f"- LDS bank conflicts: {100 * conf:.2f}% of LDS-active cycles (SQ_LDS_BANK_CONFLICT "
             f"{mean('SQ_LDS_BANK_CONFLICT'):.4g}, SQ_LDS_IDX_ACTIVE {mean('SQ_LDS_IDX_ACTIVE'):.4g})",
             f"- per wave ({waves:.0f} waves): MFMA {mean('SQ_INSTS_MFMA') / waves:.0f}, VALU "
             f"{mean('SQ_INSTS_VALU') / waves:.0f}, LDS {mean('SQ_INSTS_LDS') / waves:.0f} instructions"]
    return "\n".join(lines) + "\n"


def traffic_summary(args):
    from bench import algorithmic_bytes, kernel_source_hash
    import workloads
    fak, fc = counter_values(args.fetch, "FETCH_SIZE")
    wak, wc = counter_values(args.write, "WRITE_SIZE")
    kname = " + ".join(sorted(fak, key=KERNELS[MODE].index))
    # a step's readings: the sum over the pass's kernels of their mean per dispatch
    fa = [sum(statistics.mean(v) for v in fak.values())]
    wa = [sum(statistics.mean(v) for v in wak.values())]
    # a step's duration: the sum over the pass's kernels of their mean dispatch
    # (one row per counter and dispatch; duplicates do not move the means)
    by_kind = {}
    for d in (args.fetch, args.write):
        for r in read_csv(os.path.join(d, "run_counter_collection.csv")):
            if is_attn(r["Kernel_Name"]):
                by_kind.setdefault(short_name(r["Kernel_Name"]), []).append(
                    int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    dur_ns = sum(statistics.mean(v) for v in by_kind.values())
    kib = args.copy_mib * 1024.0
    # the calibration copies are the big ones (the library's own small copies read ~KiB)
    fcal = max(fc)
    wcal = max(wc)
    ff = kib / fcal
    fw = kib / wcal
    fetch_b = statistics.mean(fa) * ff * 1024
    write_b = statistics.mean(wa) * fw * 1024
    w = workloads.ALL[args.workload]
    alg = algorithmic_bytes(w, 2 if w.dtype != "f32" else 4)
    if MODE == "bwd":  # the backward reads q, k, v, out, dout, lse and writes dq, dk, dv (+ delta)
        e = 2
        alg = float(w.total_q * w.hq * (w.d_qk + 2 * w.d_v) * e + w.total_q * w.hq * 4 * 2
                    + w.total_kv * w.hkv * (w.d_qk + w.d_v) * e * 2 + w.total_q * w.hq * w.d_qk * e)
    lines = [f"# HBM traffic: {short_name(kname)}, workload {args.workload}", "",
             "Commands (one PMC pass each, run from the repository root on one MI355X):", "",
             "```", args.pmc_cmd.replace("{COUNTER}", "FETCH_SIZE").replace("{DIR}", "prof_fetch"),
             args.pmc_cmd.replace("{COUNTER}", "WRITE_SIZE").replace("{DIR}", "prof_write"), "```", "",
             f"Calibration: bench.py --copy-calibration-mib {args.copy_mib} copies {args.copy_mib} MiB "
             f"device to device (reads and writes {kib:.0f} KiB each).", "",
             "| counter | copy reading (KiB) | factor | attention readings (KiB/dispatch) | "
             "attention bytes/launch |", "|---|---|---|---|---|",
             f"| FETCH_SIZE | {fcal:.1f} | {ff:.3f} | {', '.join(f'{x:.0f}' for x in fa)} | "
             f"{fetch_b:.4g} |",
             f"| WRITE_SIZE | {wcal:.1f} | {fw:.3f} | {', '.join(f'{x:.0f}' for x in wa)} | "
             f"{write_b:.4g} |", "",
             f"- HBM bytes per launch (fetch + write, calibrated): {fetch_b + write_b:.4g}",
             f"- algorithmic bytes per launch (q, k, v, out, lse once): {alg:.4g}",
             f"- ratio: {(fetch_b + write_b) / alg:.2f}",
             f"- HBM rate in these runs: {(fetch_b + write_b) / dur_ns:.1f} GB/s over a mean step of "
             f"{dur_ns / 1e3:.1f} us ({100 * (fetch_b + write_b) / dur_ns / 8000:.1f}% of 8 TB/s)",
             f"- kernel source sha256[:16]: {kernel_source_hash(MODE)}"]
    data = {"workload": args.workload, "kernel": kname, "pass": MODE,
            "kernel_source_sha256_16": kernel_source_hash(MODE),
            "hbm_bytes_per_launch": fetch_b + write_b,
            "fetch_bytes_per_launch": fetch_b, "write_bytes_per_launch": write_b,
            "fetch_factor": ff, "write_factor": fw, "algorithmic_bytes": alg,
            "pmc_mean_dispatch_ns": dur_ns}
    return "\n".join(lines) + "\n", data


def main():
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--workload", required=True)
    ap.add_argument("--out-dir", default=os.path.join(ROOT, "profiles"))
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--trace")
    ap.add_argument("--trace-cmd", default="")
    ap.add_argument("--bench-json")
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--pmc-cmd", default="")
    ap.add_argument("--copy-mib", type=int, default=1024)
    ap.add_argument("--counters")
    ap.add_argument("--counters-cmd", default="")
    ap.add_argument("--mode", default="fwd", choices=sorted(KERNELS),
                    help="which pass's kernels the runs time: forward, backward or decode")
    args = ap.parse_args()
    global MODE
    MODE = args.mode
    tag = args.workload if MODE == "fwd" else f"{args.workload}_{MODE}"
    os.makedirs(args.out_dir, exist_ok=True)
    first = {"fwd": None, "bwd": "attn_bwd", "decode": "attn_decode"}[MODE]
    if args.trace:
        txt = trace_summary(args)
        kname = first or ("attn_fwd16p_kernel" if "attn_fwd16p" in txt else "attn_fwd_kernel")
        p = os.path.join(args.out_dir, f"{kname}_{tag}_trace.md")
        with open(p, "w") as f:
            f.write(txt)
        print("wrote", p)
    if args.counters:
        txt = counters_summary(args)
        kname = first or ("attn_fwd16p_kernel" if "attn_fwd16p" in txt else "attn_fwd_kernel")
        p = os.path.join(args.out_dir, f"{kname}_{tag}_counters.md")
        with open(p, "w") as f:
            f.write(txt)
        print("wrote", p)
    if args.fetch and args.write:
        txt, data = traffic_summary(args)
        kname = first or data["kernel"]
        p = os.path.join(args.out_dir, f"{kname}_{tag}_hbm.md")
        with open(p, "w") as f:
            f.write(txt)
        pj = os.path.join(args.out_dir, f"traffic_attn_{MODE}_{args.workload}.json")
        with open(pj, "w") as f:
            json.dump(data, f, indent=1)
        print("wrote", p, pj)


if __name__ == "__main__":
    main()
