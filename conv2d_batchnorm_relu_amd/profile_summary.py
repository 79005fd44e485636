"""Per-kernel counter summary of rocprofv3 passes over the benchmark's workloads.

Input: a directory tree <root>/<workload>/<pass>/..._counter_collection.csv, one rocprofv3
--pmc run per (workload, pass) of ``python3 -m conv2d_batchnorm_relu_amd.profile_run``.
The passes (each within one run's hardware counter limits):

    sq     MfmaUtil SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_MFMA SQ_INSTS_VALU_MFMA_MOPS_BF16
           SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_WAVES GRBM_GUI_ACTIVE
    fetch  FETCH_SIZE
    write  WRITE_SIZE

and the workload ``copy`` (a 512 MiB device copy) with the fetch and write passes, whose
known bytes calibrate the two HBM byte counters:

    python -m conv2d_batchnorm_relu_amd.profile_summary --root <root> \\
        --md profiles/counters_bench_workloads.md --json profiles/counters_bench_workloads.json

For every workload and kernel (grouped by kernel name and grid size) it reports the
dispatches, the mean per dispatch of: MFMA utilisation (rocprofv3's MfmaUtil, the MFMA
busy cycles over GPU-active cycles times SIMDs), MFMA instructions, bf16 MFMA flops
(SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512), the LDS bank-conflict share of LDS-active cycles,
and HBM bytes read and written (FETCH_SIZE and WRITE_SIZE scaled by the copy's factors).
The json carries the sha256 of the library's sources, so a reader can tell whether the
figures still describe the kernels in the tree.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import statistics
from collections import defaultdict

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "conv2d_batchnorm_relu_amd", "csrc")
COPY_BYTES = 512 << 20


def sources_sha256() -> str:
    """sha256 over the library's kernel and host sources (sorted by name)."""
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        if f.endswith((".hip", ".cpp", ".h", ".inc")):
            h.update(f.encode())
            with open(os.path.join(CSRC, f), "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()


def short_name(name: str) -> str:
    """Kernel name without return type, namespaces and parameter list; template
    arguments kept (they tell the kernel's variants apart)."""
    n = name.strip()
    if n.startswith("void "):
        n = n[5:]
    depth, cut = 0, len(n)
    for i, ch in enumerate(n):   # the parameter list: the first '(' outside template brackets
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0 and not n.startswith("(anonymous", i):
            cut = i
            break
    n = n[:cut]
    n = re.sub(r"\(anonymous namespace\)::", "", n)
    n = re.sub(r"\bcbr::", "", n)
    return n


def read_pass(d):
    """{(kernel, grid, wg): {counter: [values per dispatch]}, '_dur': [...]} of one pass."""
    out = defaultdict(lambda: defaultdict(list))
    seen = set()
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f, newline="") as fh:
            for r in csv.DictReader(fh):
                key = (short_name(r["Kernel_Name"]), int(r["Grid_Size"]), int(r["Workgroup_Size"]))
                out[key][r["Counter_Name"]].append(float(r["Counter_Value"]))
                did = (f, r["Dispatch_Id"])
                if did not in seen:
                    seen.add(did)
                    out[key]["_dur_ns"].append(float(r["End_Timestamp"]) - float(r["Start_Timestamp"]))
    return out


def calibration(root):
    """Bytes per counted KiB for FETCH_SIZE and WRITE_SIZE, from the copy workload: the
    dispatches with the largest counts are the 512 MiB copies."""
    fac = {}
    for pas, counter in (("fetch", "FETCH_SIZE"), ("write", "WRITE_SIZE")):
        data = read_pass(os.path.join(root, "copy", pas))
        best = max((v for k in data for v in data[k].get(counter, [])), default=0.0)
        fac[counter] = COPY_BYTES / best if best > 0 else None
        fac[counter + "_kib"] = best
    return fac


def summarize(root):
    cal = calibration(root)
    result = {"sources_sha256": sources_sha256(), "copy_bytes": COPY_BYTES,
              "fetch_bytes_per_kib": cal["FETCH_SIZE"], "write_bytes_per_kib": cal["WRITE_SIZE"],
              "copy_fetch_kib": cal["FETCH_SIZE_kib"], "copy_write_kib": cal["WRITE_SIZE_kib"], "workloads": {}}
    for wdir in sorted(glob.glob(os.path.join(root, "*"))):
        wname = os.path.basename(wdir)
        if wname == "copy" or not os.path.isdir(wdir):
            continue
        passes = {p: read_pass(os.path.join(wdir, p)) for p in ("sq", "fetch", "write")}
        keys = sorted(set().union(*[set(v) for v in passes.values()]), key=lambda k: (k[0], k[1]))
        rows = []
        for key in keys:
            def mean(p, c):
                v = passes[p].get(key, {}).get(c, [])
                return statistics.fmean(v) if v else None
            sq = passes["sq"].get(key, {})
            fetch_kib, write_kib = mean("fetch", "FETCH_SIZE"), mean("write", "WRITE_SIZE")
            lds_act, lds_conf = mean("sq", "SQ_LDS_IDX_ACTIVE"), mean("sq", "SQ_LDS_BANK_CONFLICT")
            durs = [d for p in passes.values() for d in p.get(key, {}).get("_dur_ns", [])]
            mops = mean("sq", "SQ_INSTS_VALU_MFMA_MOPS_BF16")
            rows.append({
                "kernel": key[0], "grid": key[1], "workgroup": key[2],
                "dispatches": len(sq.get("_dur_ns", [])) or len(passes["fetch"].get(key, {}).get("_dur_ns", [])),
                "duration_us_median": round(statistics.median(durs) / 1e3, 2) if durs else None,
                "mfma_util_pct": None if mean("sq", "MfmaUtil") is None else round(mean("sq", "MfmaUtil"), 2),
                "mfma_busy_cycles": mean("sq", "SQ_VALU_MFMA_BUSY_CYCLES"),
                "mfma_insts": mean("sq", "SQ_INSTS_MFMA"),
                "mfma_bf16_flops": None if mops is None else mops * 512,
                "lds_bank_conflict_pct_of_lds_active": (None if not lds_act or lds_conf is None
                                                         else round(100 * lds_conf / lds_act, 2)),
                "waves": mean("sq", "SQ_WAVES"),
                "fetch_kib": fetch_kib, "write_kib": write_kib,
                "fetch_bytes": None if fetch_kib is None or cal["FETCH_SIZE"] is None else int(fetch_kib * cal["FETCH_SIZE"]),
                "write_bytes": None if write_kib is None or cal["WRITE_SIZE"] is None else int(write_kib * cal["WRITE_SIZE"]),
            })
        result["workloads"][wname] = rows
    return result


def fmt(v, scale=1.0, nd=1):
    return "-" if v is None else f"{v / scale:,.{nd}f}"


def write_md(res, path, command):
    lines = ["# Per-kernel counters of the benchmark workloads (rocprofv3)", "",
             "Made by `python -m conv2d_batchnorm_relu_amd.profile_summary` from one rocprofv3 --pmc run per",
             "(workload, pass) of `python3 -m conv2d_batchnorm_relu_amd.profile_run --workload <w> --reps 5`:", "",
             "```", command.strip(), "```", "",
             f"Library sources sha256: `{res['sources_sha256']}`.", "",
             "HBM bytes: FETCH_SIZE and WRITE_SIZE (KiB, summed over the chip) times the factors of a "
             f"{res['copy_bytes'] >> 20} MiB device copy: {fmt(res['fetch_bytes_per_kib'], 1, 2)} B per fetched KiB "
             f"(copy counted {fmt(res['copy_fetch_kib'], 1, 0)} KiB), {fmt(res['write_bytes_per_kib'], 1, 2)} B per "
             f"written KiB (counted {fmt(res['copy_write_kib'], 1, 0)} KiB).", "",
             "MFMA util: rocprofv3's MfmaUtil (MFMA-busy SIMD cycles over GPU-active cycles x SIMDs). "
             "MFMA GFLOP: SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512. LDS conflict: SQ_LDS_BANK_CONFLICT over "
             "SQ_LDS_IDX_ACTIVE. Durations: median dispatch time under counter collection (serialised).", ""]
    for wname, rows in res["workloads"].items():
        lines += [f"## {wname}", "",
                  "| kernel | grid | disp. | us | MFMA util % | MFMA insts | MFMA GFLOP | LDS conflict % | read MB | written MB |",
                  "|---|---|---|---|---|---|---|---|---|---|"]
        for r in rows:
            lines.append(f"| `{r['kernel'][:90]}` | {r['grid']} | {r['dispatches']} | {fmt(r['duration_us_median'], 1, 1)} | "
                         f"{fmt(r['mfma_util_pct'], 1, 1)} | {fmt(r['mfma_insts'], 1, 0)} | "
                         f"{fmt(r['mfma_bf16_flops'], 1e9, 2)} | {fmt(r['lds_bank_conflict_pct_of_lds_active'], 1, 1)} | "
                         f"{fmt(r['fetch_bytes'], 1e6, 1)} | {fmt(r['write_bytes'], 1e6, 1)} |")
        lines.append("")
    with open(path, "w") as f:
        f.write("\n".join(lines))


def write_trace_md(stats_csv, path, command, note="", title="all bench workloads"):
    """Markdown table of a rocprofv3 --kernel-trace --stats kernel_stats.csv: calls and
    average / min / max duration per kernel, longest total first."""
    rows = []
    with open(stats_csv, newline="") as fh:
        for r in csv.DictReader(fh):
            rows.append((short_name(r["Name"]), int(r["Calls"]), float(r["TotalDurationNs"]), float(r["AverageNs"]),
                         float(r["MinNs"]), float(r["MaxNs"])))
    rows.sort(key=lambda r: -r[2])
    lines = [f"# Kernel durations, {title} (rocprofv3 --kernel-trace --stats)", "",
             "Command (`<repo>` is the repository root, `<out>` the output directory):", "", "```",
             command.strip(), "```", "", f"Library sources sha256: `{sources_sha256()}`.", ""]
    if note:
        lines += [note.strip(), ""]
    lines += ["| kernel | calls | avg us | min us | max us |", "|---|---|---|---|---|"]
    for name, calls, _, avg, mn, mx in rows:
        lines.append(f"| `{name[:90]}` | {calls} | {avg / 1e3:.1f} | {mn / 1e3:.1f} | {mx / 1e3:.1f} |")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--root", help="counter passes: <root>/<workload>/<pass>/*counter_collection.csv")
    ap.add_argument("--md", required=True)
    ap.add_argument("--json")
    ap.add_argument("--trace-stats", help="instead: summarise this kernel_stats.csv of a kernel-trace run")
    ap.add_argument("--note", default="", help="a paragraph added under the command (trace summaries)")
    ap.add_argument("--command", default="", help="the profiling command line(s), quoted in the summary")
    ap.add_argument("--title", default="all bench workloads", help="what the traced run covered (trace summaries)")
    args = ap.parse_args(argv)
    if args.trace_stats:
        write_trace_md(args.trace_stats, args.md, args.command, args.note, args.title)
        print(f"wrote {args.md}")
        return
    res = summarize(args.root)
    with open(args.json, "w") as f:
        json.dump(res, f, indent=1)
    write_md(res, args.md, args.command)
    print(f"wrote {args.md} and {args.json} ({len(res['workloads'])} workloads)")


if __name__ == "__main__":
    main()
