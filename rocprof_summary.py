#!/usr/bin/env python3
"""Summarise rocprofv3 output of bench.py runs into profiles/.

Inputs (rocprofv3 CSV output directories):
  --trace DIR   from  rocprofv3 --kernel-trace --stats --output-format csv -d DIR -o bench -- python3 bench.py ...
  --fetch DIR   from  rocprofv3 --pmc FETCH_SIZE --output-format csv -d DIR -o bench -- python3 bench.py ... --calibrate-copy MIB
  --write DIR   from  rocprofv3 --pmc WRITE_SIZE --output-format csv -d DIR -o bench -- python3 bench.py ... --calibrate-copy MIB

Outputs:
  profiles/<prefix>_kernel_trace.md          per-kernel calls / average / min / max duration
  profiles/<kernel>_<workload>_traffic.json  HBM-side bytes per launch of each library kernel

FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are scaled by what they read for
the calibration copy (one plain device-to-device copy of MIB MiB, which reads
and writes exactly MIB MiB): scale = true bytes / counted bytes.
"""

import argparse
import collections
import csv
import json
import os
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)


def short_name(full: str) -> str:
    """'void sv::chain_rowstats_kernel<1, true, 8>(...)' -> 'chain_rowstats'."""
    n = full.replace("(anonymous namespace)::", "").split("(")[0].split("<")[0].split("::")[-1]
    return n[:-len("_kernel")] if n.endswith("_kernel") else n


def read_counters(d: str) -> dict:
    path = os.path.join(d, "bench_counter_collection.csv")
    per = collections.defaultdict(list)
    for r in csv.DictReader(open(path)):
        per[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return per


def calibration_scale(per: dict, mib: int) -> float:
    """True bytes over counted bytes for the largest plain-copy dispatch."""
    counted = max(max(v) for k, v in per.items() if "copyBuffer" in k or "direct_copy" in k) * 1024.0
    return mib * 2 ** 20 / counted


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--trace", required=True)
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--calibrate-mib", type=int, default=256)
    ap.add_argument("--workload", default="llama_chain")
    ap.add_argument("--prefix", default="llama_chain")
    ap.add_argument("--command", required=True, help="the bench command of the kernel-trace run")
    ap.add_argument("--pmc-command", help="the bench command of the counter runs (default: --command)")
    ap.add_argument("--out", default=os.path.join(ROOT, "profiles"))
    args = ap.parse_args()
    pmc_cmd = args.pmc_command or args.command
    os.makedirs(args.out, exist_ok=True)

    from bench import kernel_source_digest

    digest = kernel_source_digest()
    rows = list(csv.DictReader(open(os.path.join(args.trace, "bench_kernel_stats.csv"))))
    lines = [f"# rocprofv3 kernel trace: {args.prefix}", "",
             "Command (run from the repository root on one MI355X):", "",
             "```", f"rocprofv3 --kernel-trace --stats --output-format csv -d <dir> -o bench -- {args.command}", "```",
             "", f"Kernel sources digest: `{digest}`", "",
             "| kernel | calls | average (us) | min (us) | max (us) | share of GPU time |",
             "|---|---:|---:|---:|---:|---:|"]
    for r in rows:
        lines.append(f"| {short_name(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f}% |")
    with open(os.path.join(args.out, f"{args.prefix}_kernel_trace.md"), "w") as f:
        f.write("\n".join(lines) + "\n")

    if args.fetch and args.write:
        fetch, write = read_counters(args.fetch), read_counters(args.write)
        fs, wsc = calibration_scale(fetch, args.calibrate_mib), calibration_scale(write, args.calibrate_mib)
        for full, vals in fetch.items():
            if "sv::" not in full:
                continue
            name = short_name(full)
            fb = sum(vals) / len(vals) * 1024.0 * fs
            wv = write.get(full, [0.0])
            wb = sum(wv) / len(wv) * 1024.0 * wsc
            rec = {
                "kernel": name, "workload": args.workload, "kernel_source_digest": digest,
                "traffic_bytes_per_launch": fb + wb, "fetch_bytes_per_launch": fb, "write_bytes_per_launch": wb,
                "fetch_scale": fs, "write_scale": wsc, "launches_counted": len(vals),
                "calibration": f"one plain device copy of {args.calibrate_mib} MiB",
                "commands": [f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir> -o bench -- {pmc_cmd} "
                             f"--calibrate-copy {args.calibrate_mib}",
                             f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir> -o bench -- {pmc_cmd} "
                             f"--calibrate-copy {args.calibrate_mib}"],
            }
            with open(os.path.join(args.out, f"{name}_{args.workload}_traffic.json"), "w") as f:
                json.dump(rec, f, indent=1)
            print(f"{name}: fetch {fb / 1e6:.2f} MB + write {wb / 1e6:.3f} MB per launch")
    print("\n".join(lines))


if __name__ == "__main__":
    main()
