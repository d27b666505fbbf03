#!/usr/bin/env python3
"""Summarise rocprofv3 output of bench.py runs into profiles/.

Inputs (rocprofv3 CSV output directories):
  --trace DIR   from  rocprofv3 --kernel-trace --stats --output-format csv -d DIR -o bench -- python3 bench.py ...
  --fetch DIR   from  rocprofv3 --pmc FETCH_SIZE --output-format csv -d DIR -o bench -- python3 bench.py ... --calibrate-copy MIB
  --write DIR   from  rocprofv3 --pmc WRITE_SIZE --output-format csv -d DIR -o bench -- python3 bench.py ... --calibrate-copy MIB
  --sq DIR      from  rocprofv3 --pmc <SQ_COUNTERS> --output-format csv -d DIR -o bench -- python3 bench.py ...
  --lat DIR     from  rocprofv3 --pmc <LAT_COUNTERS> --output-format csv -d DIR -o bench -- python3 bench.py ...
  --mem D1,D2,D3  from three runs, rocprofv3 --pmc <MEM_PASSES[i]> --output-format csv -d Di -o bench -- python3 bench.py ...

Outputs:
  profiles/<prefix>_kernel_trace.md          per-kernel calls / average / min / max duration
  profiles/<kernel>_<workload>_traffic.json  HBM-side bytes per launch of each library kernel
  profiles/<prefix>_sq_counters.md           per-kernel SQ counters and the VALU floor
  profiles/<prefix>_latency_counters.md      per-kernel L2 read latency and waiting
  profiles/<prefix>_memory_counters.md       per-kernel L2-to-memory latency, DRAM credit stalls, TLB misses

FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are scaled by what they read for
the calibration copy (one plain device-to-device copy of MIB MiB, which reads
and writes exactly MIB MiB): scale = true bytes / counted bytes.
"""

import argparse
import collections
import csv
import json
import os
import statistics
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)


def short_name(full: str) -> str:
    """'void sv::chain_rowstats_kernel<1, true, 8>(...)' -> 'chain_rowstats'."""
    n = full.replace("(anonymous namespace)::", "").split("(")[0].split("<")[0].split("::")[-1]
    return n[:-len("_kernel")] if n.endswith("_kernel") else n


def trace_durations(d: str) -> dict:
    """Per-dispatch durations (us, in dispatch order) per kernel from the kernel trace, if present."""
    path = os.path.join(d, "bench_kernel_trace.csv")
    if not os.path.exists(path):
        return {}
    per = collections.defaultdict(list)
    for r in sorted(csv.DictReader(open(path)), key=lambda r: int(r["Start_Timestamp"])):
        per[r["Kernel_Name"]].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    return per


def event_region_average(durs: list, steps: int, warmup: int):
    """bench.py runs warmup steps, three timed regions of `steps` steps and
    last the region with an event pair attached to each dispatch: the
    average over that last region's dispatches (a kernel launched n times
    per step has n * steps of them)."""
    total = warmup + 4 * steps
    if not durs or len(durs) % total:
        return None
    n = len(durs) // total * steps
    return sum(durs[-n:]) / n


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


CUS, SIMDS_PER_CU, CLOCK_HZ = 256, 4, 2.4e9
SQ_COUNTERS = ("SQ_WAVES SQ_BUSY_CYCLES SQ_WAVE_CYCLES SQ_INSTS_VALU SQ_ACTIVE_INST_VALU SQ_WAIT_INST_ANY "
               "SQ_INSTS_VMEM_RD SQ_INSTS_SALU GRBM_GUI_ACTIVE")


def sq_summary(d: str, prefix: str, command: str) -> str:
    """Per-kernel SQ counters (averages per dispatch) and what follows from
    them without assuming counter units: instructions per wave, the fraction
    of wave-cycles spent waiting for an instruction's operands, and the VALU
    floor, the time the SIMDs need just to issue the kernel's VALU
    instructions (a wave64 instruction occupies a 16-lane SIMD for 4 cycles;
    1024 SIMDs at 2.4 GHz)."""
    per = collections.defaultdict(lambda: collections.defaultdict(list))
    for r in csv.DictReader(open(os.path.join(d, "bench_counter_collection.csv"))):
        per[r["Kernel_Name"]][r["Counter_Name"]].append(float(r["Counter_Value"]))
    lines = [f"# rocprofv3 SQ counters: {prefix}", "", "Command (run from the repository root on one MI355X):", "",
             "```", f"rocprofv3 --pmc {SQ_COUNTERS} --output-format csv -d <dir> -o bench -- {command}", "```", "",
             "Averages per dispatch. VALU floor = SQ_INSTS_VALU x 4 cycles / (1024 SIMDs x 2.4 GHz): the time the "
             "chip needs only to issue the kernel's vector instructions (packed fp32 is not used). Wait fraction = "
             "SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES.", "",
             "| kernel | dispatches | waves | VALU / wave | SALU / wave | VMEM reads / wave | VALU floor (us) | "
             "wait fraction |", "|---|---:|---:|---:|---:|---:|---:|---:|"]
    for full, c in per.items():
        if "sv::" not in full:
            continue
        a = {k: sum(v) / len(v) for k, v in c.items()}
        waves = a.get("SQ_WAVES", 0.0)
        if not waves:
            continue
        floor = a["SQ_INSTS_VALU"] * 4 / (CUS * SIMDS_PER_CU * CLOCK_HZ) * 1e6
        lines.append(f"| {short_name(full)} | {len(c['SQ_WAVES'])} | {waves:.0f} | {a['SQ_INSTS_VALU'] / waves:.0f} | "
                     f"{a['SQ_INSTS_SALU'] / waves:.0f} | {a['SQ_INSTS_VMEM_RD'] / waves:.1f} | {floor:.2f} | "
                     f"{a['SQ_WAIT_INST_ANY'] / a['SQ_WAVE_CYCLES']:.2f} |")
    return "\n".join(lines) + "\n"


LAT_COUNTERS = ("SQ_WAVES SQ_WAVE_CYCLES SQ_WAIT_ANY SQ_INST_LEVEL_VMEM SQ_ACTIVE_INST_ANY SQ_LEVEL_WAVES "
                "SQ_BUSY_CU_CYCLES SQ_INSTS_VALU_TRANS_F32 TCP_TCC_READ_REQ_LATENCY_sum TCP_TCC_READ_REQ_sum")


def latency_summary(d: str, prefix: str, command: str) -> str:
    """Per-kernel memory latency and waiting (averages per dispatch): the mean
    latency of an L1-to-L2 read request in cycles (TCP_TCC_READ_REQ_LATENCY
    over TCP_TCC_READ_REQ, the L2's misses to HBM included), the fraction of
    wave-cycles spent waiting for anything (SQ_WAIT_ANY over SQ_WAVE_CYCLES:
    memory counters, barriers, dependencies) and the transcendental
    instructions per wave."""
    per = collections.defaultdict(lambda: collections.defaultdict(list))
    for r in csv.DictReader(open(os.path.join(d, "bench_counter_collection.csv"))):
        per[r["Kernel_Name"]][r["Counter_Name"]].append(float(r["Counter_Value"]))
    lines = [f"# rocprofv3 latency counters: {prefix}", "", "Command (run from the repository root on one MI355X):", "",
             "```", f"rocprofv3 --pmc {LAT_COUNTERS} --output-format csv -d <dir> -o bench -- {command}", "```", "",
             "Averages per dispatch. L2 read latency = TCP_TCC_READ_REQ_LATENCY_sum / TCP_TCC_READ_REQ_sum (cycles "
             "from an L1 request to its data, L2 misses included); wait fraction = SQ_WAIT_ANY / SQ_WAVE_CYCLES.", "",
             "| kernel | waves | L2 read requests | L2 read latency (cycles) | wait fraction | transcendentals / wave |",
             "|---|---:|---:|---:|---:|---:|"]
    for full, c in per.items():
        if "sv::" not in full:
            continue
        a = {k: sum(v) / len(v) for k, v in c.items()}
        waves = a.get("SQ_WAVES", 0.0)
        if not waves:
            continue
        req = a["TCP_TCC_READ_REQ_sum"]
        lat = a["TCP_TCC_READ_REQ_LATENCY_sum"] / req if req else float("nan")
        lines.append(f"| {short_name(full)} | {waves:.0f} | {req:.0f} | {lat:.0f} | "
                     f"{a['SQ_WAIT_ANY'] / a['SQ_WAVE_CYCLES']:.2f} | {a['SQ_INSTS_VALU_TRANS_F32'] / waves:.0f} |")
    return "\n".join(lines) + "\n"


# One counter pass each (the TCC block collects at most four counters per pass).
MEM_PASSES = ("TCC_EA0_RDREQ_sum TCC_EA0_RDREQ_LEVEL_sum TCC_HIT_sum TCC_MISS_sum",
              "TCC_EA0_RDREQ_DRAM_sum TCC_EA0_RDREQ_DRAM_CREDIT_STALL_sum",
              "TCP_UTCL1_TRANSLATION_MISS_sum TCP_UTCL1_TRANSLATION_HIT_sum TCP_PENDING_STALL_CYCLES_sum "
              "TA_BUSY_avr TA_ADDR_STALLED_BY_TC_CYCLES_sum")


def memory_summary(dirs: list, prefix: str, command: str) -> str:
    """Per-kernel memory-side counters (averages per dispatch, three passes):
    the L2's read requests to memory and its hit rate, the mean time a read
    request to memory stays in flight (TCC_EA0_RDREQ_LEVEL over
    TCC_EA0_RDREQ, in L2 cycles, by Little's law), the cycles the L2 waited
    for DRAM credits per request to DRAM (the memory controllers' queues
    full), and the address-translation miss rate of the vector L1."""
    per = collections.defaultdict(lambda: collections.defaultdict(list))
    for d in dirs:
        for r in csv.DictReader(open(os.path.join(d, "bench_counter_collection.csv"))):
            per[r["Kernel_Name"]][r["Counter_Name"]].append(float(r["Counter_Value"]))
    lines = [f"# rocprofv3 memory-side counters: {prefix}", "", "Commands (run from the repository root on one MI355X), "
             "one counter pass each:", "", "```"]
    lines += [f"rocprofv3 --pmc {p} --output-format csv -d <dir{i + 1}> -o bench -- {command}"
              for i, p in enumerate(MEM_PASSES)]
    lines += ["```", "", "Averages per dispatch. Memory latency = TCC_EA0_RDREQ_LEVEL_sum / TCC_EA0_RDREQ_sum (L2 "
              "cycles a read request to memory is in flight); DRAM credit stalls = TCC_EA0_RDREQ_DRAM_CREDIT_STALL_sum "
              "/ TCC_EA0_RDREQ_DRAM_sum (cycles the L2 waited for the memory controllers per request); TLB misses = "
              "TCP_UTCL1_TRANSLATION_MISS / (MISS + HIT).", "",
              "| kernel | L2 reads to memory | L2 hit rate | memory latency (L2 cycles) | DRAM credit stalls per request "
              "| TLB miss rate |", "|---|---:|---:|---:|---:|---:|"]
    for full, c in per.items():
        if "sv::" not in full:
            continue
        a = {k: sum(v) / len(v) for k, v in c.items()}
        rq = a.get("TCC_EA0_RDREQ_sum", 0.0)
        dram = a.get("TCC_EA0_RDREQ_DRAM_sum", 0.0)
        if not rq or not dram:
            continue
        hits = a["TCC_HIT_sum"] / (a["TCC_HIT_sum"] + a["TCC_MISS_sum"])
        tlb = a["TCP_UTCL1_TRANSLATION_MISS_sum"] / (a["TCP_UTCL1_TRANSLATION_MISS_sum"] +
                                                      a["TCP_UTCL1_TRANSLATION_HIT_sum"])
        lines.append(f"| {short_name(full)} | {rq:.0f} | {hits:.3f} | {a['TCC_EA0_RDREQ_LEVEL_sum'] / rq:.0f} | "
                     f"{a['TCC_EA0_RDREQ_DRAM_CREDIT_STALL_sum'] / dram:.2f} | {tlb:.4f} |")
    return "\n".join(lines) + "\n"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--trace")
    ap.add_argument("--sq", help="rocprofv3 --pmc output of the SQ counters (SQ_COUNTERS)")
    ap.add_argument("--lat", help="rocprofv3 --pmc output of the latency counters (LAT_COUNTERS)")
    ap.add_argument("--mem", help="three comma-separated rocprofv3 --pmc outputs, one per MEM_PASSES entry")
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--calibrate-mib", type=int, default=256)
    ap.add_argument("--steps", type=int, default=200, help="--steps of the traced bench.py command")
    ap.add_argument("--warmup", type=int, default=20, help="--warmup of the traced bench.py command")
    ap.add_argument("--workload", default="llama_chain")
    ap.add_argument("--prefix", default="llama_chain")
    ap.add_argument("--command", required=True, help="the bench command of the kernel-trace run")
    ap.add_argument("--pmc-command", help="the bench command of the counter runs (default: --command)")
    ap.add_argument("--out", default=os.path.join(ROOT, "profiles"))
    args = ap.parse_args()
    pmc_cmd = args.pmc_command or args.command
    os.makedirs(args.out, exist_ok=True)
    if args.sq:
        text = sq_summary(args.sq, args.prefix, pmc_cmd)
        with open(os.path.join(args.out, f"{args.prefix}_sq_counters.md"), "w") as f:
            f.write(text)
        print(text)
    if args.lat:
        text = latency_summary(args.lat, args.prefix, pmc_cmd)
        with open(os.path.join(args.out, f"{args.prefix}_latency_counters.md"), "w") as f:
            f.write(text)
        print(text)
    if args.mem:
        text = memory_summary(args.mem.split(","), args.prefix, pmc_cmd)
        with open(os.path.join(args.out, f"{args.prefix}_memory_counters.md"), "w") as f:
            f.write(text)
        print(text)
    if not args.trace:
        return

    from bench import LIBRARY_KERNELS, kernel_source_digest, kernel_sources, trace_digest

    rows = list(csv.DictReader(open(os.path.join(args.trace, "bench_kernel_stats.csv"))))
    digest = trace_digest([short_name(r["Name"]) for r in rows if short_name(r["Name"]) in LIBRARY_KERNELS])
    lines = [f"# rocprofv3 kernel trace: {args.prefix}", "",
             "Command (run from the repository root on one MI355X):", "",
             "```", f"rocprofv3 --kernel-trace --stats --output-format csv -d <dir> -o bench -- {args.command}", "```",
             "", f"Kernel sources digest: `{digest}`", "",
             "The event-timed region is bench.py's last timed region, in which an event pair is attached to "
             "each dispatch (the durations bench.py reports); its kernels run apart, the other regions' back to "
             "back.", "",
             "| kernel | calls | average (us) | median (us) | min (us) | max (us) | share of GPU time | "
             "event-timed region average (us) |",
             "|---|---:|---:|---:|---:|---:|---:|---:|"]
    durs = trace_durations(args.trace)
    for r in rows:
        d = durs.get(r["Name"], [])
        med = statistics.median(d) if d else None
        ev = event_region_average(d, args.steps, args.warmup)
        lines.append(f"| {short_name(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{'%.2f' % med if med is not None else '-'} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f}% | "
                     f"{'%.2f' % ev if ev is not None else '-'} |")
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
                "kernel": name, "workload": args.workload, "kernel_source_digest": kernel_source_digest(name),
                "kernel_sources": kernel_sources(name),
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
