"""rocprof_summary.py and bench.py's use of its files (CPU only), on small
synthetic rocprofv3 CSV files."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import rocprof_summary as rs  # noqa: E402

KERNEL = "void sv::chain_rowstats_kernel<0, true, 8>(void const*, void const*, int)"
COPY = "__amd_rocclr_copyBuffer"


def _write_csv(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


@pytest.mark.parametrize("full, short", [
    (KERNEL, "chain_rowstats"),
    ("void sv::(anonymous namespace)::tree_round_kernel<1, false>(int)", "tree_round"),
    (COPY, COPY),
])
def test_short_name(full, short):
    assert rs.short_name(full) == short


def test_event_region_is_the_last_of_the_bench_regions():
    """20 warmup steps, three timed regions of 200 and the event-timed region
    last: a kernel launched twice per step has 400 dispatches there."""
    durs = [1.0] * (2 * 20 + 3 * 2 * 200) + [3.0] * (2 * 200)
    assert rs.event_region_average(durs, 200, 20) == pytest.approx(3.0)
    assert rs.event_region_average(durs[1:], 200, 20) is None  # not a whole number of steps
    assert rs.event_region_average([], 200, 20) is None


def test_summary_scales_counters_by_the_plain_copy(tmp_path):
    trace, fetch, write, out = (str(tmp_path / d) for d in ("trace", "fetch", "write", "out"))
    _write_csv(os.path.join(trace, "bench_kernel_stats.csv"),
               ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs"],
               [[KERNEL, 10, 214000, 21400, 60.0, 20000, 23000]])
    mib = 256
    # FETCH_SIZE counts half of a 256 MiB copy (scale 2); WRITE_SIZE all of it (scale 1); KiB per dispatch
    _write_csv(os.path.join(fetch, "bench_counter_collection.csv"), ["Kernel_Name", "Counter_Value"],
               [[COPY, mib * 1024 / 2], [KERNEL, 1000.0], [KERNEL, 3000.0]])
    _write_csv(os.path.join(write, "bench_counter_collection.csv"), ["Kernel_Name", "Counter_Value"],
               [[COPY, mib * 1024], [KERNEL, 10.0], [KERNEL, 30.0]])
    subprocess.check_call([sys.executable, os.path.join(ROOT, "rocprof_summary.py"), "--trace", trace,
                           "--fetch", fetch, "--write", write, "--workload", "w", "--prefix", "w",
                           "--command", "python3 bench.py", "--out", out], stdout=subprocess.DEVNULL)
    md = open(os.path.join(out, "w_kernel_trace.md")).read()
    assert "| chain_rowstats | 10 | 21.40 | - | 20.00 | 23.00 | 60.0% | - |" in md
    assert f"Kernel sources digest: `{bench.trace_digest(['chain_rowstats'])}`" in md
    rec = json.load(open(os.path.join(out, "chain_rowstats_w_traffic.json")))
    assert rec["fetch_scale"] == pytest.approx(2.0) and rec["write_scale"] == pytest.approx(1.0)
    assert rec["fetch_bytes_per_launch"] == pytest.approx(2000.0 * 1024 * 2)
    assert rec["write_bytes_per_launch"] == pytest.approx(20.0 * 1024)
    assert rec["traffic_bytes_per_launch"] == pytest.approx(2000.0 * 2048 + 20.0 * 1024)
    assert rec["kernel_source_digest"] == bench.kernel_source_digest("chain_rowstats")
    assert rec["kernel_sources"] == bench.kernel_sources("chain_rowstats")


def test_kernel_digests_follow_each_family_sources():
    """A kernel's counters stay valid while the sources it is built from do
    not change: every family's files include the public header, the common
    header and the host dispatch, and no family reads another's header."""
    csrc = "draft_token_verification_chain_amd/csrc/"
    for k in ("chain_rowstats", "chain_final_part", "chain_row_draw", "greedy_rows", "argmax_rows", "tree_plan",
              "tree_rowstats", "tree_round", "tree_sample", "commit_tokens"):
        srcs = bench.kernel_sources(k)
        assert {"include/specverify.h", csrc + "sv_common.hpp", csrc + "specverify.hip"} <= set(srcs), k
        assert all(os.path.exists(os.path.join(ROOT, p)) for p in srcs)
    assert csrc + "sv_tree_sampled.hpp" not in bench.kernel_sources("chain_final_part")
    assert csrc + "sv_greedy_tree.hpp" not in bench.kernel_sources("tree_round")
    assert csrc + "sv_chain.hpp" in bench.kernel_sources("tree_round")  # the walk's pick lives there
    assert bench.kernel_source_digest("chain_rowstats") != bench.kernel_source_digest("greedy_rows")
    assert set(bench.kernel_sources()) >= set(bench.kernel_sources("tree_round"))


def test_bench_ignores_counters_taken_on_other_sources(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    rec = {"kernel_source_digest": bench.kernel_source_digest("k"), "traffic_bytes_per_launch": 123.0}
    (prof / "k_w_traffic.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_digest", lambda kernel=None: rec["kernel_source_digest"])
    assert bench.load_traffic("k", "w") == 123.0
    monkeypatch.setattr(bench, "kernel_source_digest", lambda kernel=None: "0" * 16)
    assert bench.load_traffic("k", "w") is None
    assert bench.load_traffic("missing", "w") is None


def test_bench_reads_the_trace_average_of_current_sources(tmp_path, monkeypatch):
    """roofline.rocprof_avg_us comes from the committed trace summary of the
    workload, and only while that trace's digest matches the sources of the
    library kernels it lists."""
    prof = tmp_path / "profiles"
    prof.mkdir()
    table = ["| kernel | calls | average (us) | median (us) | min (us) | max (us) | share of GPU time | "
             "event-timed region average (us) |",
             "|---|---:|---:|---:|---:|---:|---:|---:|",
             "| spin | 4 | 20000.00 | 20000.00 | 19000.00 | 21000.00 | 70.0% | - |",
             "| chain_rowstats | 820 | 21.75 | 21.70 | 20.10 | 27.00 | 16.0% | 21.10 |",
             "| chain_final_pick | 820 | 4.60 | 4.50 | 3.80 | 6.30 | 3.0% | 4.40 |"]
    good = bench.trace_digest(["chain_rowstats", "chain_final_pick"])
    (prof / "w_kernel_trace.md").write_text("\n".join([f"Kernel sources digest: `{good}`", ""] + table) + "\n")
    (prof / "v_kernel_trace.md").write_text("\n".join(["Kernel sources digest: `0000000000000000`", ""] + table))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "trace_digest", lambda kernels: good if sorted(kernels) == [
        "chain_final_pick", "chain_rowstats"] else "x")
    assert bench.load_trace_average("chain_rowstats", "w") == pytest.approx(21.75)
    assert bench.load_trace_average("chain_rowstats", "w", "event-timed region average (us)") == pytest.approx(21.10)
    assert bench.load_trace_average("spin", "w") == pytest.approx(20000.0)
    assert bench.load_trace_average("spin", "w", "event-timed region average (us)") is None
    assert bench.load_trace_average("chain_final_part", "w") is None
    assert bench.load_trace_average("chain_rowstats", "v") is None
    assert bench.load_trace_average("chain_rowstats", "missing") is None


def test_sq_and_latency_summaries(tmp_path):
    """Per-kernel figures from synthetic counter files: instructions per wave,
    the VALU floor (instructions x 4 cycles over 1024 SIMDs at 2.4 GHz), the
    wait fractions, the mean L2 read latency and transcendentals per wave."""
    d = str(tmp_path / "sq")
    rows = []
    for name, val in [("SQ_WAVES", 1024), ("SQ_INSTS_VALU", 1024 * 600), ("SQ_INSTS_SALU", 1024 * 50),
                      ("SQ_INSTS_VMEM_RD", 1024 * 8), ("SQ_WAIT_INST_ANY", 250), ("SQ_WAVE_CYCLES", 1000),
                      ("SQ_BUSY_CYCLES", 1), ("SQ_ACTIVE_INST_VALU", 1), ("GRBM_GUI_ACTIVE", 1)]:
        rows += [[KERNEL, name, val], [KERNEL, name, val]]
    rows.append([COPY, "SQ_WAVES", 8])
    _write_csv(os.path.join(d, "bench_counter_collection.csv"), ["Kernel_Name", "Counter_Name", "Counter_Value"], rows)
    md = rs.sq_summary(d, "w", "python3 bench.py")
    floor = 1024 * 600 * 4 / (1024 * 2.4e9) * 1e6
    assert f"| chain_rowstats | 2 | 1024 | 600 | 50 | 8.0 | {floor:.2f} | 0.25 |" in md
    assert COPY not in md
    d2 = str(tmp_path / "lat")
    rows = []
    for name, val in [("SQ_WAVES", 100), ("SQ_WAVE_CYCLES", 1000), ("SQ_WAIT_ANY", 400),
                      ("SQ_INSTS_VALU_TRANS_F32", 6400), ("TCP_TCC_READ_REQ_LATENCY_sum", 120000),
                      ("TCP_TCC_READ_REQ_sum", 100)]:
        rows.append([KERNEL, name, val])
    _write_csv(os.path.join(d2, "bench_counter_collection.csv"), ["Kernel_Name", "Counter_Name", "Counter_Value"], rows)
    md = rs.latency_summary(d2, "w", "python3 bench.py")
    assert "| chain_rowstats | 100 | 100 | 1200 | 0.40 | 64 |" in md


def test_memory_summary(tmp_path):
    """Memory-side figures from three synthetic counter passes: the L2's hit
    rate, the mean time a read request to memory is in flight (Little's
    law), DRAM credit stalls per request and the translation miss rate."""
    passes = [[("TCC_EA0_RDREQ_sum", 1000), ("TCC_EA0_RDREQ_LEVEL_sum", 1600000), ("TCC_HIT_sum", 30),
               ("TCC_MISS_sum", 970)],
              [("TCC_EA0_RDREQ_DRAM_sum", 1000), ("TCC_EA0_RDREQ_DRAM_CREDIT_STALL_sum", 280)],
              [("TCP_UTCL1_TRANSLATION_MISS_sum", 1), ("TCP_UTCL1_TRANSLATION_HIT_sum", 999),
               ("TCP_PENDING_STALL_CYCLES_sum", 5), ("TA_BUSY_avr", 5), ("TA_ADDR_STALLED_BY_TC_CYCLES_sum", 5)]]
    dirs = []
    for i, counters in enumerate(passes):
        d = str(tmp_path / f"p{i}")
        rows = [[KERNEL, n, v] for n, v in counters] + [[COPY, counters[0][0], 7]]
        _write_csv(os.path.join(d, "bench_counter_collection.csv"), ["Kernel_Name", "Counter_Name", "Counter_Value"],
                   rows)
        dirs.append(d)
    md = rs.memory_summary(dirs, "w", "python3 bench.py")
    assert "| chain_rowstats | 1000 | 0.030 | 1600 | 0.28 | 0.0010 |" in md
    assert COPY not in md
    for p in rs.MEM_PASSES:
        assert p in md
