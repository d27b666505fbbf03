#!/usr/bin/env python3
"""Throughput of batched draft-token verification on one MI355X.

One step = one sv_verify_chain call over one batch of the Llama-scale
workload (B = 64 sequences, k = 4 drafts, V = 128256, bfloat16 logits,
temperature 0.7): the whole path -- row normalisers of every draft and target
row, acceptance tests, first-rejection scan, residual or bonus draw.  Inputs
are resident in HBM before the timed region; several identical copies are
rotated so that successive steps read HBM rather than the 256 MB Infinity
Cache.  A spin kernel queued ahead of the timed steps builds a backlog, so the
steps run back to back on the GPU and host launch overhead stays outside the
measured time.  Two timed regions run the same K steps: the first gives the
throughput; in the second the library attaches a HIP event pair to each
kernel dispatch on its launch stream, which gives every kernel's duration
(the roofline of the dominant kernel uses these).

Prints one JSON line (see the metric, roofline and cpu_baseline fields).
Other workloads (--workload greedy_chain, deepseek_chain, eagle_tree, mtp_chain,
sampling, sampled_tree) print the same line for their own step; the default
line is the Llama-scale chain.
"""

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0        # MI355X HBM3E, published
MALL_BYTES = 256 * 2 ** 20   # Infinity Cache
METRIC = "verified draft tokens/sec and HBM GB/s (% of peak) at B=64,k=4,V=128256 bf16"
KERNEL_SOURCES = ["draft_token_verification_chain_amd/csrc/" + f for f in (
    "sv_common.hpp", "sv_tiles.hpp", "sv_chain.hpp", "sv_greedy_tree.hpp", "sv_tree_sampled.hpp", "sv_commit.hpp",
    "sv_kernels.hpp", "specverify.hip")]


def kernel_source_digest() -> str:
    """Digest of the kernel sources' code: comments and whitespace are
    dropped, so that only a change of code marks stored counters stale."""
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def load_traffic(kernel: str, workload: str):
    """HBM traffic per launch from the committed counter summary, if it was
    taken on the current kernel sources; otherwise None."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_digest") != kernel_source_digest():
        return None
    return rec.get("traffic_bytes_per_launch")


def to_device(inp, torch, W):
    import numpy as np

    def logits(a):
        if inp["dtype"] == W.BF16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    t = dict(target_logits=logits(inp["target_logits"]))
    if inp["kind"] == "chain":
        t.update(draft_logits=logits(inp["draft_logits"]),
                 draft_tokens=torch.from_numpy(inp["draft_tokens"]).cuda(),
                 temperature=torch.from_numpy(inp["temperature"]).cuda(),
                 uniforms=torch.from_numpy(inp["uniforms"]).cuda())
    elif inp["kind"] == "greedy":
        t.update(draft_tokens=torch.from_numpy(inp["draft_tokens"]).cuda())
    elif inp["kind"] == "tree_sampled":
        t.update(draft_logits=logits(inp["draft_logits"]),
                 node_tokens=torch.from_numpy(inp["node_tokens"]).cuda(),
                 parent=torch.from_numpy(inp["parent"]).cuda(),
                 temperature=torch.from_numpy(inp["temperature"]).cuda(),
                 uniforms=torch.from_numpy(inp["uniforms"]).cuda())
    else:
        t.update(node_tokens=torch.from_numpy(inp["node_tokens"]).cuda(),
                 parent=torch.from_numpy(inp["parent"]).cuda())
    return t


def check_against_oracle(inp, got: dict) -> dict:
    """The timed steps' outputs (every step verifies the same batch) against
    the oracle's: bit-exact outside the oracle's band."""
    import numpy as np

    import oracle

    ref = {"chain": oracle.verify_chain, "greedy": oracle.verify_greedy, "tree": oracle.verify_tree,
           "tree_sampled": oracle.verify_tree_sampled}[inp["kind"]](inp)
    mism = (got["accepted_len"] != ref["accepted_len"]) | (got["emitted"] != ref["emitted"]).any(axis=1)
    if got.get("accepted_nodes") is not None and ref.get("accepted_nodes") is not None:
        mism |= (got["accepted_nodes"] != ref["accepted_nodes"]).any(axis=1)
    band = ref.get("band", np.zeros(mism.shape, bool))
    return {"sequences": int(mism.size), "banded": int(band.sum()),
            "banded_differing": int((mism & band).sum()), "differing_outside_band": int((mism & ~band).sum())}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(inp, seconds: float, threads: int = 0):
    """The oracle as it stands, on this host's cores (or on `threads` of
    them), repeated on the same batch for about `seconds`."""
    import oracle

    fn = {"chain": oracle.verify_chain, "greedy": oracle.verify_greedy, "tree": oracle.verify_tree,
          "tree_sampled": oracle.verify_tree_sampled}[inp["kind"]]
    default = oracle.max_threads()
    if threads:
        oracle.set_num_threads(threads)
    try:
        fn(inp)  # warm-up (page faults, thread pool)
        reps, t0 = 0, time.perf_counter()
        while True:
            fn(inp)
            reps += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
        used = oracle.max_threads()
    finally:
        oracle.set_num_threads(default)
    return reps, el, used


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="llama_chain",
                    choices=["llama_chain", "greedy_chain", "deepseek_chain", "eagle_tree", "mtp_chain",
                             "sampling", "sampled_tree"])
    ap.add_argument("--seed", type=int, default=1)
    ap.add_argument("--copies", type=int, default=0, help="input copies rotated (0 = enough to exceed 2x the MALL)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--accept-prob", action="store_true",
                    help="chain workloads: also return accept_prob (tau of every draft, also past the first "
                         "rejection), which makes the library read every row")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="before the timed region, run one plain device copy of MIB MiB (a reference "
                         "kernel of known traffic for hardware counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library runs on a single MI355X and the workload is "
              "one GPU's batch (sequences are independent, so a batch splits across GPUs with no exchange).",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import draft_token_verification_chain_amd as svl
    import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    svl.load()
    cfg = W.WORKLOADS[args.workload]
    inp = W.make_inputs(args.workload, args.seed)
    kind = inp["kind"]
    es = 2 if inp["dtype"] == W.BF16 else 4
    in_bytes = sum(v.nbytes for k, v in inp.items() if isinstance(v, np.ndarray))
    copies = args.copies or max(1, math.ceil(2 * MALL_BYTES / in_bytes))
    dev = [to_device(inp, torch, W) for _ in range(copies)]
    B, V = inp["B"], inp["V"]

    if kind == "chain":
        k = inp["k"]
        out = dict(accepted_len=torch.empty(B, dtype=torch.int32, device="cuda"),
                   emitted=torch.empty((B, k + 1), dtype=torch.int32, device="cuda"),
                   accept_prob=(torch.empty((B, k), dtype=torch.float32, device="cuda") if args.accept_prob
                                else None))
        ws = torch.empty(svl.chain_workspace_bytes(B, k, V, inp["dtype"]), dtype=torch.uint8, device="cuda")

        def step(i):
            t = dev[i % copies]
            svl.verify_chain(t["draft_tokens"], t["draft_logits"], t["target_logits"], t["temperature"],
                             t["uniforms"], workspace=ws, out=out)
        units = B * k if k > 0 else B       # verified draft tokens (sampled tokens when k == 0) per step
        # k == 0: one workgroup per row from 256 rows of at most 256 segments
        # (64 vectors of 16 bytes each)
        nseg = -(-(-(-V // (16 // es))) // 64)  # ceil(ceil(V / (16 / es)) / 64)
        draw_kernel = "chain_row_draw" if B >= 256 and nseg <= 256 else "chain_final_part"
        # every draft row and target rows 0..k-1 once; without accept_prob,
        # from 6 drafts and 128 MiB of rows the library streams positions
        # 0..s-1 first and the rest only for sequences that accept all of them
        chain_s = (max(1, k // 4) if not args.accept_prob and k >= 6 and 2 * B * k * V * es >= 128 << 20 else k)
    elif kind == "greedy":
        k = inp["k"]
        out = dict(accepted_len=torch.empty(B, dtype=torch.int32, device="cuda"),
                   emitted=torch.empty((B, k + 1), dtype=torch.int32, device="cuda"))
        ws = torch.empty(svl.greedy_workspace_bytes(B, k, V, inp["dtype"]), dtype=torch.uint8, device="cuda")

        def step(i):
            t = dev[i % copies]
            svl.verify_greedy(t["draft_tokens"], t["target_logits"], workspace=ws, out=out)
        units = B * k
        # rows 0..s-1 of every sequence; at 256 MiB of rows and more the library
        # reads rows s..k only for sequences accepting their first s drafts
        s_first = (k + 1) // 2 if k >= 1 and B * (k + 1) * V * es >= 256 << 20 else k + 1
    elif kind == "tree_sampled":
        N = inp["N"]
        md = inp["max_depth"]
        out = dict(accepted_len=torch.empty(B, dtype=torch.int32, device="cuda"),
                   emitted=torch.empty((B, md + 1), dtype=torch.int32, device="cuda"),
                   accepted_nodes=torch.empty((B, md + 1), dtype=torch.int32, device="cuda"))
        ws = torch.empty(svl.tree_sampled_workspace_bytes(B, N, V, inp["dtype"]), dtype=torch.uint8, device="cuda")

        def step(i):
            t = dev[i % copies]
            svl.verify_tree_sampled(t["node_tokens"], t["parent"], md, t["draft_logits"], t["target_logits"],
                                    t["temperature"], t["uniforms"], workspace=ws, out=out)
        units = B * (N - 1)                 # verified draft nodes per step
        inner = int(np.count_nonzero(np.bincount(inp["parent"][1:], minlength=N)))
    else:
        N = inp["N"]
        md = inp["max_depth"]
        out = dict(accepted_len=torch.empty(B, dtype=torch.int32, device="cuda"),
                   emitted=torch.empty((B, md + 1), dtype=torch.int32, device="cuda"),
                   accepted_nodes=torch.empty((B, md + 1), dtype=torch.int32, device="cuda"))
        ws = torch.empty(svl.tree_workspace_bytes(B, N, V, inp["dtype"]), dtype=torch.uint8, device="cuda")

        def step(i):
            t = dev[i % copies]
            svl.verify_tree(t["node_tokens"], t["parent"], md, t["target_logits"], workspace=ws, out=out)
        units = B * (N - 1)                 # verified draft nodes per step
        # from 96 MiB of rows the library streams the root rows, then only the
        # rows below an accepted depth-1 node (from 192 MiB and 48 nodes: depths
        # 1-2 below an accepted depth-1 node, then depths 3+ below an accepted
        # depth-3 node); those rows are counted below, from the outcome
        tree_two_phase = N > 1 and B * N * V * es >= 96 << 20
        tree_ranges = ([(1, 2), (3, N)] if B * N * V * es >= 192 << 20 and N >= 48 else [(1, N)])

    unit = "sampled tokens/s" if kind == "chain" and inp["k"] == 0 else "verified draft tokens/s"
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    if args.calibrate_copy:
        src = torch.ones(args.calibrate_copy * 2 ** 18, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # algorithmic bytes per launch of every streaming kernel of the step, and
    # its launches per step; where they depend on the outcome (the rows a
    # draw or a later phase reads), from this batch's (identical in every copy)
    kernel_bytes, kernel_launches = {}, {}
    if kind == "chain":
        a = out["accepted_len"].cpu().numpy()
        T = inp["temperature"]
        k = inp["k"]
        if k > 0:
            kernel_bytes["chain_rowstats"] = 2 * B * chain_s * V * es
            if chain_s < k:
                kernel_bytes["chain_rowstats_rest"] = int((a >= chain_s).sum()) * 2 * (k - chain_s) * V * es
        # the final draw: both rows at a rejection, the bonus row after full
        # acceptance, the row's argmax at temperature 0 (with no drafts: row 0)
        draw = 0
        for b in range(B):
            if T[b] > 0:
                draw += (2 if a[b] < k else 1) * V * es
            elif a[b] == k:
                draw += V * es
        kernel_bytes[draw_kernel] = draw
    elif kind == "greedy":
        kernel_bytes["greedy_rows"] = B * s_first * V * es
        if s_first <= inp["k"]:
            a = out["accepted_len"].cpu().numpy()
            kernel_bytes["greedy_rows_rest"] = int((a >= s_first).sum()) * (inp["k"] + 1 - s_first) * V * es
    elif kind == "tree_sampled":
        # the target and draft rows of every inner node (a leaf's rows are read
        # only when a walk ends there; those and the walk's passes over the rows
        # of the nodes it visits come on top, uncounted)
        kernel_bytes["tree_rowstats"] = B * 2 * inner * V * es
    elif tree_two_phase:
        # each later phase lists the nodes of its depth range whose ancestor at
        # the range's first depth is accepted (node acceptance from the rows'
        # argmax, host-side bookkeeping for the byte count only)
        par, tok = inp["parent"], inp["node_tokens"]
        top = np.argmax(W.values(inp["target_logits"], inp["dtype"]), axis=-1)
        depth = np.zeros(N, np.int64)
        for n in range(1, N):
            depth[n] = depth[par[n]] + 1
        rest_rows = 0
        for b in range(B):
            acc = np.zeros(N, bool)
            acc[0] = True
            for n in range(1, N):
                acc[n] = acc[par[n]] and tok[b, n] == top[b, par[n]]
            for lo, hi in tree_ranges:
                for n in range(1, N):
                    a = n
                    while depth[a] > lo:
                        a = par[a]
                    rest_rows += int(lo <= depth[n] <= hi and acc[a])
        kernel_bytes["tree_root_rows"] = B * V * es
        kernel_bytes["tree_rows_rest"] = rest_rows * V * es / len(tree_ranges)
        kernel_launches["tree_rows_rest"] = len(tree_ranges)
    else:
        kernel_bytes["argmax_rows"] = B * N * V * es
    step_bytes = sum(v * kernel_launches.get(name, 1) for name, v in kernel_bytes.items())

    def timed(profiled: bool) -> float:
        """K steps back to back behind a ~20 ms spin kernel (so that host launch
        overhead stays outside the measurement); returns ms per step."""
        if profiled:
            svl.profile_begin(8 * args.steps)
        torch.cuda._sleep(int(50e6))
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(args.steps):
            step(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    # timed region 1: the throughput (no per-kernel events), K steps timed three
    # times; the median is reported (the spread between back-to-back runs on one
    # machine is about 1 us per step, mostly in the gaps between kernels)
    ms_repeats = [timed(False) for _ in range(3)]
    ms_per_step = sorted(ms_repeats)[1]
    # timed region 2: the same steps, each kernel's own dispatch timed by HIP events
    # (per-kernel durations for the roofline; the events themselves add gaps between
    # kernels, so this region's step time is reported separately)
    ms_profiled = timed(True)
    prof = svl.profile_end()
    s_per_step = ms_per_step * 1e-3

    kernels = {name: dict(launches=n, avg_us=1e3 * tot / max(n, 1)) for name, (n, tot) in prof.items()}
    missing = [name for name in kernel_bytes if name not in kernels]
    if missing:
        raise RuntimeError(f"bench.py expects kernels the library did not launch: {missing}")
    # the dominant kernel: the streaming kernel with the most time per step
    dominant = max(kernel_bytes, key=lambda name: kernels[name]["avg_us"] * kernel_launches.get(name, 1))
    dominant_bytes = kernel_bytes[dominant]
    dom_us = kernels[dominant]["avg_us"]
    achieved = dominant_bytes / (dom_us * 1e-6) / 1e9
    traffic = load_traffic(dominant, args.workload)

    result = {
        "metric": METRIC if args.workload == "llama_chain" else f"{unit[:-2]}/sec ({cfg['name']})",
        "value": units / s_per_step,
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "ms_per_step_repeats": ms_repeats,
        "ms_per_step_with_kernel_events": ms_profiled,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": W.DTYPE_NAMES[inp["dtype"]],
        "data": "synthetic (seeded generator, shapes of the named workload)",
        "config": {"workload": cfg["name"], "B": B, "k": inp.get("k"), "N": inp.get("N"), "V": V,
                   "logits": W.DTYPE_NAMES[inp["dtype"]], "temperature": cfg.get("temperature"),
                   "seed": args.seed, "input_copies_rotated": copies, "parallelism": "single GPU",
                   "accept_prob": bool(args.accept_prob) if kind == "chain" else None},
        "hbm_gbs": step_bytes / s_per_step / 1e9,
        "hbm_frac_of_peak": step_bytes / s_per_step / 1e9 / PEAK_HBM_GBS,
        "algorithmic_bytes_per_step": step_bytes,
        "bytes_per_verified_token": step_bytes / units,
        # every sequence emits its accepted tokens plus one final token
        "emitted_tokens_per_s": float(out["accepted_len"].sum().item() + B) / s_per_step,
        "kernels_us": {n: round(v["avg_us"], 3) for n, v in kernels.items()},
        "kernels_bytes_per_launch": {n: int(v) for n, v in kernel_bytes.items()},
        "roofline": {"bound": "hbm", "kernel": dominant, "achieved": achieved, "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS, "traffic": traffic,
                     "bytes_per_launch": dominant_bytes, "avg_launch_us": dom_us,
                     "traffic_gbs": traffic / (dom_us * 1e-6) / 1e9 if traffic else None},
    }

    if not args.no_cpu:
        reps, el, threads = cpu_baseline(inp, args.cpu_seconds)
        reps1, el1, _ = cpu_baseline(inp, args.cpu_seconds / 2, threads=1)
        result["cpu_baseline"] = {"value": units * reps / el, "unit": unit, "cores": threads,
                                  "kind": "oracle",
                                  "sample": f"the full {cfg['name']} batch (B={B}) x {reps} repetitions, {el:.1f} s",
                                  "value_1thread": units * reps1 / el1,
                                  "sample_1thread": f"the same batch x {reps1} repetitions on one thread, {el1:.1f} s",
                                  "cpu_model": cpu_model()}
        result["parity"] = check_against_oracle(inp, {key: (v.cpu().numpy() if v is not None else None)
                                                      for key, v in out.items()})
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
