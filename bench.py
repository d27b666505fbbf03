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
The line's `workloads` object holds every workload's step time, rate,
dominant kernel (the one with the most time per step) and its fraction of
peak, and the in-run parity against the oracle: the tiny chain, the greedy
chain, the DeepSeek-scale chain, the EAGLE-style trees, MTP single-token
verify, temperature sampling and the sampled tree.  --workload NAME puts
another workload in the headline place; --no-workloads measures it alone.
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
CSRC = "draft_token_verification_chain_amd/csrc/"
KERNEL_SOURCES = [CSRC + f for f in (
    "sv_common.hpp", "sv_tiles.hpp", "sv_chain.hpp", "sv_greedy_tree.hpp", "sv_tree_sampled.hpp", "sv_commit.hpp",
    "sv_kernels.hpp", "specverify.hip")] + ["include/specverify.h"]
# The sources each kernel family's code comes from (its header and the ones it
# includes, the public header and the host dispatch that sets its launch).
_BASE = ["include/specverify.h", CSRC + "sv_common.hpp", CSRC + "specverify.hip"]
KERNEL_FAMILY_SOURCES = {
    "chain": _BASE + [CSRC + "sv_tiles.hpp", CSRC + "sv_chain.hpp"],
    "greedy": _BASE + [CSRC + "sv_tiles.hpp", CSRC + "sv_greedy_tree.hpp"],
    "tree_sampled": _BASE + [CSRC + "sv_tiles.hpp", CSRC + "sv_chain.hpp", CSRC + "sv_tree_sampled.hpp"],
    "commit": _BASE + [CSRC + "sv_commit.hpp"],
}
_FAMILY_OF = [("tree_rowstats", "tree_sampled"), ("tree_round", "tree_sampled"), ("tree_sample", "tree_sampled"),
              ("chain_", "chain"), ("greedy_", "greedy"), ("argmax_rows", "greedy"), ("tree_", "greedy"),
              ("commit_", "commit")]


def kernel_sources(kernel: str = None) -> list:
    """The source files a library kernel is built from (all kernel sources
    when no kernel, or an unknown one, is named)."""
    if kernel:
        for prefix, fam in _FAMILY_OF:
            if kernel.startswith(prefix):
                return KERNEL_FAMILY_SOURCES[fam]
    return KERNEL_SOURCES


def sources_digest(paths) -> str:
    """Digest of the code of source files: comments and whitespace are
    dropped, so that only a change of code changes it."""
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def kernel_source_digest(kernel: str = None) -> str:
    """Digest of what a kernel is built from (kernel_sources): stored counters
    of the kernel stay valid while it does not change."""
    return sources_digest(kernel_sources(kernel))


def trace_digest(kernels) -> str:
    """Digest of the sources of every library kernel of a kernel trace."""
    return sources_digest(sorted({p for k in kernels for p in kernel_sources(k)}))


def load_trace_average(kernel: str, workload: str, column: str = "average (us)"):
    """The kernel's average duration (us) in the committed rocprofv3 kernel
    trace of the workload (by default over all its dispatches; "event-timed
    region average (us)": over the region whose durations bench.py reports),
    if that trace was taken on the current sources of its kernels; otherwise
    None."""
    path = os.path.join(ROOT, "profiles", f"{workload}_kernel_trace.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"Kernel sources digest: `([0-9a-f]+)`", text)
    rows, col = {}, None
    for line in text.splitlines():
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        if cells and cells[0] == "kernel" and column in cells:
            col = cells.index(column)
        elif col is not None and len(cells) > col and re.fullmatch(r"\d+", cells[1]):
            if re.fullmatch(r"[0-9.]+", cells[col]):
                rows[cells[0]] = float(cells[col])
    lib = [k for k in rows if k in LIBRARY_KERNELS]
    if not m or kernel not in rows or m.group(1) != trace_digest(lib):
        return None
    return rows[kernel]


# The library's kernels (launch names; the profile summaries use the same names).
LIBRARY_KERNELS = {"chain_rowstats", "chain_prefix", "chain_rowstats_rest", "chain_accept", "chain_final_part",
                   "chain_final_pick", "chain_row_draw", "chain_small", "clear_slots", "chain_fused", "argmax_rows",
                   "greedy_rows", "greedy_rows_rest", "greedy_fused",
                   "greedy_small",
                   "greedy_finalize", "tree_root_rows", "tree_root_plan", "tree_plan", "tree_rows_rest",
                   "tree_finalize",
                   "tree_rowstats", "tree_round", "tree_sample", "commit_tokens"}


def fused_group_rows(rows: int) -> int:
    """Lanes per row when one wave combines `rows` rows' partials."""
    G = 64
    while G > 1 and G * rows > 64:
        G //= 2
    return G


def fused_group(k: int) -> int:
    """Lanes per row when one wave combines a chain's 2k rows."""
    return fused_group_rows(2 * k)


def load_traffic(kernel: str, workload: str):
    """HBM traffic per launch from the committed counter summary, if it was
    taken on the current kernel sources; otherwise None."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_digest") != kernel_source_digest(kernel):
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


# The headline workload first, then every other workload of the line's
# `workloads` object: the five named configurations (tiny chain, Llama-scale
# chain, greedy chain, DeepSeek-scale chain, EAGLE-style tree) and the further
# shapes (MTP single-token verify, temperature sampling, the sampled tree, the
# EAGLE-style tree with distinct sibling tokens).
WORKLOAD_ORDER = ["llama_chain", "tiny_chain", "greedy_chain", "deepseek_chain", "eagle_tree", "eagle_tree_distinct",
                  "mtp_chain", "sampling", "sampled_tree"]


class Workload:
    """One workload's inputs resident in HBM, its outputs and workspace, and
    its step (one library call over one batch)."""

    def __init__(self, name, seed, copies, accept_prob, torch, svl, W):
        import numpy as np

        self.name = name
        self.cfg = W.WORKLOADS[name]
        self.inp = inp = W.make_inputs(name, seed)
        self.kind = kind = inp["kind"]
        self.es = es = 2 if inp["dtype"] == W.BF16 else 4
        in_bytes = sum(v.nbytes for v in inp.values() if isinstance(v, np.ndarray))
        # enough copies to exceed twice the Infinity Cache (at most 32: a batch
        # of a few MB is latency-bound whether or not it stays in a cache)
        self.copies = copies or max(1, min(32, math.ceil(2 * MALL_BYTES / in_bytes)))
        self.dev = dev = [to_device(inp, torch, W) for _ in range(self.copies)]
        B, V = inp["B"], inp["V"]
        self.accept_prob = accept_prob and kind == "chain"
        i32 = dict(dtype=torch.int32, device="cuda")
        if kind in ("chain", "greedy"):
            k = inp["k"]
            self.out = dict(accepted_len=torch.empty(B, **i32), emitted=torch.empty((B, k + 1), **i32))
        else:
            md = inp["max_depth"]
            self.out = dict(accepted_len=torch.empty(B, **i32), emitted=torch.empty((B, md + 1), **i32),
                            accepted_nodes=torch.empty((B, md + 1), **i32))
        out = self.out
        if kind == "chain":
            k = inp["k"]
            out["accept_prob"] = (torch.empty((B, k), dtype=torch.float32, device="cuda") if self.accept_prob
                                  else None)
            ws = torch.empty(svl.chain_workspace_bytes(B, k, V, inp["dtype"]), dtype=torch.uint8, device="cuda")

            def step(i):
                t = dev[i % self.copies]
                svl.verify_chain(t["draft_tokens"], t["draft_logits"], t["target_logits"], t["temperature"],
                                 t["uniforms"], workspace=ws, out=out)
            self.units = B * k if k > 0 else B
        elif kind == "greedy":
            k = inp["k"]
            ws = torch.empty(svl.greedy_workspace_bytes(B, k, V, inp["dtype"]), dtype=torch.uint8, device="cuda")

            def step(i):
                t = dev[i % self.copies]
                svl.verify_greedy(t["draft_tokens"], t["target_logits"], workspace=ws, out=out)
            self.units = B * k
        elif kind == "tree_sampled":
            N, md = inp["N"], inp["max_depth"]
            ws = torch.empty(svl.tree_sampled_workspace_bytes(B, N, V, inp["dtype"]), dtype=torch.uint8,
                             device="cuda")

            def step(i):
                t = dev[i % self.copies]
                svl.verify_tree_sampled(t["node_tokens"], t["parent"], md, t["draft_logits"], t["target_logits"],
                                        t["temperature"], t["uniforms"], workspace=ws, out=out)
            self.units = B * (inp["N"] - 1)
        else:
            N, md = inp["N"], inp["max_depth"]
            ws = torch.empty(svl.tree_workspace_bytes(B, N, V, inp["dtype"]), dtype=torch.uint8, device="cuda")

            def step(i):
                t = dev[i % self.copies]
                svl.verify_tree(t["node_tokens"], t["parent"], md, t["target_logits"], workspace=ws, out=out)
            self.units = B * (inp["N"] - 1)
        self.ws = ws
        self.step = step
        self.unit = ("sampled tokens/s" if kind == "chain" and inp["k"] == 0 else
                     "verified draft nodes/s" if kind in ("tree", "tree_sampled") else "verified draft tokens/s")

    def outputs(self):
        return {key: (v.cpu().numpy() if v is not None else None) for key, v in self.out.items()}

    def kernel_bytes(self, got, W):
        """Algorithmic bytes per launch of every streaming kernel of the step,
        and launches per step; where they depend on the outcome (the rows a draw
        or a later phase reads), from this batch's outputs (identical in every
        copy)."""
        import numpy as np

        inp, es, kind = self.inp, self.es, self.kind
        B, V = inp["B"], inp["V"]
        kb, launches = {}, {}
        if kind == "chain":
            k = inp["k"]
            a = got["accepted_len"]
            T = inp["temperature"]
            # every draft row and target rows 0..k-1 once; without accept_prob,
            # from 6 drafts and 128 MiB of rows the library streams positions
            # 0..s-1 first and the rest only for sequences that accept all of them
            s = (max(1, k // 4) if not self.accept_prob and k >= 6 and 2 * B * k * V * es >= 128 << 20 else k)
            if k > 0:
                kb["chain_rowstats"] = 2 * B * s * V * es
                if s < k:
                    kb["chain_rowstats_rest"] = int((a >= s).sum()) * 2 * (k - s) * V * es
            # the final draw: both rows at a rejection, the bonus row after full
            # acceptance, the row's argmax at temperature 0 (with no drafts: row 0);
            # plain sampling: one workgroup per row from 256 rows of at most 256 segments
            nseg = -(-(-(-V // (16 // es))) // 64)
            draw_kernel = "chain_row_draw" if k == 0 and B >= 256 and nseg <= 256 else "chain_final_part"
            draw = 0
            for b in range(B):
                if T[b] > 0:
                    draw += (2 if a[b] < k else 1) * V * es
                elif a[b] == k:
                    draw += V * es
            kb[draw_kernel] = draw
            # small chains: the whole verification in one launch, one workgroup per sequence
            nT = -(-V * es // 8192)
            if B <= 256 and (k > 0 or B < 256) and nseg <= 64 and 2 * k * nT <= 160 and (2 * k + 1) * V * es <= 144 << 10:
                kb = {"chain_small": kb.pop("chain_rowstats", 0) + kb.pop(draw_kernel)}
            elif 0 < k == s and B * -(-nseg // 16) <= 2048 and 2 * k <= 64 and nT <= 8 * fused_group(k):
                # rows and draw in one launch (after a launch that clears the partial slots)
                kb = {"chain_fused": kb.pop("chain_rowstats") + kb.pop(draw_kernel)}
        elif kind == "greedy":
            k = inp["k"]
            s = (k + 1) // 2 if k >= 1 and B * (k + 1) * V * es >= 256 << 20 else k + 1
            kb["greedy_rows"] = B * s * V * es
            if s <= k:
                kb["greedy_rows_rest"] = int((got["accepted_len"] >= s).sum()) * (k + 1 - s) * V * es
                # both phases in one launch when the first s rows' partials fit one wave
                if -(-V * es // 8192) <= 8 * fused_group_rows(s):
                    kb = {"greedy_fused": kb["greedy_rows"] + kb["greedy_rows_rest"]}
            # small greedy chains: one launch, one workgroup per sequence
            if B <= 256 and (k + 1) * -(-V * es // 8192) <= 16:
                kb = {"greedy_small": B * (k + 1) * V * es}
        elif kind == "tree_sampled":
            N, par = inp["N"], inp["parent"]
            # the target and draft rows of every inner node
            inner = int(np.count_nonzero(np.bincount(par[1:], minlength=N)))
            kb["tree_rowstats"] = B * 2 * inner * V * es
            # the walk's passes (from the outputs and the tree): every rejected
            # child costs one pass over its parent's two rows; the final draw's
            # masses one more pass (two rows after a rejection at that node, the
            # target row otherwise), and a walk ending at a leaf first forms the
            # leaf's target-row statistics (one row)
            kids = [[i for i in range(1, N) if par[i] == n] for n in range(N)]
            T = inp["temperature"]
            walk = 0
            for b in range(B):
                if got["accepted_len"][b] < 0 or not T[b] > 0:
                    continue
                path = [0] + [int(x) for x in got["accepted_nodes"][b] if x >= 0]
                rejected_last = 0
                for depth, n in enumerate(path):
                    nxt = path[depth + 1] if depth + 1 < len(path) else None
                    rej = sum(1 for c in kids[n] if nxt is None or c < nxt)
                    walk += rej * 2 * V * es
                    rejected_last = rej
                last = path[-1]
                walk += (2 if rejected_last else 1) * V * es + (V * es if not kids[last] else 0)
            launches["tree_round"] = 7
            kb["tree_round"] = walk / 7
        else:
            N = inp["N"]
            tree_two_phase = N > 1 and B * N * V * es >= 96 << 20
            if tree_two_phase:
                # each later phase lists the nodes of its depth range whose ancestor
                # at the range's first depth is accepted (node acceptance from the
                # outputs: the accepted path; every node of the range below an
                # accepted depth-lo ancestor is listed)
                ranges = ([(1, 2), (3, N)] if B * N * V * es >= 192 << 20 and N >= 48 else [(1, N)])
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
                    for lo, hi in ranges:
                        for n in range(1, N):
                            an = n
                            while depth[an] > lo:
                                an = par[an]
                            rest_rows += int(lo <= depth[n] <= hi and acc[an])
                # trees of at most 256 nodes: the root rows and the first plan in one launch
                kb["tree_root_plan" if N <= 256 else "tree_root_rows"] = B * V * es
                kb["tree_rows_rest"] = rest_rows * V * es / len(ranges)
                launches["tree_rows_rest"] = len(ranges)
            else:
                kb["argmax_rows"] = B * N * V * es
        return kb, launches

    def timed(self, svl, torch, steps, profiled):
        """K steps back to back behind a ~20 ms spin kernel (so that host launch
        overhead stays outside the measurement); returns ms per step."""
        if profiled:
            svl.profile_begin(16 * steps)
        torch.cuda._sleep(int(50e6))
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(steps):
            self.step(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps


def measure(wl, svl, torch, W, steps, warmup):
    """Times one workload: the median of three timed regions of `steps`
    steps without per-kernel events (the throughput), then one region with an
    event pair attached to each kernel dispatch (per-kernel durations); the
    dominant kernel is the one with the most time per step."""
    for i in range(warmup):
        wl.step(i)
    torch.cuda.synchronize()
    got = wl.outputs()
    kb, launches = wl.kernel_bytes(got, W)
    reps = [wl.timed(svl, torch, steps, False) for _ in range(3)]
    ms = sorted(reps)[1]
    ms_prof = wl.timed(svl, torch, steps, True)
    prof = svl.profile_end()
    kernels = {name: dict(launches=n, avg_us=1e3 * tot / max(n, 1)) for name, (n, tot) in prof.items()}
    per_step = {name: v["launches"] / steps for name, v in kernels.items()}
    missing = [name for name in kb if name not in kernels]
    if missing:
        raise RuntimeError(f"{wl.name}: bench.py expects kernels the library did not launch: {missing}")
    step_bytes = sum(v * launches.get(name, 1) for name, v in kb.items())
    # the dominant kernel: the kernel with the most time per step
    dominant = max(kernels, key=lambda name: kernels[name]["avg_us"] * per_step[name])
    dom_us = kernels[dominant]["avg_us"]
    dom_bytes = kb.get(dominant)
    return dict(ms=ms, reps=reps, ms_prof=ms_prof, got=got, kb=kb, launches=launches, kernels=kernels,
                per_step=per_step, step_bytes=step_bytes, dominant=dominant, dom_us=dom_us, dom_bytes=dom_bytes)


def workload_record(wl, m, parity):
    """The `workloads` entry of one workload."""
    s = m["ms"] * 1e-3
    frac = (m["dom_bytes"] / (m["dom_us"] * 1e-6) / 1e9 / PEAK_HBM_GBS) if m["dom_bytes"] else None
    rec = {"name": wl.cfg["name"], "B": wl.inp["B"], "k": wl.inp.get("k"), "N": wl.inp.get("N"), "V": wl.inp["V"],
           "logits": DTYPE_NAMES[wl.inp["dtype"]], "step_us": round(m["ms"] * 1e3, 2),
           "value": wl.units / s, "unit": wl.unit,
           "hbm_gbs": m["step_bytes"] / s / 1e9, "hbm_frac_of_peak": m["step_bytes"] / s / 1e9 / PEAK_HBM_GBS,
           "algorithmic_bytes_per_step": m["step_bytes"],
           "dominant_kernel": m["dominant"], "dominant_us": round(m["dom_us"], 3),
           "dominant_bytes_per_launch": m["dom_bytes"], "dominant_frac_of_peak": frac,
           "kernels_us": {n: round(v["avg_us"], 3) for n, v in m["kernels"].items()},
           "kernel_launches_per_step": {n: round(v, 3) for n, v in m["per_step"].items()}}
    if parity is not None:
        rec["parity"] = parity
    return rec


DTYPE_NAMES = {0: "f32", 1: "bf16"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="llama_chain", choices=WORKLOAD_ORDER)
    ap.add_argument("--seed", type=int, default=1)
    ap.add_argument("--copies", type=int, default=0, help="input copies rotated (0 = enough to exceed 2x the MALL)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu", action="store_true", help="no oracle leg (no cpu_baseline, no parity)")
    ap.add_argument("--no-workloads", action="store_true",
                    help="measure the chosen workload only (no `workloads` object)")
    ap.add_argument("--workload-steps", type=int, default=200, help="timed steps of each further workload")
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

    import torch

    import draft_token_verification_chain_amd as svl
    import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    svl.load()
    print(f"[bench] {args.workload}: generating inputs", file=sys.stderr, flush=True)
    wl = Workload(args.workload, args.seed, args.copies, args.accept_prob, torch, svl, W)
    if args.calibrate_copy:
        src = torch.ones(args.calibrate_copy * 2 ** 18, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    m = measure(wl, svl, torch, W, args.steps, args.warmup)
    s_per_step = m["ms"] * 1e-3
    dominant, dom_us = m["dominant"], m["dom_us"]
    dom_bytes = m["dom_bytes"]
    achieved = dom_bytes / (dom_us * 1e-6) / 1e9 if dom_bytes else None
    traffic = load_traffic(dominant, args.workload)
    rocprof_us = load_trace_average(dominant, args.workload, "event-timed region average (us)")
    rocprof_b2b_us = load_trace_average(dominant, args.workload)
    inp, cfg = wl.inp, wl.cfg
    B, V, kind = inp["B"], inp["V"], wl.kind
    result = {
        "metric": METRIC if args.workload == "llama_chain" else f"{wl.unit[:-2]}/sec ({cfg['name']})",
        "value": wl.units / s_per_step,
        "unit": wl.unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": m["ms"],
        "ms_per_step_repeats": m["reps"],
        "ms_per_step_with_kernel_events": m["ms_prof"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": W.DTYPE_NAMES[inp["dtype"]],
        "data": "synthetic (seeded generator, shapes of the named workload)",
        "config": {"workload": cfg["name"], "B": B, "k": inp.get("k"), "N": inp.get("N"), "V": V,
                   "logits": W.DTYPE_NAMES[inp["dtype"]], "temperature": cfg.get("temperature"),
                   "seed": args.seed, "input_copies_rotated": wl.copies, "parallelism": "single GPU",
                   "accept_prob": bool(args.accept_prob) if kind == "chain" else None},
        "hbm_gbs": m["step_bytes"] / s_per_step / 1e9,
        "hbm_frac_of_peak": m["step_bytes"] / s_per_step / 1e9 / PEAK_HBM_GBS,
        "algorithmic_bytes_per_step": m["step_bytes"],
        "bytes_per_verified_token": m["step_bytes"] / wl.units,
        # every sequence emits its accepted tokens plus one final token
        "emitted_tokens_per_s": float((m["got"]["accepted_len"].clip(min=0) + 1).sum()) / s_per_step,
        "kernels_us": {n: round(v["avg_us"], 3) for n, v in m["kernels"].items()},
        "kernels_bytes_per_launch": {n: int(v) for n, v in m["kb"].items()},
        # achieved: algorithmic bytes per launch over the kernel's average duration,
        # measured with HIP events attached to its dispatches on its launch stream
        "roofline": {"bound": "hbm", "kernel": dominant, "achieved": achieved, "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS if achieved else None, "traffic": traffic,
                     "bytes_per_launch": dom_bytes, "avg_launch_us": dom_us, "duration_source": "hip_events",
                     "traffic_gbs": traffic / (dom_us * 1e-6) / 1e9 if traffic else None,
                     # the same kernel in the committed rocprofv3 trace of this command (null
                     # once its sources have changed): its average over the event-timed
                     # region, the fraction that gives, and its average over all dispatches,
                     # most of them back to back (slower by the preceding kernel's tail)
                     "rocprof_avg_us": rocprof_us,
                     "frac_rocprof": (dom_bytes / (rocprof_us * 1e-6) / 1e9 / PEAK_HBM_GBS
                                      if rocprof_us and dom_bytes else None),
                     "rocprof_avg_us_all_dispatches": rocprof_b2b_us},
    }

    if not args.no_cpu:
        reps, el, threads = cpu_baseline(inp, args.cpu_seconds)
        reps1, el1, _ = cpu_baseline(inp, args.cpu_seconds / 2, threads=1)
        result["cpu_baseline"] = {"value": wl.units * reps / el, "unit": wl.unit, "cores": threads,
                                  "kind": "oracle",
                                  "sample": f"the full {cfg['name']} batch (B={B}) x {reps} repetitions, {el:.1f} s",
                                  "value_1thread": wl.units * reps1 / el1,
                                  "sample_1thread": f"the same batch x {reps1} repetitions on one thread, {el1:.1f} s",
                                  "cpu_model": cpu_model()}
        result["parity"] = check_against_oracle(inp, m["got"])

    if not args.no_workloads:
        first = wl
        records = {}
        for name in WORKLOAD_ORDER:
            if name == args.workload:
                records[name] = workload_record(first, m, result.get("parity"))
                continue
            del wl
            torch.cuda.empty_cache()
            print(f"[bench] {name}: generating inputs", file=sys.stderr, flush=True)
            wl = Workload(name, args.seed, 0, args.accept_prob, torch, svl, W)
            mw = measure(wl, svl, torch, W, args.workload_steps, min(args.warmup, 20))
            parity = None if args.no_cpu else check_against_oracle(wl.inp, mw["got"])
            records[name] = workload_record(wl, mw, parity)
            print(f"[bench] {name}: {records[name]['step_us']} us per step", file=sys.stderr, flush=True)
        result["workloads"] = records
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
