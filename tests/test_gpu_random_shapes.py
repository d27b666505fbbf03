"""Parity on seeded random shapes.

Each case draws a chain, greedy, greedy-tree or sampled-tree verification
problem from a counter-based generator of its own: batch size, number of drafts (0 to 12), vocabulary size
(log-uniform over 2 .. 150000, so most tails are ragged and odd sizes take the
element-load path), logit type, per-sequence temperatures with some of them 0,
and the draft's distance from the target (near copies to unrelated rows).  The
sizes are capped (24 M logits per case) so that the oracle finishes each case
in about a second.  Trees take random shapes too (node count, branching and
depth bounds, siblings that may share a token).  Every output is compared with
the oracle's: chains and sampled trees bit-exactly outside the 1e-5 band,
greedy chains and trees exactly.
"""

import numpy as np
import pytest

import workloads as W
from gpu_common import compare_chain, compare_tree_sampled, run_chain, run_greedy, run_tree, run_tree_sampled

pytestmark = pytest.mark.gpu

MAX_ELEMENTS = 24_000_000  # B * (2k + 1) * V per case


@pytest.fixture(scope="module")
def svl():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import draft_token_verification_chain_amd as svl

    svl.load()
    return svl


def _shape(case: int, rows_per_seq):
    """(B, k, V, dtype) of a case, B reduced to fit MAX_ELEMENTS."""
    g = np.random.Generator(np.random.Philox(key=[2024, case]))
    k = int(g.integers(0, 13))
    V = int(np.exp(g.uniform(np.log(2.0), np.log(150000.0))))
    dt = W.BF16 if g.random() < 0.5 else W.F32
    B = int(g.integers(1, 301))
    B = max(1, min(B, MAX_ELEMENTS // (rows_per_seq(k) * V)))
    return g, B, k, V, dt


CHAIN_CASES = list(range(64))


@pytest.mark.parametrize("case", CHAIN_CASES)
def test_random_chain_shapes(svl, orc, case):
    g, B, k, V, dt = _shape(case, lambda k: 2 * k + 1)
    T = g.uniform(0.2, 1.6, size=B).astype(np.float32)
    T[g.random(B) < 0.2] = 0.0
    sigma = float(np.exp(g.uniform(np.log(0.02), np.log(3.0))))
    zipf = 1.1 if g.random() < 0.5 else None
    inp = W.chain_inputs(B, k, V, dt, 100 + case, target_sigma=float(g.uniform(1.0, 4.0)), zipf_s=zipf,
                         draft_sigma=sigma, temperature=T)
    label = f"case {case}: B{B} k{k} V{V} {W.DTYPE_NAMES[dt]} sigma {sigma:.3g}"
    print(f"[random shapes] chain {label}", flush=True)
    got = run_chain(svl, inp)
    ref = orc.verify_chain(inp)
    stats = compare_chain(inp, got, ref, label)
    print(f"[random shapes] chain {label}: {stats}", flush=True)


GREEDY_CASES = list(range(32))


@pytest.mark.parametrize("case", GREEDY_CASES)
def test_random_greedy_shapes(svl, orc, case):
    g, B, k, V, dt = _shape(1000 + case, lambda k: k + 1)
    match_p = float(g.uniform(0.3, 1.0))
    inp = W.greedy_inputs(B, k, V, dt, 200 + case, target_sigma=float(g.uniform(1.0, 4.0)), match_p=match_p)
    label = f"case {case}: B{B} k{k} V{V} {W.DTYPE_NAMES[dt]} match {match_p:.2f}"
    print(f"[random shapes] greedy {label}", flush=True)
    got = run_greedy(svl, inp)
    ref = orc.verify_greedy(inp)
    assert (got["accepted_len"] == ref["accepted_len"]).all(), label
    assert (got["emitted"] == ref["emitted"]).all(), label


def _tree(g, max_nodes: int):
    """A random parent array: branching and depth bounds, then a node count
    that fits them."""
    branch = int(g.integers(1, 7))
    depth = int(g.integers(1, 13))
    cap = sum(branch ** d for d in range(depth + 1))
    N = int(g.integers(1, min(max_nodes, cap) + 1))
    return W.random_tree(N, int(g.integers(0, 2 ** 31)), branch, depth), depth


TREE_CASES = list(range(24))


@pytest.mark.parametrize("case", TREE_CASES)
def test_random_greedy_tree_shapes(svl, orc, case):
    g = np.random.Generator(np.random.Philox(key=[2025, case]))
    parent, depth = _tree(g, 256)
    N = parent.size
    V = int(np.exp(g.uniform(np.log(2.0), np.log(150000.0))))
    dt = W.BF16 if g.random() < 0.5 else W.F32
    B = max(1, min(int(g.integers(1, 65)), MAX_ELEMENTS // (N * V)))
    inp = W.tree_inputs(B, N, V, dt, 300 + case, target_sigma=float(g.uniform(1.0, 4.0)), max_depth=depth,
                        match_p=float(g.uniform(0.3, 1.0)), parent=parent, distinct_siblings=bool(g.random() < 0.5))
    label = f"case {case}: B{B} N{N} depth {inp['max_depth']} V{V} {W.DTYPE_NAMES[dt]}"
    print(f"[random shapes] tree {label}", flush=True)
    got = run_tree(svl, inp)
    ref = orc.verify_tree(inp)
    for key in ("accepted_len", "emitted", "accepted_nodes"):
        np.testing.assert_array_equal(got[key], ref[key], err_msg=f"{label}: {key}")


SAMPLED_TREE_CASES = list(range(24))


@pytest.mark.parametrize("case", SAMPLED_TREE_CASES)
def test_random_sampled_tree_shapes(svl, orc, case):
    g = np.random.Generator(np.random.Philox(key=[2026, case]))
    parent, depth = _tree(g, 128)
    N = parent.size
    V = int(np.exp(g.uniform(np.log(2.0), np.log(150000.0))))
    dt = W.BF16 if g.random() < 0.5 else W.F32
    B = max(1, min(int(g.integers(1, 33)), MAX_ELEMENTS // (2 * N * V)))
    T = g.uniform(0.2, 1.6, size=B).astype(np.float32)
    T[g.random(B) < 0.2] = 0.0
    sigma = float(np.exp(g.uniform(np.log(0.02), np.log(3.0))))
    inp = W.sampled_tree_inputs(B, N, V, dt, 400 + case, target_sigma=float(g.uniform(1.0, 4.0)),
                                zipf_s=1.1 if g.random() < 0.5 else None, draft_sigma=sigma, temperature=T,
                                max_depth=depth, parent=parent)
    label = f"case {case}: B{B} N{N} depth {inp['max_depth']} V{V} {W.DTYPE_NAMES[dt]} sigma {sigma:.3g}"
    print(f"[random shapes] sampled tree {label}", flush=True)
    got = run_tree_sampled(svl, inp)
    ref = orc.verify_tree_sampled(inp)
    stats = compare_tree_sampled(got, ref, label)
    print(f"[random shapes] sampled tree {label}: {stats}", flush=True)
