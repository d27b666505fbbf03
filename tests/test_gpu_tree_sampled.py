"""Parity of sampled tree verification (sv_verify_tree_sampled, through the C
ABI) with the fp64 CPU oracle.

accepted_len, emitted and accepted_nodes must match bit-exactly, except for
sequences the oracle flags as lying within 1e-5 of an acceptance threshold or
CDF boundary (counted and reported).  Rule: multi-step speculative sampling
(SpecInfer, Miao et al. 2023), the rule the EAGLE work uses for sampled
trees; the pages' section "EAGLE" keeps the longest path that passes.
"""

import json
import os

import numpy as np
import pytest

import workloads as W
from gpu_common import compare_tree_sampled, run_tree_sampled

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def svl():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import draft_token_verification_chain_amd as svl

    svl.load()
    return svl


def _record(label, stats):
    path = os.environ.get("SV_PARITY_LOG")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps(dict(kind="tree_sampled", case=label, **stats)) + "\n")
    print(f"[parity] tree_sampled {label} {stats}", flush=True)


def _check(svl, orc, inp, label):
    print(f"[case] {label}", flush=True)
    got = run_tree_sampled(svl, inp)
    ref = orc.verify_tree_sampled(inp)
    _record(label, compare_tree_sampled(got, ref, label))
    return got, ref


SHAPES = [
    # B, N, V, dtype, temperature (None: mixed, a quarter of the rows at 0)
    (8, 20, 3001, W.F32, 0.8),
    (6, 64, 5000, W.BF16, 0.7),
    (5, 33, 4097, W.BF16, None),
    (3, 100, 1000, W.F32, 1.2),
    (4, 24, 10000, W.BF16, 0.8),     # three tiles per row: an odd count, the last wave's second tile absent
    (4, 1, 2000, W.BF16, 0.9),       # the root alone: a plain draw from its target row
    (3, 64, 128257, W.BF16, 0.6),    # odd V: element loads, many segments
    (2, 40, 65536, W.F32, 0.5),
]


def _temps(B, T, seed):
    if T is not None:
        return T
    t = np.random.default_rng(seed).uniform(0.3, 1.3, B).astype(np.float32)
    t[::4] = 0.0
    return t


@pytest.mark.parametrize("seed", [1, 2, 3])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"B{s[0]}N{s[1]}V{s[2]}{W.DTYPE_NAMES[s[3]]}")
def test_small_shapes(svl, orc, shape, seed):
    B, N, V, dt, T = shape
    inp = W.sampled_tree_inputs(B, N, V, dt, seed, temperature=_temps(B, T, seed), draft_sigma=(0.3, 2.5))
    _check(svl, orc, inp, f"B{B}N{N}V{V}dt{dt}s{seed}")


# Batches on both sides of the normaliser cache's bound.  With P workgroups
# per sequence (about 1024 / B, at most a quarter of the segments), round 0
# combines every node's normalisers when N <= 4 P, one node per wave; above
# that every entry into a node combines its partials.
BATCHES = [
    (128, 24, 8200, W.F32),   # P = 8: cached, three nodes per workgroup
    (300, 16, 5000, W.F32),   # P = 4: N = 4 P exactly, one node on every wave
    (200, 24, 6000, W.BF16),  # P = 3: not cached
    (1100, 8, 600, W.BF16),   # P = 1 (one workgroup per sequence and round): not cached
    (1500, 3, 1000, W.F32),   # P = 1, cached (three nodes on three waves)
]


@pytest.mark.parametrize("shape", BATCHES, ids=lambda s: f"B{s[0]}N{s[1]}V{s[2]}{W.DTYPE_NAMES[s[3]]}")
def test_batch_sizes_around_the_normaliser_cache(svl, orc, shape):
    B, N, V, dt = shape
    inp = W.sampled_tree_inputs(B, N, V, dt, 11, temperature=_temps(B, None, 11), draft_sigma=(0.3, 2.5))
    _check(svl, orc, inp, f"batch B{B}N{N}V{V}dt{dt}")


@pytest.mark.parametrize("seed", [1, 2])
def test_full_sampled_tree_workload(svl, orc, seed):
    inp = W.make_inputs("sampled_tree", seed)
    got, ref = _check(svl, orc, inp, f"sampled_tree s{seed}")
    assert (got["accepted_len"] >= 0).all()


def test_linear_deep_and_wide_star_trees(svl, orc):
    """A chain-shaped tree of depth 63 and a one-level tree of 300 children
    (up to 300 sequential rejections at the root)."""
    lin = np.arange(-1, 63, dtype=np.int32)
    inp = W.sampled_tree_inputs(4, 64, 3000, W.BF16, 4, parent=lin, max_depth=63, draft_sigma=0.3)
    _check(svl, orc, inp, "linear64")
    star = np.zeros(301, dtype=np.int32)
    star[0] = -1
    inp = W.sampled_tree_inputs(3, 301, 2000, W.F32, 5, parent=star, max_depth=1, draft_sigma=3.0)
    _check(svl, orc, inp, "star300")


def test_max_nodes(svl, orc):
    inp = W.sampled_tree_inputs(2, 1024, 600, W.BF16, 6, max_branch=8, max_depth=12, draft_sigma=(0.5, 2.0))
    _check(svl, orc, inp, "N1024")


def test_identical_rows_keep_first_children(svl, orc):
    inp = W.sampled_tree_inputs(6, 48, 4000, W.BF16, 7)
    inp["draft_logits"] = inp["target_logits"].copy()
    got, ref = _check(svl, orc, inp, "identical")
    assert (got["accepted_len"] == ref["accepted_len"]).all()


def test_per_sequence_parents_and_invalid_trees(svl, orc):
    inp = W.sampled_tree_inputs(4, 24, 1500, W.F32, 8)
    par = np.stack([W.random_tree(24, s) for s in (11, 12, 13, 14)]).astype(np.int32)
    par[2, 9] = 15  # a parent after its child: sequence 2 is invalid
    inp["parent"] = par
    inp["max_depth"] = 23
    got, ref = _check(svl, orc, inp, "per-sequence")
    assert got["accepted_len"][2] == -1 and (got["emitted"][2] == -1).all()
    inp["max_depth"] = 1  # now deeper nodes make every sequence with depth > 1 invalid
    _check(svl, orc, inp, "too-deep")


def test_determinism(svl, orc):
    inp = W.sampled_tree_inputs(6, 64, 20000, W.BF16, 9)
    a = run_tree_sampled(svl, inp)
    for _ in range(3):
        b = run_tree_sampled(svl, inp)
        for k in a:
            np.testing.assert_array_equal(a[k], b[k])


def test_gpu_sampled_tree_distribution_chi_square(svl, orc):
    """The chi-square of the oracle's pin, through the GPU: 5 * 10^5 trials on
    the two-level tree (V = 8); each emitted token follows the target row of
    the token before it."""
    from scipy import special, stats

    rng = np.random.default_rng(4242)
    V = 8
    root_t = (1.5 * rng.standard_normal(V)).astype(np.float32)
    root_d = (root_t + rng.standard_normal(V)).astype(np.float32)
    F = (1.5 * rng.standard_normal((V, V))).astype(np.float32)
    G = (F + rng.standard_normal((V, V))).astype(np.float32)
    H = (1.5 * rng.standard_normal((V, V))).astype(np.float32)
    acc, em = [], []
    for blk in range(2):
        inp = W.sampled_tree_trials(root_t, root_d, F, G, H, 1.0, 250_000, seed=93, block=blk)
        r = run_tree_sampled(svl, inp)
        if blk == 0:  # element by element too: every trial sequence of the first block
            _record("chi-square trials", compare_tree_sampled(r, orc.verify_tree_sampled(inp), "trials"))
        acc.append(r["accepted_len"])
        em.append(r["emitted"])
    acc, em = np.concatenate(acc), np.concatenate(em)
    sm = lambda x: special.softmax(np.asarray(x, np.float64), axis=-1)  # noqa: E731
    pv = [stats.chisquare(np.bincount(em[:, 0], minlength=V), sm(root_t) * len(acc)).pvalue]
    for j, table in ((1, F), (2, H)):
        sel = acc >= j
        obs = np.bincount(em[sel, j - 1] * V + em[sel, j], minlength=V * V).reshape(V, V)
        n_prev = obs.sum(axis=1)
        keep = n_prev > 0
        exp = n_prev[:, None] * sm(table)
        pv.append(stats.chisquare(obs[keep].ravel(), exp[keep].ravel(), ddof=int(keep.sum()) - 1).pvalue)
    print(f"[chi2] sampled tree p-values {pv}", flush=True)
    assert min(pv) > 1e-4, pv


def test_hand_derived_golden_examples_on_gpu(svl):
    """The hand-derived examples of tests/golden, through the GPU (chain and
    sampled tree): the GPU reproduces the values derived by hand."""
    from gpu_common import run_chain

    here = os.path.join(os.path.dirname(__file__), "golden")
    g = json.load(open(os.path.join(here, "tree_sampled_v3_hand.json")))
    cases, B, N, V = g["cases"], len(g["cases"]), g["N"], g["V"]
    lg = lambda key: np.log(np.array([c[key] for c in cases], np.float64)).astype(np.float32)  # noqa: E731
    inp = dict(B=B, N=N, V=V, dtype=W.F32, node_tokens=np.array([c["node_tokens"] for c in cases], np.int32),
               parent=np.array([c["parent"] for c in cases], np.int32), max_depth=g["max_depth"],
               target_logits=lg("target_probs"), draft_logits=lg("draft_probs"),
               temperature=np.full(B, g["temperature"], np.float32),
               uniforms=np.array([c["uniforms"] for c in cases], np.float32))
    got = run_tree_sampled(svl, inp)
    for i, c in enumerate(cases):
        assert got["accepted_len"][i] == c["accepted_len"], c["why"]
        assert got["emitted"][i].tolist() == c["emitted"], c["why"]
        assert got["accepted_nodes"][i].tolist() == c["accepted_nodes"], c["why"]
    g = json.load(open(os.path.join(here, "chain_v4_hand.json")))
    cases, B, k, V = g["cases"], len(g["cases"]), g["k"], g["V"]
    t = np.log(np.array(g["target_probs"], np.float64)).astype(np.float32)
    d = np.log(np.array(g["draft_probs"], np.float64)).astype(np.float32)
    inp = dict(B=B, k=k, V=V, dtype=W.F32, draft_tokens=np.array([c["draft_tokens"] for c in cases], np.int32),
               draft_logits=np.broadcast_to(d, (B, k, V)).copy(),
               target_logits=np.broadcast_to(t, (B, k + 1, V)).copy(),
               temperature=np.full(B, g["temperature"], np.float32),
               uniforms=np.array([c["uniforms"] for c in cases], np.float32))
    got = run_chain(svl, inp)
    for i, c in enumerate(cases):
        assert got["accepted_len"][i] == c["accepted_len"], c["why"]
        assert got["emitted"][i].tolist() == c["emitted"], c["why"]
        np.testing.assert_allclose(got["accept_prob"][i], c["accept_prob"], atol=1e-6, err_msg=c["why"])


@pytest.mark.parametrize("kids", [5, 6, 7, 12])
def test_walks_ending_around_the_last_round(svl, orc, kids):
    """A root whose `kids` children all carry tokens the target row gives
    almost no mass: every child is rejected, so the walk needs `kids` passes
    over the root's rows and then the final draw.  With seven rounds the
    draw then falls in the last round (5), in the finisher from the masses
    the last round wrote (6), or the finisher forms the pending pass from the
    last round's state and goes on from there (7, 12)."""
    B, V = 8, 3000
    star = np.full(kids + 1, 0, dtype=np.int32)
    star[0] = -1
    inp = W.sampled_tree_inputs(B, kids + 1, V, W.F32, 40 + kids, parent=star, max_depth=1, draft_sigma=0.5)
    for b in range(B):
        toks = inp["node_tokens"][b, 1:]
        inp["target_logits"][b, 0, toks] = -30.0  # p(x) ~ 1e-13 relative: certain rejection
        inp["draft_logits"][b, 0, toks] = 8.0
    got, ref = _check(svl, orc, inp, f"star{kids}")
    assert (ref["accepted_len"] == 0).all()  # the oracle rejected every child


# Trees whose walks are fixed by their logits: at every inner node the first
# R children carry tokens the node's target row gives almost no mass and its
# draft row much (certain rejections, each one pass), and the next child a
# token the target row favours and the draft row does not (certainly kept,
# whatever the residual).  parent, rejections per level, whether the last kept
# node has children (all rejected), and the state the seven rounds leave.
RESUME_CASES = [
    ([-1, 0, 0, 0, 0, 0, 0, 0], [6], "leaf: entered in the last round"),
    ([-1, 0, 0, 0, 0, 0, 0, 0, 7, 7], [6, 2], "first pass (c = 1) at depth 1 pending"),
    ([-1, 0, 0, 0, 0, 0, 5, 5, 5, 5], [4, 4], "third pass at depth 1 pending, one more child"),
    ([-1, 0, 0, 0, 0, 4, 4, 4, 4, 8, 8, 8, 8], [3, 3, 3], "three levels, walk ends at a leaf"),
    ([-1, 0, 0, 0, 3, 3, 3, 3, 3, 3, 3, 3, 3], [2, 8], "eight passes at depth 1, four in the finisher, a leaf"),
]


@pytest.mark.parametrize("case", RESUME_CASES, ids=[c[2] for c in RESUME_CASES])
def test_walks_going_on_after_the_rounds(svl, orc, case):
    """Walks longer than the rounds: the finisher goes on from the state the
    last round left (a leaf to enter, a pending pass at c = 1 or later, a
    node's remaining children) and keeps the path the rounds wrote."""
    parent, rejections, label = np.array(case[0], np.int32), case[1], case[2]
    N, V, B = len(parent), 3000, 8
    depth = np.zeros(N, np.int64)
    for i in range(1, N):
        depth[i] = depth[parent[i]] + 1
    for dt in (W.F32, W.BF16):
        inp = W.sampled_tree_inputs(B, N, V, dt, 60 + N, parent=parent, max_depth=int(depth.max()),
                                    draft_sigma=0.5)
        tl, dl = W.values(inp["target_logits"], dt).copy(), W.values(inp["draft_logits"], dt).copy()
        want = []
        for b in range(B):
            path, n, level = [], 0, 0
            while True:
                kids = [i for i in range(1, N) if parent[i] == n]
                if not kids:
                    break
                R = rejections[level] if level < len(rejections) else len(kids)
                toks = 11 + 37 * np.arange(len(kids)) + 5 * b
                inp["node_tokens"][b, kids] = toks
                tl[b, n, toks[:R]], dl[b, n, toks[:R]] = -30.0, 8.0       # certain rejections
                if R < len(kids):
                    tl[b, n, toks[R]], dl[b, n, toks[R]] = 12.0, -30.0    # certainly kept
                    path.append(kids[R])
                    n, level = kids[R], level + 1
                else:
                    break
            want.append(path)
        inp["target_logits"], inp["draft_logits"] = W.to_dtype(tl, dt), W.to_dtype(dl, dt)
        got, ref = _check(svl, orc, inp, f"resume {label} dt{dt}")
        for b in range(B):
            assert ref["accepted_nodes"][b][:len(want[b])].tolist() == want[b]
            assert ref["accepted_len"][b] == len(want[b])


@pytest.mark.parametrize("V", [1, 2, 9, 64, 257, 512, 2049, 4096])
def test_vocabulary_sizes_at_segment_edges(svl, orc, V):
    for dt in (W.BF16, W.F32):
        inp = W.sampled_tree_inputs(4, 9, V, dt, V, temperature=_temps(4, None, V), draft_sigma=(0.3, 2.0))
        _check(svl, orc, inp, f"edge V{V} dt{dt}")


@pytest.mark.parametrize("case", [(5000.0, 0.7, W.BF16), (-1.0e5, 1.0, W.F32), (0.0, 0.05, W.F32), (0.0, 100.0, W.BF16)],
                         ids=lambda c: f"off{c[0]:g}-T{c[1]:g}-{W.DTYPE_NAMES[c[2]]}")
def test_logits_at_the_edges_of_the_declared_range(svl, orc, case):
    """Large common offsets and extreme temperatures, inside the header's
    preconditions (|l| / T < 10^6, |l_v - max l| / T < 700)."""
    offset, T, dt = case
    inp = W.sampled_tree_inputs(8, 24, 5000, dt, 33, target_sigma=1.0 if T < 0.1 else 3.0, zipf_s=None,
                                draft_sigma=(0.2, 1.5), temperature=np.float32(T))
    for key in ("target_logits", "draft_logits"):
        inp[key] = W.to_dtype(W.values(inp[key], dt) + np.float32(offset), dt)
    _check(svl, orc, inp, f"extreme off{offset:g} T{T:g} dt{dt}")
