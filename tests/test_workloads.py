"""The seeded input generators (CPU only): the structure the workloads state.

The generators hold none of the verification arithmetic; these checks cover
the properties that the parity and bench inputs rely on.
"""
import numpy as np
import pytest

import workloads as W


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_eagle_tree_distinct_siblings_carry_distinct_tokens(seed):
    inp = W.make_inputs("eagle_tree_distinct", seed, B=4, V=3000)
    par = inp["parent"]
    for b in range(inp["B"]):
        for n in range(inp["N"]):
            kids = np.flatnonzero(par[1:] == n) + 1
            toks = inp["node_tokens"][b, kids]
            assert len(set(toks.tolist())) == len(toks), (seed, b, n, toks)


def test_tree_parent_array_is_topological_and_within_depth():
    inp = W.make_inputs("eagle_tree", 5, B=2, V=500)
    par = inp["parent"]
    assert all(0 <= par[i] < i for i in range(1, inp["N"]))
    depth = np.zeros(inp["N"], int)
    for i in range(1, inp["N"]):
        depth[i] = depth[par[i]] + 1
    assert depth.max() <= inp["max_depth"]


def test_tree_match_rate_follows_match_p():
    # a child of the EAGLE-style workload carries its parent row's first argmax
    # with probability match_p, independently of its siblings
    inp = W.make_inputs("eagle_tree", 7, B=64, V=400)
    vals = W.values(inp["target_logits"], inp["dtype"])
    top = np.argmax(vals, axis=-1)
    par = inp["parent"]
    hit = (inp["node_tokens"][:, 1:] == top[:, par[1:]]).mean()
    assert abs(hit - 0.6) < 0.03, hit


@pytest.mark.parametrize("name", sorted(W.WORKLOADS))
def test_named_workloads_have_their_stated_shapes(name):
    c = W.WORKLOADS[name]
    small = dict(B=2, V=700)
    inp = W.make_inputs(name, 1, **small)
    assert inp["kind"] == c["kind"] and inp["B"] == 2 and inp["V"] == 700
    if c["kind"] in ("chain", "greedy"):
        k = c["k"]
        assert inp["target_logits"].shape == (2, k + 1, 700)
        assert inp["draft_tokens"].shape == (2, k)
    else:
        N = c["N"]
        assert inp["target_logits"].shape == (2, N, 700)
        assert inp["node_tokens"].shape == (2, N)


@pytest.mark.parametrize("dt,kw", [(W.F32, dict(draft_sigma=2e-3, offset=(-4.0, 4.0))), (W.BF16, dict(density=0.3))],
                         ids=["f32", "bf16"])
def test_near_copy_chain_forces_one_rejection_with_a_small_residual(orc, dt, kw):
    """The near-copy chain generator: every sequence rejects exactly at its
    reject_at (the oracle decides), its residual has small mass, and the bf16
    draft rows differ from the target rows by one bf16 unit on about the
    stated fraction of entries."""
    inp = W.near_copy_chain_inputs(12, 3, 3000, dt, seed=5, **kw)
    ref = orc.verify_chain(inp)
    np.testing.assert_array_equal(ref["accepted_len"], inp["reject_at"])
    assert ref["final_mass"].max() < 0.05
    if dt == W.BF16:
        t = inp["target_logits"][:, :3].astype(np.int32)
        d = inp["draft_logits"].astype(np.int32)
        moved = t != d
        assert abs(moved.mean() - 0.3) < 0.02
        assert np.abs(t - d)[moved].max() == 1  # one unit of the bf16 bit pattern


def test_near_copy_tree_walks_take_their_three_paths(orc):
    """The near-copy tree generator forces the oracle's walk into the path of
    its mode b % 3: all three root children rejected; node 1 kept and its
    children rejected; node 1 rejected, node 2 kept and its child rejected."""
    inp = W.near_copy_tree_inputs(9, 3000, W.F32, seed=6, draft_sigma=2e-3)
    ref = orc.verify_tree_sampled(inp)
    want = {0: [-1, -1, -1], 1: [1, -1, -1], 2: [2, -1, -1]}
    for b in range(inp["B"]):
        assert ref["accepted_nodes"][b].tolist() == want[b % 3], b
    assert ref["final_mass"].max() < 0.05


@pytest.mark.parametrize("dt", [W.F32, W.BF16], ids=["f32", "bf16"])
def test_flat_tail_chain_has_its_stated_mass_profile(orc, dt):
    """The flat-tail chain generator: every sequence rejects its one draft,
    the residual's mass is about 0.22, the two vocabulary halves' masses
    differ by more than 0.2 (a coarse lower bound of W), the tail holds over
    90% of p, and under p the tokens lie on average about 8 binary orders
    below the top one."""
    V = 128256
    inp = W.flat_tail_chain_inputs(4, V, dt, seed=5)
    ref = orc.verify_chain(inp)
    assert (ref["accepted_len"] == 0).all()
    assert ((ref["final_mass"] > 0.205) & (ref["final_mass"] < 0.24)).all()
    t = W.values(inp["target_logits"][:, 0], dt).astype(np.float64)
    d = W.values(inp["draft_logits"][:, 0], dt).astype(np.float64)
    p = np.exp(t - t.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    q = np.exp(d - d.max(1, keepdims=True))
    q /= q.sum(1, keepdims=True)
    halves = np.abs(p[:, :V // 2].sum(1) - q[:, :V // 2].sum(1))
    assert ((halves > 0.2) & (halves <= ref["final_mass"] + 1e-12)).all()
    assert (p[:, 0] < 0.1).all()
    depth = (p * np.log2(p.max(1, keepdims=True) / p)).sum(1)
    assert ((depth > 7) & (depth < 10)).all()
