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
