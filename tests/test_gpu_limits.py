"""GPU parity at the limits the C ABI declares (include/specverify.h):
SV_MAX_VOCAB = 2^20 tokens, SV_MAX_DRAFTS = 64 drafts, SV_MAX_TREE_NODES =
1024 nodes, and batches far larger than the benchmark's.  Same bar as the
other parity tests: bit-exact outside the oracle's 1e-5 band, accept_prob
within 1e-5.
"""

import json
import os

import numpy as np
import pytest

import workloads as W
from gpu_common import compare_chain, compare_tree_sampled, run_chain, run_greedy, run_tree, run_tree_sampled

pytestmark = pytest.mark.gpu

VMAX = 1 << 20


@pytest.fixture(scope="module")
def svl():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import draft_token_verification_chain_amd as svl

    svl.load()
    return svl


def _record(kind, label, stats):
    path = os.environ.get("SV_PARITY_LOG")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps(dict(kind=kind, case=label, **stats)) + "\n")
    print(f"[parity] {kind} {label} {stats}", flush=True)


def _chain(svl, orc, inp, label):
    print(f"[case] {label}", flush=True)
    got = run_chain(svl, inp)
    ref = orc.verify_chain(inp)
    _record("chain", label, compare_chain(inp, got, ref, label))
    return got, ref


@pytest.mark.parametrize("V", [VMAX, VMAX - 3], ids=["Vmax", "Vmax-3"])
@pytest.mark.parametrize("dt", [W.BF16, W.F32], ids=["bf16", "f32"])
def test_chain_at_max_vocabulary(svl, orc, dt, V):
    temps = np.array([0.7, 1.3, 0.0], np.float32)
    inp = W.chain_inputs(3, 3, V, dt, 21, target_sigma=3.0, zipf_s=1.1, draft_sigma=(0.3, 2.0), temperature=temps)
    _chain(svl, orc, inp, f"V{V}dt{dt}")


def test_chain_with_max_drafts_at_full_vocabulary(svl, orc):
    """k = 64 at V = 128256: a near-copy draft keeps long prefixes, so the
    acceptance ballot and the draw run over all 64 positions."""
    inp = W.chain_inputs(2, 64, 128256, W.BF16, 22, target_sigma=3.0, zipf_s=1.1, draft_sigma=0.05,
                         temperature=np.array([0.7, 1.0], np.float32))
    got, ref = _chain(svl, orc, inp, "k64")
    assert ref["accepted_len"].max() > 8  # long prefixes were exercised


def test_chain_with_max_drafts_mixed(svl, orc):
    inp = W.chain_inputs(6, 64, 3001, W.F32, 23, target_sigma=2.0, draft_sigma=(0.02, 1.5),
                         temperature=np.array([0.5, 0.0, 1.0, 0.8, 0.0, 1.2], np.float32))
    _chain(svl, orc, inp, "k64-mixed")


@pytest.mark.parametrize("k", [0, 1, 4])
def test_chain_very_large_batch(svl, orc, k):
    """Tens of thousands of sequences: the once-per-sequence acceptance kernel
    and grids far beyond one round of resident workgroups."""
    B = 20000 if k else 60000
    temps = np.random.default_rng(24).uniform(0.3, 1.3, B).astype(np.float32)
    temps[::7] = 0.0
    inp = W.chain_inputs(B, k, 515, W.F32, 24 + k, target_sigma=2.0, draft_sigma=(0.2, 2.0), temperature=temps)
    _chain(svl, orc, inp, f"B{B}k{k}")


@pytest.mark.parametrize("dt", [W.BF16, W.F32], ids=["bf16", "f32"])
def test_greedy_at_max_vocabulary(svl, orc, dt):
    inp = W.greedy_inputs(4, 5, VMAX, dt, 25)
    got, ref = run_greedy(svl, inp), orc.verify_greedy(inp)
    np.testing.assert_array_equal(got["accepted_len"], ref["accepted_len"])
    np.testing.assert_array_equal(got["emitted"], ref["emitted"])


def test_greedy_with_max_drafts(svl, orc):
    inp = W.greedy_inputs(8, 64, 20000, W.BF16, 26, match_p=0.97)
    got, ref = run_greedy(svl, inp), orc.verify_greedy(inp)
    np.testing.assert_array_equal(got["accepted_len"], ref["accepted_len"])
    np.testing.assert_array_equal(got["emitted"], ref["emitted"])
    assert ref["accepted_len"].max() > 16


def test_tree_with_max_nodes(svl, orc):
    parent = W.random_tree(1024, 27, max_branch=8, max_depth=12)
    inp = W.tree_inputs(2, 1024, 32768, W.BF16, 27, parent=parent, max_depth=12, match_p=0.9)
    got, ref = run_tree(svl, inp), orc.verify_tree(inp)
    for key in ("accepted_len", "emitted", "accepted_nodes"):
        np.testing.assert_array_equal(got[key], ref[key])


def test_tree_three_phases_with_max_nodes(svl, orc):
    """1024 nodes and 256 MiB of rows: root rows, depths 1-2 below an accepted
    depth-1 node, then deeper nodes below an accepted depth-3 node."""
    parent = W.random_tree(1024, 28, max_branch=8, max_depth=12)
    inp = W.tree_inputs(4, 1024, 32768, W.BF16, 28, parent=parent, max_depth=12, match_p=0.9)
    assert 4 * 1024 * 32768 * 2 >= 192 << 20
    got, ref = run_tree(svl, inp), orc.verify_tree(inp)
    for key in ("accepted_len", "emitted", "accepted_nodes"):
        np.testing.assert_array_equal(got[key], ref[key])
    assert ref["accepted_len"].max() >= 4


def test_greedy_two_phases_at_max_vocabulary(svl, orc):
    inp = W.greedy_inputs(24, 5, VMAX, W.BF16, 29)
    assert 24 * 6 * VMAX * 2 >= 256 << 20
    got, ref = run_greedy(svl, inp), orc.verify_greedy(inp)
    np.testing.assert_array_equal(got["accepted_len"], ref["accepted_len"])
    np.testing.assert_array_equal(got["emitted"], ref["emitted"])


def test_chain_two_phases_at_max_vocabulary(svl, orc):
    """Without accept_prob: positions 0-1, then 2-7 for sequences accepting both."""
    inp = W.chain_inputs(4, 8, VMAX, W.F32, 30, target_sigma=3.0, zipf_s=1.1, draft_sigma=[0.02, 3.0, 0.02, 3.0])
    assert 2 * 4 * 8 * VMAX * 4 >= 128 << 20
    print("[case] chain two phases at V = 2^20", flush=True)
    got = run_chain(svl, inp, accept_prob=False)
    ref = orc.verify_chain(inp)
    _record("chain", "two phases at V = 2^20", compare_chain(inp, got, ref, "two phases at V = 2^20"))


def test_sampled_tree_at_max_vocabulary(svl, orc):
    inp = W.sampled_tree_inputs(2, 16, VMAX, W.F32, 28, draft_sigma=(0.5, 2.0))
    print("[case] sampled tree Vmax", flush=True)
    got, ref = run_tree_sampled(svl, inp), orc.verify_tree_sampled(inp)
    _record("tree_sampled", "Vmax", compare_tree_sampled(got, ref, "Vmax"))
