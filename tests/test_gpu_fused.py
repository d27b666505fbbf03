"""The one-launch chain path: rows streamed and the final draw made in one
launch (chain_fused_kernel), its drawing workgroups reading the row
statistics that its streaming workgroups publish, tagged for the call (a
graph being captured clears the slots first, clear_slots_kernel).

Checked here: which calls take it (the draw fits one round of 2048
workgroups, the 2k rows' partials fit one wave: 2k <= 64 and at most 8
partials per lane), parity with the oracle on both sides of each bound, and
that the drawing workgroups give bit-identical outputs, accept_prob
included, when they read no published statistic and compute them all
themselves (sv_set_handoff_polls(0)), the path a wait that outlasted its
bound would take.
"""

import numpy as np
import pytest

import workloads as W
from gpu_common import chain_tensors, compare_chain, run_chain, run_greedy, run_tree

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def svl():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import draft_token_verification_chain_amd as svl

    svl.load()
    return svl


def _inputs(B, k, V, dt, seed):
    """Mixed temperatures; every other temperature-0 sequence drafts the
    target's argmax at every position, so that it accepts all its drafts and
    its final token is the bonus row's argmax (the chunks' argmax records)."""
    T = np.where(np.arange(B) % 7 == 3, 0.0, 0.8).astype(np.float32)
    inp = W.chain_inputs(B, k, V, dt, seed, target_sigma=3.0, zipf_s=1.1, draft_sigma=(0.05, 2.0), temperature=T)
    for b in range(3, B, 14):
        inp["draft_tokens"][b] = np.argmax(W.values(inp["target_logits"][b, :k], dt), axis=1)
    return inp


FUSED_PATH = [
    # B, k, V, dtype, expect the one-launch path
    (8, 4, 128256, W.BF16, True),     # the Llama-scale row shape
    (2, 4, 131072, W.F32, True),      # 64 tiles per row: 8 partials per lane of 8
    (2, 4, 131073, W.F32, False),     # 65 tiles
    (2, 32, 16384, W.F32, True),      # 64 rows, one lane each, 8 tiles per row
    (2, 33, 1024, W.F32, False),      # 66 rows
    (2048, 1, 4096, W.F32, True),     # 2048 draw workgroups
    (2049, 1, 4096, W.F32, False),    # 2049: the acceptance kernel instead
    (16, 4, 8192, W.BF16, False),     # the one-workgroup-per-sequence path
]


@pytest.mark.parametrize("shape", FUSED_PATH, ids=lambda s: f"B{s[0]}k{s[1]}V{s[2]}{W.DTYPE_NAMES[s[3]]}")
def test_fused_path_and_its_bounds(svl, orc, shape):
    B, k, V, dt, fused = shape
    inp = _inputs(B, k, V, dt, 21)
    label = f"fused path B{B} k{k} V{V} {W.DTYPE_NAMES[dt]}"
    print(f"[fused] {label}", flush=True)
    svl.profile_begin(64)
    got = run_chain(svl, inp)
    launched = set(svl.profile_end())
    stats = compare_chain(inp, got, orc.verify_chain(inp), label)
    print(f"[fused] {label}: {stats} {sorted(launched)}", flush=True)
    assert ("chain_fused" in launched) == fused, launched
    if fused:
        assert launched == {"chain_fused", "chain_final_pick"}, launched  # eager: no clearing launch


COMPUTED = [
    # B, k, V, dtype -- ragged tails, the element-load path, one row per lane,
    # temperature 0 mixed in
    (8, 4, 128256, W.BF16),
    (5, 3, 50001, W.F32),
    (3, 1, 262144, W.BF16),
    (2, 32, 3000, W.BF16),
    (64, 2, 9000, W.F32),
]


@pytest.mark.parametrize("shape", COMPUTED, ids=lambda s: f"B{s[0]}k{s[1]}V{s[2]}{W.DTYPE_NAMES[s[3]]}")
def test_fused_draw_computing_every_statistic_itself(svl, orc, shape):
    B, k, V, dt = shape
    inp = _inputs(B, k, V, dt, 22)
    label = f"computed statistics B{B} k{k} V{V} {W.DTYPE_NAMES[dt]}"
    print(f"[fused] {label}", flush=True)
    svl.profile_begin(64)
    read = run_chain(svl, inp)
    assert "chain_fused" in set(svl.profile_end())
    prev = svl.set_handoff_polls(0)
    try:
        computed = run_chain(svl, inp)
    finally:
        svl.set_handoff_polls(prev)
    for key in ("accepted_len", "emitted"):
        np.testing.assert_array_equal(computed[key], read[key], err_msg=f"{label}: {key}")
    assert computed["accept_prob"].tobytes() == read["accept_prob"].tobytes(), label
    stats = compare_chain(inp, computed, orc.verify_chain(inp), label)
    print(f"[fused] {label}: {stats}", flush=True)


def _np(out):
    return {key: (v.cpu().numpy() if v is not None else None) for key, v in out.items()}


def _same(a, b, label):
    for key in ("accepted_len", "emitted"):
        np.testing.assert_array_equal(a[key], b[key], err_msg=f"{label}: {key}")
    assert a["accept_prob"].tobytes() == b["accept_prob"].tobytes(), label


def test_fused_workspace_reuse_garbage_and_graphs(svl, orc):
    """One workspace, filled with random bytes first, through eager calls on
    different inputs (each call's slots carry its own tag, so what earlier
    calls or the random bytes left is never read as this call's) and through
    the replays of a graph captured on it (whose one tag is cleared before
    every replay), with eager calls on the same workspace in between: every
    result matches the oracle, and the same inputs give the same bits."""
    import torch

    B, k, V, dt = 24, 4, 50048, W.BF16
    sets = [_inputs(B, k, V, dt, s) for s in (31, 32, 33)]
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)
    ws = torch.randint(0, 256, (svl.chain_workspace_bytes(B, k, V, dt),), dtype=torch.uint8, device="cuda",
                       generator=gen)

    def eager(inp):
        t = chain_tensors(inp)
        o = svl.verify_chain(t["draft_tokens"], t["draft_logits"], t["target_logits"], t["temperature"],
                             t["uniforms"], workspace=ws)
        torch.cuda.synchronize()
        return _np(o)

    svl.profile_begin(64)
    first = [eager(inp) for inp in sets]
    assert "chain_fused" in set(svl.profile_end())
    for i, (inp, got) in enumerate(zip(sets, first)):
        compare_chain(inp, got, orc.verify_chain(inp), f"reused workspace, call {i}")
    _same(eager(sets[0]), first[0], "the first inputs again")

    static = chain_tensors(sets[0])
    out = dict(accepted_len=torch.empty(B, dtype=torch.int32, device="cuda"),
               emitted=torch.empty((B, k + 1), dtype=torch.int32, device="cuda"),
               accept_prob=torch.empty((B, k), dtype=torch.float32, device="cuda"))

    def step():
        svl.verify_chain(static["draft_tokens"], static["draft_logits"], static["target_logits"],
                         static["temperature"], static["uniforms"], workspace=ws, out=out)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep, i in enumerate((1, 2, 0, 0, 2)):
        fresh = chain_tensors(sets[i])
        for key in static:
            static[key].copy_(fresh[key])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _same(_np(out), first[i], f"graph replay {rep} (inputs {i})")
        j = (i + 1) % len(sets)
        _same(eager(sets[j]), first[j], f"eager call {rep} between replays (inputs {j})")


GREEDY_FUSED = [
    # B, k, V, dtype, match rate, expect both phases in one launch (rows of >= 256 MiB take two phases)
    (256, 5, 128256, W.BF16, 0.7, True),    # the greedy workload: s = 3, 32 tiles per row
    (64, 4, 262144, W.F32, 0.8, True),      # s = 2: 128 tiles per row, 4 partials per lane of 32
    (40, 15, 211111, W.BF16, 0.9, True),    # s = 8, odd V: element loads
    (16, 15, 300000, W.F32, 0.9, False),    # s = 8: 147 tiles per row, more than one wave holds
]


@pytest.mark.parametrize("shape", GREEDY_FUSED, ids=lambda s: f"B{s[0]}k{s[1]}V{s[2]}{W.DTYPE_NAMES[s[3]]}")
def test_greedy_two_phases_in_one_launch(svl, orc, shape):
    """Two-phase greedy chains run both phases in one launch (greedy_fused)
    when the first phase's partials of a sequence fit one wave; the outputs
    equal the oracle's, and equal themselves bit for bit when the second
    phase's checks compute every first-phase partial themselves."""
    B, k, V, dt, match_p, fused = shape
    inp = W.greedy_inputs(B, k, V, dt, 23, match_p=match_p)
    label = f"greedy B{B} k{k} V{V} {W.DTYPE_NAMES[dt]}"
    print(f"[fused] {label}", flush=True)
    ref = orc.verify_greedy(inp)
    svl.profile_begin(64)
    got = run_greedy(svl, inp)
    launched = set(svl.profile_end())
    print(f"[fused] {label}: {sorted(launched)}, mean accepted {got['accepted_len'].mean():.2f}", flush=True)
    assert launched == ({"greedy_fused", "greedy_finalize"} if fused
                        else {"greedy_rows", "greedy_rows_rest", "greedy_finalize"}), launched
    for key in ("accepted_len", "emitted"):
        np.testing.assert_array_equal(got[key], ref[key], err_msg=f"{label}: {key}")
    if fused:
        prev = svl.set_handoff_polls(0)
        try:
            computed = run_greedy(svl, inp)
        finally:
            svl.set_handoff_polls(prev)
        for key in ("accepted_len", "emitted"):
            np.testing.assert_array_equal(computed[key], ref[key], err_msg=f"{label}: {key}, computed")


TREE_ROOT_PLAN = [
    # B, N, V, dtype, max_depth, distinct siblings, expect the root rows and the first plan in one launch
    (16, 64, 128256, W.BF16, 6, False, True),   # the EAGLE-style workload's shape: three phases
    (16, 64, 128256, W.BF16, 6, True, True),
    (8, 256, 32768, W.F32, 8, False, True),     # 256 nodes, one per thread of the plan's workgroup
    (4, 300, 50000, W.BF16, 8, False, False),   # 300 nodes: tree_root_rows, then tree_plan
    (12, 100, 50001, W.BF16, 5, True, True),    # two phases, odd V: element loads
]


@pytest.mark.parametrize("shape", TREE_ROOT_PLAN,
                         ids=lambda s: f"B{s[0]}N{s[1]}V{s[2]}{W.DTYPE_NAMES[s[3]]}{'d' if s[5] else ''}")
def test_tree_root_rows_and_first_plan_in_one_launch(svl, orc, shape):
    """Greedy trees streamed in phases run the root rows and the first plan
    in one launch (tree_root_plan) up to 256 nodes; the outputs equal the
    oracle's, also when the plan computes the root's partials itself."""
    B, N, V, dt, depth, distinct, merged = shape
    inp = W.tree_inputs(B, N, V, dt, 24, target_sigma=3.0, max_depth=depth, match_p=0.7,
                        distinct_siblings=distinct)
    assert B * N * V * (2 if dt == W.BF16 else 4) >= 96 << 20
    label = f"tree B{B} N{N} V{V} {W.DTYPE_NAMES[dt]}"
    print(f"[fused] {label}", flush=True)
    ref = orc.verify_tree(inp)
    svl.profile_begin(64)
    got = run_tree(svl, inp)
    launched = set(svl.profile_end())
    print(f"[fused] {label}: {sorted(launched)}, mean accepted {got['accepted_len'].mean():.2f}", flush=True)
    assert ("tree_root_plan" in launched) == merged and ("tree_root_rows" in launched) == (not merged), launched
    for key in ("accepted_len", "emitted", "accepted_nodes"):
        np.testing.assert_array_equal(got[key], ref[key], err_msg=f"{label}: {key}")
    if merged:
        prev = svl.set_handoff_polls(0)
        try:
            computed = run_tree(svl, inp)
        finally:
            svl.set_handoff_polls(prev)
        for key in ("accepted_len", "emitted", "accepted_nodes"):
            np.testing.assert_array_equal(computed[key], ref[key], err_msg=f"{label}: {key}, computed")


def test_fused_emitted_distribution_chi_square(svl, orc):
    """The one-launch chain path's draws, bit-exact with the oracle outside
    the band, are distributed as speculative sampling says: 40 calls of 2048
    trials at V = 16, k = 4 (each call takes chain_fused), and the token
    emitted at position j given j accepted drafts follows target row j
    (chi-square)."""
    from scipy import special, stats

    rng = np.random.default_rng(2031)
    t = (1.5 * rng.standard_normal((5, 16))).astype(np.float32)
    d = (t[:4] + rng.standard_normal((4, 16))).astype(np.float32)
    accs, ems = [], []
    for blk in range(40):
        inp = W.repeated_trials(t, d, 1.0, 2048, seed=78, block=blk)
        if blk == 0:
            svl.profile_begin(16)
        got = run_chain(svl, inp)
        if blk == 0:
            assert "chain_fused" in set(svl.profile_end())
        compare_chain(inp, got, orc.verify_chain(inp), f"fused chi block{blk}")
        accs.append(got["accepted_len"])
        ems.append(got["emitted"])
    acc, em = np.concatenate(accs), np.concatenate(ems)
    for j in range(5):
        sel = acc >= j
        counts = np.bincount(em[sel, j], minlength=16)
        p = special.softmax(t[j].astype(np.float64))
        assert stats.chisquare(counts, p * sel.sum()).pvalue > 1e-4, j
