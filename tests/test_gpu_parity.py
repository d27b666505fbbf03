"""Parity of the HIP path (through the C ABI) with the fp64 CPU oracle.

accepted_len and emitted must match bit-exactly, except for sequences the
oracle flags as lying within 1e-5 of an acceptance threshold or CDF boundary
(those are counted and reported); accept_prob must agree within 1e-5
absolute.  Greedy and tree results are integer decisions on raw logits and
must match exactly everywhere.
"""

import json
import os

import numpy as np
import pytest

import workloads as W
from gpu_common import chain_tensors, compare_chain, dev, dev_logits, run_chain, run_greedy, run_tree

pytestmark = pytest.mark.gpu


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


def _check_chain(svl, orc, inp, label):
    got = run_chain(svl, inp)
    ref = orc.verify_chain(inp)
    stats = compare_chain(inp, got, ref, label)
    _record("chain", label, stats)
    return got, ref


# ------------------------------------------------------------ small shapes ---

SMALL_CHAIN = [
    # B, k, V, dtype, temperature -- several tiles with ragged tails; odd V takes the element-load path
    (7, 4, 9000, W.BF16, 0.7),
    (5, 3, 5000, W.F32, 1.0),
    (3, 1, 1000, W.BF16, 1.3),
    (4, 8, 4097, W.BF16, 0.5),
    (2, 0, 3000, W.F32, 0.9),
    (6, 5, 128257, W.BF16, 0.8),
    (3, 2, 7001, W.F32, 0.6),
    (2, 64, 600, W.BF16, 1.0),
    (1, 4, 1024, W.F32, 1.0),
]


@pytest.mark.parametrize("seed", [1, 2, 3])
@pytest.mark.parametrize("shape", SMALL_CHAIN, ids=lambda s: f"B{s[0]}k{s[1]}V{s[2]}{W.DTYPE_NAMES[s[3]]}")
def test_small_chain_parity(svl, orc, shape, seed):
    B, k, V, dt, T = shape
    inp = W.chain_inputs(B, k, V, dt, seed, target_sigma=3.0, zipf_s=1.1, draft_sigma=(0.2, 3.0), temperature=T)
    _check_chain(svl, orc, inp, f"B{B}k{k}V{V}dt{dt}s{seed}")


@pytest.mark.parametrize("dt", [W.BF16, W.F32])
def test_mixed_temperatures_including_zero(svl, orc, dt):
    B, k, V = 12, 4, 6000
    T = np.array([0.0, 0.7, 0.0, 1.3, 0.3, 0.0, 1.0, 0.0, 0.5, 2.0, 0.0, 0.9], np.float32)
    inp = W.chain_inputs(B, k, V, dt, 5, target_sigma=2.0, draft_sigma=0.5, temperature=T)
    # give the greedy rows some accepted drafts
    top = np.argmax(W.values(inp["target_logits"], dt), axis=-1)
    for b in np.flatnonzero(T == 0):
        inp["draft_tokens"][b, :2] = top[b, :2]
    got, ref = _check_chain(svl, orc, inp, f"mixedT dt{dt}")
    assert (got["accepted_len"][T == 0] >= 2).all()


def test_identical_rows_accept_every_draft(svl, orc):
    inp = W.chain_inputs(16, 5, 9000, W.BF16, 3, target_sigma=3.0, draft_sigma=0.0, temperature=0.8)
    inp["uniforms"][:, :5] = np.float32(1.0) - np.float32(2.0 ** -24)
    got, ref = _check_chain(svl, orc, inp, "identical rows")
    assert (got["accepted_len"] == 5).all()
    assert (got["accept_prob"] == 1.0).all()


def test_unaligned_logits_take_the_element_path(svl, orc):
    import torch

    B, k, V = 3, 3, 4096
    inp = W.chain_inputs(B, k, V, W.BF16, 7, target_sigma=3.0, draft_sigma=1.0, temperature=0.7)
    ref = orc.verify_chain(inp)
    # same logits, but stored one element past a 16-byte boundary
    def shifted(arr):
        flat = dev_logits(np.concatenate([np.zeros(1, np.uint16), arr.reshape(-1)]), W.BF16)
        return flat[1:].view(arr.shape)

    d, t = shifted(inp["draft_logits"]), shifted(inp["target_logits"])
    assert d.data_ptr() % 16 != 0
    out = svl.verify_chain(dev(inp["draft_tokens"]), d, t, dev(inp["temperature"]), dev(inp["uniforms"]))
    torch.cuda.synchronize()
    got = {kk: v.cpu().numpy() for kk, v in out.items()}
    _record("chain", "unaligned", compare_chain(inp, got, ref, "unaligned"))


def test_empty_batch_is_a_no_op(svl):
    import torch

    e = torch.empty((0, 4, 100), dtype=torch.bfloat16, device="cuda")
    out = svl.verify_chain(torch.empty((0, 3), dtype=torch.int32, device="cuda"), e[:, :3], e,
                           torch.empty(0, device="cuda"), torch.empty((0, 4), device="cuda"))
    torch.cuda.synchronize()
    assert out["accepted_len"].numel() == 0



# Small chains run in one launch (one workgroup per sequence) while the batch
# is at most 256 sequences, every row has at most 64 segments and a
# sequence's 2k + 1 rows hold at most 144 KiB (without drafts: below 256
# sequences); each shape here sits on one side of one bound.
SMALL_PATH = [
    # B, k, V, dtype, expect the one-launch path
    (16, 4, 8192, W.BF16, True),     # 144 KiB exactly
    (16, 4, 8200, W.BF16, False),    # just above it
    (256, 2, 4096, W.BF16, True),    # the largest batch
    (257, 2, 4096, W.BF16, False),
    (8, 0, 16384, W.F32, True),      # 64 segments of fp32
    (8, 0, 16385, W.F32, False),     # 65 segments
    (255, 0, 2048, W.F32, True),     # no drafts, below the row draw's batch size
    (256, 0, 2048, W.F32, False),    # the row draw
]


@pytest.mark.parametrize("shape", SMALL_PATH, ids=lambda s: f"B{s[0]}k{s[1]}V{s[2]}{W.DTYPE_NAMES[s[3]]}")
def test_small_chain_path_and_its_bounds(svl, orc, shape):
    B, k, V, dt, small = shape
    inp = W.chain_inputs(B, k, V, dt, 9, target_sigma=3.0, zipf_s=1.1, draft_sigma=(0.2, 3.0),
                         temperature=np.where(np.arange(B) % 5 == 0, 0.0, 0.8).astype(np.float32))
    svl.profile_begin(64)
    got, ref = _check_chain(svl, orc, inp, f"small path B{B}k{k}V{V}dt{dt}")
    launched = set(svl.profile_end())
    assert (launched == {"chain_small"}) == small, launched



# Small greedy chains run in one launch too: at most 256 sequences whose k + 1
# rows fit in 16 tiles of 8 KiB (one per wave).
GREEDY_SMALL_PATH = [
    # B, k, V, dtype, expect the one-launch path
    (16, 3, 16384, W.BF16, True),    # 4 rows of 4 tiles
    (16, 3, 16385, W.BF16, False),   # 4 rows of 5
    (256, 1, 1000, W.F32, True),
    (257, 1, 1000, W.F32, False),
    (2, 15, 512, W.F32, True),       # 16 tiles
    (2, 16, 512, W.F32, False),      # 17
]


@pytest.mark.parametrize("shape", GREEDY_SMALL_PATH, ids=lambda s: f"B{s[0]}k{s[1]}V{s[2]}{W.DTYPE_NAMES[s[3]]}")
def test_small_greedy_path_and_its_bounds(svl, orc, shape):
    B, k, V, dt, small = shape
    inp = W.greedy_inputs(B, k, V, dt, 12, match_p=0.85)
    svl.profile_begin(64)
    got = run_greedy(svl, inp)
    launched = set(svl.profile_end())
    ref = orc.verify_greedy(inp)
    np.testing.assert_array_equal(got["accepted_len"], ref["accepted_len"])
    np.testing.assert_array_equal(got["emitted"], ref["emitted"])
    assert (launched == {"greedy_small"}) == small, launched


# ------------------------------------------------------------ full workloads ---

@pytest.mark.parametrize("seed", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("workload", ["tiny_chain", "llama_chain", "deepseek_chain"])
def test_full_chain_workloads(svl, orc, workload, seed):
    inp = W.make_inputs(workload, seed)
    _check_chain(svl, orc, inp, f"{workload} seed{seed}")


@pytest.mark.parametrize("seed", [1, 2, 3, 4, 5])
def test_full_greedy_workload(svl, orc, seed):
    inp = W.make_inputs("greedy_chain", seed)
    got = run_greedy(svl, inp)
    ref = orc.verify_greedy(inp)
    np.testing.assert_array_equal(got["accepted_len"], ref["accepted_len"])
    np.testing.assert_array_equal(got["emitted"], ref["emitted"])
    _record("greedy", f"greedy_chain seed{seed}", dict(n=inp["B"], mean_accepted=float(got["accepted_len"].mean())))


# Calls whose target rows reach 256 MiB stream them in two phases: the first
# half of each sequence's rows, then the rest only for sequences whose drafts
# all match in the first half.
TWO_PHASE = [
    # B, k, V, dtype, match_p -- rows per phase: (k+1)//2 then the rest (the
    # bf16 vector path takes two phases in the full greedy workload above)
    (64, 4, 262144, W.F32, 0.8),
    (96, 1, 350000, W.F32, 0.8),
    (40, 15, 211111, W.BF16, 0.9),   # odd V: element loads
    (128, 5, 100000, W.F32, 1.0),    # every sequence takes the second phase
    (128, 5, 100000, W.F32, 0.0),    # none does
    (20, 63, 60001, W.F32, 0.95),    # V * 4 not a multiple of 16: element loads
]


@pytest.fixture(scope="module")
def two_phase_ws(svl):
    """One workspace for every two-phase case, 0xFF bytes at first and then
    whatever the earlier cases left in it."""
    import torch

    nbytes = max(svl.greedy_workspace_bytes(B, k, V, dt) for B, k, V, dt, _ in TWO_PHASE)
    return torch.full((nbytes,), 0xFF, dtype=torch.uint8, device="cuda")


@pytest.mark.parametrize("case", list(range(len(TWO_PHASE))) + [0],
                         ids=[f"case{i}" for i in range(len(TWO_PHASE))] + ["case0-again"])
def test_greedy_two_phase(svl, orc, two_phase_ws, case):
    """Parity on sizes that take the two phases.  Rows a call skips keep the
    partials of earlier calls in the shared workspace, which must never reach
    its results; the first case runs again last, over the others' partials."""
    import torch

    B, k, V, dt, mp = TWO_PHASE[case]
    assert B * (k + 1) * V * (2 if dt == W.BF16 else 4) >= 256 << 20
    inp = W.greedy_inputs(B, k, V, dt, 60 + case, match_p=mp)
    out = svl.verify_greedy(dev(inp["draft_tokens"].astype(np.int32)), dev_logits(inp["target_logits"], dt),
                            workspace=two_phase_ws)
    torch.cuda.synchronize()
    ref = orc.verify_greedy(inp)
    got = {key: v.cpu().numpy() for key, v in out.items()}
    np.testing.assert_array_equal(got["accepted_len"], ref["accepted_len"])
    np.testing.assert_array_equal(got["emitted"], ref["emitted"])
    s = (k + 1) // 2
    _record("greedy", f"two-phase B{B} k{k} V{V} p{mp}",
            dict(n=B, second_phase=int((ref["accepted_len"] >= s).sum()),
                 mean_accepted=float(ref["accepted_len"].mean())))


@pytest.mark.parametrize("seed", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("name", ["eagle_tree", "eagle_tree_distinct"])
def test_full_tree_workload(svl, orc, name, seed):
    inp = W.make_inputs(name, seed)
    got = run_tree(svl, inp)
    ref = orc.verify_tree(inp)
    for key in ("accepted_len", "emitted", "accepted_nodes"):
        np.testing.assert_array_equal(got[key], ref[key], err_msg=key)
    _record("tree", f"{name} seed{seed}", dict(n=inp["B"], mean_accepted=float(got["accepted_len"].mean())))


def test_determinism(svl):
    inp = W.make_inputs("llama_chain", 1)
    a = run_chain(svl, inp)
    b = run_chain(svl, inp)
    for key in a:
        np.testing.assert_array_equal(a[key], b[key])


# ------------------------------------------------------------ greedy / tree edges ---

def _next_above(bits, dtype):
    """The representable value just above a stored logit (bit patterns)."""
    if dtype == W.BF16:
        b = int(bits)
        return np.uint16(b + 1 if b < 0x8000 else (b - 1 if b != 0x8000 else 0x0001))
    return np.nextafter(np.float32(bits), np.float32(np.inf))


def _plant_tile_ties(t, dtype, rng):
    """Give every row a new strict maximum stored twice, in two different tiles
    (tiles hold 64 * 8 vectors of 16 bytes): even rows on both sides of a tile
    boundary, odd rows in the first and the last tile.  The first argmax is
    then the lower of the two indices."""
    ve = 8 if dtype == W.BF16 else 4
    tile = 64 * 8 * ve
    V = t.shape[-1]
    assert V > 2 * tile
    rows = t.reshape(-1, V)
    vals = W.values(rows, dtype)
    for r in range(rows.shape[0]):
        top = rows[r, int(np.argmax(vals[r]))]
        new = _next_above(top, dtype)
        if r % 2 == 0:
            bnd = tile * int(rng.integers(1, (V - 1) // tile + 1))
            i1, i2 = bnd - 1, bnd
        else:
            i1, i2 = int(rng.integers(0, tile)), int(rng.integers((V - 1) // tile * tile, V))
        rows[r, i1] = new
        rows[r, i2] = new


@pytest.mark.parametrize("dt", [W.BF16, W.F32])
@pytest.mark.parametrize("V", [20000, 20001])
def test_greedy_ties_across_tile_boundaries(svl, orc, dt, V):
    inp = W.greedy_inputs(24, 4, V, dt, 2, match_p=0.7)
    _plant_tile_ties(inp["target_logits"], dt, np.random.default_rng(0))
    top = np.argmax(W.values(inp["target_logits"], dt), axis=-1)
    inp["draft_tokens"][::2] = top[::2, :4]
    got = run_greedy(svl, inp)
    ref = orc.verify_greedy(inp)
    np.testing.assert_array_equal(got["accepted_len"], ref["accepted_len"])
    np.testing.assert_array_equal(got["emitted"], ref["emitted"])


def test_temperature_zero_chain_matches_greedy_with_ties(svl, orc):
    B, k, V = 16, 4, 20000
    inp = W.chain_inputs(B, k, V, W.BF16, 4, target_sigma=2.0, draft_sigma=1.0, temperature=0.0)
    _plant_tile_ties(inp["target_logits"], W.BF16, np.random.default_rng(1))
    top = np.argmax(W.values(inp["target_logits"], W.BF16), axis=-1)
    inp["draft_tokens"][::2] = top[::2, :k]
    got, ref = _check_chain(svl, orc, inp, "T0 ties")
    g = run_greedy(svl, dict(inp, kind="greedy"))
    np.testing.assert_array_equal(got["emitted"], g["emitted"])


def test_tree_per_sequence_parents_and_invalid_trees(svl, orc):
    B, N, V = 6, 40, 3000
    base = W.tree_inputs(B, N, V, W.BF16, 9, max_depth=6)
    parents = np.stack([W.random_tree(N, 100 + b) for b in range(B)]).astype(np.int32)
    parents[4, 7] = 9          # parent index not below the node: invalid
    inp = dict(base, parent=parents)
    depth = np.zeros(N, int)
    for i in range(1, N):
        depth[i] = depth[parents[5, i]] + 1
    inp["max_depth"] = 6
    got = run_tree(svl, inp)
    ref = orc.verify_tree(inp)
    for key in ("accepted_len", "emitted", "accepted_nodes"):
        np.testing.assert_array_equal(got[key], ref[key], err_msg=key)
    assert got["accepted_len"][4] == -1


# Trees whose rows reach 96 MiB are streamed in two phases: the root rows,
# then only the rows below a depth-1 node that carries the root's argmax.
# From 192 MiB and 48 nodes, in three: the root rows, depths 1-2 below an
# accepted depth-1 node, then depths 3 and more below an accepted depth-3 node.
def _tree_two_phase_case(case):
    V = 128256
    if case.startswith("per-sequence parents"):
        B, N = (8, 64) if case.endswith("three phases") else (12, 40)
        if case.endswith("three phases"):
            V = 200003
        inp = W.tree_inputs(B, N, V, W.BF16, 21, max_depth=6)
        parents = np.stack([W.random_tree(N, 200 + b) for b in range(B)]).astype(np.int32)
        # tokens that follow each sequence's own tree (the argmax of the parent's row, or another token)
        top = np.argmax(W.values(inp["target_logits"], W.BF16), axis=-1)
        rng = np.random.default_rng(21)
        tokens = inp["node_tokens"].copy()
        for b in range(B):
            for i in range(1, N):
                g = int(top[b, parents[b, i]])
                tokens[b, i] = g if rng.random() < 0.6 else (g + 1 + int(rng.integers(0, V - 1))) % V
        parents[4, 7] = 9          # parent index not below the node: invalid
        parents[B - 3, 30] = -3    # negative parent: invalid
        return dict(inp, parent=parents, node_tokens=tokens)
    if case == "chain":
        return W.tree_inputs(48, 11, V, W.BF16, 22, parent=np.arange(-1, 10, dtype=np.int32), match_p=0.8)
    if case == "star":
        return W.tree_inputs(16, 31, V, W.BF16, 23, parent=np.array([-1] + [0] * 30, np.int32), match_p=0.3)
    if case == "f32 element loads":
        return W.tree_inputs(8, 40, 100001, W.F32, 24)
    if case == "two nodes":
        return W.tree_inputs(400, 2, V, W.BF16, 25, parent=np.array([-1, 0], np.int32), match_p=0.5)
    if case == "all match":
        return W.tree_inputs(16, 64, V, W.BF16, 26, match_p=1.0)
    if case == "none match":
        return W.tree_inputs(16, 64, V, W.BF16, 27, match_p=0.0)
    raise ValueError(case)


TREE_TWO_PHASE = ["per-sequence parents", "chain", "star", "f32 element loads", "two nodes", "all match",
                  "none match", "per-sequence parents, three phases"]


@pytest.fixture(scope="module")
def tree_two_phase_ws(svl):
    """One workspace for every two-phase tree case, 0xFF bytes at first and
    then whatever the earlier cases left in it."""
    import torch

    return torch.full((svl.tree_workspace_bytes(400, 64, 128256, W.BF16),), 0xFF, dtype=torch.uint8, device="cuda")


@pytest.mark.parametrize("case", TREE_TWO_PHASE + TREE_TWO_PHASE[:1],
                         ids=TREE_TWO_PHASE + ["per-sequence parents again"])
def test_tree_two_phase(svl, orc, tree_two_phase_ws, case):
    """Parity on trees that take the two phases, on one shared workspace: the
    partials of rows a call skips are stale and must never reach its results
    (nor may a malformed tree's rows)."""
    import torch

    inp = _tree_two_phase_case(case)
    B, N, V, dt = inp["B"], inp["N"], inp["V"], inp["dtype"]
    assert B * N * V * (2 if dt == W.BF16 else 4) >= 96 << 20
    assert svl.tree_workspace_bytes(B, N, V, dt) <= tree_two_phase_ws.numel()
    out = svl.verify_tree(dev(inp["node_tokens"].astype(np.int32)), dev(inp["parent"].astype(np.int32)),
                          int(inp["max_depth"]), dev_logits(inp["target_logits"], dt), workspace=tree_two_phase_ws)
    torch.cuda.synchronize()
    ref = orc.verify_tree(inp)
    for key in ("accepted_len", "emitted", "accepted_nodes"):
        np.testing.assert_array_equal(out[key].cpu().numpy(), ref[key], err_msg=key)
    _record("tree", f"two-phase {case}", dict(n=B, mean_accepted=float(ref["accepted_len"].mean())))


def test_tree_linear_and_star_shapes(svl, orc):
    V = 5000
    for parent in (np.arange(-1, 11, dtype=np.int32), np.array([-1] + [0] * 30, np.int32)):
        N = parent.size
        inp = W.tree_inputs(8, N, V, W.F32, 3, parent=parent, match_p=0.8)
        got = run_tree(svl, inp)
        ref = orc.verify_tree(inp)
        for key in ("accepted_len", "emitted", "accepted_nodes"):
            np.testing.assert_array_equal(got[key], ref[key], err_msg=key)


# ------------------------------------------------------------ distribution on the GPU ---

def test_gpu_emitted_distribution_chi_square(svl, orc):
    """10^6 trials at V = 16, k = 4 through the GPU: bit-exact with the oracle
    outside the band, and the emitted token at position j given j accepted
    drafts is distributed as the target row j (chi-square)."""
    from scipy import special, stats

    rng = np.random.default_rng(2024)
    t = (1.5 * rng.standard_normal((5, 16))).astype(np.float32)
    d = (t[:4] + rng.standard_normal((4, 16))).astype(np.float32)
    accs, ems = [], []
    for blk in range(5):
        inp = W.repeated_trials(t, d, 1.0, 200_000, seed=77, block=blk)
        got, ref = _check_chain(svl, orc, inp, f"chi block{blk}")
        accs.append(got["accepted_len"])
        ems.append(got["emitted"])
    acc, em = np.concatenate(accs), np.concatenate(ems)
    for j in range(5):
        sel = acc >= j
        counts = np.bincount(em[sel, j], minlength=16)
        p = special.softmax(t[j].astype(np.float64))
        assert stats.chisquare(counts, p * sel.sum()).pvalue > 1e-4


def test_gpu_plain_sampling_chi_square(svl, orc):
    """k = 0 through the GPU: 10^6 trials at V = 16 and T = 0.8, bit-exact
    with the oracle outside the band, and the sampled token distributed as
    softmax(t / T) (chi-square)."""
    from scipy import special, stats

    rng = np.random.default_rng(2024)
    t = (1.5 * rng.standard_normal((1, 16))).astype(np.float32)
    inp = W.repeated_trials(t, np.zeros((0, 16), np.float32), 0.8, 1_000_000, seed=92)
    got, ref = _check_chain(svl, orc, inp, "chi k0")
    counts = np.bincount(got["emitted"][:, 0], minlength=16)
    p = special.softmax(t[0].astype(np.float64) / np.float64(np.float32(0.8)))
    assert stats.chisquare(counts, p * 1_000_000).pvalue > 1e-4


def _rows(inp, lo, hi):
    """Sequences lo..hi-1 of a chain batch."""
    out = dict(inp, B=hi - lo)
    for key, v in inp.items():
        if isinstance(v, np.ndarray) and v.ndim >= 1 and v.shape[0] == inp["B"]:
            out[key] = v[lo:hi]
    return out


ROW_DRAW = [(0, V, dt) for V, dt in [(128256, W.BF16), (131072, W.BF16), (131073, W.BF16), (65536, W.F32),
                                      (30001, W.F32), (70001, W.BF16), (1, W.BF16), (700, W.F32)]] + \
           [(1, 129280, W.BF16), (3, 65536, W.F32), (2, 70001, W.BF16), (4, 131073, W.BF16), (1, 2, W.F32)]


@pytest.mark.parametrize("k,V,dt", ROW_DRAW)
def test_row_draw_matches_split_batches(svl, orc, k, V, dt):
    """With no drafts, from 256 sequences on, the draw of a row of at most 256
    segments runs in one workgroup; smaller batches take the two-kernel draw.
    With drafts the two batch sizes take the two-kernel draw with the
    acceptance computed in every workgroup (64 sequences) or once per
    sequence by its own kernel (256).  Every form computes the same tiles,
    weights, segment masses and pick: one batch of 256 sequences and the same
    sequences as four batches of 64 give bit-identical outputs, which match
    the oracle outside the band.  Temperature 0 sequences take the argmax."""
    B = 256
    temps = np.where(np.arange(B) % 7 == 3, 0.0, np.linspace(0.3, 1.6, B)).astype(np.float32)
    inp = W.chain_inputs(B, k, V, dt, 77 + k, target_sigma=3.0, draft_sigma=(0.2, 1.5), temperature=temps)
    whole, ref = _check_chain(svl, orc, inp, f"row draw k{k} V{V}")
    parts = [run_chain(svl, _rows(inp, lo, lo + 64)) for lo in range(0, B, 64)]
    for key in ("accepted_len", "emitted", "accept_prob"):
        if whole[key] is not None:
            np.testing.assert_array_equal(whole[key], np.concatenate([p[key] for p in parts]), err_msg=key)


# Without accept_prob, chains of at least 6 drafts and 128 MiB of rows stream
# positions 0 .. max(1, k/4)-1 first and the remaining positions only for
# sequences that accept all of those.  Outputs must equal the one-pass
# results (with accept_prob) exactly, whichever schedule runs.
def _no_prob_case(case):
    if case in ("llama_chain", "deepseek_chain", "mtp_chain"):
        return W.make_inputs(case, 3)
    if case == "300 sequences f32":
        return W.chain_inputs(300, 2, 60000, W.F32, 31, target_sigma=3.0, draft_sigma=(0.2, 1.5))
    if case == "acceptance kernel":
        return W.chain_inputs(200, 3, 128256, W.BF16, 32, target_sigma=3.0, draft_sigma=(0.2, 1.5))
    if case == "temperature 0 mix, two phases":
        temps = np.where(np.arange(40) % 3 == 0, 0.0, 0.8).astype(np.float32)
        inp = W.chain_inputs(40, 8, 128256, W.BF16, 33, target_sigma=3.0, draft_sigma=(0.05, 1.0), temperature=temps)
        top = np.argmax(W.values(inp["target_logits"], W.BF16), axis=-1)
        inp["draft_tokens"][::3] = top[::3, :8]      # greedy sequences that accept
        inp["draft_tokens"][3, 1] = top[3, 0]        # ... and one that stops at position 1
        return inp
    if case == "64 drafts, two phases":
        return W.chain_inputs(8, 64, 65536, W.BF16, 34, target_sigma=1.0, draft_sigma=(0.01, 0.3))
    if case == "16 drafts element loads, two phases":
        return W.chain_inputs(12, 16, 100001, W.F32, 35, target_sigma=2.0, draft_sigma=(0.05, 0.5))
    if case == "256 sequences f32, two phases":
        return W.chain_inputs(256, 6, 30000, W.F32, 36, target_sigma=3.0, draft_sigma=(0.1, 1.0))
    if case == "acceptance kernel, two phases":
        return W.chain_inputs(130, 6, 128256, W.BF16, 37, target_sigma=3.0, draft_sigma=(0.1, 1.0))
    raise ValueError(case)


NO_PROB = ["llama_chain", "deepseek_chain", "mtp_chain", "300 sequences f32", "acceptance kernel",
           "temperature 0 mix, two phases", "64 drafts, two phases", "16 drafts element loads, two phases",
           "256 sequences f32, two phases", "acceptance kernel, two phases"]


@pytest.mark.parametrize("case", NO_PROB)
def test_chain_without_accept_prob(svl, orc, case):
    inp = _no_prob_case(case)
    if case.endswith("two phases") or case == "deepseek_chain":
        assert inp["k"] >= 6 and 2 * inp["B"] * inp["k"] * inp["V"] * (2 if inp["dtype"] == W.BF16 else 4) >= 128 << 20
    full = run_chain(svl, inp)
    ref = orc.verify_chain(inp)
    lean = run_chain(svl, inp, accept_prob=False)
    assert lean["accept_prob"] is None
    for key in ("accepted_len", "emitted"):
        np.testing.assert_array_equal(lean[key], full[key], err_msg=key)
    stats = compare_chain(inp, lean, ref, f"no accept_prob {case}")
    _record("chain", f"no accept_prob {case}", dict(stats, mean_accepted=float(lean["accepted_len"].mean())))


@pytest.mark.parametrize("fill", [0xFF, 0x7F], ids=["ff", "7f"])
def test_chain_two_phases_on_a_garbage_workspace(svl, orc, fill):
    """The second phase leaves the partials of skipped positions as the
    workspace held them: NaNs (0xFF) or huge values (0x7F) there must never
    reach the outputs."""
    import torch

    inp = _no_prob_case("temperature 0 mix, two phases")
    ws = torch.full((svl.chain_workspace_bytes(inp["B"], inp["k"], inp["V"], inp["dtype"]),), fill,
                    dtype=torch.uint8, device="cuda")
    got = run_chain(svl, inp, accept_prob=False, workspace=ws)
    compare_chain(inp, got, orc.verify_chain(inp), f"two phases, workspace {fill:#x}")


# ------------------------------------------------------------ NEXT rows ---

@pytest.mark.parametrize("seed", [1, 2, 3])
@pytest.mark.parametrize("workload", ["mtp_chain", "sampling"])
def test_full_mtp_and_sampling_workloads(svl, orc, workload, seed):
    """Single-token MTP verification (k = 1, B = 256, V = 129280) and plain
    temperature sampling (k = 0, B = 256)."""
    inp = W.make_inputs(workload, seed)
    _check_chain(svl, orc, inp, f"{workload} seed{seed}")


@pytest.mark.parametrize("with_history", [True, False])
@pytest.mark.parametrize("B", [1, 37, 3000])
def test_commit_tokens_parity(svl, orc, B, with_history):
    import torch

    rng = np.random.default_rng(B)
    width, cap = 5, 64
    acc = rng.integers(-1, width, B).astype(np.int32)
    acc[::13] = width  # one more than the row holds: refused
    em = rng.integers(0, 128256, (B, width)).astype(np.int32)
    lens = rng.integers(0, cap, B).astype(np.int32)
    hist = rng.integers(0, 9, (B, cap)).astype(np.int32)
    ref = orc.commit_tokens(acc, em, lens, hist if with_history else None)
    sl = dev(lens)
    h = dev(hist) if with_history else None
    out = svl.commit_tokens(dev(acc), dev(em), sl, h)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(sl.cpu().numpy(), ref["seq_len"])
    if with_history:
        np.testing.assert_array_equal(h.cpu().numpy(), ref["history"])
    offs = out["packed_offsets"].cpu().numpy()
    np.testing.assert_array_equal(offs, ref["packed_offsets"])
    np.testing.assert_array_equal(out["packed"].cpu().numpy()[:offs[B]], ref["packed"])
    np.testing.assert_array_equal(out["status"].cpu().numpy(), ref["status"])


@pytest.mark.parametrize("with_history", [True, False])
def test_commit_tokens_rows_that_would_overflow(svl, orc, with_history):
    """Counts and lengths at the int32 limit: the GPU refuses and commits the
    same rows as the oracle, with no wrap-around."""
    import torch

    imax = int(np.iinfo(np.int32).max)
    acc = np.array([imax, 1, 2, 0, 2, imax - 1], np.int32)
    em = np.arange(18, dtype=np.int32).reshape(6, 3)
    lens = np.array([5, imax - 2, imax - 2, imax, 3, 0], np.int32)
    hist = np.zeros((6, 8), np.int32) if with_history else None
    ref = orc.commit_tokens(acc, em, lens, hist)
    sl = dev(lens)
    h = dev(hist) if with_history else None
    out = svl.commit_tokens(dev(acc), dev(em), sl, h)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out["status"].cpu().numpy(), ref["status"])
    np.testing.assert_array_equal(sl.cpu().numpy(), ref["seq_len"])
    offs = out["packed_offsets"].cpu().numpy()
    np.testing.assert_array_equal(offs, ref["packed_offsets"])
    np.testing.assert_array_equal(out["packed"].cpu().numpy()[:offs[-1]], ref["packed"])
    if with_history:
        np.testing.assert_array_equal(h.cpu().numpy(), ref["history"])


def test_verify_then_commit_on_device(svl, orc):
    """A decode step without host synchronisation: verification, then the commit
    of its output into per-sequence histories, all on one stream."""
    import torch

    inp = W.make_inputs("llama_chain", 3)
    B, k = inp["B"], inp["k"]
    t = chain_tensors(inp)
    lens = np.arange(B, dtype=np.int32) % 50
    hist = np.zeros((B, 64), np.int32)
    sl, h = dev(lens), dev(hist)
    out = svl.verify_chain(t["draft_tokens"], t["draft_logits"], t["target_logits"], t["temperature"],
                           t["uniforms"])
    com = svl.commit_tokens(out["accepted_len"], out["emitted"], sl, h)
    torch.cuda.synchronize()
    ref_v = orc.verify_chain(inp)
    got_v = dict(accepted_len=out["accepted_len"].cpu().numpy(), emitted=out["emitted"].cpu().numpy(),
                 accept_prob=out["accept_prob"].cpu().numpy())
    compare_chain(inp, got_v, ref_v, "verify+commit")
    ref_c = orc.commit_tokens(got_v["accepted_len"], got_v["emitted"], lens, hist)
    np.testing.assert_array_equal(sl.cpu().numpy(), ref_c["seq_len"])
    np.testing.assert_array_equal(h.cpu().numpy(), ref_c["history"])
    np.testing.assert_array_equal(com["packed"].cpu().numpy()[:ref_c["packed_offsets"][B]], ref_c["packed"])


@pytest.mark.parametrize("shape", [(600, 2, 9000, W.BF16), (700, 1, 9000, W.F32), (700, 1, 4097, W.BF16),
                                   (1200, 0, 5000, W.BF16), (300, 2, 60000, W.F32), (300, 1, 64007, W.BF16),
                                   (600, 0, 30001, W.F32), (2500, 0, 4097, W.BF16)],
                         ids=lambda s: f"B{s[0]}k{s[1]}V{s[2]}{W.DTYPE_NAMES[s[3]]}")
def test_large_batch_final_draw(svl, orc, shape):
    """Batches large enough that each final-draw wave handles several tiles,
    with ragged row ends, a last chunk only partly inside the row and
    unaligned row lengths."""
    B, k, V, dt = shape
    inp = W.chain_inputs(B, k, V, dt, 11, target_sigma=3.0, zipf_s=1.1, draft_sigma=(0.2, 3.0),
                         temperature=(0.3, 1.3))
    _check_chain(svl, orc, inp, f"pipelined B{B}k{k}V{V}dt{dt}")


@pytest.mark.parametrize("fill", [0xFF, 0x7F], ids=["ff", "7f"])
def test_workspace_needs_no_initialisation(svl, orc, fill):
    """Every entry point on a workspace whose bytes all hold `fill` (0xFF: NaN
    floats and -1 integers; 0x7F: huge values) gives the oracle's results, as
    the header promises: no call reads workspace memory it has not written."""
    import torch

    from gpu_common import compare_tree_sampled, tree_sampled_tensors

    def ws(nbytes):
        return torch.full((nbytes,), fill, dtype=torch.uint8, device="cuda")

    temps = np.array([0.7, 0.0, 1.2, 0.5, 0.9, 0.0], np.float32)
    chains = [W.chain_inputs(6, 3, 5000, W.BF16, 91, draft_sigma=(0.3, 2.0), temperature=temps),   # inline acceptance
              W.chain_inputs(700, 1, 20000, W.BF16, 92, draft_sigma=(0.3, 2.0)),                 # acceptance kernel
              W.chain_inputs(9, 0, 3001, W.F32, 93, temperature=np.linspace(0, 1.5, 9, dtype=np.float32))]
    for i, inp in enumerate(chains):
        got = run_chain(svl, inp, workspace=ws(svl.chain_workspace_bytes(inp["B"], inp["k"], inp["V"], inp["dtype"])))
        compare_chain(inp, got, orc.verify_chain(inp), f"chain {i} fill {fill:#x}")
    g = W.greedy_inputs(20, 4, 7000, W.F32, 94)
    out = svl.verify_greedy(dev(g["draft_tokens"].astype(np.int32)), dev_logits(g["target_logits"], g["dtype"]),
                            workspace=ws(svl.greedy_workspace_bytes(20, 4, 7000, W.F32)))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out["emitted"].cpu().numpy(), orc.verify_greedy(g)["emitted"])
    t = W.tree_inputs(8, 30, 6000, W.BF16, 95)
    out = svl.verify_tree(dev(t["node_tokens"].astype(np.int32)), dev(t["parent"].astype(np.int32)),
                          int(t["max_depth"]), dev_logits(t["target_logits"], t["dtype"]),
                          workspace=ws(svl.tree_workspace_bytes(8, 30, 6000, W.BF16)))
    torch.cuda.synchronize()
    ref = orc.verify_tree(t)
    for key in ("accepted_len", "emitted", "accepted_nodes"):
        np.testing.assert_array_equal(out[key].cpu().numpy(), ref[key], key)
    # the sampled tree with and without the round-0 normaliser cache
    for inp in (W.sampled_tree_inputs(6, 40, 9000, W.BF16, 96, draft_sigma=(0.3, 2.0)),
                W.sampled_tree_inputs(200, 24, 6000, W.BF16, 97, draft_sigma=(0.3, 2.0))):
        ts = tree_sampled_tensors(inp)
        B, N, V = inp["B"], inp["N"], inp["V"]
        out = svl.verify_tree_sampled(ts["node_tokens"], ts["parent"], int(inp["max_depth"]), ts["draft_logits"],
                                      ts["target_logits"], ts["temperature"], ts["uniforms"],
                                      workspace=ws(svl.tree_sampled_workspace_bytes(B, N, V, inp["dtype"])))
        torch.cuda.synchronize()
        got = {key: (v.cpu().numpy() if v is not None else None) for key, v in out.items()}
        compare_tree_sampled(got, orc.verify_tree_sampled(inp), f"sampled tree B{B} fill {fill:#x}")


# Vocabulary sizes at the edges of the work units: a 16-byte vector (8 bf16 or
# 4 f32), a segment (64 vectors), the draw's wave tile (4 segments) and the
# streaming tile (8 segments), one below and one above each, and V = 1.
EDGE_V = [1, 2, 7, 8, 9, 63, 64, 65, 255, 256, 257, 511, 512, 513, 2047, 2048, 2049, 4095, 4096, 4097]


@pytest.mark.parametrize("V", EDGE_V)
def test_vocabulary_sizes_at_tile_and_segment_edges(svl, orc, V):
    temps = np.array([0.7, 0.0, 1.2, 0.4, 1.0], np.float32)
    for dt in (W.BF16, W.F32):
        inp = W.chain_inputs(5, 2, V, dt, V, draft_sigma=(0.3, 2.0), temperature=temps)
        _check_chain(svl, orc, inp, f"edge V{V} dt{dt}")
        k0 = W.chain_inputs(5, 0, V, dt, V + 1, temperature=temps)
        _check_chain(svl, orc, k0, f"edge k0 V{V} dt{dt}")
        g = W.greedy_inputs(5, 2, V, dt, V)
        got, ref = run_greedy(svl, g), orc.verify_greedy(g)
        np.testing.assert_array_equal(got["accepted_len"], ref["accepted_len"])
        np.testing.assert_array_equal(got["emitted"], ref["emitted"])
        t = W.tree_inputs(4, 9, V, dt, V)
        got, ref = run_tree(svl, t), orc.verify_tree(t)
        for key in ("accepted_len", "emitted", "accepted_nodes"):
            np.testing.assert_array_equal(got[key], ref[key], key)


# Logits at the edges of the header's preconditions (|l| / T < 10^6, and
# |l_v - max l| / T < 700 within a row): large common offsets (the
# distributions do not change, but the integer references and the split
# temperature scale work at large magnitudes), a very small and a very large
# temperature.  The drafts drawn before the shift remain samples of the
# shifted draft rows.
EXTREMES = [
    (5000.0, 0.7, W.BF16, 3.0),
    (-5000.0, 0.7, W.BF16, 3.0),
    (1.0e5, 1.0, W.F32, 3.0),
    (-1.0e5, 1.0, W.F32, 3.0),
    (0.0, 0.05, W.F32, 1.0),
    (0.0, 100.0, W.BF16, 3.0),
]


@pytest.mark.parametrize("case", EXTREMES, ids=lambda c: f"off{c[0]:g}-T{c[1]:g}-{W.DTYPE_NAMES[c[2]]}")
def test_logits_at_the_edges_of_the_declared_range(svl, orc, case):
    offset, T, dt, sigma = case
    inp = W.chain_inputs(16, 3, 5000, dt, 31, target_sigma=sigma, draft_sigma=(0.2, 1.5),
                         temperature=np.float32(T))
    for key in ("target_logits", "draft_logits"):
        inp[key] = W.to_dtype(W.values(inp[key], dt) + np.float32(offset), dt)
    _check_chain(svl, orc, inp, f"extreme off{offset:g} T{T:g} dt{dt}")


def test_out_of_range_draft_tokens_are_rejected(svl, orc):
    """The header's rule for a draft token outside [0, V): it is rejected
    (tau = 0) and never used as an index.  The oracle refuses such inputs, so
    the check is by properties: acceptance stops at or before the bad
    position, its accept_prob is 0 and the final token is a valid id; the
    other sequences still match the oracle exactly."""
    V = 3001
    temps = np.array([0.8, 1.1, 0.0, 0.6] * 4, np.float32)
    inp = W.chain_inputs(16, 4, V, W.F32, 41, draft_sigma=0.05, temperature=temps)  # near-copy drafts: long prefixes
    bad = {1: (1, V), 5: (2, -7), 9: (0, V + 1000), 14: (3, -1)}  # sequence: (position, token)
    for b, (j, tok) in bad.items():
        inp["draft_tokens"][b, j] = tok
    got = run_chain(svl, inp)
    for b, (j, tok) in bad.items():
        a = int(got["accepted_len"][b])
        assert a <= j, (b, a, j)
        if a == j:
            assert got["accept_prob"][b, j] == 0.0
        assert 0 <= got["emitted"][b, a] < V
        assert (got["emitted"][b, :a] == inp["draft_tokens"][b, :a]).all()
        assert (got["emitted"][b, a + 1:] == -1).all()
    keep = np.array([b for b in range(16) if b not in bad])
    sub = {key: (val[keep] if isinstance(val, np.ndarray) and val.ndim and val.shape[0] == 16 else val)
           for key, val in inp.items()}
    sub["B"] = keep.size
    ref = orc.verify_chain(sub)
    compare_chain(sub, {key: (v[keep] if v is not None else None) for key, v in got.items()}, ref, "valid rows")
    # greedy: an out-of-range id never equals the argmax
    g = W.greedy_inputs(8, 4, V, W.BF16, 42, match_p=1.0)
    g["draft_tokens"][3, 2] = V + 3
    g["draft_tokens"][6, 0] = -2
    gg = run_greedy(svl, g)
    assert gg["accepted_len"][3] == 2 and gg["accepted_len"][6] == 0
    assert ((gg["emitted"] >= 0) | (gg["emitted"] == -1)).all() and (gg["emitted"] < V).all()
    # greedy tree: a node with an out-of-range token is never accepted
    t = W.tree_inputs(4, 16, V, W.F32, 43, match_p=1.0)
    t["node_tokens"][:, 1:] = np.where(np.arange(1, 16) % 3 == 0, V + 9, t["node_tokens"][:, 1:])
    tt = run_tree(svl, t)
    for b in range(4):
        path = [n for n in tt["accepted_nodes"][b] if n >= 0]
        assert all(n % 3 != 0 for n in path), path


@pytest.mark.parametrize("workload", ["llama_chain", "deepseek_chain", "mtp_chain"])
def test_accept_prob_precision(svl, orc, workload):
    """A guard on the precision of the row normalisers, ten times tighter than
    the 1e-5 the results are held to: accept_prob = min(1, p/q) is within
    1e-6 of the oracle's fp64 value (measured maxima are about 3e-7)."""
    inp = W.make_inputs(workload, 3)
    got, ref = run_chain(svl, inp), orc.verify_chain(inp)
    err = np.abs(got["accept_prob"].astype(np.float64) - ref["accept_prob"])
    assert err.max() < 1e-6, err.max()
