"""Parity in the high-acceptance regime: draws from residuals of small mass.

When the draft distribution nearly equals the target's, a rejection leaves a
residual max(0, p - q) of small total mass W, and every CDF boundary C / W of
the final draw is a ratio of two small sums.  The pages require the output to
follow the target distribution after any rejection ("Accelerating Sonar
through speculation", section "Target-Draft"), so these draws must match the
fp64 oracle bit-exactly outside the 1e-5 band like any other.

The inputs force one rejection per sequence on near-copy draft rows (see
workloads.near_copy_chain_inputs and near_copy_tree_inputs): float32 rows with
small Gaussian noise (with and without a per-sequence logit offset, which
leaves the distribution unchanged but makes the logits of the two rows
differ by up to 4), and bfloat16 rows that differ from the target's in a
sparse set of one-unit bumps.  Each batch is verified with several sets of
final-draw uniforms; every draw is compared with the oracle's.  The residual
masses of the compared draws span about 1e-2 to 1e-5 (chains) and 5e-3 to
3e-6 (trees, after one to three rejections at a node).

The chain draw forms a residual whose mass the acceptance can bound below by
0.2 in a cheaper way (each term as e_t (1 - 2^delta), without the correction
of the normalisers' ratio), and every other residual in full.  The last test
draws from residuals on both sides of that threshold, many of them within a
factor of two of it, through both ways of obtaining the descriptor.  The
cheap form's error grows with how far below the top token the mass lies
(the exponentials' rounded exponents); flat-tail rows, whose mass lies about
8 binary orders down and whose residual (about 0.22) the tile masses already
show, put it at that edge.
"""

import numpy as np
import pytest

import workloads as W
from gpu_common import chain_tensors, compare_chain, compare_tree_sampled, tree_sampled_tensors

pytestmark = pytest.mark.gpu

V = 128256


@pytest.fixture(scope="module")
def svl():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import draft_token_verification_chain_amd as svl

    svl.load()
    return svl


def _decades(mass):
    """Counts of draws per decade of residual mass ("<1e-06" below 1e-6)."""
    edges = [0.0, 1e-6, 1e-5, 1e-4, 1e-3, 1e-2, 1e-1, 1.0]
    h, _ = np.histogram(mass, bins=edges)
    return {("<1e-06" if lo == 0.0 else f"{lo:.0e}"): int(c) for lo, c in zip(edges[:-1], h)}


# name, dtype, generator keywords, B, sets of final-draw uniforms.  B covers the
# two ways the final draw's workgroups obtain the draw's descriptor: each
# recomputes its sequence's acceptance (B * chunks <= 2048), or an acceptance
# kernel writes it once per sequence (larger batches).
CHAIN_CASES = [
    ("f32 sigma 2e-2 offset", W.F32, dict(draft_sigma=2e-2, offset=(-4.0, 4.0)), 64, 32),
    ("f32 sigma 2e-3 offset", W.F32, dict(draft_sigma=2e-3, offset=(-4.0, 4.0)), 128, 16),
    ("f32 sigma 2e-4 offset", W.F32, dict(draft_sigma=2e-4, offset=(-4.0, 4.0)), 64, 32),
    ("f32 sigma 2e-4", W.F32, dict(draft_sigma=2e-4), 128, 16),
    ("bf16 density 0.3", W.BF16, dict(density=0.3), 128, 16),
    ("bf16 density 0.3 acceptance kernel", W.BF16, dict(density=0.3), 256, 8),
    ("bf16 density 0.03", W.BF16, dict(density=0.03), 192, 11),
]


@pytest.mark.parametrize("case", CHAIN_CASES, ids=[c[0] for c in CHAIN_CASES])
def test_chain_small_residual(svl, orc, case):
    import torch

    name, dt, kw, B, R = case
    inp = W.near_copy_chain_inputs(B, 2, V, dt, seed=11, **kw)
    t = chain_tensors(inp)
    ru = np.random.Generator(np.random.Philox(key=[11, 77]))
    masses, banded, banded_diff, forced = [], 0, 0, 0
    for r in range(R):
        inp["uniforms"][:, 2] = ru.random(B, dtype=np.float32)
        t["uniforms"].copy_(torch.from_numpy(inp["uniforms"]))
        out = svl.verify_chain(t["draft_tokens"], t["draft_logits"], t["target_logits"], t["temperature"],
                               t["uniforms"])
        torch.cuda.synchronize()
        got = {k: (v.cpu().numpy() if v is not None else None) for k, v in out.items()}
        ref = orc.verify_chain(inp)
        st = compare_chain(inp, got, ref, f"{name} set {r}")
        banded += st["banded"]
        banded_diff += st["banded_mismatch"]
        forced += int((ref["accepted_len"] == inp["reject_at"]).sum())
        masses.append(ref["final_mass"])
    mass = np.concatenate(masses)
    print(f"[small residual] chain {name}: {mass.size} draws, {forced} forced rejections, banded {banded} "
          f"(differing {banded_diff}), mass decades {_decades(mass)}", flush=True)
    assert forced == B * R
    assert mass.max() < 0.05


TREE_CASES = [
    ("f32 sigma 2e-3 offset", W.F32, dict(draft_sigma=2e-3, offset=(-4.0, 4.0)), 48, 16),
    ("f32 sigma 2e-4", W.F32, dict(draft_sigma=2e-4), 48, 16),
    ("bf16 density 0.3", W.BF16, dict(density=0.3), 48, 16),
]


@pytest.mark.parametrize("case", TREE_CASES, ids=[c[0] for c in TREE_CASES])
def test_tree_small_residual(svl, orc, case):
    import torch

    name, dt, kw, B, R = case
    inp = W.near_copy_tree_inputs(B, V, dt, seed=13, **kw)
    t = tree_sampled_tensors(inp)
    ru = np.random.Generator(np.random.Philox(key=[13, 77]))
    want_nodes = np.array([[-1, -1, -1], [1, -1, -1], [2, -1, -1]])[np.arange(B) % 3]
    masses, banded, banded_diff = [], 0, 0
    for r in range(R):
        inp["uniforms"][:, 0] = ru.random(B, dtype=np.float32)
        t["uniforms"].copy_(torch.from_numpy(inp["uniforms"]))
        out = svl.verify_tree_sampled(t["node_tokens"], t["parent"], int(inp["max_depth"]), t["draft_logits"],
                                      t["target_logits"], t["temperature"], t["uniforms"])
        torch.cuda.synchronize()
        got = {k: (v.cpu().numpy() if v is not None else None) for k, v in out.items()}
        ref = orc.verify_tree_sampled(inp)
        assert (ref["accepted_nodes"] == want_nodes).all()
        st = compare_tree_sampled(got, ref, f"{name} set {r}")
        banded += st["banded"]
        banded_diff += st["banded_mismatch"]
        masses.append(ref["final_mass"])
    mass = np.concatenate(masses)
    print(f"[small residual] tree {name}: {mass.size} draws, banded {banded} (differing {banded_diff}), "
          f"mass decades {_decades(mass)}", flush=True)
    assert mass.max() < 0.05


# name, generator, B, sets of final-draw uniforms.  The near-copy rows force a
# rejection in every sequence; the ordinary chain rows reject where their
# uniforms say.  B = 256 takes the acceptance kernel.
THRESHOLD_CASES = [
    ("f32 sigma 0.6 offset", lambda B: W.near_copy_chain_inputs(B, 2, V, W.F32, seed=17, draft_sigma=0.6,
                                                                offset=(-4.0, 4.0)), 64, 16),
    ("f32 sigma 0.6 offset acceptance kernel",
     lambda B: W.near_copy_chain_inputs(B, 2, V, W.F32, seed=19, draft_sigma=0.6, offset=(-4.0, 4.0)), 256, 4),
    ("bf16 sigma 0.4", lambda B: W.chain_inputs(B, 4, V, W.BF16, seed=17, target_sigma=3.0, zipf_s=1.1,
                                                 draft_sigma=0.4, temperature=0.7), 128, 16),
    ("bf16 sigma 0.4 acceptance kernel",
     lambda B: W.chain_inputs(B, 4, V, W.BF16, seed=19, target_sigma=3.0, zipf_s=1.1, draft_sigma=0.4,
                              temperature=0.7), 256, 8),
]


@pytest.mark.parametrize("case", THRESHOLD_CASES, ids=[c[0] for c in THRESHOLD_CASES])
def test_chain_residual_mass_threshold(svl, orc, case):
    import torch

    name, make, B, R = case
    inp = make(B)
    k = inp["k"]
    t = chain_tensors(inp)
    ru = np.random.Generator(np.random.Philox(key=[17, 77]))
    masses, banded, banded_diff = [], 0, 0
    for r in range(R):
        inp["uniforms"][:, k] = ru.random(B, dtype=np.float32)
        t["uniforms"].copy_(torch.from_numpy(inp["uniforms"]))
        out = svl.verify_chain(t["draft_tokens"], t["draft_logits"], t["target_logits"], t["temperature"],
                               t["uniforms"])
        torch.cuda.synchronize()
        got = {kk: (v.cpu().numpy() if v is not None else None) for kk, v in out.items()}
        ref = orc.verify_chain(inp)
        st = compare_chain(inp, got, ref, f"{name} set {r}")
        banded += st["banded"]
        banded_diff += st["banded_mismatch"]
        masses.append(ref["final_mass"][ref["accepted_len"] < k])
    mass = np.concatenate(masses)
    below, near, above = int((mass < 0.2).sum()), int(((mass >= 0.2) & (mass < 0.4)).sum()), int((mass >= 0.4).sum())
    print(f"[residual threshold] chain {name}: {mass.size} residual draws, W < 0.2: {below}, "
          f"0.2 <= W < 0.4: {near}, W >= 0.4: {above}, banded {banded} (differing {banded_diff})", flush=True)
    # both forms of the draw are exercised, and near the threshold
    assert below >= mass.size // 10 and near >= mass.size // 10


FLAT_CASES = [("f32", W.F32, 64, 16), ("f32 acceptance kernel", W.F32, 256, 4),
              ("bf16", W.BF16, 64, 16), ("bf16 acceptance kernel", W.BF16, 256, 4)]


@pytest.mark.parametrize("case", FLAT_CASES, ids=[c[0] for c in FLAT_CASES])
def test_chain_cheap_form_on_flat_tails(svl, orc, case):
    import torch

    name, dt, B, R = case
    inp = W.flat_tail_chain_inputs(B, V, dt, seed=23)
    t = chain_tensors(inp)
    ru = np.random.Generator(np.random.Philox(key=[23, 77]))
    masses, banded, banded_diff = [], 0, 0
    for r in range(R):
        inp["uniforms"][:, 1] = ru.random(B, dtype=np.float32)
        t["uniforms"].copy_(torch.from_numpy(inp["uniforms"]))
        out = svl.verify_chain(t["draft_tokens"], t["draft_logits"], t["target_logits"], t["temperature"],
                               t["uniforms"])
        torch.cuda.synchronize()
        got = {kk: (v.cpu().numpy() if v is not None else None) for kk, v in out.items()}
        ref = orc.verify_chain(inp)
        st = compare_chain(inp, got, ref, f"flat tail {name} set {r}")
        banded += st["banded"]
        banded_diff += st["banded_mismatch"]
        assert (ref["accepted_len"] == 0).all()
        masses.append(ref["final_mass"])
    mass = np.concatenate(masses)
    print(f"[residual threshold] flat tail {name}: {mass.size} draws, W {mass.min():.3f}..{mass.max():.3f}, "
          f"banded {banded} (differing {banded_diff})", flush=True)
    assert mass.min() > 0.2
    assert banded < mass.size // 5  # the residual's boundaries lie apart: most draws are compared
