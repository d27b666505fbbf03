"""Pins of the fp64 CPU oracle against facts it did not compute itself.

Every test here runs on the CPU (no GPU marker).  The pins are: a hand-derived
worked example, library routines (scipy logsumexp / softmax, numpy argmax,
cumsum + searchsorted), closed forms (total variation, geometric acceptance
lengths), invariants of the scheme (at most k accepted and k+1 emitted;
identical distributions accept everything; temperature 0 is argmax matching),
brute force on tiny trees, and statistical tests of the distribution the
scheme guarantees (the emitted token is distributed as the target's).  Planted
mistakes in the oracle must fail the statistical tests, which shows their power.

Scheme: "Accelerating Sonar through speculation" (Perplexity, 2025), sections
"Speculative decoding", "Target-Draft" and "EAGLE"; acceptance and residual
rule from Leviathan et al., first in the pages' references.
"""

import json
import os

import numpy as np
import pytest
from scipy import special, stats

import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------ O1: normalisers ---

@pytest.mark.parametrize("dtype", [W.F32, W.BF16])
@pytest.mark.parametrize("T", [0.3, 0.7, 1.0, 1.3])
def test_logz_matches_scipy_logsumexp(orc, dtype, T):
    rng = np.random.default_rng(11)
    V = 5003
    raw = (3.0 * rng.standard_normal((6, V)) + W.zipf_bias(V, 1.1, 3)).astype(np.float32)
    logits = W.to_dtype(raw, dtype)
    vals = W.values(logits, dtype).astype(np.float64)
    got = orc.row_logz(logits, dtype, T)
    want = special.logsumexp(vals / np.float64(np.float32(T)), axis=-1)
    np.testing.assert_allclose(got, want, rtol=1e-13, atol=1e-12)


def test_constant_rows_are_uniform(orc):
    """Constant logits give P = 1/V: every draft accepted (p = q) and the bonus
    draw is the inverse CDF of the uniform distribution, y = floor(u V)."""
    B, k, V = 64, 3, 1000
    rng = np.random.default_rng(5)
    u = rng.random((B, k + 1), dtype=np.float32)
    # keep u V away from integers so the rounding of the cumulative sums is moot
    frac = (u[:, k].astype(np.float64) * V) % 1.0
    u[:, k] = np.where((frac < 1e-3) | (frac > 1 - 1e-3), np.float32(0.5 / V), u[:, k])
    inp = dict(B=B, k=k, V=V, dtype=W.F32,
               draft_tokens=rng.integers(0, V, (B, k)).astype(np.int32),
               draft_logits=np.full((B, k, V), 0.25, np.float32),
               target_logits=np.full((B, k + 1, V), -1.5, np.float32),
               temperature=np.full(B, 0.8, np.float32), uniforms=u)
    r = orc.verify_chain(inp)
    assert (r["accepted_len"] == k).all()
    np.testing.assert_allclose(r["accept_prob"], 1.0, atol=1e-12)
    np.testing.assert_array_equal(r["emitted"][:, k], np.floor(u[:, k].astype(np.float64) * V).astype(np.int32))


# ------------------------------------------------------------ worked example ---

def test_hand_derived_golden_example(orc):
    g = json.load(open(os.path.join(GOLDEN, "chain_v4_hand.json")))
    V, k = g["V"], g["k"]
    t = np.log(np.array(g["target_probs"], np.float64)).astype(np.float32)
    d = np.log(np.array(g["draft_probs"], np.float64)).astype(np.float32)
    cases = g["cases"]
    B = len(cases)
    inp = dict(B=B, k=k, V=V, dtype=W.F32,
               draft_tokens=np.array([c["draft_tokens"] for c in cases], np.int32),
               draft_logits=np.broadcast_to(d, (B, k, V)).copy(),
               target_logits=np.broadcast_to(t, (B, k + 1, V)).copy(),
               temperature=np.full(B, g["temperature"], np.float32),
               uniforms=np.array([c["uniforms"] for c in cases], np.float32))
    r = orc.verify_chain(inp)
    for i, c in enumerate(cases):
        assert r["accepted_len"][i] == c["accepted_len"], c["why"]
        assert r["emitted"][i].tolist() == c["emitted"], c["why"]
        np.testing.assert_allclose(r["accept_prob"][i], c["accept_prob"], atol=1e-6, err_msg=c["why"])
    assert not r["band"].any()


# ------------------------------------------------------------ invariants ---

@pytest.mark.parametrize("seed", range(1, 6))
@pytest.mark.parametrize("k", [0, 1, 4, 8])
def test_output_bounds(orc, seed, k):
    """At most k drafts accepted and at most k+1 tokens emitted; the accepted
    prefix is the drafts themselves; the rest is -1 padding."""
    inp = W.chain_inputs(32, k, 257, W.F32, seed, target_sigma=2.0, draft_sigma=1.5,
                         temperature=(0.3, 1.3))
    r = orc.verify_chain(inp)
    a, em = r["accepted_len"], r["emitted"]
    assert ((a >= 0) & (a <= k)).all()
    for b in range(inp["B"]):
        assert (em[b, :a[b]] == inp["draft_tokens"][b, :a[b]]).all()
        assert 0 <= em[b, a[b]] < inp["V"]
        assert (em[b, a[b] + 1:] == -1).all()
    assert ((r["accept_prob"] >= 0) & (r["accept_prob"] <= 1)).all()


@pytest.mark.parametrize("dtype", [W.F32, W.BF16])
@pytest.mark.parametrize("T", [0.0, 0.5, 1.0])
def test_identical_distributions_accept_every_draft(orc, dtype, T):
    inp = W.chain_inputs(40, 5, 777, dtype, 9, target_sigma=3.0, draft_sigma=0.0, temperature=T)
    assert (inp["draft_logits"] == inp["target_logits"][:, :5]).all()
    inp["uniforms"][:, :5] = np.float32(1.0) - np.float32(2.0 ** -24)  # the largest uniform
    r = orc.verify_chain(inp)
    assert (r["accepted_len"] == 5).all()
    assert (r["accept_prob"] == 1.0).all()


@pytest.mark.parametrize("dtype", [W.F32, W.BF16])
def test_temperature_zero_is_argmax_matching(orc, dtype):
    inp = W.chain_inputs(48, 4, 300, dtype, 4, target_sigma=2.0, draft_sigma=1.0, temperature=0.0)
    # make half of the drafts the target's argmax so that acceptances happen
    top = np.argmax(W.values(inp["target_logits"], dtype), axis=-1)
    x = inp["draft_tokens"]
    x[::2] = top[::2, :4]
    r = orc.verify_chain(inp)
    g = orc.verify_greedy(dict(inp, kind="greedy"))
    np.testing.assert_array_equal(r["accepted_len"], g["accepted_len"])
    np.testing.assert_array_equal(r["emitted"], g["emitted"])
    # and against numpy's first-occurrence argmax directly
    for b in range(inp["B"]):
        a = 0
        while a < 4 and x[b, a] == top[b, a]:
            a += 1
        assert r["accepted_len"][b] == a
        assert r["emitted"][b, a] == top[b, a]
    assert not r["band"].any()


def test_thread_count_does_not_change_results(orc):
    inp = W.chain_inputs(24, 4, 2000, W.BF16, 2, target_sigma=3.0, zipf_s=1.1, draft_sigma=1.0, temperature=0.7)
    orc.set_num_threads(1)
    r1 = orc.verify_chain(inp)
    orc.set_num_threads(max(2, os.cpu_count() or 2))
    r8 = orc.verify_chain(inp)
    for key in r1:
        np.testing.assert_array_equal(r1[key], r8[key])


# ------------------------------------------------------------ closed forms ---

def _softmax_rows(vals, T):
    return special.softmax(np.asarray(vals, np.float64) / np.float64(np.float32(T)), axis=-1)


def test_residual_mass_is_total_variation(orc):
    """At a rejection the residual mass W = sum max(0, p - q) equals
    1 - sum min(p, q); after full acceptance W = 1."""
    inp = W.chain_inputs(200, 3, 600, W.F32, 13, target_sigma=2.0, draft_sigma=(0.2, 3.0),
                         temperature=(0.3, 1.3))
    r = orc.verify_chain(inp)
    tv = W.values(inp["target_logits"], W.F32)
    dv = W.values(inp["draft_logits"], W.F32)
    for b in range(inp["B"]):
        a = r["accepted_len"][b]
        T = inp["temperature"][b]
        if a < 3:
            p = _softmax_rows(tv[b, a], T)
            q = _softmax_rows(dv[b, a], T)
            want = 1.0 - np.minimum(p, q).sum()
        else:
            want = 1.0
        assert abs(r["final_mass"][b] - want) < 1e-12


def test_accept_prob_matches_scipy_softmax(orc):
    inp = W.chain_inputs(30, 4, 900, W.BF16, 21, target_sigma=3.0, zipf_s=1.1, draft_sigma=1.0, temperature=0.7)
    r = orc.verify_chain(inp)
    tv = W.values(inp["target_logits"], W.BF16)
    dv = W.values(inp["draft_logits"], W.BF16)
    for b in range(inp["B"]):
        for i in range(4):
            x = inp["draft_tokens"][b, i]
            p = _softmax_rows(tv[b, i], 0.7)[x]
            q = _softmax_rows(dv[b, i], 0.7)[x]
            assert abs(r["accept_prob"][b, i] - min(1.0, p / q)) < 1e-12


def test_inverse_cdf_brute_force_over_uniform_grid(orc):
    """With rejection forced at position 0, the token drawn for a grid of
    uniforms equals numpy's searchsorted over the normalised cumulative residual,
    and each token's share of the grid is its residual probability."""
    V, n = 12, 4096
    rng = np.random.default_rng(3)
    t = rng.standard_normal((2, V)).astype(np.float32)
    d = rng.standard_normal((1, V)).astype(np.float32)
    d[0, 0] = 8.0  # q(0) ~ 1 while p(0) is small: drafting token 0 is rejected at u0 = 0.999
    grid = ((np.arange(n) + 0.5) / n).astype(np.float32)
    inp = dict(B=n, k=1, V=V, dtype=W.F32, draft_tokens=np.zeros((n, 1), np.int32),
               draft_logits=np.broadcast_to(d, (n, 1, V)).copy(),
               target_logits=np.broadcast_to(t, (n, 2, V)).copy(),
               temperature=np.ones(n, np.float32),
               uniforms=np.stack([np.full(n, 0.999, np.float32), grid], axis=1))
    r = orc.verify_chain(inp)
    assert (r["accepted_len"] == 0).all()
    p = _softmax_rows(t[0], 1.0)
    q = _softmax_rows(d[0], 1.0)
    w = np.maximum(p - q, 0.0)
    cdf = np.cumsum(w) / w.sum()
    want = np.searchsorted(cdf, grid.astype(np.float64), side="right")
    np.testing.assert_array_equal(r["emitted"][:, 0], want)
    share = np.bincount(r["emitted"][:, 0], minlength=V) / n
    np.testing.assert_allclose(share, w / w.sum(), atol=1.0 / n + 1e-12)
    # u = 0 selects the first token with positive residual mass
    inp["uniforms"][:, 1] = 0.0
    r0 = orc.verify_chain(inp)
    assert (r0["emitted"][:, 0] == np.flatnonzero(w > 0)[0]).all()


# ------------------------------------------------------------ distribution ---

V_CHI, K_CHI, N_CHI, BLOCKS = 16, 4, 1_000_000, 5


def _chi_rows():
    rng = np.random.default_rng(2024)
    t = (1.5 * rng.standard_normal((K_CHI + 1, V_CHI))).astype(np.float32)
    d = (t[:K_CHI] + rng.standard_normal((K_CHI, V_CHI))).astype(np.float32)
    return t, d


def _run_trials(orc, t, d, T=1.0):
    acc, em = [], []
    per = N_CHI // BLOCKS
    for blk in range(BLOCKS):
        inp = W.repeated_trials(t, d, T, per, seed=77, block=blk)
        r = orc.verify_chain(inp)
        acc.append(r["accepted_len"])
        em.append(r["emitted"])
    return np.concatenate(acc), np.concatenate(em)


def _chi_pvalues(t, acc, em, T=1.0):
    out = []
    for j in range(K_CHI + 1):
        sel = acc >= j
        counts = np.bincount(em[sel, j], minlength=V_CHI)
        p = _softmax_rows(t[j], T)
        out.append(stats.chisquare(counts, p * sel.sum()).pvalue)
    return np.array(out)


@pytest.fixture(scope="module")
def chi_trials(orc):
    t, d = _chi_rows()
    acc, em = _run_trials(orc, t, d)
    return t, d, acc, em


def test_emitted_token_follows_target_distribution(chi_trials):
    """10^6 seeded trials, V = 16, k = 4: given the first j drafts accepted, the
    token at position j (accepted draft or final draw) is distributed as the
    target row j, for every j = 0..k (chi-square)."""
    t, d, acc, em = chi_trials
    pv = _chi_pvalues(t, acc, em)
    assert (pv > 1e-4).all(), pv


def test_acceptance_rate_is_overlap(chi_trials):
    """P(draft j accepted | drafts < j accepted) = sum_v min(p_v, q_v) (binomial)."""
    t, d, acc, em = chi_trials
    for j in range(K_CHI):
        n = (acc >= j).sum()
        hits = (acc >= j + 1).sum()
        alpha = np.minimum(_softmax_rows(t[j], 1.0), _softmax_rows(d[j], 1.0)).sum()
        z = (hits - n * alpha) / np.sqrt(n * alpha * (1 - alpha))
        assert abs(z) < 5, (j, alpha, hits / n)


@pytest.mark.parametrize("T", [0.5, 1.0, 2.5])
def test_plain_sampling_follows_target_distribution(orc, T):
    """k = 0 (no drafts): over 10^6 seeded trials at V = 16 the sampled token
    is distributed as softmax(t / T) (chi-square), and the same counts reject
    a softmax at a wrong temperature, so the test has the power to see one."""
    t, _ = _chi_rows()
    inp = W.repeated_trials(t[:1], np.zeros((0, V_CHI), np.float32), T, N_CHI, seed=91)
    r = orc.verify_chain(inp)
    assert (r["accepted_len"] == 0).all()
    counts = np.bincount(r["emitted"][:, 0], minlength=V_CHI)
    assert stats.chisquare(counts, _softmax_rows(t[0], T) * N_CHI).pvalue > 1e-4
    assert stats.chisquare(counts, _softmax_rows(t[0], 1.7) * N_CHI).pvalue < 1e-12


@pytest.mark.parametrize("mutation", ["MUT_SAMPLE_TARGET_AT_MISMATCH", "MUT_RESIDUAL_SWAPPED",
                                      "MUT_ROWS_SHIFTED", "MUT_ACCEPT_INVERTED"])
def test_planted_mistakes_fail_the_distribution_test(orc, mutated, mutation):
    t, d = _chi_rows()
    mutated(getattr(orc, mutation))
    acc, em = _run_trials(orc, t, d)
    assert _chi_pvalues(t, acc, em).min() < 1e-12


# ------------------------------------------------------------ greedy ---

@pytest.mark.parametrize("dtype", [W.F32, W.BF16])
def test_greedy_matches_numpy_argmax_with_planted_ties(orc, dtype):
    B, k, V = 64, 5, 1531
    inp = W.greedy_inputs(B, k, V, dtype, 8, match_p=0.8)
    t = inp["target_logits"]
    rng = np.random.default_rng(1)
    # plant exact ties: copy each row's maximum to an earlier and a later index
    vals = W.values(t, dtype)
    later = np.zeros((B, k + 1), np.int64)
    for b in range(0, B, 2):
        for j in range(k + 1):
            m = int(np.argmax(vals[b, j]))
            lo = int(rng.integers(0, m)) if m > 0 else m
            hi = int(rng.integers(m + 1, V)) if m + 1 < V else m
            t[b, j, lo] = t[b, j, m]
            t[b, j, hi] = t[b, j, m]
            later[b, j] = hi
    top = np.argmax(W.values(t, dtype), axis=-1)
    np.testing.assert_array_equal(orc.row_argmax(t, dtype), top)
    # drafts: the first argmax, except that some tied rows draft a later tied copy
    # (a tie is not a match: only the lowest index is the argmax)
    x = top[:, :k].copy()
    x[0::4, 1] = later[0::4, 1]
    x[1::3, 2] = (x[1::3, 2] + 1) % V
    inp["draft_tokens"] = x.astype(np.int32)
    r = orc.verify_greedy(inp)
    for b in range(B):
        a = 0
        while a < k and x[b, a] == top[b, a]:
            a += 1
        assert r["accepted_len"][b] == a
        assert r["emitted"][b, :a].tolist() == x[b, :a].tolist()
        assert r["emitted"][b, a] == top[b, a]
        assert (r["emitted"][b, a + 1:] == -1).all()


def test_greedy_planted_last_index_tie_is_caught(orc, mutated):
    V = 100
    t = np.zeros((1, 1, V), np.float32)
    t[0, 0, [10, 70]] = 5.0
    inp = dict(B=1, k=0, V=V, dtype=W.F32, draft_tokens=np.zeros((1, 0), np.int32), target_logits=t)
    assert orc.verify_greedy(inp)["emitted"][0, 0] == 10
    mutated(orc.MUT_ARGMAX_LAST)
    assert orc.verify_greedy(inp)["emitted"][0, 0] == 70


def test_greedy_generator_mean_accepted_length(orc):
    """Drafts match the target argmax independently with probability 0.8, so
    P(a >= i) = 0.8^i and E[a] = sum_{i=1..5} 0.8^i = 2.68928."""
    inp = W.greedy_inputs(20000, 5, 64, W.BF16, 3, match_p=0.8)
    a = orc.verify_greedy(inp)["accepted_len"]
    want = sum(0.8 ** i for i in range(1, 6))
    se = a.std() / np.sqrt(a.size)
    assert abs(a.mean() - want) < 5 * se
    for i in range(1, 6):
        assert abs((a >= i).mean() - 0.8 ** i) < 5 * np.sqrt(0.8 ** i * (1 - 0.8 ** i) / a.size)


# ------------------------------------------------------------ tree ---

def _brute_force_tree(parent, tokens, top):
    """Enumerate every root path; keep the deepest whose every edge matches."""
    N = len(parent)
    best, best_path = 0, []
    for n in range(N):
        path = [n]
        while path[-1] != 0:
            path.append(int(parent[path[-1]]))
        path = path[::-1]  # root ... n
        ok = all(tokens[path[i + 1]] == top[path[i]] for i in range(len(path) - 1))
        if ok and len(path) - 1 > best:
            best, best_path = len(path) - 1, path[1:]
    end = best_path[-1] if best_path else 0
    return best, [int(tokens[m]) for m in best_path] + [int(top[end])], best_path


@pytest.mark.parametrize("seed", range(1, 9))
def test_tree_matches_brute_force(orc, seed):
    N, V, B = 14, 6, 32
    inp = W.tree_inputs(B, N, V, W.F32, seed, max_branch=3, max_depth=5, match_p=0.7)
    r = orc.verify_tree(inp)
    top = np.argmax(W.values(inp["target_logits"], W.F32), axis=-1)
    for b in range(B):
        d, em, nodes = _brute_force_tree(inp["parent"], inp["node_tokens"][b], top[b])
        assert r["accepted_len"][b] == d
        assert r["emitted"][b, :d + 1].tolist() == em
        assert (r["emitted"][b, d + 1:] == -1).all()
        assert r["accepted_nodes"][b, :d].tolist() == nodes


def test_linear_tree_is_chain_greedy(orc):
    N, V, B = 9, 50, 40
    parent = np.arange(-1, N - 1, dtype=np.int32)
    inp = W.tree_inputs(B, N, V, W.BF16, 5, parent=parent, match_p=0.85)
    r = orc.verify_tree(inp)
    g = orc.verify_greedy(dict(kind="greedy", B=B, k=N - 1, V=V, dtype=W.BF16,
                               draft_tokens=inp["node_tokens"][:, 1:].copy(),
                               target_logits=inp["target_logits"]))
    np.testing.assert_array_equal(r["accepted_len"], g["accepted_len"])
    np.testing.assert_array_equal(r["emitted"], g["emitted"])


def test_star_tree_accepts_at_most_one(orc):
    N, V, B = 20, 30, 50
    parent = np.zeros(N, np.int32)
    parent[0] = -1
    inp = W.tree_inputs(B, N, V, W.F32, 6, parent=parent, match_p=0.3)
    r = orc.verify_tree(inp)
    assert (r["accepted_len"] <= 1).all()
    assert (r["accepted_len"] == 1).any()


def test_tree_equal_depth_tie_takes_lowest_index(orc, mutated):
    # root with two children that both carry the root's argmax
    N, V = 3, 8
    t = np.zeros((1, N, V), np.float32)
    t[0, 0, 5] = 3.0
    t[0, 1, 1] = 3.0
    t[0, 2, 2] = 3.0
    inp = dict(B=1, N=N, V=V, dtype=W.F32, node_tokens=np.array([[0, 5, 5]], np.int32),
               parent=np.array([-1, 0, 0], np.int32), max_depth=1, target_logits=t)
    r = orc.verify_tree(inp)
    assert r["accepted_len"][0] == 1 and r["accepted_nodes"][0, 0] == 1
    assert r["emitted"][0].tolist() == [5, 1]
    mutated(orc.MUT_TREE_TIE_HIGHEST)
    r = orc.verify_tree(inp)
    assert r["accepted_nodes"][0, 0] == 2 and r["emitted"][0].tolist() == [5, 2]


def test_tree_invalid_parent_or_depth_marks_sequence(orc):
    N, V = 4, 8
    t = np.zeros((2, N, V), np.float32)
    parent = np.array([[-1, 0, 3, 1], [-1, 0, 1, 2]], np.int32)  # seq 0: parent[2] = 3 >= 2
    inp = dict(B=2, N=N, V=V, dtype=W.F32, node_tokens=np.zeros((2, N), np.int32),
               parent=parent, max_depth=2, target_logits=t)  # seq 1 has depth 3 > 2
    r = orc.verify_tree(inp)
    assert r["accepted_len"].tolist() == [-1, -1]
    assert (r["emitted"] == -1).all() and (r["accepted_nodes"] == -1).all()


# ------------------------------------------------------------ commit ---

def test_commit_matches_list_semantics(orc):
    """Appending each sequence's a+1 committed tokens, written as list
    concatenation, against the oracle's index arithmetic."""
    rng = np.random.default_rng(12)
    B, width, cap = 300, 6, 40
    acc = rng.integers(-1, width, B).astype(np.int32)
    acc[::17] = width + 2  # more tokens than the row holds: refused
    em = rng.integers(0, 1000, (B, width)).astype(np.int32)
    lens = rng.integers(0, cap, B).astype(np.int32)
    hist = rng.integers(0, 1000, (B, cap)).astype(np.int32)
    r = orc.commit_tokens(acc, em, lens, hist)
    packed, offs = [], [0]
    for b in range(B):
        old = list(hist[b, :lens[b]])
        a = int(acc[b])
        ok = 0 <= a < width and lens[b] + a + 1 <= cap
        new = list(em[b, :a + 1]) if ok else []
        assert list(r["history"][b, :lens[b] + len(new)]) == old + new
        assert list(r["history"][b, lens[b] + len(new):]) == list(hist[b, lens[b] + len(new):])
        assert r["seq_len"][b] == lens[b] + len(new)
        assert r["status"][b] == (0 if ok else (2 if a < 0 else 1))
        packed += new
        offs.append(offs[-1] + len(new))
    assert r["packed"].tolist() == packed
    assert r["packed_offsets"].tolist() == offs
    # without a history nothing limits the lengths
    r2 = orc.commit_tokens(acc, em, lens)
    assert (r2["seq_len"] == lens + np.where((acc >= 0) & (acc < width), acc + 1, 0)).all()


def test_commit_refuses_rows_that_would_overflow(orc):
    """A count of INT32_MAX, or (without a history, which has no capacity) a
    length that would pass INT32_MAX, is refused with status 1 and leaves the
    sequence untouched; a length that reaches INT32_MAX exactly is committed."""
    imax = int(np.iinfo(np.int32).max)
    acc = np.array([imax, 1, 2, 0], np.int32)
    em = np.arange(12, dtype=np.int32).reshape(4, 3)
    lens = np.array([5, imax - 2, imax - 2, imax], np.int32)
    r = orc.commit_tokens(acc, em, lens)
    assert r["status"].tolist() == [1, 0, 1, 1]
    assert r["seq_len"].tolist() == [5, imax, imax - 2, imax]
    assert r["packed"].tolist() == [3, 4]
    assert r["packed_offsets"].tolist() == [0, 0, 2, 2, 2]


# ------------------------------------------------------------ sampled tree ---
# Multi-step speculative sampling (SpecInfer, Miao et al. 2023; the rule the
# EAGLE work applies to its trees): the pages give no rule for sampled trees.

def _chain_as_tree(inp):
    """A chain laid out as a linear tree: node i >= 1 carries draft i-1 and is
    scored by rows i-1; u_tree[i] = u_chain[i-1], u_tree[0] = u_chain[k]."""
    B, k, V = inp["B"], inp["k"], inp["V"]
    N = k + 1
    draft = np.zeros((B, N, V), dtype=inp["draft_logits"].dtype)
    draft[:, :k] = inp["draft_logits"]
    tok = np.zeros((B, N), np.int32)
    tok[:, 1:] = inp["draft_tokens"]
    u = np.empty((B, N), np.float32)
    u[:, 1:] = inp["uniforms"][:, :k]
    u[:, 0] = inp["uniforms"][:, k]
    return dict(B=B, N=N, V=V, dtype=inp["dtype"], node_tokens=tok, parent=np.arange(-1, N - 1, dtype=np.int32),
                max_depth=k, draft_logits=draft, target_logits=inp["target_logits"],
                temperature=inp["temperature"], uniforms=u)


@pytest.mark.parametrize("seed", [1, 2, 3])
@pytest.mark.parametrize("dtype", [W.F32, W.BF16])
def test_sampled_linear_tree_is_chain(orc, seed, dtype):
    """On a linear tree (one child per node) the walk is chain speculative
    sampling: same accepted lengths, tokens and band flags, T = 0 included."""
    B = 96
    temps = np.random.default_rng(seed).uniform(0.3, 1.3, B).astype(np.float32)
    temps[::4] = 0.0
    inp = W.chain_inputs(B, 4, 3001, dtype, seed, target_sigma=2.0, zipf_s=1.1, draft_sigma=(0.2, 2.5),
                         temperature=temps)
    c = orc.verify_chain(inp)
    t = orc.verify_tree_sampled(_chain_as_tree(inp))
    np.testing.assert_array_equal(t["accepted_len"], c["accepted_len"])
    np.testing.assert_array_equal(t["emitted"], c["emitted"])
    np.testing.assert_array_equal(t["band"], c["band"])
    for b in range(B):
        a = c["accepted_len"][b]
        np.testing.assert_array_equal(t["accepted_nodes"][b, :a], np.arange(1, a + 1))


def _first_child_path(parent):
    path, n = [], 0
    while True:
        kids = np.flatnonzero(parent == n)
        kids = kids[kids > 0]
        if kids.size == 0:
            return path
        n = int(kids[0])
        path.append(n)


@pytest.mark.parametrize("dtype", [W.F32, W.BF16])
@pytest.mark.parametrize("T", [0.5, 1.0])
def test_sampled_tree_identical_rows_keep_first_child(orc, dtype, T):
    """Draft rows equal to target rows give tau = 1 for every tested child, so
    the walk keeps the lowest-index child at every node down to a leaf."""
    inp = W.sampled_tree_inputs(8, 40, 2000, dtype, 5, temperature=T)
    inp["draft_logits"] = inp["target_logits"].copy()
    r = orc.verify_tree_sampled(inp)
    path = _first_child_path(inp["parent"])
    assert (r["accepted_len"] == len(path)).all()
    for b in range(inp["B"]):
        np.testing.assert_array_equal(r["accepted_nodes"][b, :len(path)], path)
        np.testing.assert_array_equal(r["emitted"][b, :len(path)], inp["node_tokens"][b, path])


def _distinct_siblings(inp):
    """Give equal-token siblings distinct tokens that miss the parent's argmax."""
    tok = inp["node_tokens"].copy()
    par = inp["parent"]
    V = inp["V"]
    top = np.argmax(W.values(inp["target_logits"], inp["dtype"]), axis=-1)
    for b in range(inp["B"]):
        for n in range(inp["N"]):
            seen = set()
            for i in np.flatnonzero(par == n):
                if i == 0:
                    continue
                y = int(tok[b, i])
                while y in seen:
                    y = (y + 1) % V
                    if y == top[b, n]:
                        y = (y + 1) % V
                seen.add(y)
                tok[b, i] = y
    inp["node_tokens"] = tok
    return inp


@pytest.mark.parametrize("seed", [1, 2])
def test_sampled_tree_temperature_zero_is_greedy_tree(orc, seed):
    """At T = 0 every distribution is one-hot at its first argmax: a child is
    kept iff its token is the parent's target argmax, and the final token is
    the last kept node's argmax -- the greedy tree, when siblings differ."""
    inp = _distinct_siblings(W.tree_inputs(12, 48, 1500, W.BF16, seed, match_p=0.7))
    rng = np.random.default_rng(seed)
    inp["draft_logits"] = W.to_dtype(2.0 * rng.standard_normal(inp["target_logits"].shape, dtype=np.float32), W.BF16)
    inp["temperature"] = np.zeros(inp["B"], np.float32)
    inp["uniforms"] = rng.random((inp["B"], inp["N"]), dtype=np.float32)
    g = orc.verify_tree(inp)
    s = orc.verify_tree_sampled(inp)
    np.testing.assert_array_equal(s["accepted_len"], g["accepted_len"])
    np.testing.assert_array_equal(s["emitted"], g["emitted"])
    np.testing.assert_array_equal(s["accepted_nodes"], g["accepted_nodes"])


def test_sampled_tree_invalid_parent_or_depth_marks_sequence(orc):
    inp = W.sampled_tree_inputs(3, 12, 500, W.F32, 2)
    par = np.tile(inp["parent"], (3, 1))
    par[1, 5] = 7            # a parent after its child
    inp["parent"] = par
    r = orc.verify_tree_sampled(inp)
    assert r["accepted_len"][1] == -1 and (r["emitted"][1] == -1).all() and (r["accepted_nodes"][1] == -1).all()
    assert (r["accepted_len"][[0, 2]] >= 0).all()
    inp["parent"] = inp["parent"][0].copy()
    inp["max_depth"] = 0
    r = orc.verify_tree_sampled(inp)
    assert (r["accepted_len"] == -1).all()


V_TREE, N_TREE, TREE_BLOCKS = 8, 1_000_000, 5


def _tree_tables():
    rng = np.random.default_rng(4242)
    V = V_TREE
    root_t = (1.5 * rng.standard_normal(V)).astype(np.float32)
    root_d = (root_t + rng.standard_normal(V)).astype(np.float32)
    F = (1.5 * rng.standard_normal((V, V))).astype(np.float32)
    G = (F + rng.standard_normal((V, V))).astype(np.float32)
    H = (1.5 * rng.standard_normal((V, V))).astype(np.float32)
    return root_t, root_d, F, G, H


def _run_tree_trials(orc, tables, T=1.0):
    acc, em, nodes = [], [], []
    per = N_TREE // TREE_BLOCKS
    for blk in range(TREE_BLOCKS):
        r = orc.verify_tree_sampled(W.sampled_tree_trials(*tables, T, per, seed=91, block=blk))
        acc.append(r["accepted_len"])
        em.append(r["emitted"])
        nodes.append(r["accepted_nodes"])
    return np.concatenate(acc), np.concatenate(em), np.concatenate(nodes)


def _tree_chi_pvalues(tables, acc, em, T=1.0):
    """p-values of: y1 ~ p_root; y2 | y1 ~ F[y1]; y3 | y2 ~ H[y2]."""
    root_t, root_d, F, G, H = tables
    V = V_TREE
    out = [stats.chisquare(np.bincount(em[:, 0], minlength=V), _softmax_rows(root_t, T) * len(acc)).pvalue]
    for j, table in ((1, F), (2, H)):
        sel = acc >= j
        prev, cur = em[sel, j - 1], em[sel, j]
        obs = np.bincount(prev * V + cur, minlength=V * V).reshape(V, V)
        n_prev = obs.sum(axis=1)
        exp = n_prev[:, None] * _softmax_rows(table, T)
        keep = n_prev > 0
        out.append(stats.chisquare(obs[keep].ravel(), exp[keep].ravel(), ddof=int(keep.sum()) - 1).pvalue)
    return np.array(out)


@pytest.fixture(scope="module")
def tree_chi_trials(orc):
    tables = _tree_tables()
    return (tables,) + _run_tree_trials(orc, tables)


def test_sampled_tree_tokens_follow_target_distribution(tree_chi_trials):
    """10^6 seeded trials on a two-level tree (3 children, 2 grandchildren
    each; V = 8; siblings drawn independently from the draft rows): the first
    token follows the root's target row and each later token the target row
    of the token before it (chi-square)."""
    tables, acc, em, nodes = tree_chi_trials
    pv = _tree_chi_pvalues(tables, acc, em)
    assert (pv > 1e-4).all(), pv


def test_sampled_tree_sibling_acceptance_rates(tree_chi_trials):
    """At the root, child 1 is kept with probability sum min(p, q); given its
    rejection, child 2 with probability sum min(r, q) where r is the
    normalised residual max(0, p - q) (binomial z-scores)."""
    tables, acc, em, nodes = tree_chi_trials
    root_t, root_d = tables[0], tables[1]
    p, q = _softmax_rows(root_t, 1.0), _softmax_rows(root_d, 1.0)
    r = np.maximum(p - q, 0.0)
    r /= r.sum()
    first = nodes[:, 0]
    for n, hits, alpha in ((len(first), (first == 1).sum(), np.minimum(p, q).sum()),
                           ((first != 1).sum(), (first == 2).sum(), np.minimum(r, q).sum())):
        z = (hits - n * alpha) / np.sqrt(n * alpha * (1 - alpha))
        assert abs(z) < 5, (alpha, hits / n)


@pytest.mark.parametrize("mutation", ["MUT_TREE_STALE_RESIDUAL", "MUT_SAMPLE_TARGET_AT_MISMATCH"])
def test_sampled_tree_planted_mistakes_fail_the_distribution_test(orc, mutated, mutation):
    tables = _tree_tables()
    mutated(getattr(orc, mutation))
    acc, em, nodes = _run_tree_trials(orc, tables)
    assert _tree_chi_pvalues(tables, acc, em).min() < 1e-12


def test_sampled_tree_hand_derived_golden_example(orc):
    g = json.load(open(os.path.join(GOLDEN, "tree_sampled_v3_hand.json")))
    V, N, cases = g["V"], g["N"], g["cases"]
    B = len(cases)
    lg = lambda key: np.log(np.array([c[key] for c in cases], np.float64)).astype(np.float32)  # noqa: E731
    inp = dict(B=B, N=N, V=V, dtype=W.F32, node_tokens=np.array([c["node_tokens"] for c in cases], np.int32),
               parent=np.array([c["parent"] for c in cases], np.int32), max_depth=g["max_depth"],
               target_logits=lg("target_probs"), draft_logits=lg("draft_probs"),
               temperature=np.full(B, g["temperature"], np.float32),
               uniforms=np.array([c["uniforms"] for c in cases], np.float32))
    r = orc.verify_tree_sampled(inp)
    for i, c in enumerate(cases):
        assert r["accepted_len"][i] == c["accepted_len"], c["why"]
        assert r["emitted"][i].tolist() == c["emitted"], c["why"]
        assert r["accepted_nodes"][i].tolist() == c["accepted_nodes"], c["why"]
    assert not r["band"].any()
