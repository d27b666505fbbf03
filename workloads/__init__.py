"""Seeded synthetic inputs for batched draft-token verification.

This module only *constructs inputs*: Gaussian and Zipf-biased logits, their
rounding to bfloat16, draft tokens drawn for the drafting stage, the
pre-generated uniforms, and random draft trees.  None of the verification
arithmetic (row normalisers, acceptance test, first-rejection scan, residual
distribution, inverse CDF) lives here.  The CPU oracle and the GPU library
consume the arrays produced here unchanged, so both see bit-identical inputs.

Random streams: every purpose (target noise, draft noise, vocabulary
permutation, draft sampling, uniforms, tree shape, ...) draws from its own
numpy ``Philox`` generator keyed by ``(seed, purpose)``.  Generation loops over
sequences in a fixed order, so an input set is a pure function of
``(shape, seed)``.

Draft tokens are drawn from the draft model's temperature softmax with the
Gumbel-max construction: ``argmax_v(d_v / T + G_v)`` with ``G_v`` iid standard
Gumbel is distributed exactly as ``softmax(d / T)``, without computing any
normaliser.  At ``T == 0`` the draft is its own argmax (greedy drafting).

Logits are returned as ``numpy.float32`` arrays (dtype code ``F32``) or as
``numpy.uint16`` bfloat16 bit patterns (dtype code ``BF16``).
"""

from __future__ import annotations

import numpy as np

F32 = 0
BF16 = 1
DTYPE_NAMES = {F32: "f32", BF16: "bf16"}

_PURPOSE = {
    "target": 1,
    "draft": 2,
    "perm": 3,
    "draft_tokens": 4,
    "uniforms": 5,
    "tree": 6,
    "temperature": 7,
    "sigma": 8,
    "tree_tokens": 9,
    "greedy_tokens": 10,
    "tree_uniforms": 11,
}


def rng_for(seed: int, purpose: str) -> np.random.Generator:
    """Philox stream for one random purpose of one seed."""
    return np.random.Generator(np.random.Philox(key=[int(seed), _PURPOSE[purpose]]))


# ---------------------------------------------------------------- bfloat16 ---

def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest, ties to even.

    Inputs must be finite.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float32, exactly."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_dtype(x: np.ndarray, dtype: int) -> np.ndarray:
    """Round float values to the storage dtype (float32 array or bf16 bits)."""
    if dtype == BF16:
        return bf16_bits(x)
    if dtype == F32:
        return np.ascontiguousarray(x, dtype=np.float32)
    raise ValueError(f"unknown dtype code {dtype}")


def values(arr: np.ndarray, dtype: int) -> np.ndarray:
    """Stored logits -> their exact float32 values."""
    return bf16_to_f32(arr) if dtype == BF16 else np.asarray(arr, dtype=np.float32)


# ------------------------------------------------------------ primitives ---

def zipf_bias(V: int, s: float, seed: int) -> np.ndarray:
    """Zipf log-frequency bias over a seeded vocabulary permutation.

    Token v gets rank ``perm[v]`` (0 = most frequent) and bias
    ``-s * ln(1 + rank)``; a Zipf(s) frequency law is ``freq ~ rank**-s``, and the
    additive normalising constant cancels in any softmax.
    """
    perm = rng_for(seed, "perm").permutation(V)
    return (-s * np.log1p(perm.astype(np.float64))).astype(np.float32)


def _other_token(rng: np.random.Generator, avoid: int, V: int) -> int:
    """Uniform over the V-1 tokens different from ``avoid`` (``avoid`` itself
    when V = 1, where there is no other token)."""
    if V < 2:
        return avoid
    r = int(rng.integers(0, V - 1))
    return r if r < avoid else r + 1


def gumbel_max_tokens(vals: np.ndarray, temperature: float, rng: np.random.Generator) -> np.ndarray:
    """Draft tokens for rows ``vals[..., V]`` drawn from softmax(vals / T).

    Gumbel-max: argmax(vals / T + G) with G iid standard Gumbel.  T == 0 gives
    the (first) argmax, i.e. greedy drafting.
    """
    v64 = np.asarray(vals, dtype=np.float64)
    if temperature > 0:
        g = rng.gumbel(size=v64.shape)
        return np.argmax(v64 / float(temperature) + g, axis=-1).astype(np.int32)
    return np.argmax(v64, axis=-1).astype(np.int32)


# ------------------------------------------------------------ chain ---

def chain_inputs(B: int, k: int, V: int, dtype: int, seed: int, *,
                 target_sigma: float = 2.0, zipf_s: float | None = None,
                 draft_sigma=0.5, temperature=1.0) -> dict:
    """Inputs for chain verification.

    target logits  t[b, j, :] = target_sigma * N(0,1) (+ Zipf bias), j = 0..k
    draft logits   d[b, i, :] = t[b, i, :] + sigma_b * N(0,1),      i = 0..k-1
    (both rounded to ``dtype``; draft noise is added to the rounded target).
    ``draft_sigma`` / ``temperature``: a scalar, a (lo, hi) tuple meaning a
    per-sequence uniform draw, or an explicit length-B sequence.
    Draft tokens x[b, i] ~ softmax(d[b, i, :] / T_b) (Gumbel-max).
    uniforms u[b, 0..k] float32 in [0, 1): u[b, i] tests draft i, u[b, k] drives
    the final (residual or bonus) sample.
    """
    temps = _per_seq(temperature, B, seed, "temperature")
    sigmas = _per_seq(draft_sigma, B, seed, "sigma")
    bias = zipf_bias(V, zipf_s, seed) if zipf_s else None
    rt, rd, rx = rng_for(seed, "target"), rng_for(seed, "draft"), rng_for(seed, "draft_tokens")
    np_dt = np.uint16 if dtype == BF16 else np.float32
    target = np.empty((B, k + 1, V), dtype=np_dt)
    draft = np.empty((B, k, V), dtype=np_dt)
    tokens = np.empty((B, k), dtype=np.int32)
    for b in range(B):
        t = (target_sigma * rt.standard_normal((k + 1, V), dtype=np.float32))
        if bias is not None:
            t = t + bias
        target[b] = to_dtype(t, dtype)
        tv = values(target[b, :k], dtype)
        d = tv + np.float32(sigmas[b]) * rd.standard_normal((k, V), dtype=np.float32)
        draft[b] = to_dtype(d, dtype)
        tokens[b] = gumbel_max_tokens(values(draft[b], dtype), float(temps[b]), rx)
    uniforms = rng_for(seed, "uniforms").random((B, k + 1), dtype=np.float32)
    return dict(kind="chain", B=B, k=k, V=V, dtype=dtype, draft_tokens=tokens,
                draft_logits=draft, target_logits=target,
                temperature=temps.astype(np.float32), uniforms=uniforms,
                draft_sigma=sigmas.astype(np.float32))


def _per_seq(spec, B: int, seed: int, purpose: str) -> np.ndarray:
    if isinstance(spec, tuple):
        lo, hi = spec
        return rng_for(seed, purpose).uniform(lo, hi, size=B).astype(np.float32)
    arr = np.asarray(spec, dtype=np.float32)
    if arr.ndim == 0:
        return np.full(B, float(arr), dtype=np.float32)
    assert arr.shape == (B,)
    return arr


def repeated_trials(target_vals: np.ndarray, draft_vals: np.ndarray, temperature: float,
                    n: int, seed: int, block: int = 0) -> dict:
    """``n`` independent trials of one fixed (draft, target) row set.

    ``target_vals`` [k+1, V] and ``draft_vals`` [k, V] are float32 values used as
    F32 logits; every trial draws its own draft tokens (from softmax(d / T)) and
    uniforms.  ``block`` selects a sub-stream so that large trial counts can be
    produced block by block.
    """
    k1, V = target_vals.shape
    k = k1 - 1
    rx = np.random.Generator(np.random.Philox(key=[int(seed), 1000 + 2 * int(block)]))
    ru = np.random.Generator(np.random.Philox(key=[int(seed), 1001 + 2 * int(block)]))
    dv = np.broadcast_to(draft_vals.astype(np.float32), (n, k, V))
    tokens = gumbel_max_tokens(dv, temperature, rx)
    return dict(kind="chain", B=n, k=k, V=V, dtype=F32, draft_tokens=tokens,
                draft_logits=np.ascontiguousarray(dv),
                target_logits=np.ascontiguousarray(np.broadcast_to(target_vals.astype(np.float32), (n, k1, V))),
                temperature=np.full(n, temperature, dtype=np.float32),
                uniforms=ru.random((n, k + 1), dtype=np.float32))


# ------------------------------------------------------------ near-copy drafts ---

# The largest float32 below 1: a test uniform that rejects every draft whose
# acceptance probability is below 1 - 2^-24.
U_MAX = np.float32(1.0) - np.float32(2.0 ** -24)


def bump_bf16(bits: np.ndarray, mask: np.ndarray, up: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns moved by one unit in the last place where ``mask``:
    away from zero where ``up``, towards zero elsewhere (finite, nonzero inputs)."""
    out = np.array(bits, dtype=np.uint16, copy=True)
    step = np.where(up, 1, -1).astype(np.int32)
    out[mask] = (out[mask].astype(np.int32) + step[mask]).astype(np.uint16)
    return out


def near_copy_chain_inputs(B: int, k: int, V: int, dtype: int, seed: int, *, draft_sigma: float = 0.0,
                           density: float = 0.0, offset=0.0, temperature=0.7, target_sigma: float = 3.0,
                           zipf_s: float | None = 1.1) -> dict:
    """Chain inputs whose draft rows nearly copy the target rows, with every
    sequence forced to reject one draft (so that the final draw is a residual
    of small mass).

    target logits  t[b, j, :] = target_sigma * N(0,1) (+ Zipf bias), j = 0..k
    draft logits   float32: d[b, i, :] = t[b, i, :] + offset_b + draft_sigma * N(0,1)
                   bfloat16: d = t, with a random subset of density ``density`` of
                   each row moved one bf16 unit up or down (equally likely)
    ``offset``: a scalar or a (lo, hi) tuple (per-sequence uniform draw); a shift
    of a whole row leaves its distribution unchanged.
    Rejection position j_b uniform in 0..k-1.  Drafts before j_b are drawn from
    the draft softmax and tested with u = 0 (always kept); the draft at j_b is
    the token with the largest d - t (the largest draft/target ratio) and is
    tested with u = U_MAX; u[b, k] drives the residual draw.  Drafts after j_b
    are drawn from the draft softmax (never tested).
    """
    assert k >= 1
    temps = _per_seq(temperature, B, seed, "temperature")
    offs = _per_seq(offset, B, seed, "sigma")
    bias = zipf_bias(V, zipf_s, seed) if zipf_s else None
    rt, rd, rx = rng_for(seed, "target"), rng_for(seed, "draft"), rng_for(seed, "draft_tokens")
    ru = rng_for(seed, "uniforms")
    np_dt = np.uint16 if dtype == BF16 else np.float32
    target = np.empty((B, k + 1, V), dtype=np_dt)
    draft = np.empty((B, k, V), dtype=np_dt)
    tokens = np.empty((B, k), dtype=np.int32)
    uniforms = ru.random((B, k + 1), dtype=np.float32)
    reject_at = rx.integers(0, k, size=B).astype(np.int32)
    for b in range(B):
        t = target_sigma * rt.standard_normal((k + 1, V), dtype=np.float32)
        if bias is not None:
            t = t + bias
        target[b] = to_dtype(t, dtype)
        if dtype == BF16:
            mask = rd.random((k, V)) < density
            up = rd.random((k, V)) < 0.5
            draft[b] = bump_bf16(target[b, :k], mask, up)
        else:
            tv = values(target[b, :k], F32)
            draft[b] = tv + np.float32(offs[b]) + np.float32(draft_sigma) * rd.standard_normal((k, V), dtype=np.float32)
        dv = values(draft[b], dtype)
        tokens[b] = gumbel_max_tokens(dv, float(temps[b]), rx)
        j = int(reject_at[b])
        diff = dv[j].astype(np.float64) - values(target[b, j], dtype).astype(np.float64)
        tokens[b, j] = int(np.argmax(diff))
        uniforms[b, :j] = 0.0
        uniforms[b, j] = U_MAX
    return dict(kind="chain", B=B, k=k, V=V, dtype=dtype, draft_tokens=tokens, draft_logits=draft,
                target_logits=target, temperature=temps.astype(np.float32), uniforms=uniforms,
                reject_at=reject_at)



def flat_tail_chain_inputs(B: int, V: int, dtype: int, seed: int, *, tail: int = 8192, gap: float = 6.2,
                           shift: float = 0.5, noise: float = 0.3, draft_sigma: float = 0.05) -> dict:
    """Chain inputs (k = 1, T = 1) whose rows put most of their mass in a flat
    tail far below the top token, with a residual of moderate mass that the
    rows' coarse masses already show, every sequence forced to reject.

    target logits  t[b, j, v] = noise * N(0,1) + o_v, with o_0 = 0 (the top
                   token), o_v = -gap on ``tail`` tokens spread evenly over the
                   vocabulary, and o_v = -40 elsewhere (no mass)
    draft logits   d[b, 0, v] = t[b, 0, v] + draft_sigma * N(0,1) + shift (v < V/2), - shift (v >= V/2)
    (both rounded to ``dtype``).  With the defaults the tail carries about 92%
    of the mass, the mean of log2(p_max / p_v) under p is about 8, the
    residual's mass W is about 0.23 and the two halves' masses alone differ
    by about 0.22; the residual lives on about tail/2 tokens, so its CDF
    boundaries lie far more than 1e-5 apart.  The draft token is the one with
    the largest d - t, tested with u = U_MAX; u[b, 1] drives the residual draw.
    """
    base = near_copy_chain_inputs(B, 1, V, F32, seed, draft_sigma=draft_sigma, target_sigma=noise, zipf_s=None,
                                  temperature=1.0)
    off = np.full(V, -40.0, dtype=np.float32)
    off[np.linspace(1, V - 1, tail).astype(np.int64)] = -gap
    off[0] = 0.0
    half = np.where(np.arange(V) < V // 2, shift, -shift).astype(np.float32)
    t = values(base["target_logits"], F32) + off
    d = values(base["draft_logits"], F32) + off + half
    target, draft = to_dtype(t, dtype), to_dtype(d, dtype)
    diff = values(draft[:, 0], dtype).astype(np.float64) - values(target[:, 0], dtype).astype(np.float64)
    tokens = np.argmax(diff, axis=-1).astype(np.int32).reshape(B, 1)
    uniforms = base["uniforms"]
    uniforms[:, 0] = U_MAX
    return dict(kind="chain", B=B, k=1, V=V, dtype=dtype, draft_tokens=tokens, draft_logits=draft,
                target_logits=target, temperature=base["temperature"], uniforms=uniforms,
                reject_at=np.zeros(B, dtype=np.int32))

# Tree of the near-copy sampled-tree inputs: the root has children 1, 2, 3;
# node 1 has children 4, 5, 6 and node 2 has child 7.
NEAR_COPY_TREE = np.array([-1, 0, 0, 0, 1, 1, 1, 2], dtype=np.int32)


def near_copy_tree_inputs(B: int, V: int, dtype: int, seed: int, *, draft_sigma: float = 0.0,
                          density: float = 0.0, offset=0.0, temperature=0.7, target_sigma: float = 3.0,
                          zipf_s: float | None = 1.1) -> dict:
    """Sampled-tree inputs on NEAR_COPY_TREE whose draft rows nearly copy the
    target rows (as for near_copy_chain_inputs), with the walk forced into one
    of three paths (sequence b takes mode b % 3):

      0: the three children of the root are rejected; the final token is drawn
         at the root after three rejections;
      1: node 1 is kept, its three children are rejected; the final draw is at
         node 1 after three rejections;
      2: node 1 is rejected, node 2 kept, its one child rejected; the final
         draw is at node 2 after one rejection.

    A child meant to be rejected carries, among the tokens not yet used by
    its siblings, the one with the largest d - t of its parent's rows (so its
    draft probability exceeds its target probability) and is tested with
    u = U_MAX; a child meant to be kept carries the token with the smallest
    d - t (u = 0).  u[b, 0] drives the final draw.
    """
    parent = NEAR_COPY_TREE
    N = parent.shape[0]
    temps = _per_seq(temperature, B, seed, "temperature")
    offs = _per_seq(offset, B, seed, "sigma")
    bias = zipf_bias(V, zipf_s, seed) if zipf_s else None
    rt, rd = rng_for(seed, "target"), rng_for(seed, "draft")
    np_dt = np.uint16 if dtype == BF16 else np.float32
    target = np.empty((B, N, V), dtype=np_dt)
    draft = np.empty((B, N, V), dtype=np_dt)
    tokens = np.zeros((B, N), dtype=np.int32)
    uniforms = rng_for(seed, "tree_uniforms").random((B, N), dtype=np.float32)
    keep = {0: (), 1: (1,), 2: (2,)}
    for b in range(B):
        t = target_sigma * rt.standard_normal((N, V), dtype=np.float32)
        if bias is not None:
            t = t + bias
        target[b] = to_dtype(t, dtype)
        if dtype == BF16:
            mask = rd.random((N, V)) < density
            up = rd.random((N, V)) < 0.5
            draft[b] = bump_bf16(target[b], mask, up)
        else:
            draft[b] = (values(target[b], F32) + np.float32(offs[b]) +
                        np.float32(draft_sigma) * rd.standard_normal((N, V), dtype=np.float32))
        mode = b % 3
        for n in range(N):
            kids = [i for i in range(1, N) if parent[i] == n]
            if not kids:
                continue
            diff = values(draft[b, n], dtype).astype(np.float64) - values(target[b, n], dtype).astype(np.float64)
            order = np.argsort(-diff, kind="stable")
            hi, lo = 0, V - 1
            for i in kids:
                if i in keep[mode]:
                    tokens[b, i] = int(order[lo])
                    lo -= 1
                    uniforms[b, i] = 0.0
                else:
                    tokens[b, i] = int(order[hi])
                    hi += 1
                    uniforms[b, i] = U_MAX
    return dict(kind="tree_sampled", B=B, N=N, V=V, dtype=dtype, node_tokens=tokens, parent=parent.copy(),
                max_depth=2, draft_logits=draft, target_logits=target, temperature=temps.astype(np.float32),
                uniforms=uniforms)


# ------------------------------------------------------------ greedy ---

def greedy_inputs(B: int, k: int, V: int, dtype: int, seed: int, *,
                  target_sigma: float = 2.0, match_p: float = 0.8) -> dict:
    """Inputs for greedy (temperature 0) chain verification.

    target logits t[b, j, :] = target_sigma * N(0,1), j = 0..k, rounded to dtype.
    draft token x[b, i] = first argmax of t[b, i, :] with probability match_p,
    otherwise uniform over the other V-1 tokens.
    """
    rt, rx = rng_for(seed, "target"), rng_for(seed, "greedy_tokens")
    np_dt = np.uint16 if dtype == BF16 else np.float32
    target = np.empty((B, k + 1, V), dtype=np_dt)
    tokens = np.empty((B, k), dtype=np.int32)
    for b in range(B):
        target[b] = to_dtype(target_sigma * rt.standard_normal((k + 1, V), dtype=np.float32), dtype)
        top = np.argmax(values(target[b, :k], dtype), axis=-1)
        for i in range(k):
            hit = rx.random() < match_p
            tokens[b, i] = int(top[i]) if hit else _other_token(rx, int(top[i]), V)
    return dict(kind="greedy", B=B, k=k, V=V, dtype=dtype, draft_tokens=tokens, target_logits=target)


# ------------------------------------------------------------ tree ---

def random_tree(N: int, seed: int, max_branch: int = 4, max_depth: int = 6) -> np.ndarray:
    """Parent array of a random rooted tree: parent[0] = -1, parent[i] < i.

    Node i attaches to a uniform choice among earlier nodes of depth < max_depth
    that have fewer than max_branch children.
    """
    rng = rng_for(seed, "tree")
    parent = np.full(N, -1, dtype=np.int32)
    depth = np.zeros(N, dtype=np.int64)
    children = np.zeros(N, dtype=np.int64)
    for i in range(1, N):
        cand = [j for j in range(i) if depth[j] < max_depth and children[j] < max_branch]
        if not cand:
            raise ValueError("tree bounds too tight for N nodes")
        p = int(cand[int(rng.integers(0, len(cand)))])
        parent[i] = p
        depth[i] = depth[p] + 1
        children[p] += 1
    return parent


def tree_inputs(B: int, N: int, V: int, dtype: int, seed: int, *,
                target_sigma: float = 2.0, max_branch: int = 4, max_depth: int = 6,
                match_p: float = 0.6, parent: np.ndarray | None = None,
                distinct_siblings: bool = False) -> dict:
    """Inputs for greedy static-tree verification.

    One parent array shared by all B sequences; target logits per node
    t[b, n, :] = target_sigma * N(0,1) rounded to dtype (row n is the target's
    prediction for the children of node n).  Node 0 is the root (its token is
    never matched); node i >= 1 carries the first argmax of its parent's row with
    probability match_p, otherwise a uniform other token.  With
    distinct_siblings, as the draft's top candidates are in a draft tree, the
    children of a node carry distinct tokens: a child takes the argmax with
    probability match_p only if no earlier sibling has it, and otherwise a
    uniform token that differs from the argmax and from its earlier siblings'.
    """
    if parent is None:
        parent = random_tree(N, seed, max_branch, max_depth)
    rt, rx = rng_for(seed, "target"), rng_for(seed, "tree_tokens")
    np_dt = np.uint16 if dtype == BF16 else np.float32
    target = np.empty((B, N, V), dtype=np_dt)
    tokens = np.empty((B, N), dtype=np.int32)
    for b in range(B):
        target[b] = to_dtype(target_sigma * rt.standard_normal((N, V), dtype=np.float32), dtype)
        top = np.argmax(values(target[b], dtype), axis=-1)
        tokens[b, 0] = int(rx.integers(0, V))
        taken: dict[int, set] = {}
        for i in range(1, N):
            g = int(top[parent[i]])
            if not distinct_siblings:
                tokens[b, i] = g if rx.random() < match_p else _other_token(rx, g, V)
                continue
            used = taken.setdefault(int(parent[i]), set())
            if g not in used and rx.random() < match_p:
                y = g
            else:
                y = _other_token(rx, g, V)
                while y in used and len(used) < V - 1:
                    y = _other_token(rx, g, V)
            used.add(y)
            tokens[b, i] = y
    depth = np.zeros(N, dtype=np.int64)
    for i in range(1, N):
        depth[i] = depth[parent[i]] + 1
    return dict(kind="tree", B=B, N=N, V=V, dtype=dtype, node_tokens=tokens,
                parent=parent.astype(np.int32), max_depth=int(max(max_depth, depth.max())),
                target_logits=target)


def sampled_tree_inputs(B: int, N: int, V: int, dtype: int, seed: int, *,
                        target_sigma: float = 3.0, zipf_s: float | None = 1.1, draft_sigma=1.0,
                        temperature=0.7, max_branch: int = 4, max_depth: int = 6,
                        parent: np.ndarray | None = None) -> dict:
    """Inputs for sampled (stochastic) tree verification.

    One parent array shared by all B sequences.  For every node n:
    target row t[b, n, :] = target_sigma * N(0,1) (+ Zipf bias) and draft row
    d[b, n, :] = t[b, n, :] + sigma_b * N(0,1), both rounded to dtype (row n
    predicts the children of node n).  The children of node n carry tokens
    drawn independently from softmax(d[b, n, :] / T_b) (Gumbel-max), as a
    drafter sampling its tree would.  uniforms u[b, :N] in [0, 1): u[b, i]
    tests node i >= 1, u[b, 0] drives the final draw.
    """
    if parent is None:
        parent = random_tree(N, seed, max_branch, max_depth)
    temps = _per_seq(temperature, B, seed, "temperature")
    sigmas = _per_seq(draft_sigma, B, seed, "sigma")
    bias = zipf_bias(V, zipf_s, seed) if zipf_s else None
    rt, rd, rx = rng_for(seed, "target"), rng_for(seed, "draft"), rng_for(seed, "tree_tokens")
    np_dt = np.uint16 if dtype == BF16 else np.float32
    target = np.empty((B, N, V), dtype=np_dt)
    draft = np.empty((B, N, V), dtype=np_dt)
    tokens = np.empty((B, N), dtype=np.int32)
    for b in range(B):
        t = target_sigma * rt.standard_normal((N, V), dtype=np.float32)
        if bias is not None:
            t = t + bias
        target[b] = to_dtype(t, dtype)
        dv = values(target[b], dtype) + np.float32(sigmas[b]) * rd.standard_normal((N, V), dtype=np.float32)
        draft[b] = to_dtype(dv, dtype)
        tokens[b, 0] = int(rx.integers(0, V))
        if N > 1:
            rows = values(draft[b][parent[1:]], dtype)  # the draft row of each node's parent
            tokens[b, 1:] = gumbel_max_tokens(rows, float(temps[b]), rx)
    depth = np.zeros(N, dtype=np.int64)
    for i in range(1, N):
        depth[i] = depth[parent[i]] + 1
    uniforms = rng_for(seed, "tree_uniforms").random((B, N), dtype=np.float32)
    return dict(kind="tree_sampled", B=B, N=N, V=V, dtype=dtype, node_tokens=tokens,
                parent=parent.astype(np.int32), max_depth=int(max(max_depth, depth.max())),
                draft_logits=draft, target_logits=target, temperature=temps.astype(np.float32),
                uniforms=uniforms, draft_sigma=sigmas.astype(np.float32))


# Two-level tree of the sampled-tree trials: the root has three children, each
# child two (N = 10).
TRIAL_TREE = np.array([-1, 0, 0, 0, 1, 1, 2, 2, 3, 3], dtype=np.int32)


def sampled_tree_trials(root_t: np.ndarray, root_d: np.ndarray, F: np.ndarray, G: np.ndarray,
                        H: np.ndarray, temperature: float, n: int, seed: int, block: int = 0) -> dict:
    """``n`` independent trials of sampled tree verification on TRIAL_TREE.

    Logit tables (float32 values, used as F32 logits; V = len(root_t)): the
    root has target row root_t and draft row root_d; a child with token y has
    target row F[y] and draft row G[y]; a grandchild with token z has target
    row H[z].  Children are drawn independently from softmax(root_d / T),
    grandchildren of a child with token y from softmax(G[y] / T).  A target
    that depends on the last token only then gives the first three emitted
    tokens the laws softmax(root_t / T), softmax(F[y1] / T), softmax(H[y2] / T).
    """
    V = root_t.shape[0]
    N = TRIAL_TREE.shape[0]
    rx = np.random.Generator(np.random.Philox(key=[int(seed), 3000 + 2 * int(block)]))
    ru = np.random.Generator(np.random.Philox(key=[int(seed), 3001 + 2 * int(block)]))
    tok = np.zeros((n, N), dtype=np.int32)
    tok[:, 1:4] = gumbel_max_tokens(np.broadcast_to(root_d, (n, 3, V)), temperature, rx)
    for c in (1, 2, 3):
        kids = [i for i in range(N) if TRIAL_TREE[i] == c]
        tok[:, kids] = gumbel_max_tokens(G[tok[:, c]][:, None, :].repeat(len(kids), axis=1), temperature, rx)
    target = np.zeros((n, N, V), dtype=np.float32)
    draft = np.zeros((n, N, V), dtype=np.float32)
    target[:, 0] = root_t
    draft[:, 0] = root_d
    target[:, 1:4] = F[tok[:, 1:4]]
    draft[:, 1:4] = G[tok[:, 1:4]]
    target[:, 4:] = H[tok[:, 4:]]
    return dict(kind="tree_sampled", B=n, N=N, V=V, dtype=F32, node_tokens=tok, parent=TRIAL_TREE.copy(),
                max_depth=2, draft_logits=draft, target_logits=target,
                temperature=np.full(n, temperature, dtype=np.float32),
                uniforms=ru.random((n, N), dtype=np.float32))


# ------------------------------------------------------------ the named workloads ---

WORKLOADS = {
    "tiny_chain": dict(name="tiny chain verify", kind="chain", B=1, k=4, V=1024, dtype=F32,
            target_sigma=2.0, zipf_s=None, draft_sigma=0.5, temperature=1.0),
    "llama_chain": dict(name="Llama-scale chain verify", kind="chain", B=64, k=4, V=128256, dtype=BF16,
            target_sigma=3.0, zipf_s=1.1, draft_sigma=1.0, temperature=0.7),
    "greedy_chain": dict(name="greedy chain verify", kind="greedy", B=256, k=5, V=128256, dtype=BF16,
            target_sigma=2.0, match_p=0.8),
    "deepseek_chain": dict(name="DeepSeek-scale chain verify", kind="chain", B=32, k=8, V=129280, dtype=F32,
            target_sigma=3.0, zipf_s=1.1, draft_sigma=(0.2, 3.0), temperature=(0.3, 1.3)),
    # each child's token equals its parent's target argmax with probability 0.6,
    # independently of its siblings
    "eagle_tree": dict(name="EAGLE-style static tree verify", kind="tree", B=16, N=64, V=128256, dtype=BF16,
            target_sigma=2.0, max_branch=4, max_depth=6, match_p=0.6, distinct_siblings=False),
    # the same trees with distinct sibling tokens, as a draft tree's top
    # candidates are (at most one child of a node can match)
    "eagle_tree_distinct": dict(name="EAGLE-style static tree verify, distinct siblings", kind="tree", B=16, N=64,
            V=128256, dtype=BF16, target_sigma=2.0, max_branch=4, max_depth=6, match_p=0.6,
            distinct_siblings=True),
    # one draft token per sequence, as in the single-token multi-token-prediction
    # schedule (the target scores 2 tokens per sequence of the decode batch)
    "mtp_chain": dict(name="MTP single-token verify", kind="chain", B=256, k=1, V=129280, dtype=BF16,
            target_sigma=3.0, zipf_s=1.1, draft_sigma=1.0, temperature=0.7),
    # plain temperature sampling of one target row per sequence (no drafts)
    "sampling": dict(name="temperature sampling", kind="chain", B=256, k=0, V=128256, dtype=BF16,
            target_sigma=3.0, zipf_s=1.1, draft_sigma=1.0, temperature=0.7),
    # the tree of the EAGLE-style workload, verified by sampling (children drawn
    # from the draft rows, logits generated like the Llama-scale chain)
    "sampled_tree": dict(name="sampled tree verify", kind="tree_sampled", B=16, N=64, V=128256, dtype=BF16,
            target_sigma=3.0, zipf_s=1.1, draft_sigma=1.0, temperature=0.7, max_branch=4, max_depth=6),
}


def make_inputs(workload: str, seed: int = 1, **override) -> dict:
    """Inputs for one of the named workloads in WORKLOADS (sizes may be overridden)."""
    c = dict(WORKLOADS[workload])
    c.update(override)
    kind = c.pop("kind")
    c.pop("name")
    if kind == "chain":
        return chain_inputs(c.pop("B"), c.pop("k"), c.pop("V"), c.pop("dtype"), seed, **c)
    if kind == "greedy":
        return greedy_inputs(c.pop("B"), c.pop("k"), c.pop("V"), c.pop("dtype"), seed, **c)
    if kind == "tree":
        return tree_inputs(c.pop("B"), c.pop("N"), c.pop("V"), c.pop("dtype"), seed, **c)
    if kind == "tree_sampled":
        return sampled_tree_inputs(c.pop("B"), c.pop("N"), c.pop("V"), c.pop("dtype"), seed, **c)
    raise ValueError(kind)
