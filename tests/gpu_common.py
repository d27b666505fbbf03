"""Helpers of the GPU parity tests: numpy inputs -> device tensors, and the
comparison of GPU outputs with the oracle's."""

import numpy as np
import torch

import workloads as W

BAND_EPS = 1e-5
PROB_TOL = 1e-5


def _host(arr, dtype=None):
    """A C-contiguous, writable array (copied only when needed) for torch.from_numpy."""
    return np.require(arr, dtype=dtype, requirements=["C", "W"])


def dev_logits(arr, dtype, device="cuda"):
    if dtype == W.BF16:
        return torch.from_numpy(_host(arr).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(_host(arr, np.float32)).to(device)


def dev(arr, device="cuda"):
    return torch.from_numpy(_host(arr)).to(device)


def chain_tensors(inp, device="cuda"):
    return dict(draft_tokens=dev(inp["draft_tokens"].astype(np.int32), device),
                draft_logits=dev_logits(inp["draft_logits"], inp["dtype"], device),
                target_logits=dev_logits(inp["target_logits"], inp["dtype"], device),
                temperature=dev(inp["temperature"].astype(np.float32), device),
                uniforms=dev(inp["uniforms"].astype(np.float32), device))


def run_chain(svl, inp, **kw):
    t = chain_tensors(inp)
    out = svl.verify_chain(t["draft_tokens"], t["draft_logits"], t["target_logits"], t["temperature"],
                           t["uniforms"], **kw)
    torch.cuda.synchronize()
    return {k: (v.cpu().numpy() if v is not None else None) for k, v in out.items()}


def run_greedy(svl, inp):
    out = svl.verify_greedy(dev(inp["draft_tokens"].astype(np.int32)),
                            dev_logits(inp["target_logits"], inp["dtype"]))
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def run_tree(svl, inp):
    out = svl.verify_tree(dev(inp["node_tokens"].astype(np.int32)), dev(inp["parent"].astype(np.int32)),
                          int(inp["max_depth"]), dev_logits(inp["target_logits"], inp["dtype"]))
    torch.cuda.synchronize()
    return {k: (v.cpu().numpy() if v is not None else None) for k, v in out.items()}


def compare_chain(inp, got, ref, label=""):
    """Bit-exact accepted_len / emitted outside the oracle's band; accept_prob
    within PROB_TOL absolute everywhere.  Returns the band statistics."""
    band = ref["band"]
    mism = (got["accepted_len"] != ref["accepted_len"]) | (got["emitted"] != ref["emitted"]).any(axis=1)
    bad = np.flatnonzero(mism & ~band)
    assert bad.size == 0, (
        f"{label}: {bad.size} sequences differ outside the band, e.g. b={bad[0]}: "
        f"gpu a={got['accepted_len'][bad[0]]} em={got['emitted'][bad[0]].tolist()} "
        f"oracle a={ref['accepted_len'][bad[0]]} em={ref['emitted'][bad[0]].tolist()}")
    if got.get("accept_prob") is not None and inp["k"] > 0:
        err = np.abs(got["accept_prob"].astype(np.float64) - ref["accept_prob"])
        assert err.max() <= PROB_TOL, f"{label}: accept_prob error {err.max():.3g}"
    return dict(n=int(band.size), banded=int(band.sum()), banded_mismatch=int((mism & band).sum()))


def tree_sampled_tensors(inp, device="cuda"):
    return dict(node_tokens=dev(inp["node_tokens"].astype(np.int32), device),
                parent=dev(inp["parent"].astype(np.int32), device),
                draft_logits=dev_logits(inp["draft_logits"], inp["dtype"], device),
                target_logits=dev_logits(inp["target_logits"], inp["dtype"], device),
                temperature=dev(inp["temperature"].astype(np.float32), device),
                uniforms=dev(inp["uniforms"].astype(np.float32), device))


def run_tree_sampled(svl, inp, **kw):
    t = tree_sampled_tensors(inp)
    out = svl.verify_tree_sampled(t["node_tokens"], t["parent"], int(inp["max_depth"]), t["draft_logits"],
                                  t["target_logits"], t["temperature"], t["uniforms"], **kw)
    torch.cuda.synchronize()
    return {k: (v.cpu().numpy() if v is not None else None) for k, v in out.items()}


def compare_tree_sampled(got, ref, label=""):
    """Bit-exact accepted_len / emitted / accepted_nodes outside the oracle's
    band.  Returns the band statistics."""
    band = ref["band"]
    mism = ((got["accepted_len"] != ref["accepted_len"]) | (got["emitted"] != ref["emitted"]).any(axis=1) |
            (got["accepted_nodes"] != ref["accepted_nodes"]).any(axis=1))
    bad = np.flatnonzero(mism & ~band)
    assert bad.size == 0, (
        f"{label}: {bad.size} sequences differ outside the band, e.g. b={bad[0]}: "
        f"gpu a={got['accepted_len'][bad[0]]} em={got['emitted'][bad[0]].tolist()} "
        f"nodes={got['accepted_nodes'][bad[0]].tolist()} oracle a={ref['accepted_len'][bad[0]]} "
        f"em={ref['emitted'][bad[0]].tolist()} nodes={ref['accepted_nodes'][bad[0]].tolist()}")
    return dict(n=int(band.size), banded=int(band.sum()), banded_mismatch=int((mism & band).sum()))
