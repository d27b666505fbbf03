"""Serving-loop use of the C ABI on the GPU: a verification step and the
device-side commit captured once in a HIP graph and replayed on new inputs,
and independent batches verified concurrently on two streams.  Results are
checked against the fp64 oracle (bit-exact outside the 1e-5 band)."""

import numpy as np
import pytest

import workloads as W
from gpu_common import chain_tensors, compare_chain, dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def svl():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import draft_token_verification_chain_amd as svl

    svl.load()
    return svl


def _inputs(seed, B=32, k=4, V=20000):
    return W.chain_inputs(B, k, V, W.BF16, seed, target_sigma=3.0, zipf_s=1.1, draft_sigma=(0.3, 2.0),
                          temperature=(0.4, 1.2))


def _np(out):
    return {key: (v.cpu().numpy() if v is not None else None) for key, v in out.items()}


def test_graph_capture_and_replay(svl, orc):
    """verify_chain + commit_tokens captured once; every replay, on freshly
    copied inputs and with eager work in between, matches the oracle."""
    import torch

    sets = [_inputs(s) for s in (31, 32, 33, 34)]
    B, k, V = sets[0]["B"], sets[0]["k"], sets[0]["V"]
    static = chain_tensors(sets[0])
    ws = torch.zeros(svl.chain_workspace_bytes(B, k, V, W.BF16), dtype=torch.uint8, device="cuda")
    out = dict(accepted_len=torch.empty(B, dtype=torch.int32, device="cuda"),
               emitted=torch.empty((B, k + 1), dtype=torch.int32, device="cuda"),
               accept_prob=torch.empty((B, k), dtype=torch.float32, device="cuda"))
    lens0 = (np.arange(B, dtype=np.int32) * 3) % 40
    sl = dev(lens0.copy())
    hist = dev(np.zeros((B, 64), np.int32))
    com = dict(packed_offsets=torch.empty(B + 1, dtype=torch.int32, device="cuda"),
               packed=torch.empty(B * (k + 1), dtype=torch.int32, device="cuda"),
               status=torch.empty(B, dtype=torch.int32, device="cuda"))

    def step():
        svl.verify_chain(static["draft_tokens"], static["draft_logits"], static["target_logits"],
                         static["temperature"], static["uniforms"], workspace=ws, out=out)
        svl.commit_tokens(out["accepted_len"], out["emitted"], sl, hist, out=com)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    for rep, inp in enumerate(sets + sets[:2]):
        fresh = chain_tensors(inp)
        for key in static:
            static[key].copy_(fresh[key])
        sl.copy_(dev(lens0.copy()))
        hist.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = _np(out)
        ref = orc.verify_chain(inp)
        compare_chain(inp, got, ref, f"graph replay {rep}")
        ref_c = orc.commit_tokens(got["accepted_len"], got["emitted"], lens0, np.zeros((B, 64), np.int32))
        np.testing.assert_array_equal(sl.cpu().numpy(), ref_c["seq_len"])
        np.testing.assert_array_equal(hist.cpu().numpy(), ref_c["history"])
        # eager work between replays (a separate call with its own buffers)
        other = sets[(rep + 1) % len(sets)]
        t = chain_tensors(other)
        eager = svl.verify_chain(t["draft_tokens"], t["draft_logits"], t["target_logits"], t["temperature"],
                                 t["uniforms"])
        torch.cuda.synchronize()
        compare_chain(other, _np(eager), orc.verify_chain(other), f"eager between replays {rep}")


def test_two_streams_concurrently(svl, orc):
    """Two batches on two streams, each with its own workspace, in flight
    together for several rounds."""
    import torch

    a_inp, b_inp = _inputs(41, B=48), _inputs(42, B=40, k=2, V=30011)
    ta, tb = chain_tensors(a_inp), chain_tensors(b_inp)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for _ in range(4):
        with torch.cuda.stream(s1):
            oa = svl.verify_chain(ta["draft_tokens"], ta["draft_logits"], ta["target_logits"], ta["temperature"],
                                  ta["uniforms"])
        with torch.cuda.stream(s2):
            ob = svl.verify_chain(tb["draft_tokens"], tb["draft_logits"], tb["target_logits"], tb["temperature"],
                                  tb["uniforms"])
        outs.append((oa, ob))
    torch.cuda.synchronize()
    ra, rb = orc.verify_chain(a_inp), orc.verify_chain(b_inp)
    for i, (oa, ob) in enumerate(outs):
        compare_chain(a_inp, _np(oa), ra, f"stream 1 round {i}")
        compare_chain(b_inp, _np(ob), rb, f"stream 2 round {i}")
