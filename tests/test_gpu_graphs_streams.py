"""Serving-loop use of the C ABI on the GPU: every verification entry point
(the sampled chain together with the device-side commit, greedy, the greedy
tree, the sampled tree) captured once in a HIP graph and replayed on new
inputs with eager calls in between, and independent batches verified
concurrently on two streams.  Results are checked against the fp64 oracle
(bit-exact outside the 1e-5 band)."""

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


@pytest.mark.parametrize("B,k", [(32, 4), (256, 1), (256, 0)])
def test_graph_capture_and_replay(svl, orc, B, k):
    """verify_chain + commit_tokens captured once; every replay, on freshly
    copied inputs and with eager work in between, matches the oracle.  At 256
    sequences the draw after drafts takes its acceptance from its own kernel,
    and plain sampling runs one workgroup per sequence."""
    import torch

    sets = [_inputs(s, B=B, k=k) for s in (31, 32, 33, 34)]
    V = sets[0]["V"]
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


def test_graph_replay_chain_two_phases(svl, orc):
    """sv_verify_chain without accept_prob at a size that streams positions
    0..1 first and the rest only for sequences accepting both (k = 8, 164 MB
    of rows), captured once and replayed on inputs with other acceptance
    patterns, with eager calls in between."""
    import torch

    B, k, V = 40, 8, 128256
    sets = [W.chain_inputs(B, k, V, W.BF16, s, target_sigma=3.0, draft_sigma=sig)
            for s, sig in ((81, (0.05, 0.6)), (82, (0.5, 2.5)))]
    assert 2 * B * k * V * 2 >= 128 << 20
    static = chain_tensors(sets[0])
    ws = torch.zeros(svl.chain_workspace_bytes(B, k, V, W.BF16), dtype=torch.uint8, device="cuda")
    out = dict(accepted_len=torch.empty(B, dtype=torch.int32, device="cuda"),
               emitted=torch.empty((B, k + 1), dtype=torch.int32, device="cuda"), accept_prob=None)
    g = _capture(lambda: svl.verify_chain(static["draft_tokens"], static["draft_logits"], static["target_logits"],
                                          static["temperature"], static["uniforms"], workspace=ws, out=out))

    def check(inp, rep):
        compare_chain(inp, _np(out), orc.verify_chain(inp), f"two-phase graph replay {rep}")

    def eager(inp, rep):
        t = chain_tensors(inp)
        e = svl.verify_chain(t["draft_tokens"], t["draft_logits"], t["target_logits"], t["temperature"],
                             t["uniforms"], accept_prob=False)
        torch.cuda.synchronize()
        compare_chain(inp, _np(e), orc.verify_chain(inp), f"two-phase eager {rep}")

    _replay_each(g, static, sets + sets[:1], chain_tensors, check, eager)


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


def _capture(step):
    """A HIP graph of step(), after one warm-up call on a side stream."""
    import torch

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
    return g


def _replay_each(g, static, sets, to_tensors, check, eager):
    """Replays g once per input set (copied into the captured tensors), with
    an eager call on other buffers between replays; checks every result."""
    import torch

    for rep, inp in enumerate(sets):
        fresh = to_tensors(inp)
        for key in static:
            static[key].copy_(fresh[key])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        check(inp, rep)
        other = sets[(rep + 1) % len(sets)]
        eager(other, rep)


def test_graph_replay_greedy_and_tree(svl, orc):
    """sv_verify_greedy and sv_verify_tree captured once each and replayed on
    new inputs; every replay matches the oracle exactly."""
    import torch

    from gpu_common import dev_logits, run_greedy, run_tree

    gsets = [W.greedy_inputs(48, 5, 20011, W.BF16, s, match_p=0.7) for s in (51, 52, 53)]
    B, k, V = 48, 5, 20011
    to_g = lambda inp: dict(draft_tokens=dev(inp["draft_tokens"].astype(np.int32)),
                            target_logits=dev_logits(inp["target_logits"], inp["dtype"]))
    gs = to_g(gsets[0])
    gws = torch.zeros(svl.greedy_workspace_bytes(B, k, V, W.BF16), dtype=torch.uint8, device="cuda")
    gout = dict(accepted_len=torch.empty(B, dtype=torch.int32, device="cuda"),
                emitted=torch.empty((B, k + 1), dtype=torch.int32, device="cuda"))
    g = _capture(lambda: svl.verify_greedy(gs["draft_tokens"], gs["target_logits"], workspace=gws, out=gout))

    def check_g(inp, rep):
        ref = orc.verify_greedy(inp)
        np.testing.assert_array_equal(gout["accepted_len"].cpu().numpy(), ref["accepted_len"], f"replay {rep}")
        np.testing.assert_array_equal(gout["emitted"].cpu().numpy(), ref["emitted"], f"replay {rep}")

    def eager_g(inp, rep):
        np.testing.assert_array_equal(run_greedy(svl, inp)["emitted"], orc.verify_greedy(inp)["emitted"])

    _replay_each(g, gs, gsets + gsets[:1], to_g, check_g, eager_g)

    tsets = [W.tree_inputs(12, 40, 9001, W.F32, s, match_p=0.6) for s in (61, 62, 63)]
    B, N, V, md = 12, 40, 9001, int(tsets[0]["max_depth"])
    to_t = lambda inp: dict(node_tokens=dev(inp["node_tokens"].astype(np.int32)),
                            parent=dev(inp["parent"].astype(np.int32)),
                            target_logits=dev_logits(inp["target_logits"], inp["dtype"]))
    ts = to_t(tsets[0])
    tws = torch.zeros(svl.tree_workspace_bytes(B, N, V, W.F32), dtype=torch.uint8, device="cuda")
    tout = dict(accepted_len=torch.empty(B, dtype=torch.int32, device="cuda"),
                emitted=torch.empty((B, md + 1), dtype=torch.int32, device="cuda"),
                accepted_nodes=torch.empty((B, md + 1), dtype=torch.int32, device="cuda"))
    g = _capture(lambda: svl.verify_tree(ts["node_tokens"], ts["parent"], md, ts["target_logits"], workspace=tws,
                                         out=tout))

    def check_t(inp, rep):
        ref = orc.verify_tree(inp)
        for key in ("accepted_len", "emitted", "accepted_nodes"):
            np.testing.assert_array_equal(tout[key].cpu().numpy(), ref[key], f"replay {rep} {key}")

    def eager_t(inp, rep):
        np.testing.assert_array_equal(run_tree(svl, inp)["emitted"], orc.verify_tree(inp)["emitted"])

    _replay_each(g, ts, tsets + tsets[:1], to_t, check_t, eager_t)


def test_graph_replay_greedy_two_phase(svl, orc):
    """sv_verify_greedy at a size that reads its rows in two phases, captured
    once and replayed on inputs with other match patterns: which sequences the
    second phase streams is decided on the device at every replay."""
    import torch

    from gpu_common import dev_logits, run_greedy

    B, k, V = 72, 5, 156000
    assert B * (k + 1) * V * 4 >= 256 << 20
    gsets = [W.greedy_inputs(B, k, V, W.F32, s, match_p=p) for s, p in ((71, 0.8), (72, 1.0), (73, 0.5))]
    to_g = lambda inp: dict(draft_tokens=dev(inp["draft_tokens"].astype(np.int32)),
                            target_logits=dev_logits(inp["target_logits"], inp["dtype"]))
    gs = to_g(gsets[0])
    gws = torch.zeros(svl.greedy_workspace_bytes(B, k, V, W.F32), dtype=torch.uint8, device="cuda")
    gout = dict(accepted_len=torch.empty(B, dtype=torch.int32, device="cuda"),
                emitted=torch.empty((B, k + 1), dtype=torch.int32, device="cuda"))
    g = _capture(lambda: svl.verify_greedy(gs["draft_tokens"], gs["target_logits"], workspace=gws, out=gout))

    def check_g(inp, rep):
        ref = orc.verify_greedy(inp)
        np.testing.assert_array_equal(gout["accepted_len"].cpu().numpy(), ref["accepted_len"], f"replay {rep}")
        np.testing.assert_array_equal(gout["emitted"].cpu().numpy(), ref["emitted"], f"replay {rep}")

    def eager_g(inp, rep):
        np.testing.assert_array_equal(run_greedy(svl, inp)["emitted"], orc.verify_greedy(inp)["emitted"])

    _replay_each(g, gs, gsets + gsets[:1], to_g, check_g, eager_g)


def test_graph_replay_sampled_tree(svl, orc):
    """sv_verify_tree_sampled (rowstats, the walk rounds with their
    double-buffered state, the finisher) captured once and replayed on new
    inputs, with eager sampled-tree calls in between."""
    import torch

    from gpu_common import compare_tree_sampled, run_tree_sampled, tree_sampled_tensors

    temps = np.array([0.7, 1.1, 0.0, 0.5, 0.9, 1.3, 0.0, 0.8, 0.6, 1.0], np.float32)
    sets = [W.sampled_tree_inputs(10, 48, 12007, W.BF16, s, temperature=temps, draft_sigma=(0.3, 2.5))
            for s in (71, 72, 73)]
    B, N, V, md = 10, 48, 12007, int(sets[0]["max_depth"])
    static = tree_sampled_tensors(sets[0])
    ws = torch.zeros(svl.tree_sampled_workspace_bytes(B, N, V, W.BF16), dtype=torch.uint8, device="cuda")
    out = dict(accepted_len=torch.empty(B, dtype=torch.int32, device="cuda"),
               emitted=torch.empty((B, md + 1), dtype=torch.int32, device="cuda"),
               accepted_nodes=torch.empty((B, md + 1), dtype=torch.int32, device="cuda"))
    g = _capture(lambda: svl.verify_tree_sampled(static["node_tokens"], static["parent"], md,
                                                 static["draft_logits"], static["target_logits"],
                                                 static["temperature"], static["uniforms"], workspace=ws, out=out))

    def check(inp, rep):
        compare_tree_sampled(_np(out), orc.verify_tree_sampled(inp), f"graph replay {rep}")

    def eager(inp, rep):
        compare_tree_sampled(run_tree_sampled(svl, inp), orc.verify_tree_sampled(inp), f"eager {rep}")

    _replay_each(g, static, sets + sets[:2], tree_sampled_tensors, check, eager)


def test_sampled_trees_on_two_streams(svl, orc):
    """Two sampled-tree batches in flight together on two streams, each with
    its own workspace."""
    import torch

    from gpu_common import compare_tree_sampled, tree_sampled_tensors

    a_inp = W.sampled_tree_inputs(12, 40, 9001, W.F32, 81, draft_sigma=(0.3, 2.0))
    b_inp = W.sampled_tree_inputs(7, 64, 20000, W.BF16, 82, draft_sigma=(0.3, 2.0))
    ta, tb = tree_sampled_tensors(a_inp), tree_sampled_tensors(b_inp)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for _ in range(3):
        with torch.cuda.stream(s1):
            oa = svl.verify_tree_sampled(ta["node_tokens"], ta["parent"], int(a_inp["max_depth"]),
                                         ta["draft_logits"], ta["target_logits"], ta["temperature"], ta["uniforms"])
        with torch.cuda.stream(s2):
            ob = svl.verify_tree_sampled(tb["node_tokens"], tb["parent"], int(b_inp["max_depth"]),
                                         tb["draft_logits"], tb["target_logits"], tb["temperature"], tb["uniforms"])
        outs.append((oa, ob))
    torch.cuda.synchronize()
    ra, rb = orc.verify_tree_sampled(a_inp), orc.verify_tree_sampled(b_inp)
    for i, (oa, ob) in enumerate(outs):
        compare_tree_sampled(_np(oa), ra, f"stream 1 round {i}")
        compare_tree_sampled(_np(ob), rb, f"stream 2 round {i}")
