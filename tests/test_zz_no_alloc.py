"""sv_verify_chain_static (through the C ABI) against sv_verify_chain.

The entry point for callers that cannot allocate runs the chain verification
on the library's own per-GPU device array instead of a caller workspace.  Its
outputs must equal those of sv_verify_chain on the same inputs, call after
call on the shared array: here two calls in a row, the second with a smaller
batch of another shape and dtype, and a third that repeats the first.  Both
are also checked against the oracle (bit-exact outside the 1e-5 band).
"""

import numpy as np
import pytest

import workloads as W
from gpu_common import chain_tensors, compare_chain

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def svl():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import draft_token_verification_chain_amd as svl

    svl.load()
    return svl


def _np(out):
    return {k: (v.cpu().numpy() if v is not None else None) for k, v in out.items()}


def _both(svl, inp):
    import torch

    t = chain_tensors(inp)
    args = (t["draft_tokens"], t["draft_logits"], t["target_logits"], t["temperature"], t["uniforms"])
    got_static = svl.verify_chain_static(*args)
    torch.cuda.synchronize()
    got_static = _np(got_static)
    got_ws = _np(svl.verify_chain(*args))
    torch.cuda.synchronize()
    return got_static, got_ws


def test_static_workspace_matches_caller_workspace(svl, orc):
    first = W.make_inputs("llama_chain", 3)                      # B=64, k=4, V=128256, bf16
    second = W.chain_inputs(5, 2, 9001, W.F32, 4, target_sigma=3.0, zipf_s=1.1, draft_sigma=(0.2, 3.0),
                            temperature=(0.3, 1.3))             # smaller, f32, odd V (element loads)
    for label, inp in (("first", first), ("second, smaller", second), ("first again", first)):
        got_static, got_ws = _both(svl, inp)
        for key in ("accepted_len", "emitted", "accept_prob"):
            np.testing.assert_array_equal(got_static[key], got_ws[key], err_msg=f"{label}: {key}")
        ref = orc.verify_chain(inp)
        st = compare_chain(inp, got_static, ref, f"static workspace, {label}")
        print(f"[no-alloc] {label}: B={inp['B']} k={inp['k']} V={inp['V']} {st}", flush=True)


def test_static_workspace_refuses_batches_beyond_its_size(svl):
    import torch

    from draft_token_verification_chain_amd import SpecVerifyError

    B, k, V = 4096, 4, 128256
    assert svl.chain_workspace_bytes(B, k, V, svl.SV_BF16) > 16 << 20
    # shape-only tensors: the size check fails on the host before any launch
    tok = torch.zeros((B, k), dtype=torch.int32, device="cuda")
    d = torch.empty((B, k, V), dtype=torch.bfloat16, device="cuda")
    t = torch.empty((B, k + 1, V), dtype=torch.bfloat16, device="cuda")
    temp = torch.ones(B, device="cuda")
    u = torch.zeros((B, k + 1), device="cuda")
    with pytest.raises(SpecVerifyError) as e:
        svl.verify_chain_static(tok, d, t, temp, u)
    assert e.value.status == 2  # SV_ERR_WORKSPACE_TOO_SMALL
