"""libspecverify: batched verification of speculative-decoding draft tokens on
AMD Instinct MI355X (gfx950), behind a C ABI (include/specverify.h).

The Python names mirror the C entry points:
  verify_chain   -> sv_verify_chain   (acceptance test, first rejection, residual / bonus draw)
  verify_chain_static -> sv_verify_chain_static (the same, on the library's own device workspace)
  verify_greedy  -> sv_verify_greedy  (temperature-0 argmax matching)
  verify_tree    -> sv_verify_tree    (EAGLE-style static tree, greedy)
  verify_tree_sampled -> sv_verify_tree_sampled (sampled tree, multi-step speculative sampling)
  commit_tokens  -> sv_commit_tokens  (append the step's tokens on the device)
The shared library is loaded on first use; calls raise if it is missing.
"""

from ._binding import (  # noqa: F401
    SV_BF16,
    SV_F32,
    SpecVerifyError,
    chain_workspace_bytes,
    commit_tokens,
    greedy_workspace_bytes,
    load,
    profile_begin,
    profile_end,
    set_handoff_polls,
    status_string,
    tree_sampled_workspace_bytes,
    tree_workspace_bytes,
    verify_chain,
    verify_chain_static,
    verify_greedy,
    verify_tree,
    verify_tree_sampled,
    version,
)
