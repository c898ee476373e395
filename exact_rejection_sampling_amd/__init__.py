"""MI355X-native batched target-side verification for exact speculative decoding.

The work runs in hand-written HIP kernels for gfx950 inside libspec_verify.so (C ABI
declared in include/spec_verify.h).  This package is the thin Python binding: torch
tensors in, torch tensors out, on the current CUDA (HIP) stream.

    spec_verify_chain          rejection-sampling verification of draft chains
                               (stop_tokens= / budget= apply stop tokens and an output
                               budget inside the round)
    spec_verify_greedy         argmax-match verification (same stop options)
    spec_verify_tree           tree verification by target-sample membership
    spec_verify_tree_greedy    its temperature-0 form (argmax membership)
    spec_verify_tree_residual  multi-candidate tree verification with residual updates

prepare_* check and marshal the arguments once and return a callable that issues the
same library call again (for loops that call the verifier many times on buffers refilled
in place).
"""
from ._binding import (REQ_STATUS, SpecError, PreparedCall, chain_workspace_bytes,
                       greedy_workspace_bytes, load_library, prepare_chain, prepare_greedy,
                       prepare_tree, prepare_tree_greedy, prepare_tree_residual, spec_verify_chain,
                       spec_verify_greedy, spec_verify_tree, spec_verify_tree_greedy,
                       spec_verify_tree_residual, tree_residual_workspace_bytes, tree_workspace_bytes,
                       reset_workspaces, spec_verify_chain_static, LIB_PATH)

__all__ = ["spec_verify_chain", "spec_verify_greedy", "spec_verify_tree", "spec_verify_tree_greedy",
           "spec_verify_tree_residual", "prepare_tree_residual", "tree_residual_workspace_bytes",
           "load_library", "chain_workspace_bytes", "greedy_workspace_bytes", "tree_workspace_bytes",
           "prepare_chain", "prepare_greedy", "prepare_tree", "prepare_tree_greedy", "PreparedCall",
           "SpecError", "REQ_STATUS", "LIB_PATH", "reset_workspaces",
           "spec_verify_chain_static"]
