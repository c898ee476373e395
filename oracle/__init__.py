"""Float64 CPU oracle for exact speculative verification -- TEST INFRASTRUCTURE ONLY.

This package is the plain, slow, obviously-correct reference that the GPU library is
checked against. Only `tests/`, `__graft_entry__.smoke()` and the CPU-baseline leg of
`bench.py` may import it. The product path (the HIP library and its Python binding)
never imports, calls or links anything here, and nothing here imports the product
path: the two share no code. The only module both sides consume is the seeded input
generator `synth`, which holds none of the verifier's arithmetic.

Pages this oracle follows, cited by title and section in every function:
  [M7.1]  "M7.1 - Speculative Decoding: Draft, Verify, Accept, Reject"
  [M7.7]  "M7.7 - Draft Sources, Dependent Heads, and Hardware-Aware Trees"
  [Atlas] "Speculative decoding: proposals and verified output" (AI-atlas lesson data)
  [M16]   "Module 16: Speculative Decoding"
  [Tiny]  "Exact Speculative and Assisted Decoding for TinyRustLM"

Parity status: every public function is pinned by tests under `tests/` against
values the pages print, closed forms, or brute-force enumeration; none is
"parity unpinned".
"""
from .numerics import (NONFINITE, BADTOKEN, BADUNIFORM, QZERO, RESIDUAL_EMPTY, BADTREE, OK,
                       decode, softmax_maxshift, softmax_online, target_probs)
from .chain import verify_chain, verify_chain_one, FLAG_WINDOW
from .greedy import verify_greedy, verify_greedy_one, verify_greedy_stop_one
from .tree import verify_tree, verify_tree_one, validate_tree, tree_expected_nodes
from .tree_residual import verify_tree_residual, verify_tree_residual_one
from .tree_greedy import verify_tree_greedy, verify_tree_greedy_one
from .processors import process_row, process_rows, unpack_mask, densify_sparse_q
from . import laws

__all__ = [
    "OK", "NONFINITE", "BADTOKEN", "BADUNIFORM", "QZERO", "RESIDUAL_EMPTY", "BADTREE",
    "decode", "softmax_maxshift", "softmax_online", "target_probs",
    "verify_chain", "verify_chain_one", "FLAG_WINDOW",
    "verify_greedy", "verify_greedy_one", "verify_greedy_stop_one",
    "verify_tree", "verify_tree_one", "validate_tree", "tree_expected_nodes",
    "verify_tree_residual", "verify_tree_residual_one",
    "verify_tree_greedy", "verify_tree_greedy_one",
    "process_row", "process_rows", "unpack_mask", "densify_sparse_q",
    "laws",
]
