"""Greedy tree verification (the temperature-0 membership walk) -- the oracle.

Test infrastructure only (see the package docstring).

[M16] "Module 16: Speculative Decoding", "Verify the Tree -- and Why It's Exact": from
the root, follow the child whose token is the target's own greedy next token, until no
child matches; the accepted path is emitted, then the target's greedy next token after
it, so the output is what plain greedy decoding of the target would emit.  This is the
membership walk of tree.py with the target's sample replaced by its argmax (the limit
T -> 0 of softmax(row / T)).  Same tree layout as tree.py: node 0 is the frontier root,
row v scores the children of node v.  Readings: the argmax takes the lowest index on
ties ([Tiny] "Normative greedy pseudocode" asks for a declared tie-break), and among
siblings that repeat a token the lowest-index one is followed, as in tree.py.
  v = 0
  repeat: y = first argmax of row v
          if a child c of v has token(c) = y: accept c, v = c
          else: emit the accepted tokens, then y; stop.
"""
from __future__ import annotations

import numpy as np

from .numerics import OK, NONFINITE, BADTREE, decode, row_is_valid
from .greedy import first_argmax
from .tree import validate_tree


def verify_tree_greedy_one(L: np.ndarray, parents: np.ndarray, node_tokens: np.ndarray):
    """Returns dict(status, accepted_len, path, tokens) for one request; L [N, V] float64."""
    N, V = L.shape
    if not validate_tree(parents, node_tokens, V):
        return dict(status=BADTREE, accepted_len=-1, path=[], tokens=[])
    v = 0
    path = []
    while True:
        if not row_is_valid(L[v]):
            return dict(status=NONFINITE, accepted_len=-1, path=[], tokens=[])
        y = first_argmax(L[v])
        nxt = -1
        for c in range(v + 1, N):
            if int(parents[c]) == v and int(node_tokens[c]) == y:
                nxt = c
                break
        if nxt < 0:
            return dict(status=OK, accepted_len=len(path), path=path,
                        tokens=[int(node_tokens[c]) for c in path] + [y])
        path.append(nxt)
        v = nxt


def verify_tree_greedy(logits, parents, node_tokens, logit_dtype="bf16", requests=None):
    """Batched, in the library's output layout (see tree.verify_tree; no flags: every
    decision is an exact comparison)."""
    B, N = logits.shape[0], logits.shape[1]
    idx = list(range(B)) if requests is None else [int(r) for r in requests]
    n = len(idx)
    acc = np.full(n, -1, np.int32)
    out_tokens = np.full((n, N), -1, np.int32)
    out_nodes = np.full((n, N), -1, np.int32)
    status = np.zeros(n, np.int32)
    for j, b in enumerate(idx):
        r = verify_tree_greedy_one(decode(logits[b], logit_dtype), np.asarray(parents[b]),
                                   np.asarray(node_tokens[b]))
        status[j] = r["status"]
        if r["status"] == OK:
            acc[j] = r["accepted_len"]
            out_tokens[j, :len(r["tokens"])] = r["tokens"]
            out_nodes[j, :len(r["path"])] = r["path"]
    return dict(accepted_len=acc, out_tokens=out_tokens, out_nodes=out_nodes, status=status)
