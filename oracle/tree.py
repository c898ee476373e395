"""Tree verification by target-sample membership -- the oracle, step by step.

Test infrastructure only (see the package docstring).

Inputs of one request: the candidate tree as a parent-index array (node 0 is the
frontier root, parents[0] = -1, 0 <= parents[v] < v for v > 0 -- [M7.7] §0x0F
"Implementation Assertions" requires -1 <= parent < row), one token per node, and
one logits row per node.  Row v scores the children of node v: [M7.7] §0x07E (the
distribution that scores a candidate comes from its parent's row; a root-level
candidate is scored by the frontier row, which here is node 0's row).

Walk ([M7.7] §0x04B/§0x09: REST and SpecInfer accept a child when it matches the
token the target itself samples; [M16] "Verify the Tree": follow the matching child
down until none matches, then emit one more target token):
  v = 0
  repeat: y = inverse-CDF draw from softmax(row_v / T) with u[v];
          if some child c of v has token(c) = y: accept c, v = c
          else: stop; y is the terminal token.
If two siblings carry the same token (not a trie) the lowest-index one is taken.
Output: accepted node ids along the path, their tokens, then the terminal token.
"""
from __future__ import annotations

import numpy as np

from .numerics import OK, NONFINITE, BADUNIFORM, BADTREE, decode, row_is_valid, target_probs
from .chain import FLAG_WINDOW, inverse_cdf


def validate_tree(parents: np.ndarray, node_tokens: np.ndarray, V: int) -> bool:
    """[M7.7] §0x0F: parent index -1 only at the root, otherwise an earlier row; every
    non-root node token must be a vocabulary id (node 0's token is never read)."""
    N = len(parents)
    if N < 1 or int(parents[0]) != -1:
        return False
    for v in range(1, N):
        pv = int(parents[v])
        if not (0 <= pv < v):
            return False
        if not (0 <= int(node_tokens[v]) < V):
            return False
    return True


def verify_tree_one(L: np.ndarray, parents: np.ndarray, node_tokens: np.ndarray, u: np.ndarray,
                    temperature: float):
    """Returns dict(status, accepted_len, path, tokens, flagged) for one request.

    L: [N, V] float64 logits, one row per node.
    """
    N, V = L.shape
    if not validate_tree(parents, node_tokens, V):
        return dict(status=BADTREE, accepted_len=-1, path=[], tokens=[], flagged=False)
    flagged = False
    v = 0
    path = []
    while True:
        if not row_is_valid(L[v]):
            return dict(status=NONFINITE, accepted_len=-1, path=[], tokens=[], flagged=flagged)
        uv = float(u[v])
        if not (0.0 <= uv < 1.0):
            return dict(status=BADUNIFORM, accepted_len=-1, path=[], tokens=[], flagged=flagged)
        p, _, _ = target_probs(L[v], temperature)
        y, _, lo, hi = inverse_cdf(p, uv)
        if abs(uv - lo) < FLAG_WINDOW or abs(uv - hi) < FLAG_WINDOW:
            flagged = True
        nxt = -1
        for c in range(v + 1, N):           # children have larger indices than their parent
            if int(parents[c]) == v and int(node_tokens[c]) == y:
                nxt = c
                break
        if nxt < 0:
            toks = [int(node_tokens[c]) for c in path] + [y]
            return dict(status=OK, accepted_len=len(path), path=path, tokens=toks, flagged=flagged)
        path.append(nxt)
        v = nxt


def verify_tree(logits, parents, node_tokens, u, temperature, logit_dtype="bf16", requests=None):
    """Batched tree verification in the library's output layout:
    accepted_len [n], out_tokens [n, N], out_nodes [n, N] (-1 padded), status, flagged."""
    B, N = logits.shape[0], logits.shape[1]
    idx = list(range(B)) if requests is None else [int(r) for r in requests]
    n = len(idx)
    acc = np.full(n, -1, np.int32)
    out_tokens = np.full((n, N), -1, np.int32)
    out_nodes = np.full((n, N), -1, np.int32)
    status = np.zeros(n, np.int32)
    flagged = np.zeros(n, bool)
    for j, b in enumerate(idx):
        r = verify_tree_one(decode(logits[b], logit_dtype), np.asarray(parents[b]),
                            np.asarray(node_tokens[b]), np.asarray(u[b]), temperature)
        status[j] = r["status"]
        flagged[j] = r["flagged"]
        if r["status"] == OK:
            acc[j] = r["accepted_len"]
            out_tokens[j, :len(r["tokens"])] = r["tokens"]
            out_nodes[j, :len(r["path"])] = r["path"]
    return dict(accepted_len=acc, out_tokens=out_tokens, out_nodes=out_nodes, status=status,
                flagged=flagged)


def tree_expected_nodes(parents: np.ndarray, node_tokens: np.ndarray, probs: np.ndarray) -> float:
    """Expected number of tree nodes a membership walk reaches, root included.

    [M7.7] §0x0AA "Positional Acceptance Model": E[G] = sum_v f(v), where f(root) = 1
    and f(v) is the product, along the root-to-v path, of the probability that the
    walk selects each child.  Under target-sample membership the walk at node u
    selects child c exactly when the target draw at u equals token(c), so that
    probability is p_u(token(c)) (siblings with distinct tokens are mutually
    exclusive).  probs: [N, V] per-node target distributions.
    """
    N = len(parents)
    f = np.zeros(N)
    f[0] = 1.0
    for v in range(1, N):
        f[v] = f[int(parents[v])] * probs[int(parents[v]), int(node_tokens[v])]
    return float(f.sum())
