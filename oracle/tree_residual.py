"""Multi-candidate tree verification with residual updates -- the oracle, step by step.

Test infrastructure only (see the package docstring).

[M7.7] "M7.7 - Draft Sources, Dependent Heads, and Hardware-Aware Trees" §0x09A
("Stochastic residual update") defines the procedure at one node: the children are
tested one after another; child i, whose token X_i was drawn from its own proposal
distribution q_i, is accepted with probability min(1, p^(i-1)(X_i) / q_i(X_i)); after a
rejection the remaining target mass becomes the normalized positive residual
p^(i) = [p^(i-1) - q_i]_+ / sum_y [p^(i-1)(y) - q_i(y)]_+.  If every child is rejected,
the output is a sample of the last residual.  §0x08B explains why testing every child
against the original p instead would duplicate probability mass.

Applied to a candidate tree (the layout of the membership verifier: node 0 is the
frontier root, parents[v] < v, row v of the target logits scores v's children):
  v = 0
  repeat: res = p_v = softmax(row_v / T)
          for each child c of v in increasing index order:
              accept c iff u_acc[c] < min(1, res(x_c) / q_c(x_c))   (x_c = token of c)
              on acceptance: v = c, continue the walk from c
              on rejection:  res = [res - q_c]_+ / sum([res - q_c]_+)
          no child accepted (or no children): y = inverse-CDF draw of res with u_draw[v];
          emit the tokens of the accepted nodes, then y; stop.
q_c is the row of the draft distributions for node c (the distribution its token was
drawn from); a tree whose siblings were drawn i.i.d. repeats one row for each sibling.
Readings (the pages leave them open): children are tested in index order; each child
test consumes its own uniform u_acc[c] and the terminal draw at v uses u_draw[v]; the
residual floor is 0 and an empty residual is an error, as in the chain verifier.
"""
from __future__ import annotations

import numpy as np

from .numerics import (OK, NONFINITE, BADUNIFORM, QZERO, RESIDUAL_EMPTY, BADTREE, decode,
                       row_is_valid, target_probs)
from .chain import FLAG_WINDOW, inverse_cdf
from .tree import validate_tree


def verify_tree_residual_one(L: np.ndarray, Q: np.ndarray, parents: np.ndarray, node_tokens: np.ndarray,
                             u_acc: np.ndarray, u_draw: np.ndarray, temperature: float):
    """One request.  L: [N, V] float64 target logits; Q: [N, V] float64 proposal rows (row 0
    unused).  Returns dict(status, accepted_len, path, tokens, flagged, residuals) where
    `residuals` counts the residual updates taken along the walk."""
    N, V = L.shape
    fail = lambda code, fl: dict(status=code, accepted_len=-1, path=[], tokens=[], flagged=fl,
                                 residuals=0)
    if not validate_tree(parents, node_tokens, V):
        return fail(BADTREE, False)
    flagged = False
    v = 0
    path = []
    updates = 0
    while True:
        if not row_is_valid(L[v]):
            return fail(NONFINITE, flagged)
        res, _, _ = target_probs(L[v], temperature)
        nxt = -1
        for c in range(v + 1, N):            # children in increasing index order
            if int(parents[c]) != v:
                continue
            x = int(node_tokens[c])
            qx = float(Q[c, x])
            if not (np.isfinite(qx) and qx > 0.0):
                return fail(QZERO, flagged)
            u = float(u_acc[c])
            if not (0.0 <= u < 1.0):
                return fail(BADUNIFORM, flagged)
            a = min(1.0, float(res[x]) / qx)
            if abs(u - a) < FLAG_WINDOW:
                flagged = True
            if u < a:
                nxt = c
                break
            q = Q[c]
            if not np.isfinite(q).all() or (q < 0).any():
                return fail(RESIDUAL_EMPTY, flagged)
            g = np.maximum(res - q, 0.0)
            W = float(np.sum(g))
            if not (np.isfinite(W) and W > 0.0):
                return fail(RESIDUAL_EMPTY, flagged)
            res = g / W
            updates += 1
        if nxt >= 0:
            path.append(nxt)
            v = nxt
            continue
        ud = float(u_draw[v])
        if not (0.0 <= ud < 1.0):
            return fail(BADUNIFORM, flagged)
        y, _, lo, hi = inverse_cdf(res, ud)
        if abs(ud - lo) < FLAG_WINDOW or abs(ud - hi) < FLAG_WINDOW:
            flagged = True
        toks = [int(node_tokens[c]) for c in path] + [y]
        return dict(status=OK, accepted_len=len(path), path=path, tokens=toks, flagged=flagged,
                    residuals=updates)


def verify_tree_residual(logits, q, parents, node_tokens, u_acc, u_draw, temperature,
                         logit_dtype="bf16", q_dtype="f32", requests=None):
    """Batched, in the library's output layout: accepted_len [n], out_tokens [n, N],
    out_nodes [n, N] (-1 padded), status [n], flagged [n]."""
    B, N = logits.shape[0], logits.shape[1]
    idx = list(range(B)) if requests is None else [int(r) for r in requests]
    n = len(idx)
    acc = np.full(n, -1, np.int32)
    out_tokens = np.full((n, N), -1, np.int32)
    out_nodes = np.full((n, N), -1, np.int32)
    status = np.zeros(n, np.int32)
    flagged = np.zeros(n, bool)
    for j, b in enumerate(idx):
        r = verify_tree_residual_one(decode(logits[b], logit_dtype), decode(q[b], q_dtype),
                                     np.asarray(parents[b]), np.asarray(node_tokens[b]),
                                     np.asarray(u_acc[b]), np.asarray(u_draw[b]), temperature)
        status[j] = r["status"]
        flagged[j] = r["flagged"]
        if r["status"] == OK:
            acc[j] = r["accepted_len"]
            out_tokens[j, :len(r["tokens"])] = r["tokens"]
            out_nodes[j, :len(r["path"])] = r["path"]
    return dict(accepted_len=acc, out_tokens=out_tokens, out_nodes=out_nodes, status=status,
                flagged=flagged)
