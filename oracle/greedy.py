"""Greedy (argmax-match) verification -- the oracle, as its plain definition.

Test infrastructure only (see the package docstring).

Definition ([M7.1] §0x02D "Blockwise Decoding As The Ancestor": longest-prefix
validation is exact for greedy decoding; [Tiny] "Normative greedy pseudocode"):
  a_i = argmax_x l_{i,x} with the lowest index winning ties (the pages ask for a
  declared tie-break and never declare one; lowest index is the reading taken);
  A = the first i < gamma with x_i != a_i, else gamma;
  emitted tokens = x_0..x_{A-1}, a_A   (A + 1 tokens).
Temperature does not move an argmax, so none is taken.
"""
from __future__ import annotations

import numpy as np

from .numerics import OK, NONFINITE, BADTOKEN, decode, row_is_valid


def first_argmax(row: np.ndarray) -> int:
    """Lowest index attaining the maximum of a row without NaN."""
    return int(np.flatnonzero(row == row.max())[0])


def verify_greedy_one(L: np.ndarray, x: np.ndarray):
    """Returns (status, A, tokens) for one request; L [gamma+1, V] float64."""
    gamma = len(x)
    V = L.shape[1]
    for i in range(gamma):
        if not row_is_valid(L[i]):
            return NONFINITE, -1, []
        xi = int(x[i])
        if not (0 <= xi < V):
            return BADTOKEN, -1, []
        t = first_argmax(L[i])
        if xi != t:
            return OK, i, [int(v) for v in x[:i]] + [t]
    if not row_is_valid(L[gamma]):
        return NONFINITE, -1, []
    return OK, gamma, [int(v) for v in x] + [first_argmax(L[gamma])]


def verify_greedy(logits, tokens, logit_dtype="bf16", requests=None):
    """Batched greedy verification in the library's output layout (see verify_chain)."""
    B, R = logits.shape[0], logits.shape[1]
    idx = list(range(B)) if requests is None else [int(r) for r in requests]
    n = len(idx)
    acc = np.full(n, -1, np.int32)
    out = np.full((n, R), -1, np.int32)
    status = np.zeros(n, np.int32)
    for j, b in enumerate(idx):
        s, A, toks = verify_greedy_one(decode(logits[b], logit_dtype), np.asarray(tokens[b]))
        status[j] = s
        if s == OK:
            acc[j] = A
            out[j, :len(toks)] = toks
    return dict(accepted_len=acc, out_tokens=out, status=status)
