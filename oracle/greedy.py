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


def verify_greedy_stop_one(L: np.ndarray, x: np.ndarray, stop_tokens=(), budget=None):
    """Returns (status, A, tokens, finish) for one request; L [gamma+1, V] float64.

    Stopping as in the chain verifier ([M7.1] §0x05B, §0x06): an accepted draft in
    stop_tokens, or the one that uses up the remaining output budget, ends the round
    after itself with no target token; a target token that is a stop token or uses up the
    budget is emitted once and finishes the request; a budget of 0 emits nothing.
    finish: 1 stop token, 2 budget (a stop token wins a tie), 0 otherwise.
    """
    gamma = len(x)
    V = L.shape[1]
    stop = set(int(t) for t in stop_tokens)
    H = None if budget is None else int(budget)
    if H is not None and H <= 0:
        return OK, 0, [], 2
    for i in range(gamma):
        if not row_is_valid(L[i]):
            return NONFINITE, -1, [], 0
        xi = int(x[i])
        if not (0 <= xi < V):
            return BADTOKEN, -1, [], 0
        t = first_argmax(L[i])
        if xi != t:
            return OK, i, [int(v) for v in x[:i]] + [t], (1 if t in stop else (2 if H == i + 1 else 0))
        if xi in stop:
            return OK, i + 1, [int(v) for v in x[:i + 1]], 1
        if H == i + 1:
            return OK, i + 1, [int(v) for v in x[:i + 1]], 2
    if not row_is_valid(L[gamma]):
        return NONFINITE, -1, [], 0
    t = first_argmax(L[gamma])
    return OK, gamma, [int(v) for v in x] + [t], (1 if t in stop else (2 if H == gamma + 1 else 0))


def verify_greedy_one(L: np.ndarray, x: np.ndarray):
    """Returns (status, A, tokens) for one request; L [gamma+1, V] float64."""
    s, A, toks, _ = verify_greedy_stop_one(L, x)
    return s, A, toks


def verify_greedy(logits, tokens, logit_dtype="bf16", requests=None, stop_tokens=(), budget=None):
    """Batched greedy verification in the library's output layout (see verify_chain)."""
    B, R = logits.shape[0], logits.shape[1]
    idx = list(range(B)) if requests is None else [int(r) for r in requests]
    n = len(idx)
    acc = np.full(n, -1, np.int32)
    out = np.full((n, R), -1, np.int32)
    status = np.zeros(n, np.int32)
    finish = np.zeros(n, np.int32)
    for j, b in enumerate(idx):
        s, A, toks, fin = verify_greedy_stop_one(decode(logits[b], logit_dtype), np.asarray(tokens[b]),
                                                 stop_tokens, None if budget is None else int(budget[b]))
        status[j] = s
        if s == OK:
            acc[j] = A
            out[j, :len(toks)] = toks
            finish[j] = fin
    return dict(accepted_len=acc, out_tokens=out, status=status, finish=finish)
