"""Chain verification by rejection sampling -- the oracle, step by step in float64.

Test infrastructure only (see the package docstring).

The steps follow the pages' order and notation:
  * rows 0..gamma-1 of the target logits score draft tokens x_0..x_{gamma-1};
    row gamma is the bonus row ([M7.1] §0x04A "Verification Shape", layout B:
    p_for_draft = logits[:K], p_for_bonus = logits[K]);
  * p_i = softmax(l_i / T)  ([M7.1] §0x04F, §0x03D);
  * accept draft i iff u_i < a_i = min(1, p_i(x_i) / q_i(x_i))
    ([M16] "The Math: Speculative Sampling", the accept rule);
  * stop at the first rejection A ([M7.1] §0x03G); if every draft is accepted, A = gamma;
  * terminal weights w = max(p_A - q_A, 0) if A < gamma ([M7.1] §0x03C), else
    w = p_gamma ([M7.1] §0x03H); the terminal token is the inverse-CDF draw of
    u_gamma in vocabulary order: the first k whose running sum of w exceeds
    u_gamma * W, W = sum w  (the pages leave the sampling order open; this is the
    plain reading);
  * emitted tokens: x_0..x_{A-1} then the terminal token, A + 1 in all
    ([M16] "Code: Verify a Draft": the emitted length is always n_accepted + 1).

Readings of points the pages leave open are listed in the repository's design notes;
the ones that change results are: the strict inequality u < a with u on [0, 1), the
use of u_gamma for whichever terminal draw happens, q used exactly as stored, and the
error statuses below, checked in the order a round reaches them ([Tiny] "Normative
stochastic pseudocode" checks each row when it is reached).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

from .numerics import (OK, NONFINITE, BADTOKEN, BADUNIFORM, QZERO, RESIDUAL_EMPTY,
                       decode, row_is_valid, target_probs)

#: draws within this distance of an acceptance threshold or a CDF boundary are
#: "flagged": finite-precision implementations may legitimately decide them either way.
FLAG_WINDOW = 1e-6


@dataclass
class ChainResult:
    status: int
    accepted_len: int                    # A, or -1 on error
    tokens: List[int]                    # emitted tokens (A + 1 of them), [] on error
    flagged: bool = False
    m: List[float] = field(default_factory=list)       # per reached row: max of l/T
    logZ: List[float] = field(default_factory=list)    # per reached row: log sum exp(l/T - m)
    p_x: List[float] = field(default_factory=list)     # p_i(x_i) per reached draft row
    q_x: List[float] = field(default_factory=list)     # q_i(x_i) per reached draft row
    a: List[float] = field(default_factory=list)       # a_i per reached draft row
    W: float = float("nan")                            # terminal weight mass
    weights: Optional[np.ndarray] = None               # terminal weights w (unnormalized)
    cdf_lo: float = float("nan")                       # C_{k-1} at the chosen k
    cdf_hi: float = float("nan")                       # C_k at the chosen k
    finish: int = 0                                    # 0 open, 1 stop token emitted, 2 budget reached


def inverse_cdf(w: np.ndarray, u: float):
    """First index k with sum_{x<=k} w(x) > u * W, W = sum w (vocabulary order).

    Returns (k, W, C_{k-1}, C_k) with C the normalized running sum.  A zero-weight
    index is never returned: the running sum must strictly increase to pass u*W.
    """
    c = np.cumsum(w)
    W = float(c[-1])
    k = int(np.searchsorted(c, u * W, side="right"))
    lo = float(c[k - 1]) / W if k > 0 else 0.0
    hi = float(c[k]) / W
    return k, W, lo, hi


def verify_chain_one(L: np.ndarray, Q: np.ndarray, x: np.ndarray, u: np.ndarray,
                     temperature: float, stop_tokens=(), budget=None) -> ChainResult:
    """Verify one request.

    L: [gamma+1, V] float64 target logits; Q: [gamma, V] float64 draft probabilities;
    x: [gamma] draft tokens; u: [gamma+1] uniforms (u[i] for the accept test of draft
    i, u[gamma] for the terminal draw -- [M7.1] §0x04J: one terminal draw per round).

    Stopping ([M7.1] §0x05B "Round Progress Includes Correction Or Bonus", §0x06 "KV
    Commit And Rollback": stopping is applied before publication): an accepted draft in
    `stop_tokens` ends the round after itself, and so does the accepted draft that uses
    up the remaining output `budget` (None: no limit); neither emits a correction or a
    bonus, and no later draft is tested.  A correction or bonus that is a stop token, or
    that uses up the budget, is emitted once and finishes the request.  A budget of 0
    dispatches no round (nothing is emitted).  `finish`: 1 after a stop token, 2 when the
    budget is reached (a stop token wins a tie), else 0; accepted_len counts the emitted
    drafts.
    """
    gamma = int(len(x))
    V = int(L.shape[1])
    res = ChainResult(status=OK, accepted_len=-1, tokens=[])
    u = np.asarray(u, dtype=np.float64)

    def fail(code):
        return ChainResult(status=code, accepted_len=-1, tokens=[], flagged=res.flagged,
                           m=res.m, logZ=res.logZ, p_x=res.p_x, q_x=res.q_x, a=res.a)

    stop = set(int(t) for t in stop_tokens)
    H = None if budget is None else int(budget)
    if H is not None and H <= 0:
        return ChainResult(status=OK, accepted_len=0, tokens=[], finish=2)
    A = gamma
    end = None                 # (emitted drafts, finish) when the round stops without a draw
    for i in range(gamma):
        if not row_is_valid(L[i]):
            return fail(NONFINITE)
        xi = int(x[i])
        if not (0 <= xi < V):
            return fail(BADTOKEN)
        qx = float(Q[i, xi])
        if not (np.isfinite(qx) and qx > 0.0):
            return fail(QZERO)
        if not (0.0 <= u[i] < 1.0):
            return fail(BADUNIFORM)
        p, m, Z = target_probs(L[i], temperature)
        res.m.append(m)
        res.logZ.append(float(np.log(Z)))
        px = float(p[xi])
        a = min(1.0, px / qx)
        res.p_x.append(px)
        res.q_x.append(qx)
        res.a.append(a)
        if abs(u[i] - a) < FLAG_WINDOW:
            res.flagged = True
        if not (u[i] < a):          # first rejection: stop here
            A = i
            break
        if int(x[i]) in stop:       # an accepted stop token ends the round
            end = (i + 1, 1)
            break
        if H is not None and i + 1 == H:   # the remaining budget is used up
            end = (i + 1, 2)
            break

    if end is not None:
        res.accepted_len, res.finish = end
        res.tokens = [int(t) for t in x[:end[0]]]
        return res

    if A == gamma:
        if not row_is_valid(L[gamma]):
            return fail(NONFINITE)
        p, m, Z = target_probs(L[gamma], temperature)
        res.m.append(m)
        res.logZ.append(float(np.log(Z)))
    if not (0.0 <= u[gamma] < 1.0):
        return fail(BADUNIFORM)

    if A < gamma:
        p, _, _ = target_probs(L[A], temperature, check_backends=False)
        qrow = Q[A]
        if not np.isfinite(qrow).all() or (qrow < 0).any():
            return fail(RESIDUAL_EMPTY)
        w = np.maximum(p - qrow, 0.0)           # positive residual [p - q]_+
    else:
        w = p                                   # bonus: an ordinary target draw
    total = float(np.sum(w))
    if not (np.isfinite(total) and total > 0.0):
        return fail(RESIDUAL_EMPTY)
    k, W, lo, hi = inverse_cdf(w, float(u[gamma]))
    if abs(u[gamma] - lo) < FLAG_WINDOW or abs(u[gamma] - hi) < FLAG_WINDOW:
        res.flagged = True

    res.accepted_len = A
    res.tokens = [int(t) for t in x[:A]] + [k]
    res.finish = 1 if k in stop else (2 if H is not None and A + 1 == H else 0)
    res.W = W
    res.weights = w
    res.cdf_lo, res.cdf_hi = lo, hi
    return res


def verify_chain(logits, q, tokens, u, temperature, logit_dtype="f32", q_dtype="f32",
                 requests=None, stop_tokens=(), budget=None):
    """Batched chain verification, one request at a time.

    logits [B, gamma+1, V] (raw bf16 bits or fp32), q [B, gamma, V], tokens [B, gamma],
    u [B, gamma+1].  `requests` optionally restricts the work to a subset of request
    indices (for sampled checks at full size).

    Returns a dict of numpy arrays in the library's output layout:
      accepted_len [n] (-1 on error), out_tokens [n, gamma+1] (-1 padded),
      status [n], flagged [n] bool, stats [n, gamma+1, 4] float64 with, for each reached
      row i < gamma, (m_i, log Z_i, p_i(x_i), a_i); row gamma holds (m_gamma, log Z_gamma)
      when the bonus row is reached and W (terminal mass) in column 2; unreached
      entries are NaN.  Also `results`: the per-request ChainResult objects.
    """
    B, R, V = logits.shape[0], logits.shape[1], logits.shape[2]
    gamma = R - 1
    idx = list(range(B)) if requests is None else [int(r) for r in requests]
    n = len(idx)
    out = dict(
        accepted_len=np.full(n, -1, np.int32),
        out_tokens=np.full((n, R), -1, np.int32),
        status=np.zeros(n, np.int32),
        flagged=np.zeros(n, bool),
        finish=np.zeros(n, np.int32),
        stats=np.full((n, R, 4), np.nan),
        results=[],
    )
    for j, b in enumerate(idx):
        L = decode(logits[b], logit_dtype)
        Q = decode(q[b], q_dtype) if gamma > 0 else np.zeros((0, V))
        r = verify_chain_one(L, Q, np.asarray(tokens[b]), np.asarray(u[b]), temperature, stop_tokens,
                             None if budget is None else int(budget[b]))
        out["results"].append(r)
        out["status"][j] = r.status
        out["flagged"][j] = r.flagged
        if r.status != OK:
            continue
        out["accepted_len"][j] = r.accepted_len
        out["out_tokens"][j, :len(r.tokens)] = r.tokens
        out["finish"][j] = r.finish
        st = out["stats"][j]
        for i in range(len(r.a)):
            st[i] = (r.m[i], r.logZ[i], r.p_x[i], r.a[i])
        if len(r.m) > gamma:        # the bonus row was reached
            st[gamma, 0] = r.m[gamma]
            st[gamma, 1] = r.logZ[gamma]
        st[gamma, 2] = r.W
    return out
