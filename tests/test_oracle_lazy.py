"""Pins of the reading behind lazy row consumption (CPU only).

[M7.1] §0x03G "First Rejection Is A Semantic Stop, Not Only An Optimization": the round
stops at the first rejection and discards every later draft conditional, uniform and
target row.  So the outputs of a request whose first rejection is at A cannot depend on
anything past it: replacing target rows A+1..gamma, draft rows and tokens A+1.., and
uniforms A+1..gamma-1 with arbitrary values (NaN included) must leave every output and
every reported statistic unchanged.  The terminal uniform u[gamma] and row A's q (the
residual) are used and stay.  The same holds for greedy verification after the first
mismatch.  This is what makes reading rows lazily exact.
"""
import numpy as np

import oracle


def _perturb_chain(x_logits, q, tokens, u, acc, rng, V):
    L, Q, T, U = x_logits.copy(), q.copy(), tokens.copy(), u.copy()
    G = T.shape[1]
    for b, A in enumerate(acc):
        if A < 0 or A >= G:
            continue
        L[b, A + 1:] = rng.normal(0, 5, L[b, A + 1:].shape)
        if A + 1 <= G and rng.random() < 0.5:
            L[b, A + 1:, rng.integers(V)] = np.nan
        Q[b, A + 1:] = rng.random(Q[b, A + 1:].shape)
        T[b, A + 1:] = rng.integers(-3, V + 3, T[b, A + 1:].shape)
        U[b, A + 1:G] = rng.random(G - A - 1) * 2 - 0.5     # may leave [0, 1)
    return L, Q, T, U


def test_chain_outputs_ignore_everything_after_the_first_rejection():
    rng = np.random.default_rng(40)
    hits = 0
    for trial in range(30):
        B, G, V = 24, int(rng.integers(1, 6)), int(rng.integers(2, 30))
        L = rng.normal(0, 2, (B, G + 1, V))
        q = rng.dirichlet(np.ones(V), (B, G))
        tokens = np.array([[rng.choice(V, p=q[b, i]) for i in range(G)] for b in range(B)], np.int32)
        u = rng.random((B, G + 1)).astype(np.float32).astype(np.float64)
        T = float(rng.uniform(0.5, 1.5))
        exp = oracle.verify_chain(L, q, tokens, u, T, "f64", q_dtype="f64")
        L2, q2, t2, u2 = _perturb_chain(L, q, tokens, u, exp["accepted_len"], rng, V)
        got = oracle.verify_chain(L2, q2, t2, u2, T, "f64", q_dtype="f64")
        for key in ("accepted_len", "out_tokens", "status", "flagged"):
            np.testing.assert_array_equal(got[key], exp[key], err_msg=key)
        np.testing.assert_array_equal(got["stats"], exp["stats"])   # NaN where unreached, in both
        hits += int((exp["accepted_len"] < G).sum())
    assert hits > 200


def test_greedy_outputs_ignore_everything_after_the_first_mismatch():
    rng = np.random.default_rng(41)
    for trial in range(30):
        B, G, V = 24, int(rng.integers(1, 7)), int(rng.integers(2, 30))
        L = rng.normal(0, 2, (B, G + 1, V))
        arg = L.argmax(-1)
        tokens = np.where(rng.random((B, G)) < 0.6, arg[:, :G], rng.integers(0, V, (B, G))).astype(np.int32)
        exp = oracle.verify_greedy(L, tokens, "f64")
        L2, t2 = L.copy(), tokens.copy()
        for b, A in enumerate(exp["accepted_len"]):
            if 0 <= A < G:
                L2[b, A + 1:] = np.nan if rng.random() < 0.5 else rng.normal(0, 5, L2[b, A + 1:].shape)
                t2[b, A + 1:] = rng.integers(-3, V + 3, G - A - 1)
        got = oracle.verify_greedy(L2, t2, "f64")
        for key in ("accepted_len", "out_tokens", "status"):
            np.testing.assert_array_equal(got[key], exp[key], err_msg=key)

