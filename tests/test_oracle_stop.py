"""Pins of stop-token and output-budget handling (CPU only).

[M7.1] "M7.1 - Speculative Decoding: Draft, Verify, Accept, Reject" §0x05B: a round's
committed progress is G = min(A + 1, H), H the distance to the first emitted stop token or
the remaining output budget.  §0x06 applies stopping before publication and gives three
examples (full acceptance, a length cap after d_3, an EOS at d_2), pinned here with the
chain and greedy oracles.  The law: with a stop token, the emitted sequences (completed
with target draws until a stop token or the horizon) follow the target's own law of
stop-terminated sequences, and with a budget the emitted prefix follows the target's law
of its first H tokens (exact enumeration with one uniform inside every branch).
"""
import itertools
from collections import defaultdict

import numpy as np
import pytest

import oracle
from oracle.chain import verify_chain_one
from lawcheck import logits_for, _midpoints, prefix_table


def _rows_accept_all(V, drafts, bonus):
    """Rows where p = q puts all mass on the drafts (acceptance certain) and a one-hot
    bonus row."""
    G = len(drafts)
    P = np.zeros((G + 1, V))
    for i, d in enumerate(drafts):
        P[i, d] = 1.0
    P[G, bonus] = 1.0
    L = np.stack([logits_for(P[i], 1.0) for i in range(G + 1)])
    return L, P[:G].copy()


def test_pages_examples_chain():
    V, d, b = 6, [1, 2, 3], 4
    L, Q = _rows_accept_all(V, d, b)
    u = np.array([0.3, 0.6, 0.9, 0.5])
    run = lambda **k: verify_chain_one(L, Q, np.array(d), u, 1.0, **k)
    r = run()                                   # full acceptance, no stop
    assert (r.tokens, r.accepted_len, r.finish) == ([1, 2, 3, 4], 3, 0)
    r = run(budget=3)                           # length cap after d_3
    assert (r.tokens, r.accepted_len, r.finish) == ([1, 2, 3], 3, 2)
    r = run(stop_tokens=[2])                    # EOS at d_2
    assert (r.tokens, r.accepted_len, r.finish) == ([1, 2], 2, 1)
    r = run(budget=4)                           # the bonus uses up the budget
    assert (r.tokens, r.finish) == ([1, 2, 3, 4], 2)
    r = run(stop_tokens=[4])                    # the bonus is the stop token: counted once
    assert (r.tokens, r.finish) == ([1, 2, 3, 4], 1)
    r = run(budget=0)                           # zero budget dispatches no round
    assert (r.status, r.tokens, r.accepted_len, r.finish) == (oracle.OK, [], 0, 2)
    r = run(stop_tokens=[2], budget=2)          # both at d_2: the stop token
    assert (r.tokens, r.finish) == ([1, 2], 1)


def test_no_tests_after_a_stop():
    V, d, b = 6, [1, 2, 3], 4
    L, Q = _rows_accept_all(V, d, b)
    L = L.copy()
    L[2, 0] = np.nan                            # row 2 is invalid, but never reached
    u = np.array([0.3, 0.6, 7.0, 0.5])          # and so is u_2
    r = verify_chain_one(L, Q, np.array(d), u, 1.0, stop_tokens=[2])
    assert (r.status, r.tokens, r.finish) == (oracle.OK, [1, 2], 1)
    r = verify_chain_one(L, Q, np.array(d), u, 1.0, budget=2)
    assert (r.status, r.tokens, r.finish) == (oracle.OK, [1, 2], 2)
    assert verify_chain_one(L, Q, np.array(d), u, 1.0).status == oracle.NONFINITE


def test_rejection_before_the_stop():
    V = 6
    p0 = np.array([0.0, 0.0, 0.0, 0.0, 1.0, 0.0])     # p(d_1 = 1) = 0: always rejected
    L = np.stack([logits_for(p0, 1.0)] * 4)
    Q = np.tile(np.array([0.1, 0.5, 0.2, 0.1, 0.05, 0.05]), (3, 1))
    r = verify_chain_one(L, Q, np.array([1, 2, 3]), np.array([0.5, 0.5, 0.5, 0.5]), 1.0, stop_tokens=[2])
    assert (r.tokens, r.accepted_len, r.finish) == ([4], 0, 0)     # the correction is token 4
    r = verify_chain_one(L, Q, np.array([1, 2, 3]), np.array([0.5, 0.5, 0.5, 0.5]), 1.0, stop_tokens=[4])
    assert (r.tokens, r.finish) == ([4], 1)


def test_pages_examples_greedy():
    V = 6
    P = np.zeros((4, V))
    for i, t in enumerate([1, 2, 3, 4]):
        P[i, t] = 1.0
    L = np.stack([logits_for(P[i] * 0.9 + 0.02, 1.0) for i in range(4)])
    g = lambda **k: oracle.verify_greedy_stop_one(L, np.array([1, 2, 3]), **k)
    assert g() == (oracle.OK, 3, [1, 2, 3, 4], 0)
    assert g(budget=3) == (oracle.OK, 3, [1, 2, 3], 2)
    assert g(stop_tokens=[2]) == (oracle.OK, 2, [1, 2], 1)
    assert g(stop_tokens=[4]) == (oracle.OK, 3, [1, 2, 3, 4], 1)
    assert g(budget=0) == (oracle.OK, 0, [], 2)
    assert oracle.verify_greedy_stop_one(L, np.array([1, 5, 3]), stop_tokens=[2]) == (oracle.OK, 1, [1, 2], 1)


def _stop_law(p_of, q_of, V, gamma, T, horizon, stop, budget):
    """Emitted-token law of one round (completed with target draws until a stop token or
    `horizon`), by enumeration: every draft path x ~ q, every accept/reject branch and
    terminal token, the oracle driven with one uniform inside each branch."""
    joint = defaultdict(float)
    H = budget if budget is not None else np.inf
    for x in itertools.product(range(V), repeat=gamma):
        qrows = [np.asarray(q_of(x[:i]), np.float64) for i in range(gamma)]
        w = float(np.prod([qrows[i][x[i]] for i in range(gamma)]))
        if w == 0.0:
            continue
        L = np.stack([logits_for(p_of(x[:i]), T) for i in range(gamma + 1)])
        Q = np.stack(qrows)

        def finish(seq, mass, u):
            r = verify_chain_one(L, Q, np.array(x), u, T, stop_tokens=stop, budget=budget)
            assert r.status == oracle.OK and r.tokens == list(seq), (r.tokens, seq)
            seq = tuple(seq)
            stack = [(seq, mass)]
            while stack:          # complete with target draws until a stop token or the horizon
                s, m = stack.pop()
                if len(s) == horizon or (s and s[-1] in stop):
                    joint[s] += m
                    continue
                for k, pk in enumerate(p_of(s)):
                    if pk > 0:
                        stack.append((s + (k,), m * pk))

        def walk(i, u, mass):
            if i == gamma:                          # every draft accepted: bonus row
                for k, mk, uk in _midpoints(np.asarray(p_of(x), np.float64)):
                    u2 = u.copy(); u2[gamma] = uk
                    finish(list(x) + [k], mass * mk, u2)
                return
            p = np.asarray(p_of(x[:i]), np.float64)
            a = min(1.0, p[x[i]] / qrows[i][x[i]])
            if a > 0:
                u2 = u.copy(); u2[i] = 0.5 * a
                if x[i] in stop or i + 1 == H:       # the round ends after this draft
                    finish(list(x[:i + 1]), mass * a, u2)
                else:
                    walk(i + 1, u2, mass * a)
            if a < 1:
                u2 = u.copy(); u2[i] = 0.5 * (1 + a)
                res = np.maximum(p - qrows[i], 0.0)
                for k, mk, uk in _midpoints(res):
                    u3 = u2.copy(); u3[gamma] = uk
                    finish(list(x[:i]) + [k], mass * (1 - a) * mk, u3)

        walk(0, np.full(gamma + 1, 0.5), w)
    return joint


def _target_stop_law(p_of, V, horizon, stop):
    joint = defaultdict(float)
    stack = [((), 1.0)]
    while stack:
        s, m = stack.pop()
        if len(s) == horizon or (s and s[-1] in stop):
            joint[s] += m
            continue
        for k, pk in enumerate(p_of(s)):
            if pk > 0:
                stack.append((s + (k,), m * pk))
    return joint


@pytest.mark.parametrize("V,gamma,stop,budget", [(3, 2, [2], None), (3, 3, [0], None), (2, 3, [1], None),
                                                 (3, 3, [], 2), (3, 2, [2], 2), (3, 3, [], 1)])
def test_stop_and_budget_law(V, gamma, stop, budget):
    rng = np.random.default_rng(7 * V + gamma + len(stop) + (budget or 0))
    p_of = prefix_table(rng, V, gamma + 2)
    q_of = prefix_table(rng, V, gamma + 2)
    horizon = gamma + 1 if budget is None else budget
    got = _stop_law(p_of, q_of, V, gamma, 1.0, horizon, stop, budget)
    exp = _target_stop_law(p_of, V, horizon, stop)
    keys = set(got) | set(exp)
    assert max(abs(got.get(k, 0.0) - exp.get(k, 0.0)) for k in keys) < 1e-12
