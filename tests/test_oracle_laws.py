"""Exact-law pins of the oracle's samplers by brute-force enumeration (CPU only).

[M7.1] §0x03H (Loop 5: two-token vocabulary, K = 3, all draft paths, completion to
horizon K + 1) and §0x04G/§0x04H (Loop 10: prefix-indexed raw-logit tables,
temperature, horizon 3, all eight sequences) describe these oracles; [Tiny]
"Exactness tests" asks for exhaustive enumeration on vocabularies of 2 to 6.
The speculative joint must equal the target's own joint: a dropped term, a wrong
row, continuing after a rejection, a bonus drawn from q or an inverted ratio all
break the equality.
"""
import itertools

import numpy as np
import pytest
from scipy import stats as sst

import oracle
from oracle import laws
from oracle.chain import verify_chain_one
from lawcheck import (chain_joint, target_joint, max_joint_gap, tree_joint, prefix_table,
                      candidate_tree, rooted, logits_for)


def _context_free(rows):
    return lambda pre: rows[len(pre)]


@pytest.mark.parametrize("V,gamma", [(2, 3), (3, 2), (4, 2), (2, 1), (3, 1), (4, 3)])
def test_chain_law_context_free_rows(V, gamma):
    rng = np.random.default_rng(100 * V + gamma)
    for trial in range(3):
        P = rng.dirichlet(np.ones(V), gamma + 1)
        Q = rng.dirichlet(np.ones(V), gamma)
        if trial == 1:                      # exact zeros on both sides
            P[:, 0] = 0; P /= P.sum(1, keepdims=True)
            Q[:, -1] = 0; Q /= Q.sum(1, keepdims=True)
        T = [1.0, 0.8, 1.7][trial]
        joint, alen = chain_joint(_context_free(P), _context_free(Q), V, gamma, T)
        assert max_joint_gap(joint, target_joint(_context_free(P), V, gamma + 1)) < 1e-12
        # accepted-length law: context-free rows make alpha_i^reach = sum min(p_i, q_i)
        alphas = [laws.acceptance_rate(P[i], Q[i]) for i in range(gamma)]
        np.testing.assert_allclose(alen, laws.accepted_length_law(alphas), atol=1e-12)


@pytest.mark.parametrize("V,gamma", [(2, 2), (2, 3), (3, 2)])
def test_chain_law_prefix_indexed_tables(V, gamma):
    """Loop-10 style: rows depend on the whole prefix, so the row after a correction
    differs from the row after the rejected draft; only stop-at-first-rejection with
    the reached rows reproduces the target joint."""
    rng = np.random.default_rng(7 + V * 10 + gamma)
    p_of = prefix_table(rng, V, gamma)
    q_of = prefix_table(rng, V, gamma - 1)
    for T in (1.0, 0.6):
        joint, _ = chain_joint(p_of, q_of, V, gamma, T)
        assert max_joint_gap(joint, target_joint(p_of, V, gamma + 1)) < 1e-12


def test_loop5_two_token_k3():
    """Two-token vocabulary, K = 3: the fixed-length joint equals ordinary target decoding."""
    rng = np.random.default_rng(5)
    p_of = prefix_table(rng, 2, 3, zero_prob=0.0)
    q_of = prefix_table(rng, 2, 2, zero_prob=0.0)
    joint, _ = chain_joint(p_of, q_of, 2, 3, 1.0)
    tj = target_joint(p_of, 2, 4)
    assert len(tj) == 16
    assert max_joint_gap(joint, tj) < 1e-12


def test_negative_control_resampling_from_p_is_wrong():
    """[M16] pitfalls / [M7.1] §0x03C: correcting from p instead of the residual double
    counts.  Build that wrong law by hand and check it differs from p."""
    p = np.array([0.6, 0.3, 0.1]); q = np.array([0.2, 0.3, 0.5])
    alpha = laws.acceptance_rate(p, q)
    wrong = np.minimum(p, q) + (1 - alpha) * p
    assert np.abs(wrong - p).max() > 0.05


# ---------------------------------------------------------------- tree walk
def test_tree_law_random_trees():
    rng = np.random.default_rng(11)
    V, horizon = 3, 4
    p_of = prefix_table(rng, V, horizon)
    for trial in range(4):
        # random trie over V tokens, depth <= 3, distinct sibling tokens
        parents, tokens = [-1], [0]
        depth = [0]
        for v in range(1, 9):
            cand = [u for u in range(len(parents)) if depth[u] < 3 and
                    sum(1 for c in range(len(parents)) if parents[c] == u) < V]
            par = int(rng.choice(cand))
            used = {tokens[c] for c in range(len(parents)) if parents[c] == par}
            tok = int(rng.choice([t for t in range(V) if t not in used]))
            parents.append(par); tokens.append(tok); depth.append(depth[par] + 1)
        parents, tokens = np.array(parents), np.array(tokens)
        T = [1.0, 0.7, 1.3, 1.0][trial]
        joint, e_acc = tree_joint(p_of, parents, tokens, V, T, horizon)
        assert max_joint_gap(joint, target_joint(p_of, V, horizon)) < 1e-12
        # expected accepted nodes = E[G] - 1 from the positional model
        paths = [()]
        for v in range(1, len(parents)):
            paths.append(paths[parents[v]] + (int(tokens[v]),))
        probs = np.stack([p_of(paths[v]) for v in range(len(parents))])
        eg = oracle.tree_expected_nodes(parents, tokens, probs)
        assert e_acc == pytest.approx(eg - 1, abs=1e-12)
        assert 1 <= eg <= min(len(parents), max(depth) + 1)


def test_tree_greedy_example_with_one_hot_rows():
    """[M16] "Verify the Tree": next-token map, heads [[1,5],[2],[3],[7]] -> accepted [1,2,3],
    emitted [1,2,3,4].  One-hot target rows make the sampled walk the greedy walk."""
    import json, os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "m16_examples.json")))
    g = g["verify_tree_greedy"]
    nxt = {int(k): v for k, v in g["next_token_map"].items()}
    toks, pars = rooted(*candidate_tree(g["heads"]))
    V = 8
    N = len(toks)
    L = np.full((N, V), -np.inf)
    L[0, nxt[g["last_token"]]] = 0.0                 # frontier row
    for v in range(1, N):
        L[v, nxt[toks[v]]] = 0.0
    for u in (0.0, 0.37, 0.999):
        r = oracle.verify_tree_one(L, np.array(pars), np.array(toks), np.full(N, u), 1.0)
        assert r["status"] == oracle.OK
        assert [toks[c] for c in r["path"]] == g["accepted"]
        assert r["tokens"] == g["emitted"]


def test_tree_validation():
    V = 5
    good = np.array([-1, 0, 0, 1]), np.array([0, 1, 2, 3])
    assert oracle.validate_tree(*good, V)
    assert not oracle.validate_tree(np.array([0, 0, 0, 1]), good[1], V)     # root parent
    assert not oracle.validate_tree(np.array([-1, 0, 3, 1]), good[1], V)    # forward parent
    assert not oracle.validate_tree(np.array([-1, -1, 0, 1]), good[1], V)   # second root
    assert not oracle.validate_tree(good[0], np.array([0, 1, 5, 3]), V)     # token out of range
    L = np.zeros((4, V))
    r = oracle.verify_tree_one(L, np.array([-1, 0, 2, 1]), good[1], np.zeros(4), 1.0)
    assert r["status"] == oracle.BADTREE


def test_tree_duplicate_sibling_takes_lowest_index():
    V = 4
    L = np.full((4, V), -np.inf); L[0, 2] = 0.0; L[1:, 0] = 0.0
    parents = np.array([-1, 0, 0, 0]); tokens = np.array([0, 1, 2, 2])
    r = oracle.verify_tree_one(L, parents, tokens, np.zeros(4), 1.0)
    assert r["path"] == [2] and r["tokens"] == [2, 0]


# ---------------------------------------------------------------- greedy
def test_greedy_definition_and_ties():
    L = np.array([[0.0, 3.0, 3.0, -1.0],       # tie: lowest index 1
                  [5.0, -np.inf, 5.0, 5.0],    # tie: 0
                  [-1.0, -1.0, -0.5, -2.0]])
    s, A, toks = oracle.verify_greedy_one(L, np.array([1, 0]))
    assert (s, A, toks) == (oracle.OK, 2, [1, 0, 2])
    s, A, toks = oracle.verify_greedy_one(L, np.array([2, 0]))
    assert (s, A, toks) == (oracle.OK, 0, [1])
    s, A, toks = oracle.verify_greedy_one(L, np.array([1, 3]))
    assert (s, A, toks) == (oracle.OK, 1, [1, 0])
    # a wrong draft still emits exactly one token ([M16] Exercise 6)
    s, A, toks = oracle.verify_greedy_one(L, np.array([0, 0]))
    assert A == 0 and len(toks) == 1
    bad = L.copy(); bad[0, 0] = np.nan
    assert oracle.verify_greedy_one(bad, np.array([1, 0]))[0] == oracle.NONFINITE
    bad = L.copy(); bad[2, :] = -np.inf     # unreached unless both drafts match
    assert oracle.verify_greedy_one(bad, np.array([2, 0]))[0] == oracle.OK
    assert oracle.verify_greedy_one(bad, np.array([1, 0]))[0] == oracle.NONFINITE
    assert oracle.verify_greedy_one(L, np.array([4, 0]))[0] == oracle.BADTOKEN


def test_greedy_equals_serial_argmax_decode():
    """[M16] "Verify the Tree" (chain case): greedy verification emits exactly what serial
    greedy decoding would, for a next-token map target."""
    rng = np.random.default_rng(2)
    V = 7
    nxt = rng.integers(0, V, V)
    for trial in range(100):
        last = int(rng.integers(V))
        gamma = int(rng.integers(0, 6))
        serial = []
        t = last
        for _ in range(gamma + 1):
            t = int(nxt[t]); serial.append(t)
        drafts = [s if rng.random() < 0.7 else int(rng.integers(V)) for s in serial[:gamma]]
        ctx = [last] + drafts
        L = np.full((gamma + 1, V), -np.inf)
        for i in range(gamma + 1):
            L[i, nxt[ctx[i]]] = 0.0
        s, A, toks = oracle.verify_greedy_one(L, np.array(drafts, dtype=int))
        assert toks == serial[:A + 1]


# ---------------------------------------------------------------- Monte Carlo (secondary)
def test_chain_monte_carlo_first_token_and_length():
    """Seeded Monte Carlo as a secondary check ([M7.1] §0x04I): fresh drafts and uniforms per
    trial; chi-square on the first emitted token vs p_0 and on A vs Pr(A=a)."""
    rng = np.random.default_rng(12345)
    V, gamma, T, n = 6, 3, 1.0, 6000
    P = rng.dirichlet(np.ones(V) * 0.7, gamma + 1)
    Qr = rng.dirichlet(np.ones(V) * 0.7, gamma)
    L = np.stack([logits_for(P[i], T) for i in range(gamma + 1)])
    first = np.zeros(V); alen = np.zeros(gamma + 1)
    for _ in range(n):
        x = np.array([rng.choice(V, p=Qr[i]) for i in range(gamma)])
        u = rng.integers(0, 1 << 24, gamma + 1) * 2.0 ** -24
        r = verify_chain_one(L, Qr, x, u, T)
        first[r.tokens[0]] += 1
        alen[r.accepted_len] += 1
    exp_first = P[0] * n
    assert sst.chisquare(first, exp_first).pvalue > 1e-3
    law = laws.accepted_length_law([laws.acceptance_rate(P[i], Qr[i]) for i in range(gamma)])
    assert sst.chisquare(alen, law * n).pvalue > 1e-3
