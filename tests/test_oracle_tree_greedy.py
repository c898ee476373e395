"""Pins of the greedy tree oracle (CPU only).

[M16] "Module 16: Speculative Decoding", "Verify the Tree -- and Why It's Exact": with a
toy target given as a next-token map (0->1, 1->2, 2->3, 3->4, 4->0, 5->5, 6->6, 7->7) and
the candidate tree of heads {1, 5}, {2}, {3}, {7}, the walk accepts 1, 2, 3 and emits
1, 2, 3, 4, which is plain greedy decoding of the target.  The pages state the identity
with plain greedy decoding for every target and tree; here it is checked on random
prefix-dependent targets and random trees, together with the reduction to the greedy
chain verifier on path trees and the limit T -> 0 of the membership walk.
"""
import numpy as np
import pytest

import oracle
from oracle.tree_greedy import verify_tree_greedy_one
from oracle.tree import verify_tree_one
from lawcheck import candidate_tree, rooted


def _onehot_rows(next_of, tokens, V):
    L = np.zeros((len(tokens), V))
    for v, t in enumerate(tokens):
        L[v, next_of(t)] = 1.0
    return L


def test_pages_example_chain_map():
    chain = {0: 1, 1: 2, 2: 3, 3: 4, 4: 0, 5: 5, 6: 6, 7: 7}
    tokens, parents = rooted(*candidate_tree([[1, 5], [2], [3], [7]]))
    # node 0 is the frontier whose last token is 0; every row is the map's next token
    L = _onehot_rows(lambda t: chain[t], tokens, 8)
    r = verify_tree_greedy_one(L, np.array(parents), np.array(tokens))
    assert r["status"] == oracle.OK
    assert [tokens[c] for c in r["path"]] == [1, 2, 3]
    assert r["tokens"] == [1, 2, 3, 4] and r["accepted_len"] == 3


def _random_tree(rng, V, N, repeat_tokens):
    """Random parent array and node tokens; unless repeat_tokens, a trie (siblings carry
    distinct tokens, so a node has at most V children)."""
    parents, tokens = [-1], [0]
    used = [set()]
    for v in range(1, N):
        open_nodes = [u for u in range(v) if repeat_tokens or len(used[u]) < V]
        pv = int(open_nodes[int(rng.integers(0, len(open_nodes)))])
        t = int(rng.integers(0, V))
        if not repeat_tokens:
            t = int(rng.choice(sorted(set(range(V)) - used[pv])))
        used[pv].add(t)
        used.append(set())
        parents.append(pv)
        tokens.append(t)
    return np.array(parents), np.array(tokens)


def _paths(parents, tokens):
    paths = [()] * len(parents)
    for v in range(1, len(parents)):
        paths[v] = paths[parents[v]] + (int(tokens[v]),)
    return paths


@pytest.mark.parametrize("repeat_tokens", [False, True])
def test_emits_plain_greedy_decoding(repeat_tokens):
    rng = np.random.default_rng(13 + repeat_tokens)
    for trial in range(200):
        V = int(rng.integers(2, 6))
        N = int(rng.integers(1, 16))
        table = {}

        def nxt(prefix):                         # a random prefix-dependent greedy target
            if prefix not in table:
                table[prefix] = rng.normal(0, 1, V)
            return table[prefix]
        parents, tokens = _random_tree(rng, V, N, repeat_tokens)
        paths = _paths(parents, tokens)
        L = np.stack([nxt(paths[v]) for v in range(N)])
        r = verify_tree_greedy_one(L, parents, tokens)
        assert r["status"] == oracle.OK
        greedy, pre = [], ()
        for _ in range(len(r["tokens"])):
            row = nxt(pre)
            t = int(np.flatnonzero(row == row.max())[0])
            greedy.append(t)
            pre = pre + (t,)
        assert r["tokens"] == greedy
        # the walk stops only where no child carries the greedy token
        end = r["path"][-1] if r["path"] else 0
        kids = [int(tokens[c]) for c in range(end + 1, N) if parents[c] == end]
        assert r["tokens"][-1] not in kids
        # accepted nodes form a root path
        prev = 0
        for c in r["path"]:
            assert parents[c] == prev
            prev = c


def test_deep_acceptance_on_a_target_built_from_the_tree():
    rng = np.random.default_rng(3)
    V, N = 5, 40
    parents, tokens = _random_tree(rng, V, N, False)
    kids = {v: [c for c in range(v + 1, N) if parents[c] == v] for v in range(N)}
    # row v favours its highest-index child's token: the walk follows those to a leaf
    L = rng.normal(0, 0.1, (N, V))
    for v in range(N):
        if kids[v]:
            L[v, tokens[kids[v][-1]]] = 5.0
    r = verify_tree_greedy_one(L, parents, tokens)
    v, path = 0, []
    while kids[v]:
        v = kids[v][-1]
        path.append(v)
    assert r["path"] == path and r["accepted_len"] == len(path)


def test_path_tree_is_the_greedy_chain_verifier():
    rng = np.random.default_rng(9)
    for trial in range(300):
        G, V = int(rng.integers(0, 6)), int(rng.integers(1, 5))
        L = np.round(rng.normal(0, 1, (G + 1, V)) * 2) / 2        # ties are common
        x = rng.integers(0, V, G)
        s, A, toks = oracle.verify_greedy_one(L, x)
        r = verify_tree_greedy_one(L, np.arange(-1, G), np.concatenate([[0], x]))
        assert (r["status"], r["accepted_len"], r["tokens"]) == (s, A, toks)


def test_zero_temperature_limit_of_membership():
    rng = np.random.default_rng(21)
    for trial in range(100):
        V, N = 6, 9
        parents, tokens = _random_tree(rng, V, N, True)
        L = rng.permuted(np.tile(np.arange(V) * 0.05, (N, 1)), axis=1)   # distinct values, gaps 0.05
        r0 = verify_tree_greedy_one(L, parents, tokens)
        # at T = 1e-3 the argmax holds all but ~e^-50 of the mass: a central uniform draws it
        r1 = verify_tree_one(L, parents, tokens, np.full(N, 0.5), 1e-3)
        assert r1["tokens"] == r0["tokens"] and r1["path"] == r0["path"]


def test_ties_and_repeated_siblings():
    # row 0 ties tokens 1 and 3: the lowest index (1) is the greedy token; two children
    # carry token 1: the lower-index one (node 2) is followed
    L = np.array([[0.0, 2.0, 0.0, 2.0], [0.0, 0.0, 0.0, 1.0], [0.0, 0.0, 1.0, 1.0], [1.0, 0.0, 0.0, 0.0]])
    parents = np.array([-1, 0, 0, 0])
    tokens = np.array([0, 3, 1, 1])
    r = verify_tree_greedy_one(L, parents, tokens)
    assert r["path"] == [2] and r["tokens"] == [1, 2]


def test_statuses_in_reached_order():
    L = np.zeros((4, 5))
    L[0, 2] = 1.0
    parents, tokens = np.array([-1, 0, 0, 1]), np.array([0, 2, 4, 1])
    bad = L.copy()
    bad[2, 0] = np.nan                           # node 2 is never reached
    assert verify_tree_greedy_one(bad, parents, tokens)["status"] == oracle.OK
    bad[1, 0] = np.inf                           # node 1's row is reached
    assert verify_tree_greedy_one(bad, parents, tokens)["status"] == oracle.NONFINITE
    neg = L.copy()
    neg[1] = -np.inf
    assert verify_tree_greedy_one(neg, parents, tokens)["status"] == oracle.NONFINITE
    assert verify_tree_greedy_one(L, np.array([-1, 0, 2, 1]), tokens)["status"] == oracle.BADTREE
    assert verify_tree_greedy_one(L, parents, np.array([0, 2, 5, 1]))["status"] == oracle.BADTREE
    one = verify_tree_greedy_one(L[:1], np.array([-1]), np.array([7]))
    assert one["tokens"] == [2] and one["accepted_len"] == 0
