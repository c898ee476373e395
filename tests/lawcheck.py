"""Brute-force law checks of the oracle's samplers on tiny vocabularies.

The samplers are deterministic functions of the caller's uniforms.  Each branch of
a round (accept prefix, first rejection, terminal token) occupies an interval of
uniform values whose length is its probability.  These helpers drive the oracle
with one uniform inside every branch, check that the oracle takes that branch, and
add the branch's probability to the joint law of the emitted tokens.  Short rounds
are completed with ordinary target draws up to a common horizon, so the speculative
joint can be compared with the target's own autoregressive joint
([M7.1] §0x03H and §0x04H: enumerate draft paths, first rejections and terminal
tokens, then complete to a fixed horizon).
"""
from __future__ import annotations

import itertools
from collections import defaultdict

import numpy as np

import oracle
from oracle.chain import verify_chain_one
from oracle.tree import verify_tree_one


def logits_for(p: np.ndarray, T: float) -> np.ndarray:
    """Logits whose temperature softmax is p (zeros become -inf)."""
    T = float(np.float32(T))
    with np.errstate(divide="ignore"):
        return T * np.log(np.asarray(p, dtype=np.float64))


def _midpoints(weights: np.ndarray):
    """(k, mass_k, u_k) for every positive-mass index, u_k inside the k-th CDF interval."""
    c = np.cumsum(weights)
    W = c[-1]
    lo = 0.0
    out = []
    for k, w in enumerate(weights):
        hi = c[k] / W
        if w > 0:
            out.append((k, w / W, 0.5 * (lo + hi)))
        lo = hi
    return out


def chain_joint(p_of, q_of, V: int, gamma: int, T: float):
    """Speculative joint over sequences of length gamma + 1.

    p_of(prefix) / q_of(prefix): target / draft next-token rows given a tuple prefix.
    Returns (joint dict, accepted-length law array).
    """
    joint = defaultdict(float)
    alen = np.zeros(gamma + 1)
    for x in itertools.product(range(V), repeat=gamma):
        qrows = [np.asarray(q_of(x[:i]), dtype=np.float64) for i in range(gamma)]
        qmass = float(np.prod([qrows[i][x[i]] for i in range(gamma)])) if gamma else 1.0
        if qmass == 0.0:
            continue
        L = np.stack([logits_for(p_of(x[:i]), T) for i in range(gamma + 1)])
        Q = np.stack(qrows) if gamma else np.zeros((0, V))
        xs = np.asarray(x, dtype=np.int64)
        # thresholds along the path: accept everything that can be accepted
        probe = verify_chain_one(L, Q, xs, np.zeros(gamma + 1), T)
        assert probe.status == oracle.OK
        a = probe.a
        for r in range(gamma + 1):
            if r < gamma:
                if len(a) <= r:
                    break
                prefix_w = float(np.prod(a[:r]))
                branch_w = prefix_w * (1.0 - a[r])
                if branch_w == 0.0:
                    continue
                u = np.zeros(gamma + 1)
                u[r] = a[r]                # the smallest uniform that rejects draft r
            else:
                if len(a) < gamma:
                    continue
                branch_w = float(np.prod(a)) if gamma else 1.0
                if branch_w == 0.0:
                    continue
                u = np.zeros(gamma + 1)
            res = verify_chain_one(L, Q, xs, u, T)
            assert res.status == oracle.OK and res.accepted_len == r, (x, r, res)
            for k, mass, uk in _midpoints(res.weights):
                u2 = u.copy()
                u2[gamma] = uk
                res2 = verify_chain_one(L, Q, xs, u2, T)
                assert res2.accepted_len == r and res2.tokens[-1] == k, (x, r, k, res2)
                y = tuple(int(t) for t in x[:r]) + (k,)
                alen[r] += qmass * branch_w * mass
                # complete to the horizon with ordinary target draws
                for tail in itertools.product(range(V), repeat=gamma - r):
                    seq = y + tail
                    pr = 1.0
                    for j in range(r + 1, gamma + 1):
                        pr *= p_of(seq[:j])[seq[j]]
                    if pr > 0:
                        joint[seq] += qmass * branch_w * mass * pr
    return joint, alen


def target_joint(p_of, V: int, length: int):
    out = {}
    for seq in itertools.product(range(V), repeat=length):
        pr = 1.0
        for j in range(length):
            pr *= p_of(seq[:j])[seq[j]]
        if pr > 0:
            out[seq] = pr
    return out


def max_joint_gap(a: dict, b: dict) -> float:
    keys = set(a) | set(b)
    return max(abs(a.get(k, 0.0) - b.get(k, 0.0)) for k in keys)


def tree_joint(p_of, parents, node_tokens, V: int, T: float, horizon: int):
    """Emitted-token joint of the membership walk, completed to `horizon` tokens.

    Node v's row is the target's next-token row after the tokens on the root-to-v
    path (node 0 = the frontier, empty path).  Returns (joint, E[accepted nodes]).
    """
    N = len(parents)
    paths = [()] * N
    for v in range(1, N):
        paths[v] = paths[parents[v]] + (int(node_tokens[v]),)
    L = np.stack([logits_for(p_of(paths[v]), T) for v in range(N)])
    joint = defaultdict(float)
    e_acc = 0.0

    # enumerate draws along the walk: state = (node, uniforms so far, probability)
    stack = [(0, np.full(N, 0.5), 1.0)]
    while stack:
        v, u, w = stack.pop()
        for k, mass, uk in _midpoints(np.asarray(p_of(paths[v]), dtype=np.float64)):
            u2 = u.copy()
            u2[v] = uk
            child = next((c for c in range(v + 1, N)
                          if parents[c] == v and node_tokens[c] == k), None)
            if child is not None:
                stack.append((child, u2, w * mass))
                continue
            res = verify_tree_one(L, np.asarray(parents), np.asarray(node_tokens), u2, T)
            assert res["status"] == oracle.OK
            assert res["tokens"][-1] == k and len(res["path"]) == len(paths[v]), (res, v, k)
            y = paths[v] + (k,)
            e_acc += w * mass * len(res["path"])
            for tail in itertools.product(range(V), repeat=horizon - len(y)):
                seq = y + tail
                pr = 1.0
                for j in range(len(y), horizon):
                    pr *= p_of(seq[:j])[seq[j]]
                if pr > 0:
                    joint[seq] += w * mass * pr
    return joint, e_acc


def prefix_table(rng: np.random.Generator, V: int, depth: int, zero_prob: float = 0.25):
    """Random prefix-indexed next-token table (every prefix up to `depth` tokens).

    Some entries are exactly zero (masked tokens), but every row keeps mass.
    """
    table = {}
    for n in range(depth + 1):
        for pre in itertools.product(range(V), repeat=n):
            row = rng.random(V) + 0.05
            row[rng.random(V) < zero_prob] = 0.0
            if row.sum() == 0:
                row[rng.integers(V)] = 1.0
            table[pre] = row / row.sum()
    return lambda pre: table[tuple(pre)]


def candidate_tree(heads):
    """Cartesian candidate tree as a forest: every node of depth d branches into the
    tokens of head d+1 ([M16] "The Candidate Tree"; [M7.7] §0x07C counts its nodes).
    Returns (tokens, parents) in breadth-first order with -1 for depth-1 nodes."""
    tokens, parents = [], []
    level = [-1]
    for head in heads:
        nxt = []
        for par in level:
            for t in head:
                tokens.append(int(t))
                parents.append(par)
                nxt.append(len(tokens) - 1)
        level = nxt
    return tokens, parents


def rooted(tokens, parents):
    """Prepend the frontier as node 0: forest roots become its children."""
    return [0] + list(tokens), [-1] + [p + 1 if p >= 0 else 0 for p in parents]
