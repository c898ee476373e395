"""Pins of the residual-update tree oracle (CPU only).

[M7.7] "M7.7 - Draft Sources, Dependent Heads, and Hardware-Aware Trees" §0x09A: for
target p = (0.5, 0.3, 0.2) and two i.i.d. proposals from q = (0.4, 0.4, 0.2), the output
marginal over all nine proposal pairs, every accept/reject branch and the final residual
sample is p; testing each candidate against the original p instead is not (§0x08B).
The walk is driven with one uniform inside every branch interval (the approach of
lawcheck.py) and the emitted joint law, completed to a horizon with target draws, must
equal the target's own joint for random trees, i.i.d. and per-child proposals alike.
A path-shaped tree is the chain verifier.
"""
import itertools
from collections import defaultdict

import numpy as np
import pytest

import oracle
from oracle.tree_residual import verify_tree_residual_one
from oracle.chain import verify_chain_one
from lawcheck import logits_for, _midpoints, target_joint, max_joint_gap, prefix_table


def _paths(parents, tokens):
    N = len(parents)
    paths = [()] * N
    for v in range(1, N):
        paths[v] = paths[parents[v]] + (int(tokens[v]),)
    return paths


def residual_walk_law(p_of, q_of, parents, V, T, horizon, retest_original=False, verify_rows=None):
    """Joint law of the emitted tokens (completed to `horizon`) over the proposals (node c's
    token drawn from q_of(c, tokens of its ancestors, tokens of its earlier siblings)) and
    the walk's uniforms.

    retest_original: weight the branches as if every child were tested against the
    original p (the wrong procedure of [M7.7] §0x08B); the oracle is then not consulted.
    verify_rows: rows given to the verifier instead of the proposal rows (a proposal /
    verifier mismatch, [M7.7] §0x0AB); called like q_of.
    """
    N = len(parents)
    children = {v: [c for c in range(v + 1, N) if parents[c] == v] for v in range(N)}
    joint = defaultdict(float)
    for toks in itertools.product(range(V), repeat=N - 1):
        tokens = (0,) + toks
        paths = _paths(parents, tokens)
        sibs = [tuple(tokens[s] for s in children[parents[c]] if s < c) if c else () for c in range(N)]
        qrows = [np.zeros(V)] + [np.asarray(q_of(c, paths[parents[c]], sibs[c]), np.float64) for c in range(1, N)]
        w_prop = float(np.prod([qrows[c][tokens[c]] for c in range(1, N)]))
        if verify_rows is not None:
            qrows = [np.zeros(V)] + [np.asarray(verify_rows(c, paths[parents[c]], sibs[c]), np.float64)
                                     for c in range(1, N)]
        if w_prop == 0.0:
            continue
        L = np.stack([logits_for(p_of(paths[v]), T) for v in range(N)])
        Q = np.stack(qrows)
        stack = [(0, np.full(N, 0.5), np.full(N, 0.5), 1.0)]
        while stack:
            v, ua, ud, w = stack.pop()
            p = np.asarray(p_of(paths[v]), np.float64)
            res = p.copy()
            ua = ua.copy()
            for c in children[v]:
                x = tokens[c]
                a = min(1.0, (p if retest_original else res)[x] / qrows[c][x])
                if a > 0.0:
                    ua2 = ua.copy()
                    ua2[c] = 0.5 * a
                    stack.append((c, ua2, ud, w * a))
                if a >= 1.0:
                    w = 0.0
                    break
                ua[c] = 0.5 * (1.0 + a)
                w *= 1.0 - a
                if not retest_original:
                    g = np.maximum(res - qrows[c], 0.0)
                    res = g / g.sum()
            if w == 0.0:
                continue
            for k, mass, uk in _midpoints(p if retest_original else res):
                ud2 = ud.copy()
                ud2[v] = uk
                if not retest_original:
                    r = verify_tree_residual_one(L, Q, np.asarray(parents), np.asarray(tokens), ua, ud2, T)
                    assert r["status"] == oracle.OK, r
                    assert r["tokens"] == list(paths[v]) + [k], (r, v, k)
                y = paths[v] + (k,)
                for tail in itertools.product(range(V), repeat=horizon - len(y)):
                    seq = y + tail
                    pr = 1.0
                    for j in range(len(y), horizon):
                        pr *= p_of(seq[:j])[seq[j]]
                    if pr > 0:
                        joint[seq] += w_prop * w * mass * pr
    return joint


def test_pages_example_two_iid_proposals():
    p = np.array([0.5, 0.3, 0.2])
    q = np.array([0.4, 0.4, 0.2])
    p_of = lambda pre: p if len(pre) == 0 else np.full(3, 1 / 3)
    q_of = lambda c, pre, sib: q
    parents = [-1, 0, 0]
    first = lambda joint: np.array([sum(v for s, v in joint.items() if s[0] == k) for k in range(3)])
    joint = residual_walk_law(p_of, q_of, parents, 3, 1.0, 2)
    marg = first(joint)
    assert np.allclose(marg, p, atol=1e-12), marg
    assert max_joint_gap(joint, target_joint(p_of, 3, 2)) < 1e-12
    # the wrong procedure of testing each candidate against the original p
    wrong = residual_walk_law(p_of, q_of, parents, 3, 1.0, 2, retest_original=True)
    wmarg = first(wrong)
    assert abs(wmarg.sum() - 1.0) < 1e-12
    assert np.abs(wmarg - p).max() > 0.01, wmarg


def test_pages_degenerate_example_duplicated_mass():
    # §0x08B: every draft is token 1 and the target is Bernoulli(1/2): k independent tests
    # against p would emit 1 with probability 1 - 2^-k; the residual procedure keeps 1/2
    p = np.array([0.5, 0.5])
    q = np.array([0.0, 1.0])
    p_of = lambda pre: p if len(pre) == 0 else np.full(2, 0.5)
    for k in (2, 3):
        parents = [-1] + [0] * k
        first1 = lambda joint: sum(v for s, v in joint.items() if s[0] == 1)
        joint = residual_walk_law(p_of, lambda c, pre, sib: q, parents, 2, 1.0, 2)
        assert abs(first1(joint) - 0.5) < 1e-12
        wrong = residual_walk_law(p_of, lambda c, pre, sib: q, parents, 2, 1.0, 2, retest_original=True)
        # at least 1 - 2^-k (the pages' bound); all-rejected rounds add 2^-k * p(1)
        assert first1(wrong) >= 1 - 0.5 ** k
        assert abs(first1(wrong) - (1 - 0.5 ** k + 0.5 ** k * 0.5)) < 1e-12


@pytest.mark.parametrize("V,k,iid", [(2, 1, True), (3, 2, True), (3, 3, True), (3, 2, False), (4, 2, False)])
def test_law_depth_one(V, k, iid):
    rng = np.random.default_rng(40 * V + k + (0 if iid else 7))
    p_of = prefix_table(rng, V, 2)
    qs = [rng.dirichlet(np.ones(V)) for _ in range(k + 1)]
    q_of = (lambda c, pre, sib: qs[0]) if iid else (lambda c, pre, sib: qs[c])
    parents = [-1] + [0] * k
    joint = residual_walk_law(p_of, q_of, parents, V, 0.9, 2)
    assert max_joint_gap(joint, target_joint(p_of, V, 2)) < 1e-12


@pytest.mark.parametrize("shape", ["two_by_two", "chain_and_fan"])
def test_law_depth_two(shape):
    V = 2
    rng = np.random.default_rng(11 if shape == "two_by_two" else 12)
    p_of = prefix_table(rng, V, 3)
    q_tab = {}

    def q_of(c, pre, sib):
        # each parent's children drawn i.i.d. from a proposal that depends on the prefix
        if pre not in q_tab:
            q_tab[pre] = rng.dirichlet(np.ones(V))
        return q_tab[pre]
    parents = [-1, 0, 0, 1, 1, 2, 2] if shape == "two_by_two" else [-1, 0, 1, 1, 0]
    joint = residual_walk_law(p_of, q_of, parents, V, 1.0, 3)
    assert max_joint_gap(joint, target_joint(p_of, V, 3)) < 1e-12


def test_path_tree_is_the_chain_verifier():
    rng = np.random.default_rng(5)
    V, G = 6, 3
    for trial in range(200):
        L = rng.normal(0, 1.5, (G + 1, V))
        Q = rng.dirichlet(np.ones(V), G)
        x = np.array([rng.choice(V, p=Q[i]) for i in range(G)])
        u = rng.random(G + 1)
        # tree: node i + 1 is draft i, child of node i; node rows = chain rows
        parents = np.arange(-1, G)
        tokens = np.concatenate([[0], x])
        Qt = np.concatenate([np.zeros((1, V)), Q])
        ua = np.concatenate([[0.5], u[:G]])
        ud = np.full(G + 1, u[G])
        t = verify_tree_residual_one(L, Qt, parents, tokens, ua, ud, 1.0)
        c = verify_chain_one(L, Q, x, u, 1.0)
        assert t["status"] == c.status == oracle.OK
        assert t["tokens"] == c.tokens and t["accepted_len"] == c.accepted_len


def test_statuses_in_reached_order():
    V = 4
    p = np.array([0.25] * 4)
    L = np.stack([logits_for(p, 1.0)] * 3)
    Q = np.stack([p] * 3)
    parents = np.array([-1, 0, 0])
    tokens = np.array([0, 1, 2])
    ua, ud = np.array([0.5, 0.9, 0.9]), np.array([0.3, 0.3, 0.3])
    r = verify_tree_residual_one(L, Q, parents, tokens, ua, ud, 1.0)
    # p = q: child 1 is accepted whatever u < 1 is
    assert r["status"] == oracle.OK and r["path"] == [1]
    bad = L.copy(); bad[0, 2] = np.nan
    assert verify_tree_residual_one(bad, Q, parents, tokens, ua, ud, 1.0)["status"] == oracle.NONFINITE
    Qz = Q.copy(); Qz[1, 1] = 0.0
    assert verify_tree_residual_one(L, Qz, parents, tokens, ua, ud, 1.0)["status"] == oracle.QZERO
    assert verify_tree_residual_one(L, Q, parents, tokens, np.array([0.5, 1.0, 0.9]), ud, 1.0)["status"] == oracle.BADUNIFORM
    assert verify_tree_residual_one(L, Q, np.array([-1, 0, 2]), tokens, ua, ud, 1.0)["status"] == oracle.BADTREE
    assert verify_tree_residual_one(L, Q, parents, np.array([0, 1, 9]), ua, ud, 1.0)["status"] == oracle.BADTREE
    # the first child is rejected (p(1) = 0) and the second child's q row has a negative
    # entry only after a rejection is it read as a whole
    p0 = np.array([0.5, 0.0, 0.25, 0.25])
    L0 = np.stack([logits_for(p0, 1.0)] * 3)
    Qn = Q.copy(); Qn[1, 3] = -0.1
    assert verify_tree_residual_one(L0, Qn, parents, tokens, ua, ud, 1.0)["status"] == oracle.RESIDUAL_EMPTY
    # every child rejected, then a bad terminal uniform
    ua0 = np.array([0.5, 0.5, 0.999999])
    r = verify_tree_residual_one(L0, Q, parents, tokens, ua0, np.array([1.5, 0.3, 0.3]), 1.0)
    assert r["status"] == oracle.BADUNIFORM


def test_leaf_root_is_a_plain_target_draw():
    p = np.array([0.1, 0.2, 0.3, 0.4])
    L = logits_for(p, 0.7)[None]
    for j in range(40):
        u = (j + 0.5) / 40
        r = verify_tree_residual_one(L, np.zeros((1, 4)), np.array([-1]), np.array([0]), np.array([0.5]),
                                     np.array([u]), 0.7)
        assert r["tokens"] == [int(np.searchsorted(np.cumsum(p), u, side="right"))]


@pytest.mark.parametrize("V,k", [(2, 2), (3, 2), (3, 3), (4, 3)])
def test_law_without_replacement_proposals(V, k):
    """[M7.7] §0x0AB (Sequoia): siblings drawn without replacement, each from the draft row
    with the earlier siblings' tokens removed (uniform over the unsampled tokens once the
    draft mass is used up); verified with those rows, the emitted law is the target's."""
    from synth import without_replacement_row
    rng = np.random.default_rng(60 + 10 * V + k)
    p_of = prefix_table(rng, V, 2)
    q0 = rng.dirichlet(np.ones(V))
    if V >= 3:
        q0[rng.integers(V)] = 0.0                      # a token the draft never proposes first
        q0 /= q0.sum()
    q_of = lambda c, pre, sib: without_replacement_row(q0, sib)
    parents = [-1] + [0] * k
    joint = residual_walk_law(p_of, q_of, parents, V, 1.0, 2)
    assert max_joint_gap(joint, target_joint(p_of, V, 2)) < 1e-12


def test_without_replacement_with_iid_rows_is_wrong():
    """[M7.7] §0x0AB: without-replacement sampling changes the proposal law, so the verifier
    for i.i.d. samples (every sibling tested against the drafter's original row) is not
    exact for it."""
    from synth import without_replacement_row
    p = np.array([0.2, 0.5, 0.3])
    q0 = np.array([0.6, 0.3, 0.1])
    p_of = lambda pre: p if len(pre) == 0 else np.full(3, 1 / 3)
    parents = [-1, 0, 0]
    first = lambda joint: np.array([sum(v for s, v in joint.items() if s[0] == t) for t in range(3)])
    right = residual_walk_law(p_of, lambda c, pre, sib: without_replacement_row(q0, sib), parents, 3, 1.0, 2)
    assert np.allclose(first(right), p, atol=1e-12)
    wrong = residual_walk_law(p_of, lambda c, pre, sib: without_replacement_row(q0, sib), parents, 3, 1.0, 2,
                              verify_rows=lambda c, pre, sib: q0)
    assert abs(first(wrong).sum() - 1.0) < 1e-12
    assert np.abs(first(wrong) - p).max() > 0.01, first(wrong)
