"""GPU parity of spec_verify_tree_greedy (the temperature-0 membership walk) against the
oracle: statuses, accepted lengths, path nodes and emitted tokens bit-exact (every
decision is an exact comparison of logits)."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import synth
import exact_rejection_sampling_amd as sv
from gpu_util import DEV, say, t_logits, t_i32, to_np, compare_exact

pytestmark = pytest.mark.gpu

KEYS = ["accepted_len", "out_tokens", "out_nodes"]


def run(x, workspace_tensor=None):
    return to_np(sv.spec_verify_tree_greedy(t_logits(x.logits, x.logit_dtype), t_i32(x.node_tokens),
                                            t_i32(x.parents), workspace_tensor=workspace_tensor))


def expected(x):
    return oracle.verify_tree_greedy(x.logits, x.parents, x.node_tokens, x.logit_dtype)


def check(x):
    got, exp = run(x), expected(x)
    compare_exact(got, exp, KEYS)
    return got, exp


def test_tree_workload_shape():
    """B=32 requests, 63-node trees of depth <= 6, V=152064 bf16; children drawn from a
    noisy drafter."""
    x = synth.make_config(5, 0)
    say("tree_greedy config5 B=32 N=63 V=152064")
    got, _ = check(x)
    print("accepted", got["accepted_len"].tolist())


def test_deep_walks():
    x = synth.make_config(5, 1, boost=8.0)
    say("tree_greedy config5 deep variant")
    got, _ = check(x)
    print("accepted", got["accepted_len"].tolist())
    assert got["accepted_len"].max() >= 4


@pytest.mark.parametrize("V,dtype,N", [(1, "bf16", 3), (5, "f32", 9), (2049, "bf16", 31), (8193, "f32", 17),
                                       (40000, "bf16", 63), (65537, "f32", 7)])
def test_ragged(V, dtype, N):
    x = synth.make_tree(8, N, V, seed=3 * V + N, logit_dtype=dtype, max_depth=min(6, N - 1), max_children=4,
                        boost=6.0)
    say(f"tree_greedy ragged V={V} {dtype} N={N}")
    check(x)


def test_pages_example_next_token_map():
    """[M16] "Verify the Tree": accepted [1, 2, 3], emitted [1, 2, 3, 4]."""
    from lawcheck import candidate_tree, rooted
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "m16_examples.json")))
    g = g["verify_tree_greedy"]
    nxt = {int(k): v for k, v in g["next_token_map"].items()}
    toks, pars = rooted(*candidate_tree(g["heads"]))
    V, N = 64, len(toks)
    L = np.zeros((1, N, V), np.float32)
    L[0, 0, nxt[g["last_token"]]] = 1.0
    for v in range(1, N):
        L[0, v, nxt[toks[v]]] = 1.0
    x = synth.TreeInputs(1, N, V, np.float32(1.0), "f32", L, np.array([toks], np.int32),
                         np.array([pars], np.int32), np.zeros((1, N), np.float32))
    say("tree_greedy m16 example")
    got, _ = check(x)
    n = got["accepted_len"][0]
    assert [toks[c] for c in got["out_nodes"][0][:n]] == g["accepted"]
    assert got["out_tokens"][0][:n + 1].tolist() == g["emitted"]


def test_ties_across_chunks_take_the_lowest_index():
    """Coarse bf16 rows: the maximum repeats within and across 2048-element chunks, in
    root and helper-summarized rows alike."""
    B, N, V = 16, 15, 30000
    rng = np.random.default_rng(41)
    vals = np.round(rng.normal(0, 1, (B, N, V)) * 2) / 2
    top = vals.max() + 1.0
    for b in range(B):
        for v in range(N):
            vals[b, v, rng.choice(V, size=3, replace=False)] = top      # three-way tie
    parents = np.stack([synth.random_tree(rng, N, 4, 3) for _ in range(B)])
    tokens = rng.integers(0, V, (B, N)).astype(np.int32)
    for b in range(B):                       # make the walk go down: a child holds the tie's lowest index
        for v in range(N):
            kids = np.nonzero(parents[b] == v)[0]
            if kids.size:
                tokens[b, kids[-1]] = int(np.flatnonzero(vals[b, v] == top)[0])
    x = synth.TreeInputs(B, N, V, np.float32(1.0), "bf16", synth.f32_to_bf16_bits(vals.astype(np.float32)),
                         tokens, parents.astype(np.int32), np.zeros((B, N), np.float32))
    say("tree_greedy ties")
    got, _ = check(x)
    assert got["accepted_len"].min() >= 1


def test_path_trees_match_the_greedy_chain_kernel():
    g = synth.make_greedy(16, 6, 12000, seed=52, logit_dtype="bf16", match_prob=0.8)
    parents = np.tile(np.arange(-1, 6, dtype=np.int32), (16, 1))
    tokens = np.concatenate([np.zeros((16, 1), np.int32), g.tokens], axis=1)
    x = synth.TreeInputs(16, 7, 12000, np.float32(1.0), "bf16", g.logits, tokens, parents,
                         np.zeros((16, 7), np.float32))
    say("tree_greedy path trees vs spec_verify_greedy")
    got = run(x)
    chain = to_np(sv.spec_verify_greedy(t_logits(g.logits, "bf16"), t_i32(g.tokens)))
    np.testing.assert_array_equal(got["accepted_len"], chain["accepted_len"])
    np.testing.assert_array_equal(got["out_tokens"], chain["out_tokens"])
    np.testing.assert_array_equal(got["req_status"], chain["req_status"])


def test_bad_trees_and_rows():
    x = synth.make_tree(8, 15, 4096, seed=12, boost=8.0, logit_dtype="f32")
    x.parents[0, 0] = 0                       # root must have parent -1
    x.parents[1, 5] = 7                       # forward parent
    x.node_tokens[2, 3] = 4096                # node token out of range
    x.logits[3, 0, 11] = np.nan               # NaN in the root row
    x.logits[4, 0, :] = -np.inf               # root row entirely -inf
    x.logits[5, 0, 100] = np.inf              # +inf in the root row
    kids = np.nonzero(x.parents[6] == 0)[0]   # request 6: a child row that the walk reaches
    exp6 = oracle.verify_tree_greedy_one(x.logits[6].astype(np.float64), x.parents[6], x.node_tokens[6])
    x.logits[6, exp6["path"][0] if exp6["path"] else 0, 7] = np.nan
    leaves = [v for v in range(15) if not (x.parents[7] == v).any()]
    x.logits[7, leaves[-1], 3] = np.nan       # request 7: NaN in a leaf row (reached or not)
    say("tree_greedy bad inputs")
    got, exp = check(x)
    assert exp["status"].tolist()[:7] == [6, 6, 6, 1, 1, 1, 1]


def test_single_node_trees():
    x = synth.make_tree(4, 1, 3000, seed=4)
    say("tree_greedy N=1")
    got, _ = check(x)
    assert (got["accepted_len"] == 0).all()


def test_workspace_returns_to_zero_and_repeats():
    x = synth.make_config(5, 2, B=8, boost=6.0)
    ws = torch.zeros(sv.tree_workspace_bytes(x.B, x.N, x.V) + 512, dtype=torch.uint8, device=DEV)
    say("tree_greedy workspace reuse")
    a = run(x, workspace_tensor=ws)
    b = run(x, workspace_tensor=ws)
    torch.cuda.synchronize()
    assert int(ws.count_nonzero()) == 0
    for k in a:
        np.testing.assert_array_equal(a[k], b[k])


def _streamed_ahead_request(kind, rng, N, V):
    """One request whose root children are laid out for one outcome of the helpers' guess of
    the root child: 'hit' (the walk's child is the guess), 'tie' (two tokens share the root
    maximum; the walk takes the lower token, and so does the guess), 'miss' (the walk's child
    is node 280, past the nodes the guess looks at, while nodes 1..4 are root children too),
    'none' (no root child among nodes 1..256 has a finite logit: nothing is streamed ahead)
    and 'stay' (no root child carries the root's argmax token)."""
    par = np.full(N, 1, np.int32)
    par[0] = -1
    par[1] = 0
    rows = rng.normal(0.0, 1.0, (N, V)).astype(np.float32)
    tok = rng.permutation(V)[:N].astype(np.int32)          # distinct tokens
    kids = {"hit": [1, 2, 3, 4, 5], "tie": [1, 2, 3, 4, 5], "miss": [1, 2, 3, 4, 280],
            "none": [1, 270, 290], "stay": [1, 2, 3, 4, 5]}[kind]
    for c in kids:
        par[c] = 0
    target = {"hit": 3, "tie": 5, "miss": 280, "none": 290, "stay": None}[kind]
    if kind == "none":
        rows[0, tok[1]] = -np.inf                          # node 1 cannot be guessed
    if kind == "tie":
        lo, hi = sorted(int(t) for t in rng.choice(V, 2, replace=False))
        tok[5], tok[2] = lo, hi                            # node 2 carries the higher token
        rows[0, lo] = rows[0, hi] = 10.0
    elif target is not None:
        rows[0, tok[target]] = 10.0
    if target is not None:                                 # two more levels below the target
        a, bb = (6, 7) if target < 256 else (target + 1, target + 2)
        par[a], par[bb] = target, a
        rows[target, tok[a]] = 10.0
        rows[a, tok[bb]] = 10.0
    return par, tok, rows


def test_root_child_streamed_ahead_hit_miss_and_none():
    """The greedy tree's helpers stream one root child's row ahead of the first order; every
    outcome of that guess gives the oracle's walk, and the workspace returns to zero."""
    B, N, V = 10, 300, 5000
    rng = np.random.default_rng(97)
    kinds = ["hit", "tie", "miss", "none", "stay"] * 2
    parts = [_streamed_ahead_request(k, rng, N, V) for k in kinds]
    parents = np.stack([p[0] for p in parts])
    tokens = np.stack([p[1] for p in parts])
    logits = np.stack([p[2] for p in parts])
    x = synth.TreeInputs(B, N, V, np.float32(1.0), "f32", logits, tokens, parents, np.zeros((B, N), np.float32))
    ws = torch.zeros(sv.tree_workspace_bytes(B, N, V) + 512, dtype=torch.uint8, device=DEV)
    say("tree_greedy streamed-ahead root child: hit, tie, miss, none, stay")
    got, exp = run(x, workspace_tensor=ws), expected(x)
    compare_exact(got, exp, KEYS)
    torch.cuda.synchronize()
    assert int(ws.count_nonzero()) == 0
    want = {"hit": 3, "tie": 3, "miss": 3, "none": 3, "stay": 0}
    assert got["accepted_len"].tolist() == [want[k] for k in kinds]
