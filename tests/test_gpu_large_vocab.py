"""GPU parity at vocabularies far above the workloads' (V = 8 500 000, and the residual
tree's limit V = 2^21), where the kernels take the paths that only long rows reach: more
than 64 statistics slices per row (each decision lane loops over slices), more than 2048
terminal chunks per row (the selector re-reads chunk masses beyond the 8 it keeps in
registers), tree rows of more than 1024 chunks (the walker reads the row's summaries from
the workspace instead of staging them in LDS), and hundreds of helper blocks per row; and
trees at the node limit N = 4096, and a residual-update node with more rejected children
than a helper keeps in LDS.  Same comparisons as the workload-size tests."""
import numpy as np
import pytest

import oracle
import synth
import exact_rejection_sampling_amd as sv
from gpu_util import say, compare_chain, compare_exact, run_chain, run_greedy, run_tree, t_logits, t_f32, t_i32, to_np

pytestmark = pytest.mark.gpu

BIG = 8_500_000          # 2076 terminal chunks and 4151 wave chunks per row
TREE_KEYS = ["accepted_len", "out_tokens", "out_nodes"]


def test_chain_residual_over_eight_million_tokens():
    """One request, draft 0 rejected (u = 0.999999): the residual of a 2076-chunk row."""
    x = synth.make_chain(1, 1, BIG, seed=700, logit_dtype="bf16", sigma=3.0, boost_frac=0.001, noise=1.0,
                         temperature=1.0)
    x.u = x.u.copy()
    x.u[0, 0] = np.float32(0.999999)
    exp = oracle.verify_chain(x.logits, x.q, x.tokens, x.u, x.temperature, x.logit_dtype)
    assert exp["accepted_len"][0] == 0
    say(f"chain residual B=1 gamma=1 V={BIG}")
    print(compare_chain(run_chain(x), exp))


def test_chain_bonus_over_eight_million_tokens():
    """q = p: the draft is accepted and the 2076-chunk bonus row is sampled."""
    x = synth.make_chain(1, 1, BIG, seed=701, logit_dtype="f32", sigma=2.0, noise=0.0, temperature=1.0)
    exp = oracle.verify_chain(x.logits, x.q, x.tokens, x.u, x.temperature, x.logit_dtype)
    say(f"chain bonus B=1 gamma=1 V={BIG}")
    compare_chain(run_chain(x), exp)
    assert exp["accepted_len"][0] == 1


def test_greedy_over_eight_million_tokens():
    x = synth.make_greedy(2, 2, BIG, seed=702, logit_dtype="bf16", match_prob=0.8)
    say(f"greedy B=2 gamma=2 V={BIG}")
    compare_exact(run_greedy(x), oracle.verify_greedy(x.logits, x.tokens, x.logit_dtype),
                  ["accepted_len", "out_tokens"])


def test_trees_over_eight_million_tokens():
    """A path of three children, each boosted by +30 in its parent's row: both walks go to
    the bottom, sampling rows of 4151 chunks (summaries read from the workspace)."""
    x = synth.make_tree(1, 4, BIG, seed=703, logit_dtype="bf16", max_depth=3, max_children=1, boost=30.0)
    exp = oracle.verify_tree(x.logits, x.parents, x.node_tokens, x.u, x.temperature, x.logit_dtype)
    say(f"tree B=1 N=4 V={BIG} (path)")
    compare_exact(run_tree(x), exp, TREE_KEYS, flagged=exp["flagged"])
    say(f"tree_greedy B=1 N=4 V={BIG} (path)")
    got = to_np(sv.spec_verify_tree_greedy(t_logits(x.logits, x.logit_dtype), t_i32(x.node_tokens),
                                           t_i32(x.parents)))
    compare_exact(got, oracle.verify_tree_greedy(x.logits, x.parents, x.node_tokens, x.logit_dtype), TREE_KEYS)
    assert exp["accepted_len"][0] == 3 and got["accepted_len"][0] == 3


def test_residual_tree_at_its_vocabulary_limit():
    V = 1 << 21
    x = synth.make_tree_residual(2, 7, V, seed=704, sigma=2.0, noise=0.5, max_depth=3, max_children=3)
    say(f"tree_residual B=2 N=7 V={V}")
    got = to_np(sv.spec_verify_tree_residual(t_logits(x.logits, x.logit_dtype), t_f32(x.q), t_i32(x.node_tokens),
                                             t_i32(x.parents), t_f32(x.u_acc), t_f32(x.u_draw),
                                             float(x.temperature)))
    exp = oracle.verify_tree_residual(x.logits, x.q, x.parents, x.node_tokens, x.u_acc, x.u_draw,
                                      x.temperature, x.logit_dtype)
    compare_exact(got, exp, TREE_KEYS, flagged=exp["flagged"])
    print("accepted", got["accepted_len"].tolist())


def test_trees_with_the_most_nodes():
    """N = 4096 nodes (the limit), random trees of depth <= 40: the membership walks and the
    child searches over thousands of nodes."""
    x = synth.make_tree(3, 4096, 512, seed=705, logit_dtype="f32", max_depth=40, max_children=6, boost=12.0)
    say("tree B=3 N=4096 V=512")
    exp = oracle.verify_tree(x.logits, x.parents, x.node_tokens, x.u, x.temperature, x.logit_dtype)
    compare_exact(run_tree(x), exp, TREE_KEYS, flagged=exp["flagged"])
    say("tree_greedy B=3 N=4096 V=512")
    got = to_np(sv.spec_verify_tree_greedy(t_logits(x.logits, x.logit_dtype), t_i32(x.node_tokens),
                                           t_i32(x.parents)))
    compare_exact(got, oracle.verify_tree_greedy(x.logits, x.parents, x.node_tokens, x.logit_dtype), TREE_KEYS)
    print("accepted", exp["accepted_len"].tolist(), got["accepted_len"].tolist())


def test_residual_tree_with_hundreds_of_rejected_siblings():
    """A root with 300 children, every one proposing a token the target almost never takes
    (the target's mass sits on tokens 0..9, the drafter's on 10..511): all 300 are rejected,
    so the residual carries 300 updates -- past the 256 rejected children a helper keeps in
    LDS -- before the final draw."""
    B, N, V = 2, 301, 512
    rng = np.random.default_rng(706)
    logits = rng.normal(0, 1, (B, N, V)).astype(np.float32)
    logits[:, 0, :10] += 20.0
    q = np.zeros((B, N, V), np.float32)
    q[:, 1:, 10:] = np.float32(1.0 / (V - 10))
    parents = np.zeros((B, N), np.int32)
    parents[:, 0] = -1
    tokens = np.zeros((B, N), np.int32)
    tokens[:, 1:] = rng.integers(10, V, (B, N - 1))
    u_acc = rng.random((B, N), dtype=np.float32)
    u_draw = rng.random((B, N), dtype=np.float32)
    exp = oracle.verify_tree_residual(logits, q, parents, tokens, u_acc, u_draw, 1.0, "f32")
    assert (exp["accepted_len"] == 0).all() and (exp["status"] == 0).all()
    say("tree_residual B=2 star of 300 rejected children V=512")
    got = to_np(sv.spec_verify_tree_residual(t_f32(logits), t_f32(q), t_i32(tokens), t_i32(parents), t_f32(u_acc),
                                             t_f32(u_draw), 1.0))
    compare_exact(got, exp, TREE_KEYS, flagged=exp["flagged"])
    assert (got["out_tokens"][:, 0] < 10).all()
