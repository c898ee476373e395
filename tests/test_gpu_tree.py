"""GPU parity of spec_verify_tree against the oracle: statuses, accepted lengths, path
nodes and emitted tokens exact, except requests the oracle flags (a draw within 1e-6
of a CDF boundary)."""
import json
import os

import numpy as np
import pytest

import oracle
import synth
from gpu_util import say, run_tree, compare_exact

pytestmark = pytest.mark.gpu

KEYS = ["accepted_len", "out_tokens", "out_nodes"]


def oracle_tree(x, requests=None):
    return oracle.verify_tree(x.logits, x.parents, x.node_tokens, x.u, x.temperature,
                              x.logit_dtype, requests=requests)


def check(x):
    got = run_tree(x)
    exp = oracle_tree(x)
    compare_exact(got, exp, KEYS, flagged=exp["flagged"])
    return got, exp


def test_config5_full():
    """B=32 requests, 63-node trees of depth <= 6, V=152064 bf16, T=1."""
    x = synth.make_config(5, 0)
    say("tree config5 B=32 N=63 V=152064")
    got, exp = check(x)
    print("accepted", got["accepted_len"].tolist(), "flagged", int(exp["flagged"].sum()))


def test_config5_deep_variant():
    """Child tokens boosted by +8 in their parent's row so that walks go deep."""
    x = synth.make_config(5, 1, boost=8.0)
    say("tree config5 deep variant")
    got, exp = check(x)
    print("accepted", got["accepted_len"].tolist())
    assert got["accepted_len"].max() >= 4


@pytest.mark.parametrize("V,dtype,N,T", [(1, "bf16", 3, 1.0), (5, "f32", 9, 0.7), (2049, "bf16", 31, 1.0),
                                         (8193, "f32", 17, 1.3), (40000, "bf16", 63, 0.9),
                                         # 128 chunk summaries, the most the walker's one-wave
                                         # sample takes, and one element more
                                         (262144, "bf16", 15, 1.0), (262145, "f32", 15, 0.8)])
def test_ragged(V, dtype, N, T):
    x = synth.make_tree(8, N, V, seed=V + N, logit_dtype=dtype, temperature=T,
                        max_depth=min(6, N - 1), max_children=4, boost=6.0)
    say(f"tree ragged V={V} {dtype} N={N}")
    check(x)


def test_single_node_tree():
    x = synth.make_tree(4, 1, 3000, seed=4)
    say("tree N=1")
    got, exp = check(x)
    assert (got["accepted_len"] == 0).all()


def test_m16_greedy_tree_with_one_hot_rows():
    """[M16] "Verify the Tree": accepted [1, 2, 3], emitted [1, 2, 3, 4]."""
    from lawcheck import candidate_tree, rooted
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "m16_examples.json")))
    g = g["verify_tree_greedy"]
    nxt = {int(k): v for k, v in g["next_token_map"].items()}
    toks, pars = rooted(*candidate_tree(g["heads"]))
    V, N = 64, len(toks)
    L = np.full((1, N, V), -np.inf, np.float32)
    L[0, 0, nxt[g["last_token"]]] = 0.0
    for v in range(1, N):
        L[0, v, nxt[toks[v]]] = 0.0
    x = synth.TreeInputs(1, N, V, np.float32(1.0), "f32", L, np.array([toks], np.int32),
                         np.array([pars], np.int32), np.full((1, N), 0.5, np.float32))
    say("tree m16 example")
    got, _ = check(x)
    n = got["accepted_len"][0]
    assert [toks[c] for c in got["out_nodes"][0][:n]] == g["accepted"]
    assert got["out_tokens"][0][:n + 1].tolist() == g["emitted"]


def test_bad_trees_and_rows():
    x = synth.make_tree(6, 15, 4096, seed=12, boost=8.0)
    x.parents[0, 0] = 0                       # root must have parent -1
    x.parents[1, 5] = 7                       # forward parent
    x.node_tokens[2, 3] = 4096                # node token out of range
    x.u[3, 0] = 1.0                           # bad uniform at the root
    lg = synth.bf16_bits_to_f32(x.logits)
    lg[4, 0, 11] = np.nan                     # NaN in the root row
    x.logits = synth.f32_to_bf16_bits(lg)
    say("tree bad inputs")
    got, exp = check(x)
    assert exp["status"].tolist()[:5] == [6, 6, 6, 3, 1]


def test_repeatable():
    x = synth.make_config(5, 2, B=8, boost=6.0)
    say("tree repeatability")
    a, b = run_tree(x), run_tree(x)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k])


@pytest.mark.parametrize("T", [0.01, 100.0])
def test_extreme_temperatures(T):
    x = synth.make_tree(8, 31, 20000, seed=int(T * 10) + 5, logit_dtype="bf16", temperature=T, max_depth=4,
                        max_children=4, boost=6.0)
    say(f"tree T={T}")
    got, exp = check(x)
    print("accepted", got["accepted_len"].tolist(), "flagged", int(exp["flagged"].sum()))
