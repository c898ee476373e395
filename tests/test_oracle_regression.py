"""The oracle still produces the stored outputs of tests/golden/oracle_regression.json
(written by tests/golden/make_golden.py), and the input generator is reproducible."""
import json
import os

import numpy as np

import oracle
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden", "oracle_regression.json")


def test_oracle_matches_stored_outputs():
    cases = json.load(open(GOLD))["cases"]
    for c in cases:
        x = synth.make_config(c["config"], c["run"], **c.get("override", {}))
        if c["kind"] == "chain":
            o = oracle.verify_chain(x.logits, x.q, x.tokens, x.u, x.temperature, x.logit_dtype)
        elif c["kind"] == "greedy":
            o = oracle.verify_greedy(x.logits, x.tokens, x.logit_dtype)
        elif c["kind"] == "tree_residual":
            o = oracle.verify_tree_residual(x.logits, x.q, x.parents, x.node_tokens, x.u_acc, x.u_draw,
                                            x.temperature, x.logit_dtype)
            assert o["out_nodes"].tolist() == c["out_nodes"]
        else:
            o = oracle.verify_tree(x.logits, x.parents, x.node_tokens, x.u, x.temperature, x.logit_dtype)
            assert o["out_nodes"].tolist() == c["out_nodes"]
        assert o["accepted_len"].tolist() == c["accepted_len"]
        assert o["out_tokens"].tolist() == c["out_tokens"]
        assert o["status"].tolist() == c["status"]


def test_generator_is_reproducible_and_well_formed():
    a = synth.make_config(2, 0, B=3, V=500)
    b = synth.make_config(2, 0, B=3, V=500)
    assert np.array_equal(a.logits, b.logits) and np.array_equal(a.q, b.q)
    assert np.array_equal(a.tokens, b.tokens) and np.array_equal(a.u, b.u)
    assert a.logits.dtype == np.uint16 and a.logits.shape == (3, 6, 500)
    assert a.q.dtype == np.float32 and a.q.shape == (3, 5, 500)
    # every proposal has positive draft probability; uniforms lie on the 2^-24 grid of [0,1)
    qx = np.take_along_axis(a.q, a.tokens[..., None].astype(np.int64), 2)[..., 0]
    assert (qx > 0).all()
    k = a.u.astype(np.float64) * 2 ** 24
    assert (k == np.floor(k)).all() and (a.u >= 0).all() and (a.u < 1).all()
    c = synth.make_config(2, 1, B=3, V=500)
    assert not np.array_equal(a.logits, c.logits)


def test_generator_bf16_rounding():
    x = np.array([1.0, 1.00390625, 1.005859375, -3.3, np.inf, -np.inf], dtype=np.float32)
    bits = synth.f32_to_bf16_bits(x)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: ties to even -> 1.0
    assert bits[0] == 0x3F80 and bits[1] == 0x3F80
    assert bits[2] == 0x3F81            # 1 + 1.5*2^-8 rounds up
    assert bits[4] == 0x7F80 and bits[5] == 0xFF80
    assert abs(synth.bf16_bits_to_f32(bits[3:4])[0] + 3.3) < 0.02


def test_tree_generator_shape():
    t = synth.make_config(5, 0, B=2, N=63, V=1000)
    for b in range(2):
        par = t.parents[b]
        assert par[0] == -1 and all(0 <= par[v] < v for v in range(1, 63))
        depth = np.zeros(63, int)
        for v in range(1, 63):
            depth[v] = depth[par[v]] + 1
        assert depth.max() <= 6
        assert np.bincount(par[1:], minlength=63).max() <= 4
        for v in range(63):       # distinct sibling tokens (a trie)
            kids = np.nonzero(par == v)[0]
            assert len(set(t.node_tokens[b, kids].tolist())) == len(kids)
