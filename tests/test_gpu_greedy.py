"""GPU parity of spec_verify_greedy against the oracle: bit-exact (integer work)."""
import numpy as np
import pytest
import torch

import oracle
import synth
import exact_rejection_sampling_amd as sv
from gpu_util import DEV, say, run_greedy, compare_exact

pytestmark = pytest.mark.gpu


def oracle_greedy(x, requests=None):
    return oracle.verify_greedy(x.logits, x.tokens, x.logit_dtype, requests=requests)


def test_config4_full():
    """B=256, gamma=8, V=128256 bf16 (the greedy workload), every request compared."""
    x = synth.make_config(4, 0)
    say("greedy config4 B=256 gamma=8 V=128256")
    got = run_greedy(x)
    compare_exact(got, oracle_greedy(x), ["accepted_len", "out_tokens"])
    print("mean accepted", got["accepted_len"].mean())


@pytest.mark.parametrize("V,dtype,gamma", [(1, "bf16", 3), (2, "f32", 4), (7, "bf16", 2),
                                           (2047, "bf16", 5), (2049, "f32", 5), (8193, "bf16", 8),
                                           (32000, "f32", 0), (50257, "bf16", 6), (5000, "bf16", 63)])
def test_ragged(V, dtype, gamma):
    x = synth.make_greedy(24, gamma, V, seed=V + gamma, logit_dtype=dtype, match_prob=0.85)
    say(f"greedy ragged V={V} {dtype} gamma={gamma}")
    compare_exact(run_greedy(x), oracle_greedy(x), ["accepted_len", "out_tokens"])


def test_ties_take_the_lowest_index():
    """Coarse bf16 values make exact ties common; plant more across chunk borders."""
    B, G, V = 32, 4, 10000
    rng = np.random.default_rng(5)
    vals = np.round(rng.normal(0, 1, (B, G + 1, V)) * 2) / 2          # few distinct values
    for b in range(B):
        for i in range(G + 1):
            pos = rng.choice(V, 3, replace=False)
            vals[b, i, pos] = vals[b, i].max() + 1.0                    # a 3-way tie at the top
    x = synth.GreedyInputs(B, G, V, "bf16", synth.f32_to_bf16_bits(vals.astype(np.float32)),
                           np.zeros((B, G), np.int32))
    f = synth.bf16_bits_to_f32(x.logits)
    first = np.array([[np.flatnonzero(f[b, i] == f[b, i].max())[0] for i in range(G)] for b in range(B)])
    x.tokens = np.where(rng.random((B, G)) < 0.8, first, (first + 1) % V).astype(np.int32)
    say("greedy ties")
    compare_exact(run_greedy(x), oracle_greedy(x), ["accepted_len", "out_tokens"])


def test_negative_zero_and_masked_rows():
    B, G, V = 6, 2, 3000
    L = np.full((B, G + 1, V), -np.inf, np.float32)
    L[0, :, 10] = -0.0; L[0, :, 20] = 0.0             # -0 and +0 tie: lowest index (10)
    L[1, :, 2999] = 5.0                                 # max at the very last position
    L[2, :, 0] = -1e30; L[2, :, 5] = -1e30              # very negative but finite
    L[3, 0, 7] = 1.0; L[3, 1:, :] = -np.inf             # row 1 unreached? draft 0 must mismatch
    L[4, :, 8] = 1.0; L[4, 0, 9] = np.nan               # NaN in reached row 0
    L[5, :, 8] = 1.0; L[5, 2, 8] = np.inf               # +inf in the bonus row
    tok = np.array([[10, 10], [2999, 2999], [0, 0], [6, 0], [8, 8], [8, 8]], np.int32)
    x = synth.GreedyInputs(B, G, V, "f32", L, tok)
    say("greedy signed zero / masked rows")
    got = run_greedy(x)
    exp = oracle_greedy(x)
    compare_exact(got, exp, ["accepted_len", "out_tokens"])
    assert exp["status"].tolist() == [0, 0, 0, 0, 1, 1]


def test_bad_tokens():
    x = synth.make_greedy(4, 3, 100, seed=3, match_prob=1.0)
    x.tokens[1, 0] = 100
    x.tokens[2, 1] = -1                      # reached only if draft 0 matches (it does)
    x.tokens[3, 2] = 1 << 30
    say("greedy bad tokens")
    got = run_greedy(x)
    exp = oracle_greedy(x)
    compare_exact(got, exp, ["accepted_len", "out_tokens"])
    assert exp["status"].tolist() == [0, 2, 2, 2]


def test_greedy_matches_chain_with_one_hot_targets():
    """[M7.1] §0x02D: with one-hot target rows the chain rule is the greedy check."""
    B, G, V = 16, 5, 3000
    rng = np.random.default_rng(8)
    best = rng.integers(0, V, (B, G + 1))
    L = np.full((B, G + 1, V), -np.inf, np.float32)
    L[np.arange(B)[:, None], np.arange(G + 1)[None], best] = 0.0
    tok = np.where(rng.random((B, G)) < 0.7, best[:, :G], rng.integers(0, V, (B, G))).astype(np.int32)
    q = rng.dirichlet(np.ones(V), (B, G)).astype(np.float32)
    q[q <= 0] = 1e-30
    say("greedy vs chain one-hot")
    g = run_greedy(synth.GreedyInputs(B, G, V, "f32", L, tok))
    from gpu_util import t_f32, t_i32, to_np
    c = to_np(sv.spec_verify_chain(t_f32(L), t_f32(q), t_i32(tok),
                                   t_f32(rng.random((B, G + 1)).astype(np.float32) * 0.999), 1.0))
    np.testing.assert_array_equal(g["accepted_len"], c["accepted_len"])
    np.testing.assert_array_equal(g["out_tokens"], c["out_tokens"])


def test_repeatable():
    x = synth.make_greedy(64, 6, 70000, seed=1)
    say("greedy repeatability")
    a, b = run_greedy(x), run_greedy(x)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k])
