"""Pins of the float64 oracle against values the pages print and closed forms.

CPU only.  Every expected value here is either printed on a page (fixtures under
tests/golden/, each naming its source) or fixed by mathematics (identities, closed
forms, special cases that reduce to a textbook result).
"""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import laws
from oracle.chain import verify_chain_one, inverse_cdf
from oracle.numerics import bf16_to_f64, softmax_maxshift, softmax_online, target_probs
from lawcheck import logits_for

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- AI-atlas three-symbol trace
def test_atlas_three_symbol_trace():
    g = gold("atlas_three_symbol.json")
    p, q = np.array(g["p"]), np.array(g["q"])
    a = [laws.accept_probability(p[x], q[x]) for x in range(3)]
    np.testing.assert_allclose(a, g["accept_probability"], atol=1e-15)
    np.testing.assert_allclose(q * np.array(a), g["accepted_mass"], atol=1e-15)
    alpha = laws.acceptance_rate(p, q)
    assert alpha == pytest.approx(g["alpha"], abs=1e-15)
    assert 1 - alpha == pytest.approx(g["rejected_mass"], abs=1e-15)
    r = laws.residual_distribution(p, q)
    np.testing.assert_allclose(r, g["residual"], atol=1e-15)
    np.testing.assert_allclose(q * np.array(a) + (1 - alpha) * r, g["output"], atol=1e-15)
    law = laws.iid_output_count_law(g["iid_alpha"], g["iid_gamma"])
    np.testing.assert_allclose(law, g["iid_output_count_probs"], atol=1e-15)
    assert (law * np.arange(1, 4)).sum() == pytest.approx(g["iid_expected_count"], abs=1e-12)
    assert laws.expected_tokens(0.6, 2) == pytest.approx(g["iid_expected_count"], abs=1e-12)


def test_atlas_trace_through_the_sampler():
    """The chain sampler on the three-symbol rows: every correction is A (residual [1,0,0])."""
    g = gold("atlas_three_symbol.json")
    p, q = np.array(g["p"]), np.array(g["q"])
    L = np.stack([logits_for(p, 1.0)] * 2)
    Q = q[None, :]
    for x, a in enumerate(g["accept_probability"]):
        if a < 1:
            for ut in (0.0, 0.3, 0.999):
                r = verify_chain_one(L, Q, np.array([x]), np.array([a + 1e-9, ut]), 1.0)
                assert r.accepted_len == 0 and r.tokens == [0]
        r = verify_chain_one(L, Q, np.array([x]), np.array([0.0, 0.5]), 1.0)
        assert r.accepted_len == 1 and r.tokens[0] == x
        assert r.a[0] == pytest.approx(a, abs=1e-12)


# ---------------------------------------------------------------- Module 16 examples
def test_m16_verify_draft_example():
    g = gold("m16_examples.json")["verify_draft"]
    p, q = np.array(g["p"]), np.array(g["q"])
    assert round(laws.acceptance_rate(p, q), 3) == g["alpha_3dp"]
    assert round(1 - laws.total_variation(p, q), 3) == g["alpha_3dp"]
    np.testing.assert_allclose(laws.residual_distribution(p, q), g["residual"], atol=1e-12)
    # the printed outcome (1 accepted, emitted [0, 0]) is the rejection branch at draft 1;
    # the one-hot residual makes the correction 0 whatever the terminal uniform
    L = np.stack([logits_for(p, 1.0)] * 3)
    Q = np.stack([q, q])
    a1 = p[1] / q[1] + 1e-9
    for ut in (0.0, 0.5, 0.9999):
        r = verify_chain_one(L, Q, np.array(g["draft_tokens"]), np.array([0.3, a1, ut]), 1.0)
        assert r.accepted_len == g["printed_accepted"]
        assert r.tokens == g["printed_emitted"]
    # draft 0 (p >= q) is always accepted: a = 1
    r = verify_chain_one(L, Q, np.array(g["draft_tokens"]), np.array([0.999, 0.999, 0.5]), 1.0)
    assert r.a[0] == 1.0 and r.accepted_len == 1


def test_m16_exercise1_alpha_equals_one_minus_tv():
    g = gold("m16_examples.json")["exercise1"]
    p = np.array(g["p"])
    for case in g["cases"]:
        q = np.array(case["q"])
        assert round(laws.acceptance_rate(p, q), 3) == case["alpha_3dp"]
        assert laws.acceptance_rate(p, q) == pytest.approx(1 - laws.total_variation(p, q), abs=1e-15)


def test_m16_exercise2_gamma_sweep():
    g = gold("m16_examples.json")["exercise2"]
    tok = [round(laws.expected_tokens(g["alpha"], k), 2) for k in g["gamma"]]
    spd = [round(laws.speculative_speedup(g["alpha"], k, g["c"]), 2) for k in g["gamma"]]
    assert tok == g["tokens_per_pass_2dp"]
    assert spd == g["speedup_2dp"]
    best = max(g["gamma"], key=lambda k: laws.speculative_speedup(g["alpha"], k, g["c"]))
    assert best == g["best_gamma"]


def test_m16_exercise3_identity():
    g = gold("m16_examples.json")["exercise3"]
    p, q = np.array(g["p"]), np.array(g["q"])
    alpha = laws.acceptance_rate(p, q)
    rec = np.minimum(p, q) + laws.residual_distribution(p, q) * (1 - alpha)
    np.testing.assert_allclose(rec, p, atol=1e-15)


def test_m16_exercise4_chain_of_heads():
    g = gold("m16_examples.json")["exercise4"]
    got = [round(laws.chain_of_heads_expected_length([d ** k for k in range(1, g["heads"] + 1)]), 2)
           for d in g["decays"]]
    assert got == g["tokens_per_pass_2dp"]


# ---------------------------------------------------------------- M7.1 / M7.7 examples
def test_m71_three_token_example():
    """Values printed in the three-token example; the tables themselves were lost, so
    any completion with p(A)=0.3, q(A)=0.6, p-q = +0.25 on B and +0.05 on C is used."""
    g = gold("m71_m77_examples.json")["three_token"]
    q = np.array([g["q_A"], 0.15, 0.25])
    p = np.array([g["p_A"], q[1] + g["residual_B"], q[2] + g["residual_C"]])
    assert p.sum() == pytest.approx(1.0) and q.sum() == pytest.approx(1.0)
    assert laws.accept_probability(p[0], q[0]) == pytest.approx(g["accept_A"])
    assert laws.positive_residual(p, q).sum() == pytest.approx(g["Z"])
    r = laws.residual_distribution(p, q)
    assert round(r[1], 3) == g["p_prime_B_3dp"] and round(r[2], 3) == g["p_prime_C_3dp"]
    assert laws.acceptance_rate(p, q) == pytest.approx(g["diagonal"])
    assert laws.total_variation(p, q) == pytest.approx(g["Z"])


def test_m77_positional_chain():
    g = gold("m71_m77_examples.json")["positional"]
    h = np.array(g["h"])
    p = h * np.concatenate([[1.0], np.cumprod(1 - h)[:-1]])    # p_j = h_j prod_{i<j}(1 - h_i)
    np.testing.assert_allclose(p, g["p"], atol=1e-15)
    assert p.sum() == pytest.approx(g["p_sum"], abs=1e-15)
    assert 1 - p.sum() == pytest.approx(g["none_selected"], abs=1e-15)
    # five-node chain, each child selected w.p. 0.82: E[G] = 1 + .82 + ... + .82^4
    n, a = g["chain_nodes"], g["chain_child_prob"]
    parents = np.arange(-1, n - 1)
    node_tokens = np.ones(n, dtype=int)
    probs = np.tile([1 - a, a], (n, 1))            # token 1 (the child) w.p. 0.82
    eg = oracle.tree_expected_nodes(parents, node_tokens, probs)
    assert eg == pytest.approx(g["chain_expected"], abs=1e-12)
    assert round((g["t5"] + g["depth"] * g["c"]) / eg, 4) == g["chain_time_per_token_4dp"]
    assert laws.expected_progress([a] * (n - 1)) == pytest.approx(eg, abs=1e-12)


def test_m77_cartesian_count():
    from lawcheck import candidate_tree
    g = gold("m71_m77_examples.json")["cartesian"]
    tokens, parents = candidate_tree([[0] * b for b in g["b"]])
    assert len(tokens) == g["n_tree"]


def test_m16_candidate_tree_layout():
    from lawcheck import candidate_tree
    g = gold("m16_examples.json")["candidate_tree"]
    tokens, parents = candidate_tree(g["heads"])
    assert tokens == g["tokens"] and parents == g["parents"]


# ---------------------------------------------------------------- closed forms
@pytest.mark.parametrize("alpha", [0.0, 0.3, 0.66, 0.9, 1.0])
@pytest.mark.parametrize("gamma", [0, 1, 5, 8])
def test_closed_form_equals_survival_sum(alpha, gamma):
    assert laws.expected_tokens(alpha, gamma) == pytest.approx(
        laws.expected_progress([alpha] * gamma), rel=1e-13, abs=1e-13)
    law = laws.accepted_length_law([alpha] * gamma)
    assert law.sum() == pytest.approx(1.0, abs=1e-14) and (law >= -1e-15).all()


def test_front_vs_back_loaded_acceptance():
    """[M7.1] §0x05E: same arithmetic mean, different survival tails and E[G]."""
    front, back = [0.95, 0.90, 0.60, 0.40], [0.40, 0.60, 0.90, 0.95]
    assert np.mean(front) == pytest.approx(np.mean(back))
    assert laws.expected_progress(front) > laws.expected_progress(back)
    assert laws.survival(front)[-1] == pytest.approx(laws.survival(back)[-1])


# ---------------------------------------------------------------- numerics
def test_bf16_decode_known_patterns():
    bits = np.array([0x3F80, 0xC000, 0x7F80, 0xFF80, 0x0001, 0x4049, 0x8000], dtype=np.uint16)
    v = bf16_to_f64(bits)
    assert v[0] == 1.0 and v[1] == -2.0 and v[2] == np.inf and v[3] == -np.inf
    assert v[4] == 2.0 ** -133
    assert v[5] == 3.140625
    assert v[6] == 0.0 and np.signbit(v[6])
    assert np.isnan(bf16_to_f64(np.array([0x7FC0], dtype=np.uint16)))[0]


def test_softmax_backends_agree_and_normalize():
    rng = np.random.default_rng(7)
    for V in (1, 3, 1023, 1024, 1025, 5000):
        s = rng.normal(0, 8, V)
        s[rng.random(V) < 0.1] = -np.inf
        if np.isneginf(s).all():
            s[0] = 0.0
        p1, m1, Z1 = softmax_maxshift(s)
        p2, m2, Z2 = softmax_online(s, block=1024)
        assert m1 == m2
        np.testing.assert_allclose(p2, p1, rtol=1e-13, atol=1e-300)
        assert p1.sum() == pytest.approx(1.0, abs=1e-13)
        assert (p1[np.isneginf(s)] == 0).all()


def test_temperature_known_values():
    """softmax([0, ln 3] / 1) = [1/4, 3/4]; halving T squares the odds: [1/10, 9/10]."""
    l = np.array([0.0, np.log(3.0)])
    p, _, _ = target_probs(l, 1.0)
    np.testing.assert_allclose(p, [0.25, 0.75], atol=1e-15)
    p, _, _ = target_probs(l, 0.5)
    np.testing.assert_allclose(p, [0.1, 0.9], atol=1e-15)


def test_temperature_uses_the_fp32_value():
    l = np.array([0.0, 1.0])
    p, _, _ = target_probs(l, 0.8)
    T = float(np.float32(0.8))
    assert p[1] / p[0] == pytest.approx(np.exp(1.0 / T), rel=1e-15)


def test_inverse_cdf_uniform_weights_is_floor():
    V = 64
    w = np.ones(V)
    for k in range(0, 1 << 24, 99991):
        u = k * 2.0 ** -24
        assert inverse_cdf(w, u)[0] == int(np.floor(u * V))


def test_inverse_cdf_exact_law_on_a_grid():
    """Dyadic weights + every u on a 2^-10 grid: each index is drawn exactly w_k/W of the time;
    zero-weight indices never."""
    w = np.array([1, 0, 3, 0, 4, 0, 0, 8], dtype=float) / 16.0
    counts = np.zeros(len(w))
    M = 1 << 10
    for j in range(M):
        counts[inverse_cdf(w, j / M)[0]] += 1
    np.testing.assert_array_equal(counts / M, w)


# ---------------------------------------------------------------- special cases
def test_one_hot_target_reduces_to_greedy():
    """[M7.1] §0x02D: with p one-hot, the p/q rule is the greedy longest-prefix check."""
    rng = np.random.default_rng(3)
    V, gamma = 6, 4
    for trial in range(200):
        best = rng.integers(0, V, gamma + 1)
        L = np.full((gamma + 1, V), -np.inf)
        L[np.arange(gamma + 1), best] = 0.0
        Q = rng.dirichlet(np.ones(V), gamma)
        x = np.where(rng.random(gamma) < 0.6, best[:gamma], rng.integers(0, V, gamma))
        u = rng.random(gamma + 1)
        r = verify_chain_one(L, Q, x, u, 1.0)
        s, A, toks = oracle.verify_greedy_one(L, x)
        assert (r.accepted_len, r.tokens) == (A, toks)


def test_q_equal_p_accepts_everything():
    rng = np.random.default_rng(4)
    V, gamma = 50, 5
    for T in (0.7, 1.0, 1.3):
        L = rng.normal(0, 3, (gamma + 1, V))
        Q = np.stack([target_probs(L[i], T)[0] for i in range(gamma)])
        x = np.array([rng.choice(V, p=Q[i]) for i in range(gamma)])
        r = verify_chain_one(L, Q, x, rng.random(gamma + 1) * 0.999, T)
        assert r.accepted_len == gamma and r.a == pytest.approx([1.0] * gamma)


def test_p_zero_always_rejects_and_residual_avoids_q_excess():
    """[M7.1] §0x03D: a drafted x with p(x) = 0 is always rejected; tokens where q >= p get
    no correction mass."""
    p = np.array([0.0, 0.5, 0.5, 0.0])
    q = np.array([0.4, 0.1, 0.5, 0.0])
    L = np.stack([logits_for(p, 1.0)] * 2)
    for u0 in (0.0, 0.5):
        for ut in np.linspace(0, 0.999, 17):
            r = verify_chain_one(L, q[None], np.array([0]), np.array([u0, ut]), 1.0)
            assert r.accepted_len == 0 and r.tokens == [1]   # only B has p > q


def test_status_order_and_reached_semantics():
    V = 4
    p = np.array([0.25] * 4)
    L = np.stack([logits_for(p, 1.0)] * 3)
    Q = np.stack([p, p])
    ok = verify_chain_one(L, Q, np.array([1, 2]), np.array([0.1, 0.1, 0.1]), 1.0)
    assert ok.status == oracle.OK and ok.accepted_len == 2
    bad = L.copy(); bad[0, 1] = np.nan
    assert verify_chain_one(bad, Q, np.array([1, 2]), np.array([0.1, 0.1, 0.1]), 1.0).status == oracle.NONFINITE
    bad = L.copy(); bad[0, 1] = np.inf
    assert verify_chain_one(bad, Q, np.array([1, 2]), np.array([0.1, 0.1, 0.1]), 1.0).status == oracle.NONFINITE
    bad = L.copy(); bad[0, :] = -np.inf
    assert verify_chain_one(bad, Q, np.array([1, 2]), np.array([0.1, 0.1, 0.1]), 1.0).status == oracle.NONFINITE
    assert verify_chain_one(L, Q, np.array([4, 2]), np.array([0.1, 0.1, 0.1]), 1.0).status == oracle.BADTOKEN
    assert verify_chain_one(L, Q, np.array([-1, 2]), np.array([0.1, 0.1, 0.1]), 1.0).status == oracle.BADTOKEN
    Qz = Q.copy(); Qz[0, 1] = 0.0
    assert verify_chain_one(L, Qz, np.array([1, 2]), np.array([0.1, 0.1, 0.1]), 1.0).status == oracle.QZERO
    assert verify_chain_one(L, Q, np.array([1, 2]), np.array([1.0, 0.1, 0.1]), 1.0).status == oracle.BADUNIFORM
    assert verify_chain_one(L, Q, np.array([1, 2]), np.array([0.1, 0.1, -0.0 - 1e-9]), 1.0).status == oracle.BADUNIFORM
    # row order: a NaN row beats a bad token at the same position
    bad = L.copy(); bad[0, 0] = np.nan
    assert verify_chain_one(bad, Q, np.array([9, 2]), np.array([0.1, 0.1, 0.1]), 1.0).status == oracle.NONFINITE
    # at one position the draft's q(x) is checked before its uniform (the draft token and
    # its probability come with the proposal; the uniform is drawn by the verifier)
    assert verify_chain_one(L, Qz, np.array([1, 2]), np.array([1.5, 0.1, 0.1]), 1.0).status == oracle.QZERO
    # and an earlier position's error wins over a later one's
    Qz1 = Q.copy(); Qz1[1, 2] = 0.0
    assert verify_chain_one(L, Qz1, np.array([1, 2]), np.array([2.0, 0.1, 0.1]), 1.0).status == oracle.BADUNIFORM
    # unreached rows / tokens / uniforms do not matter: reject at draft 0 (p=0 there)
    p0 = np.array([0.0, 1.0, 0.0, 0.0])
    L2 = np.stack([logits_for(p0, 1.0), np.full(V, np.nan), np.full(V, np.nan)])
    r = verify_chain_one(L2, Q, np.array([0, 99]), np.array([0.5, 7.0, 0.3]), 1.0)
    assert r.status == oracle.OK and r.accepted_len == 0 and r.tokens == [1]
    # residual: q row at the rejected position must be finite and non-negative
    Qn = Q.copy(); Qn[0, 3] = np.nan
    L3 = np.stack([logits_for(p0, 1.0)] * 3)
    assert verify_chain_one(L3, Qn, np.array([0, 1]), np.array([0.5, 0.1, 0.1]), 1.0).status == oracle.RESIDUAL_EMPTY
    Qn = Q.copy(); Qn[0, 3] = -0.1
    assert verify_chain_one(L3, Qn, np.array([0, 1]), np.array([0.5, 0.1, 0.1]), 1.0).status == oracle.RESIDUAL_EMPTY
    # residual mass zero: p == q exactly but the draft is rejected (needs u >= a = 1: impossible);
    # force it with q(x) > p(x) elsewhere zero residual -> q dominates everywhere
    pq = np.array([0.5, 0.5, 0.0, 0.0])
    Qd = np.stack([np.array([0.5, 1.0, 0.5, 0.0]), pq])    # q_0 sums to 2: residual empty
    L4 = np.stack([logits_for(pq, 1.0)] * 3)
    assert verify_chain_one(L4, Qd, np.array([1, 0]), np.array([0.9, 0.1, 0.1]), 1.0).status == oracle.RESIDUAL_EMPTY


def test_gamma_zero_is_a_plain_target_draw():
    p = np.array([0.1, 0.2, 0.3, 0.4])
    L = logits_for(p, 0.9)[None]
    for j in range(64):
        u = j / 64
        r = verify_chain_one(L, np.zeros((0, 4)), np.zeros(0, int), np.array([u]), 0.9)
        expect = sum(u >= c for c in (0.1, 0.3, 0.6))       # CDF steps of p
        assert r.accepted_len == 0 and r.tokens == [expect]
