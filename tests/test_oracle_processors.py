"""Pins of the target logit processors (CPU only).

[Tiny] "Exact Speculative and Assisted Decoding for TinyRustLM", "Grammar and deterministic
opportunities" (q_G formula) and "Exactness tests" item 6 (test the transformed
distributions after temperature, top-k, top-p and grammar masks); [M7.1] §0x06J (p and q
are the processed rows) and §0x04G (ordered temperature and additive-bias processors).
Each processor is checked against its definition computed another way (closed form,
brute force over token subsets), and the chain verifier fed processed rows must emit the
processed target's law exactly.
"""
import itertools

import numpy as np
import pytest

import oracle
from oracle.processors import process_row, process_rows, unpack_mask
from oracle.numerics import target_probs
from lawcheck import chain_joint, target_joint, max_joint_gap


def probs(row, T):
    return target_probs(row, T)[0]


def test_grammar_mask_is_the_pages_q_G():
    rng = np.random.default_rng(1)
    for trial in range(50):
        V = int(rng.integers(2, 9))
        l = rng.normal(0, 2, V).astype(np.float32).astype(np.float64)
        A = rng.random(V) < 0.6
        if not A.any():
            A[rng.integers(V)] = True
        T = float(np.float32(rng.uniform(0.3, 2.0)))
        q = np.exp(l / T) / np.exp(l / T).sum()
        qG = q * A / (q * A).sum()
        out, _ = process_row(l, T, allowed=A)
        assert np.allclose(probs(out, T), qG, atol=1e-14)


def test_bias_precedes_temperature():
    l = np.array([0.5, -1.0, 2.0, 0.25], np.float32).astype(np.float64)
    b = np.array([1.0, 3.0, -2.0, 0.0], np.float32)
    T = 0.5
    out, _ = process_row(l, T, bias=b)
    s = l + b.astype(np.float64)
    assert np.allclose(probs(out, T), np.exp(s / T) / np.exp(s / T).sum(), atol=1e-14)
    # a -inf bias bans a token
    out, _ = process_row(l, T, bias=np.array([0, -np.inf, 0, 0], np.float32))
    assert probs(out, T)[1] == 0.0


def test_bias_sum_is_fp32():
    l = np.array([1.0, 16777216.0], np.float32).astype(np.float64)
    out, _ = process_row(l, 1.0, bias=np.array([0.0, 1.0], np.float32))
    assert out[1] == 16777216.0                     # 2^24 + 1 rounds to 2^24 in fp32


def _brute_top_k(s, k):
    order = sorted(range(len(s)), key=lambda x: -s[x])
    kth = s[order[k - 1]]
    return s >= kth


def test_top_k_keeps_the_k_largest_and_their_ties():
    rng = np.random.default_rng(2)
    for trial in range(200):
        V = int(rng.integers(1, 12))
        l = np.round(rng.normal(0, 1, V) * 2) / 2               # ties are common
        k = int(rng.integers(1, V + 2))
        out, _ = process_row(l, 1.0, top_k=k)
        kept = np.isfinite(out)
        if k >= V:
            assert kept.all()
        else:
            assert (kept == _brute_top_k(l, k)).all()
            assert kept.sum() >= k and all(l[kept].min() >= x for x in l[~kept])


def _brute_top_p(s, T, p):
    """Smallest tie-closed set of top tokens whose mass reaches p, by enumerating every
    tie-closed prefix of the values."""
    w = np.exp((s - s.max()) / T)
    w = w / w.sum()
    best = None
    for v in sorted(set(s.tolist()), reverse=True):
        S = s >= v
        if w[S].sum() >= p - 1e-15:
            best = S
            break
    return best


def test_top_p_is_the_smallest_tie_closed_nucleus():
    rng = np.random.default_rng(3)
    for trial in range(300):
        V = int(rng.integers(1, 10))
        l = np.round(rng.normal(0, 1.5, V) * 2) / 2
        T = float(np.float32(rng.uniform(0.5, 1.5)))
        p = float(rng.uniform(0.05, 0.99))
        out, flagged = process_row(l, T, top_p=p)
        if flagged:
            continue
        assert (np.isfinite(out) == _brute_top_p(l, T, p)).all()


def test_top_k_then_top_p_then_mask_order():
    # mask first: a large logit outside A never counts toward k or p
    l = np.array([5.0, 4.0, 3.0, 2.0, 1.0])
    A = np.array([False, True, True, True, True])
    out, _ = process_row(l, 1.0, allowed=A, top_k=2)
    assert np.isfinite(out).tolist() == [False, True, True, False, False]
    # top-p acts on the top-k renormalized distribution
    out, _ = process_row(l, 1.0, top_k=2, top_p=0.7)
    w = np.exp(l[:2] - 5.0)
    assert w[0] / w.sum() >= 0.7 and np.isfinite(out).tolist() == [True, False, False, False, False]
    out, _ = process_row(l, 1.0, top_k=2, top_p=0.8)
    assert np.isfinite(out).tolist() == [True, True, False, False, False]


def test_disabled_processors_are_the_identity_and_faults_stay():
    l = np.array([0.1, -0.2, 0.3], np.float32).astype(np.float64)     # stored logits are fp32 values
    out, _ = process_row(l, 0.8, top_k=0, top_p=1.0)
    assert (out == l).all()
    bad = np.array([0.1, np.nan, 0.3])
    out, _ = process_row(bad, 1.0, allowed=np.array([True, False, True]))
    assert np.isnan(out[1])                     # a masked NaN still invalidates the row
    out, _ = process_row(l, 1.0, allowed=np.zeros(3, bool))
    assert np.isneginf(out).all()               # no valid token


def test_mask_words_layout():
    V = 70
    allowed = np.zeros(V, bool)
    allowed[[0, 31, 32, 69]] = True
    words = np.zeros(3, np.uint32)
    for x in np.flatnonzero(allowed):
        words[x // 32] |= np.uint32(1) << np.uint32(x % 32)
    assert (unpack_mask(words, V) == allowed).all()


@pytest.mark.parametrize("kind", ["mask", "top_k", "top_p", "bias"])
def test_chain_on_processed_rows_emits_the_processed_law(kind):
    """The verifier run on processed target rows, with drafts from an unprocessed q, emits
    the processed target's joint law exactly (enumeration over V = 3, gamma = 2)."""
    rng = np.random.default_rng({"mask": 5, "top_k": 6, "top_p": 7, "bias": 8}[kind])
    V, G, T = 3, 2, 0.9
    raw = {}

    def raw_of(pre):
        if pre not in raw:
            raw[pre] = rng.normal(0, 1.0, V)
        return raw[pre]

    def proc(pre):
        l = raw_of(pre)
        if kind == "mask":
            out, _ = process_row(l, T, allowed=np.array([True, (len(pre) % 2) == 0, True]))
        elif kind == "top_k":
            out, _ = process_row(l, T, top_k=2)
        elif kind == "top_p":
            out, _ = process_row(l, T, top_p=0.6)
        else:
            out, _ = process_row(l, T, bias=np.array([0.5, -1.0, 0.0], np.float32))
        return probs(out, T)
    qtab = {}

    def q_of(pre):
        if pre not in qtab:
            qtab[pre] = rng.dirichlet(np.ones(V))
        return qtab[pre]
    joint, _ = chain_joint(proc, q_of, V, G, T)
    assert max_joint_gap(joint, target_joint(proc, V, G + 1)) < 1e-12


def test_process_rows_batches_like_rows():
    rng = np.random.default_rng(9)
    B, R, V = 3, 2, 40
    L = rng.normal(0, 2, (B, R, V)).astype(np.float32)
    words = rng.integers(0, 2 ** 32, (B, R, 2), dtype=np.uint64).astype(np.uint32)
    bias = rng.normal(0, 1, V).astype(np.float32)
    out, _ = process_rows(L, "f32", 0.7, bias, words, np.array([3, 0, 50]), np.array([0.9, 0.5, 1.0]))
    allowed = unpack_mask(words, V)
    for b in range(B):
        for i in range(R):
            ref, _ = process_row(L[b, i].astype(np.float64), 0.7, bias, allowed[b, i],
                                 [3, 0, 50][b], [0.9, 0.5, 1.0][b])
            assert np.array_equal(out[b, i], ref)


def test_sparse_q_rows_are_zero_outside_the_support():
    from oracle.processors import densify_sparse_q
    idx = np.array([[3, 0, 7], [1, 1, 2]])
    val = np.array([[0.5, 0.25, 0.25], [0.25, 0.25, 0.5]], np.float32)
    q = densify_sparse_q(idx, val, 8)
    assert q[0].tolist() == [0.25, 0, 0, 0.5, 0, 0, 0, 0.25]
    assert q[1].tolist() == [0, 0.5, 0.5, 0, 0, 0, 0, 0]          # a repeated index adds up
    with pytest.raises(ValueError):
        densify_sparse_q(np.array([[8]]), np.array([[1.0]]), 8)


@pytest.mark.parametrize("K", [1, 2])
def test_top_k_drafter_with_sparse_q_is_exact_and_hidden_mass_is_not(K):
    """[Tiny] "Logit and residual scratch": with a top-K drafter (mass outside the K listed
    tokens truly zero) the verifier on the sparse rows emits the target law; if the drafter
    proposes from its full distribution but only K entries reach the verifier (omitted
    probabilities not zero), the law is wrong."""
    rng = np.random.default_rng(30 + K)
    V, G, T = 3, 2, 1.0
    p_of = lambda pre, t={}: t.setdefault(pre, rng.dirichlet(np.ones(V)))
    full = {}

    def q_full(pre):
        if pre not in full:
            full[pre] = rng.dirichlet(np.ones(V))
        return full[pre]

    def topk(row):
        keep = np.argsort(-row, kind="stable")[:K]
        out = np.zeros(V)
        out[keep] = row[keep]
        return out / out.sum()
    joint, _ = chain_joint(p_of, lambda pre: topk(q_full(pre)), V, G, T)
    assert max_joint_gap(joint, target_joint(p_of, V, G + 1)) < 1e-12
    # drafts from the full q, verified against the truncated (renormalized) rows
    from lawcheck import _midpoints  # noqa: F401  (same enumeration, mismatched rows)
    joint_bad = mismatched_chain_joint(p_of, q_full, lambda pre: topk(q_full(pre)), V, G, T)
    assert max_joint_gap(joint_bad, target_joint(p_of, V, G + 1)) > 1e-3


def mismatched_chain_joint(p_of, q_draw, q_verify, V, G, T):
    """Emitted law when drafts come from q_draw but the verifier is given q_verify rows
    (accept probability min(1, p / q_verify), residual [p - q_verify]_+)."""
    from collections import defaultdict
    joint = defaultdict(float)
    for x in itertools.product(range(V), repeat=G):
        w = float(np.prod([q_draw(x[:i])[x[i]] for i in range(G)]))
        if w == 0.0:
            continue

        def walk(i, mass):
            if i == G:
                for k, pk in enumerate(p_of(x)):
                    joint[x + (k,)] += mass * pk
                return
            p, qv = p_of(x[:i]), q_verify(x[:i])
            a = 0.0 if qv[x[i]] == 0 else min(1.0, p[x[i]] / qv[x[i]])
            walk(i + 1, mass * a)
            if a < 1.0:
                res = np.maximum(p - qv, 0.0)
                res = res / res.sum()
                for k, rk in enumerate(res):
                    seq = x[:i] + (k,)
                    # complete to G + 1 tokens with target draws
                    stack = [(seq, mass * (1 - a) * rk)]
                    while stack:
                        s_, m_ = stack.pop()
                        if len(s_) == G + 1:
                            joint[s_] += m_
                            continue
                        for t, pt in enumerate(p_of(s_)):
                            stack.append((s_ + (t,), m_ * pt))
        walk(0, w)
    return joint
