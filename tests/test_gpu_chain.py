"""GPU parity of spec_verify_chain against the float64 oracle.

Statuses exact; accepted lengths and emitted tokens exact except requests the oracle
flags (a draw within 1e-6 of an acceptance threshold or CDF boundary); statistics
within the tolerances of tests/gpu_util.py.  Sizes run from tiny ragged vocabularies
to the full B=64, gamma=5, V=128256 workload in the launch configuration the benchmark
times.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import exact_rejection_sampling_amd as sv
from gpu_util import (DEV, say, run_chain, compare_chain, t_logits, t_f32, t_i32, to_np)

pytestmark = pytest.mark.gpu


def oracle_chain(x, requests=None):
    return oracle.verify_chain(x.logits, x.q, x.tokens, x.u, x.temperature, x.logit_dtype,
                               requests=requests)


@pytest.mark.parametrize("run", range(4))
def test_config1_small(run):
    x = synth.make_config(1, run)
    say(f"chain config1 run={run}")
    s = compare_chain(run_chain(x), oracle_chain(x))
    print(s)


@pytest.mark.parametrize("V,dtype,T", [
    (1, "f32", 1.0), (2, "bf16", 0.8), (7, "f32", 1.3), (33, "bf16", 0.8), (2047, "f32", 1.0),
    (2048, "bf16", 0.8), (2049, "f32", 0.8), (8191, "bf16", 1.0), (8193, "bf16", 0.5),
    (20003, "bf16", 0.8), (32000, "bf16", 0.8), (32000, "f32", 1.0),
    # 64 terminal chunks, the most the selector's one-wave pick takes, and one element more
    (262144, "bf16", 0.8), (262145, "f32", 1.0)])
def test_ragged_vocab(V, dtype, T):
    x = synth.make_chain(16, 5, V, seed=77 + V, logit_dtype=dtype, sigma=3.0, boost_frac=0.01,
                         noise=1.0, temperature=T)
    say(f"chain ragged V={V} {dtype} T={T}")
    print(compare_chain(run_chain(x), oracle_chain(x)))


@pytest.mark.parametrize("gamma", [0, 1, 2, 8, 63])
def test_gamma_edges(gamma):
    x = synth.make_chain(8, gamma, 1500, seed=500 + gamma, logit_dtype="bf16", sigma=2.0,
                         noise=0.3, temperature=0.9)
    say(f"chain gamma={gamma}")
    print(compare_chain(run_chain(x), oracle_chain(x)))


def test_config2_full():
    x = synth.make_config(2, 0)
    say("chain config2 B=64 gamma=5 V=32000 bf16")
    print(compare_chain(run_chain(x), oracle_chain(x)))


@pytest.mark.parametrize("dtype,T", [("bf16", 0.8), ("f32", 1.0)])
def test_config3_full(dtype, T):
    """Headline shape, every request compared (the oracle needs a few seconds)."""
    x = synth.make_config(3, 0, logit_dtype=dtype, temperature=T)
    say(f"chain config3 B=64 gamma=5 V=128256 {dtype} T={T}")
    got = run_chain(x)
    s = compare_chain(got, oracle_chain(x))
    acc = got["accepted_len"]
    print(s, "mean accepted", acc.mean(), "rejecting", int((acc < 5).sum()))


def test_q_in_bf16():
    x = synth.make_chain(16, 4, 3000, seed=31, logit_dtype="bf16", boost_frac=0.01)
    qb = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(x.q))
    x.q = qb                                     # the oracle sees the bf16-rounded q
    bad = np.take_along_axis(qb, x.tokens[..., None].astype(np.int64), 2)[..., 0] <= 0
    say("chain q bf16")
    got = run_chain(x, q_bf16=True)
    exp = oracle_chain(x)
    print(compare_chain(got, exp), "qzero", int(bad.any(axis=1).sum()))


def test_repeatable_and_workspace_reuse():
    x = synth.make_config(2, 3, B=32)
    say("chain repeatability")
    a = run_chain(x)
    b = run_chain(x)
    for k in a:
        np.testing.assert_array_equal(a[k].view(np.uint32) if a[k].dtype == np.float32 else a[k],
                                      b[k].view(np.uint32) if b[k].dtype == np.float32 else b[k])


def _one_request(p_rows, q_rows, tokens, u, T=1.0, dtype="f32"):
    """A single-request ChainInputs-like object from explicit rows."""
    class X: pass
    x = X()
    with np.errstate(divide="ignore"):
        L = np.log(np.asarray(p_rows, dtype=np.float64)) * float(np.float32(T))
    x.logits = L[None].astype(np.float32)
    x.logit_dtype = dtype
    x.q = np.asarray(q_rows, dtype=np.float32)[None]
    x.tokens = np.asarray(tokens, dtype=np.int32)[None]
    x.u = np.asarray(u, dtype=np.float32)[None]
    x.temperature = np.float32(T)
    return x


def test_pages_worked_examples_on_gpu():
    """The AI-atlas three-symbol trace and the Module 16 verify example, through the GPU."""
    p, q = [0.6, 0.3, 0.1], [0.2, 0.3, 0.5]
    for tok, u0 in [(2, 0.25), (2, 0.1), (0, 0.999), (1, 0.5)]:
        x = _one_request([p, p], [q], [tok], [u0, 0.7])
        say(f"atlas trace tok={tok} u={u0}")
        got = run_chain(x)
        exp = oracle_chain(x)
        compare_chain(got, exp)
        if tok == 2 and u0 > 0.2:
            assert got["out_tokens"][0].tolist() == [0, -1]     # correction is always A
    p4, q4 = [0.5, 0.3, 0.15, 0.05], [0.4, 0.4, 0.15, 0.05]
    x = _one_request([p4, p4, p4], [q4, q4], [0, 1], [0.3, 0.8, 0.42])
    say("m16 verify example")
    got = run_chain(x)
    assert got["accepted_len"].tolist() == [1] and got["out_tokens"][0].tolist() == [0, 0, -1]


def test_error_statuses():
    B, G, V = 14, 3, 4100
    x = synth.make_chain(B, G, V, seed=9, logit_dtype="f32", sigma=2.0, noise=0.3, temperature=1.0)
    L = x.logits
    # 0: NaN in reached row 0
    L[0, 0, 17] = np.nan
    # 1: whole row 0 is -inf
    L[1, 0, :] = -np.inf
    # 2: +inf in row 0
    L[2, 0, 4000] = np.inf
    # 3: draft token out of range
    x.tokens[3, 0] = V
    # 4: negative draft token
    x.tokens[4, 0] = -5
    # 5: q(x_0) = 0
    x.q[5, 0, x.tokens[5, 0]] = 0.0
    # 6: accept uniform 1.0
    x.u[6, 0] = 1.0
    # 7: NaN terminal uniform
    x.u[7, G] = np.nan
    # 8: rejected at row 0 (u just below 1 and p < q there), NaN in unreached row 2: OK
    x.q[8, 0] = 0.0
    x.q[8, 0, 5] = 1.0
    x.tokens[8, 0] = 5
    L[8, 0, 5] = -np.inf                 # p(x_0) = 0: always rejected
    L[8, 2, 9] = np.nan
    # 9: rejected at row 0, q row has a NaN entry -> residual invariant
    x.q[9, 0] = 0.0
    x.q[9, 0, 5] = 1.0
    x.tokens[9, 0] = 5
    L[9, 0, 5] = -np.inf
    x.q[9, 0, 100] = np.nan
    # 10: same, negative q entry
    x.q[10, 0] = 0.0
    x.q[10, 0, 5] = 1.0
    x.tokens[10, 0] = 5
    L[10, 0, 5] = -np.inf
    x.q[10, 0, 200] = -0.25
    # 11: untouched
    # 12: q(x_0) = 0 and a bad uniform at the same position: q is checked first
    x.q[12, 0, x.tokens[12, 0]] = 0.0
    x.u[12, 0] = 1.5
    # 13: a bad uniform at position 0 wins over q(x_1) = 0 at position 1
    x.u[13, 0] = 2.0
    x.q[13, 1, x.tokens[13, 1]] = 0.0
    say("chain error statuses")
    got = run_chain(x)
    exp = oracle_chain(x)
    compare_chain(got, exp)
    assert exp["status"].tolist() == [1, 1, 1, 2, 2, 4, 3, 3, 0, 5, 5, 0, 4, 3]
    assert (got["out_tokens"][got["req_status"] != 0] == -1).all()
    assert (got["accepted_len"][got["req_status"] != 0] == -1).all()


def test_residual_empty_when_q_dominates():
    p = [0.5, 0.5, 0.0, 0.0]
    q = [0.5, 1.0, 0.5, 0.0]          # q sums to 2: [p - q]_+ = 0 everywhere
    x = _one_request([p, p], [q], [1], [0.9, 0.2])
    say("chain residual empty")
    got = run_chain(x)
    assert got["req_status"].tolist() == [5] and oracle_chain(x)["status"].tolist() == [5]


def test_empty_batch():
    say("chain B=0")
    out = sv.spec_verify_chain(torch.zeros(0, 3, 10, device=DEV), torch.zeros(0, 2, 10, device=DEV),
                               torch.zeros(0, 2, dtype=torch.int32, device=DEV),
                               torch.zeros(0, 3, device=DEV), 1.0)
    torch.cuda.synchronize()
    assert out["accepted_len"].numel() == 0


def test_chi_square_million_trials():
    """10^6 independent trials on fixed config-1 rows (V=32, gamma=4, T=1): fresh drafts
    x_i ~ q_i and uniforms per trial; Pearson chi-square (cells with expected count < 5
    pooled) must not reject at the 0.001 level for (i) the first emitted token vs p_0,
    (ii) the correction given a rejection at draft 0 vs the normalized residual r_0,
    (iii) the bonus given all accepted vs p_gamma, (iv) the accepted length vs Pr(A = a)."""
    from scipy import stats as sst
    from oracle import laws
    base = synth.make_config(1, 0)
    n, V, G = 1_000_000, base.V, base.gamma
    rng = np.random.default_rng(2024)
    L1 = base.logits[0].astype(np.float64)
    P = np.stack([oracle.target_probs(L1[i], 1.0)[0] for i in range(G + 1)])
    Q = base.q[0].astype(np.float64)
    say("chain chi-square: building 10^6 trials")
    cq = np.cumsum(Q, axis=1)
    draws = rng.random((n, G)) * cq[:, -1][None, :]
    tokens = np.stack([np.searchsorted(cq[i], draws[:, i], side="right") for i in range(G)], 1)
    tokens = np.minimum(tokens, V - 1).astype(np.int32)
    u = (rng.integers(0, 1 << 24, (n, G + 1)) * 2.0 ** -24).astype(np.float32)
    logits = torch.from_numpy(base.logits[0]).to(DEV).unsqueeze(0).expand(n, G + 1, V).contiguous()
    q = torch.from_numpy(base.q[0]).to(DEV).unsqueeze(0).expand(n, G, V).contiguous()
    say("chain chi-square: GPU call")
    out = to_np(sv.spec_verify_chain(logits, q, t_i32(tokens), t_f32(u), 1.0))
    del logits, q
    assert (out["req_status"] == 0).all()
    acc, toks = out["accepted_len"], out["out_tokens"]

    def chi2(counts, probs):
        exp = probs * counts.sum()
        order = np.argsort(exp)
        c, e = counts[order].astype(float), exp[order]
        # pool the smallest cells until every pooled cell expects >= 5
        pc, pe, cc, ce = [], [], 0.0, 0.0
        for ci, ei in zip(c, e):
            cc += ci; ce += ei
            if ce >= 5:
                pc.append(cc); pe.append(ce); cc = ce = 0.0
        if ce > 0:
            pc[-1] += cc; pe[-1] += ce
        return sst.chisquare(pc, pe).pvalue

    first = np.bincount(toks[:, 0], minlength=V)
    p1 = chi2(first, P[0])
    rej0 = acc == 0
    r0 = laws.residual_distribution(P[0], Q[0])
    p2 = chi2(np.bincount(toks[rej0, 0], minlength=V), r0)
    allacc = acc == G
    p3 = chi2(np.bincount(toks[allacc, G], minlength=V), P[G])
    law = laws.accepted_length_law([laws.acceptance_rate(P[i], Q[i]) for i in range(G)])
    p4 = chi2(np.bincount(acc, minlength=G + 1), law)
    print(dict(first=p1, correction0=p2, bonus=p3, length=p4, n_rej0=int(rej0.sum()),
               n_all=int(allacc.sum())))
    for pv in (p1, p2, p3, p4):
        assert pv > 1e-3


def test_one_workspace_across_shapes_and_entry_points():
    """Counters sit at fixed offsets: a single zero-filled workspace serves calls of any
    size and any entry point issued in order on one stream."""
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device=DEV)
    cases = [synth.make_chain(16, 5, 32000, seed=1, boost_frac=0.01),
             synth.make_chain(8, 0, 1500, seed=2),
             synth.make_chain(33, 3, 70001, seed=3, logit_dtype="f32"),
             synth.make_chain(2, 63, 900, seed=4)]
    from gpu_util import run_greedy
    for rep in range(2):
        for x in cases:
            say(f"shared workspace chain B={x.B} gamma={x.gamma} V={x.V} rep={rep}")
            out = to_np(sv.spec_verify_chain(t_logits(x.logits, x.logit_dtype), t_f32(x.q), t_i32(x.tokens),
                                             t_f32(x.u), float(x.temperature), with_stats=True,
                                             workspace_tensor=ws))
            compare_chain(out, oracle_chain(x))
            g = synth.make_greedy(x.B, x.gamma, x.V, seed=x.V)
            say(f"shared workspace greedy B={g.B} gamma={g.gamma} V={g.V}")
            gout = to_np(sv.spec_verify_greedy(t_logits(g.logits, g.logit_dtype), t_i32(g.tokens),
                                               workspace_tensor=ws))
            exp = oracle.verify_greedy(g.logits, g.tokens, g.logit_dtype)
            np.testing.assert_array_equal(gout["out_tokens"], exp["out_tokens"])
    torch.cuda.synchronize()
    assert int(ws.count_nonzero()) == 0              # the whole workspace is back at zero


@pytest.mark.parametrize("T", [0.01, 0.05, 20.0, 1000.0])
def test_extreme_temperatures(T):
    """Near-greedy and near-uniform targets: at T = 0.01 most p(x) underflow (fp32 on the
    GPU, fp64 in the oracle: both far below any uniform), at T = 1000 the rows are almost
    flat; tokens, lengths and statistics still match outside flagged draws."""
    x = synth.make_chain(32, 4, 20000, seed=90 + int(T * 100), logit_dtype="bf16", sigma=3.0, boost_frac=0.01,
                         noise=1.0, temperature=T)
    say(f"chain T={T}")
    got = run_chain(x)
    print(compare_chain(got, oracle_chain(x)), np.bincount(got["accepted_len"][got["req_status"] == 0]).tolist())
