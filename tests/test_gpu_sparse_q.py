"""GPU parity of sparse draft rows (spec_verify_chain_ex with q_index): a top-K drafter's
rows passed as K (index, value) pairs, zero elsewhere ([Tiny] "Logit and residual scratch":
exact only when the omitted proposal probabilities are known to be zero).  The oracle runs
the unchanged verifier on the densified rows."""
import numpy as np
import pytest
import torch

import oracle
import synth
import exact_rejection_sampling_amd as sv
from gpu_util import DEV, say, compare_chain, t_logits, t_f32, t_i32, to_np

pytestmark = pytest.mark.gpu


def run_sparse(x, idx, vals, workspace_tensor=None, **kw):
    out = sv.spec_verify_chain(t_logits(x.logits, x.logit_dtype), t_f32(vals), t_i32(x.tokens), t_f32(x.u),
                               float(x.temperature), with_stats=True, q_index=t_i32(idx),
                               workspace_tensor=workspace_tensor, **kw)
    return to_np(out)


def oracle_sparse(x, idx, vals):
    q = oracle.densify_sparse_q(idx, vals, x.V)
    return oracle.verify_chain(x.logits, q, x.tokens, x.u, x.temperature, x.logit_dtype, q_dtype="f64")


def test_headline_shape_top64_drafter():
    """B=64, gamma=5, V=128256 bf16, T=0.8, drafter truncated to its 64 largest entries."""
    x, idx, vals = synth.make_chain_sparse(64, 5, 128256, 64, seed=3000, logit_dtype="bf16", sigma=3.0,
                                           boost_frac=0.01, boost=8.0, noise=1.0, temperature=0.8)
    say("chain sparse q K=64 config3 shape")
    got = run_sparse(x, idx, vals)
    print(compare_chain(got, oracle_sparse(x, idx, vals)), "rejecting", int((got["accepted_len"] < 5).sum()))


@pytest.mark.parametrize("V,K,dt", [(7, 1, "f32"), (2049, 4, "bf16"), (20003, 1000, "bf16"), (8193, 8193, "f32")])
def test_ragged_and_k_extremes(V, K, dt):
    x, idx, vals = synth.make_chain_sparse(16, 4, V, K, seed=3100 + K, logit_dtype=dt, sigma=2.0, noise=1.0,
                                           temperature=0.9)
    say(f"chain sparse q V={V} K={K} {dt}")
    compare_chain(run_sparse(x, idx, vals), oracle_sparse(x, idx, vals))


def test_full_support_matches_the_dense_call():
    x, idx, vals = synth.make_chain_sparse(16, 5, 12000, 12000, seed=3200, logit_dtype="bf16", noise=0.8)
    say("chain sparse q K=V vs dense")
    got = run_sparse(x, idx, vals)
    dense = to_np(sv.spec_verify_chain(t_logits(x.logits, "bf16"), t_f32(x.q), t_i32(x.tokens), t_f32(x.u),
                                       float(x.temperature), with_stats=True))
    for k in ("accepted_len", "out_tokens", "req_status", "stats"):
        np.testing.assert_array_equal(got[k], dense[k], err_msg=k)


def test_sparse_errors_and_repeated_indices():
    B, G, V, K = 8, 3, 3000, 16
    x, idx, vals = synth.make_chain_sparse(B, G, V, K, seed=3300, logit_dtype="f32", sigma=2.0, noise=3.0)
    idx, vals = idx.copy(), vals.copy()
    exp0 = oracle_sparse(x, idx, vals)
    rej = np.nonzero(exp0["accepted_len"] < G)[0]
    assert len(rej) >= 4
    a, b_, c, d = rej[:4]
    # a: the rejected row lists an index outside [0, V) -> RESIDUAL_EMPTY
    A = exp0["accepted_len"][a]
    j = int(np.nonzero(idx[a, A] != x.tokens[a, A])[0][0])
    idx[a, A, j] = V + 5
    # b: the rejected row has a negative value at an index other than the draft token
    B_ = exp0["accepted_len"][b_]
    j = int(np.nonzero(idx[b_, B_] != x.tokens[b_, B_])[0][0])
    vals[b_, B_, j] = -0.5
    # c: the first draft token is not listed at all -> q(x) = 0 -> QZERO
    j = int(np.nonzero(idx[c, 0] == x.tokens[c, 0])[0][0])
    other = (int(x.tokens[c, 0]) + 1) % V
    while other in idx[c, 0]:
        other = (other + 1) % V
    idx[c, 0, j] = other
    # d: the first draft token listed twice: the two values add up
    jx = int(np.nonzero(idx[d, 0] == x.tokens[d, 0])[0][0])
    jo = (jx + 1) % K
    vals[d, 0, jx] *= 0.5
    vals[d, 0, jo] = vals[d, 0, jx]
    idx[d, 0, jo] = x.tokens[d, 0]
    say("chain sparse q errors and repeated indices")
    got = run_sparse(x, idx, vals)
    assert got["req_status"][a] == oracle.RESIDUAL_EMPTY and got["req_status"][b_] == oracle.RESIDUAL_EMPTY
    assert got["req_status"][c] == oracle.QZERO
    keep = np.setdiff1d(np.arange(B), [a, b_])          # the others against the oracle
    q = oracle.densify_sparse_q(idx[keep], vals[keep], V)
    exp = oracle.verify_chain(x.logits[keep], q, x.tokens[keep], x.u[keep], x.temperature, "f32", q_dtype="f64")
    compare_chain({k: v[keep] for k, v in got.items()}, exp)


def test_workspace_returns_to_zero_with_processors():
    x, idx, vals = synth.make_chain_sparse(32, 5, 32000, 256, seed=3400, logit_dtype="bf16")
    bias, words, _, _ = synth.make_processors(32, 6, 32000, seed=3401, with_top_k=False, with_top_p=False)
    ws = torch.zeros(sv.chain_workspace_bytes(32, 5, 32000) + 512, dtype=torch.uint8, device=DEV)
    say("chain sparse q + bias/mask, workspace reuse")
    kw = dict(bias=t_f32(bias), allowed=torch.from_numpy(words.view(np.int32)).to(DEV))
    a = run_sparse(x, idx, vals, workspace_tensor=ws, **kw)
    b = run_sparse(x, idx, vals, workspace_tensor=ws, **kw)
    torch.cuda.synchronize()
    assert int(ws.count_nonzero()) == 0
    for k in a:
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)
    L, pflag = oracle.process_rows(x.logits, "bf16", x.temperature, bias, words)
    exp = oracle.verify_chain(L, oracle.densify_sparse_q(idx, vals, x.V), x.tokens, x.u, x.temperature, "f64",
                              q_dtype="f64")
    exp["flagged"] |= pflag
    compare_chain(a, exp)


def test_the_largest_sparse_rows():
    """K = 65536 entries per row (the limit) at V = 128256: every terminal item scans all of
    them to fill its chunk, and the gather sums a token's entries block-wide."""
    x, idx, vals = synth.make_chain_sparse(4, 3, 128256, 65536, seed=3500, logit_dtype="bf16", sigma=3.0,
                                           boost_frac=0.01, noise=1.0, temperature=0.8)
    say("chain sparse q K=65536 V=128256")
    got = run_sparse(x, idx, vals)
    print(compare_chain(got, oracle_sparse(x, idx, vals)), got["accepted_len"].tolist())
