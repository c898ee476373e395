"""GPU parity of lazy row consumption (spec_verify_chain_ex and spec_verify_greedy_ex with
lazy_rows = k): rows are read in groups of k, a group only when every draft before it was
accepted ([M7.1] §0x03G: the round stops at the first rejection and discards every later
row).  The outputs must equal those of the call that reads every row, bit for bit
(statistics are reported for reached rows only in both), and match the oracle as every
chain or greedy call does.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import exact_rejection_sampling_amd as sv
from gpu_util import DEV, say, compare_chain, compare_exact, t_logits, t_f32, t_i32, to_np

pytestmark = pytest.mark.gpu

KEYS = ("accepted_len", "out_tokens", "req_status", "stats")


def run(x, lazy_rows, workspace_tensor=None, q=None, **kw):
    out = sv.spec_verify_chain(t_logits(x.logits, x.logit_dtype), t_f32(x.q if q is None else q), t_i32(x.tokens),
                               t_f32(x.u), float(x.temperature), with_stats=True, lazy_rows=lazy_rows,
                               workspace_tensor=workspace_tensor, **kw)
    return to_np(out)


def same(a, b, keys=KEYS):
    for k in keys:
        if k in a or k in b:
            np.testing.assert_array_equal(a[k], b[k], err_msg=k)   # NaN positions must agree too


def test_headline_shape_every_group_width():
    """B=64, gamma=5, V=128256 bf16, T=0.8: k = 1, 2, 3 against the dense call and the oracle."""
    x = synth.make_config(3, 0)
    say("chain dense config3 (reference for lazy)")
    dense = run(x, 0)
    exp = oracle.verify_chain(x.logits, x.q, x.tokens, x.u, x.temperature, x.logit_dtype)
    compare_chain(dense, exp)
    for k in (1, 2, 3):
        say(f"chain lazy k={k} config3")
        got = run(x, k)
        same(got, dense)
    print("accepted", np.bincount(dense["accepted_len"][dense["req_status"] == 0], minlength=6).tolist())


@pytest.mark.parametrize("V,dt,gamma,k", [(1, "f32", 3, 1), (7, "bf16", 2, 1), (33, "f32", 8, 3),
                                          (2049, "bf16", 5, 2), (8193, "f32", 4, 1), (20003, "bf16", 8, 4),
                                          (32000, "bf16", 5, 6), (32000, "bf16", 5, 100), (5000, "f32", 0, 1)])
def test_ragged_shapes_and_group_widths(V, dt, gamma, k):
    x = synth.make_chain(24, gamma, V, seed=500 + V + gamma, logit_dtype=dt, sigma=2.0, noise=0.7,
                         temperature=0.9)
    say(f"chain lazy V={V} {dt} gamma={gamma} k={k}")
    got = run(x, k)
    compare_chain(got, oracle.verify_chain(x.logits, x.q, x.tokens, x.u, x.temperature, x.logit_dtype))
    same(got, run(x, 0))


def test_high_acceptance_reads_every_group():
    """q = p: every draft is accepted outside flagged draws, so every group is read and the
    bonus row is drawn from."""
    x = synth.make_chain(32, 6, 4096, seed=520, logit_dtype="f32", sigma=2.0, noise=0.0, temperature=1.0)
    say("chain lazy k=1, q = p")
    got = run(x, 1)
    exp = oracle.verify_chain(x.logits, x.q, x.tokens, x.u, x.temperature, x.logit_dtype)
    compare_chain(got, exp)
    assert (got["accepted_len"][~exp["flagged"]] == 6).mean() > 0.9
    same(got, run(x, 0))


def test_bad_rows_after_the_first_rejection_are_not_read():
    """NaN rows, bad tokens and zero q after the first rejection leave the request OK (in
    the dense call too); a NaN in a reached row is NONFINITE."""
    B, G, V = 8, 5, 3000
    x = synth.make_chain(B, G, V, seed=530, logit_dtype="f32", sigma=2.0, noise=3.0, temperature=1.0)
    x.u = x.u.copy()
    x.u[:4, 0] = np.float32(0.999999)           # requests 0-3: draft 0 rejected unless p/q >= 1
    x.u[4:, :3] = np.float32(0.0)               # requests 4-7: drafts 0-2 accepted
    exp0 = oracle.verify_chain(x.logits, x.q, x.tokens, x.u, x.temperature, x.logit_dtype)
    rej = np.nonzero(exp0["accepted_len"] == 0)[0]
    assert rej.size >= 3
    logits, tokens = x.logits.copy(), x.tokens.copy()
    logits[rej[0], 2, 7] = np.nan
    logits[rej[1], 5, :] = np.nan                # the bonus row
    tokens[rej[2], 3] = V + 5
    x.logits, x.tokens = logits, tokens
    acc = np.nonzero(exp0["accepted_len"] >= 3)[0]
    assert acc.size
    x.logits[acc[0], 2, 11] = np.nan             # a reached row (read by the group of row 2)
    exp = oracle.verify_chain(x.logits, x.q, x.tokens, x.u, x.temperature, x.logit_dtype)
    assert (exp["status"][rej[:3]] == 0).all()
    say("chain lazy k=1 with bad unreached rows")
    got = run(x, 1)
    compare_chain(got, exp)
    same(got, run(x, 0))
    assert got["req_status"][acc[0]] == oracle.NONFINITE


@pytest.mark.parametrize("k", [1, 2])
def test_stops_and_budgets(k):
    x = synth.make_config(2, 7)
    stop, budget = synth.make_stop(x.tokens, x.V, seed=540, n_stop=64, from_drafts=48)
    say(f"chain lazy k={k} with stops and budgets")
    got = run(x, k, stop_tokens=t_i32(stop), budget=t_i32(budget))
    exp = oracle.verify_chain(x.logits, x.q, x.tokens, x.u, x.temperature, x.logit_dtype,
                              stop_tokens=stop.tolist(), budget=budget)
    compare_chain(got, exp)
    keep = ~exp["flagged"]
    np.testing.assert_array_equal(got["finish"][keep], exp["finish"][keep])
    same(got, run(x, 0, stop_tokens=t_i32(stop), budget=t_i32(budget)), KEYS + ("finish",))
    assert (budget <= 0).any() and (exp["finish"] == 2).any()


def test_processors_and_sparse_rows():
    x = synth.make_config(2, 8)
    bias, words, tk, tp = synth.make_processors(x.B, x.gamma + 1, x.V, seed=550)
    kw = dict(bias=t_f32(bias), allowed=torch.from_numpy(words.view(np.int32)).to(DEV), top_k=t_i32(tk),
              top_p=t_f32(tp))
    say("chain lazy k=2 with processors")
    same(run(x, 2, **kw), run(x, 0, **kw))
    xs, idx, vals = synth.make_chain_sparse(32, 5, 20000, 128, seed=551, logit_dtype="bf16")
    say("chain lazy k=1 with sparse draft rows")
    a = run(xs, 1, q=vals, q_index=t_i32(idx))
    same(a, run(xs, 0, q=vals, q_index=t_i32(idx)))
    q = oracle.densify_sparse_q(idx, vals, xs.V)
    compare_chain(a, oracle.verify_chain(xs.logits, q, xs.tokens, xs.u, xs.temperature, xs.logit_dtype,
                                         q_dtype="f64"))


def test_many_requests_and_workspace_reuse():
    """B = 2048 requests of V = 256: many groups in flight; the workspace returns to zero
    and serves the dense call next."""
    x = synth.make_chain(2048, 5, 256, seed=560, logit_dtype="bf16", sigma=2.0, noise=1.0)
    ws = torch.zeros(sv.chain_workspace_bytes(x.B, x.gamma, x.V) + 512, dtype=torch.uint8, device=DEV)
    say("chain lazy k=1 B=2048 V=256, workspace reuse")
    a = run(x, 1, workspace_tensor=ws)
    torch.cuda.synchronize()
    assert int(ws.count_nonzero()) == 0
    b = run(x, 0, workspace_tensor=ws)
    c = run(x, 2, workspace_tensor=ws)
    torch.cuda.synchronize()
    assert int(ws.count_nonzero()) == 0
    same(a, b)
    same(c, b)
    compare_chain(a, oracle.verify_chain(x.logits, x.q, x.tokens, x.u, x.temperature, x.logit_dtype))


def run_greedy(x, lazy_rows, workspace_tensor=None, **kw):
    return to_np(sv.spec_verify_greedy(t_logits(x.logits, x.logit_dtype), t_i32(x.tokens), lazy_rows=lazy_rows,
                                       workspace_tensor=workspace_tensor, **kw))


GKEYS = ("accepted_len", "out_tokens", "req_status")


def test_greedy_workload_shape():
    """B=256, gamma=8, V=128256 bf16 (drafts match the argmax with probability 0.7): k = 1, 3,
    4 against the dense call and the oracle, bit for bit."""
    x = synth.make_config(4, 0)
    say("greedy dense config4 (reference for lazy)")
    dense = run_greedy(x, 0)
    compare_exact(dense, oracle.verify_greedy(x.logits, x.tokens, x.logit_dtype), ["accepted_len", "out_tokens"])
    for k in (1, 3, 4):
        say(f"greedy lazy k={k} config4")
        same(run_greedy(x, k), dense, GKEYS)


@pytest.mark.parametrize("V,dt,gamma,k", [(1, "f32", 3, 1), (7, "bf16", 2, 1), (2049, "bf16", 8, 3),
                                          (8193, "f32", 5, 2), (32000, "bf16", 63, 4), (5000, "f32", 0, 1)])
def test_greedy_ragged_shapes(V, dt, gamma, k):
    x = synth.make_greedy(24, gamma, V, seed=600 + V + gamma, logit_dtype=dt, match_prob=0.8)
    say(f"greedy lazy V={V} {dt} gamma={gamma} k={k}")
    got = run_greedy(x, k)
    compare_exact(got, oracle.verify_greedy(x.logits, x.tokens, x.logit_dtype), ["accepted_len", "out_tokens"])
    same(got, run_greedy(x, 0), GKEYS)


def test_greedy_bad_rows_stops_budgets_and_workspace_reuse():
    B, G, V = 64, 8, 4000
    x = synth.make_greedy(B, G, V, seed=610, logit_dtype="f32", match_prob=0.6)
    exp0 = oracle.verify_greedy(x.logits, x.tokens, x.logit_dtype)
    early = np.nonzero(exp0["accepted_len"] <= 1)[0]
    late = np.nonzero(exp0["accepted_len"] >= 4)[0]
    assert early.size >= 2 and late.size >= 1
    x.logits = x.logits.copy()
    x.logits[early[0], 6, 3] = np.nan            # unreached rows: not read, no failure
    x.logits[early[1], G, :] = np.nan
    x.logits[late[0], 2, 9] = np.nan             # a reached row: NONFINITE
    stop, budget = synth.make_stop(x.tokens, V, seed=611, n_stop=32, from_drafts=24)
    ws = torch.zeros(sv.greedy_workspace_bytes(B, G, V) + 512, dtype=torch.uint8, device=DEV)
    say("greedy lazy k=2 bad rows, stops, budgets, workspace reuse")
    kw = dict(stop_tokens=t_i32(stop), budget=t_i32(budget))
    a = run_greedy(x, 2, workspace_tensor=ws, **kw)
    torch.cuda.synchronize()
    assert int(ws.count_nonzero()) == 0
    b = run_greedy(x, 0, workspace_tensor=ws, **kw)
    c = run_greedy(x, 1, workspace_tensor=ws)
    torch.cuda.synchronize()
    assert int(ws.count_nonzero()) == 0
    same(a, b, GKEYS + ("finish",))
    exp = oracle.verify_greedy(x.logits, x.tokens, x.logit_dtype, stop_tokens=stop.tolist(), budget=budget)
    compare_exact(a, exp, ["accepted_len", "out_tokens", "finish"])
    e2 = oracle.verify_greedy(x.logits, x.tokens, x.logit_dtype)
    compare_exact(c, e2, ["accepted_len", "out_tokens"])
    assert c["req_status"][early[0]] == 0 and c["req_status"][early[1]] == 0
    assert c["req_status"][late[0]] == oracle.NONFINITE


def test_greedy_lazy_with_bias_and_mask():
    """Gates decide on processed rows too: lazy greedy with bias and masks equals the
    every-row call with them, and the oracle on the processed rows."""
    x = synth.make_greedy(48, 6, 20000, seed=620, logit_dtype="bf16", match_prob=0.75)
    bias, words, _, _ = synth.make_processors(x.B, x.gamma + 1, x.V, seed=621, bias_sigma=0.5,
                                              with_top_k=False, with_top_p=False)
    kw = dict(bias=t_f32(bias), allowed=torch.from_numpy(words.view(np.int32)).to(DEV))
    say("greedy lazy k=2 with bias and masks")
    got = run_greedy(x, 2, **kw)
    same(got, run_greedy(x, 0, **kw), GKEYS)
    L, _ = oracle.process_rows(x.logits, x.logit_dtype, 1.0, bias, words)
    compare_exact(got, oracle.verify_greedy(L, x.tokens, "f64"), ["accepted_len", "out_tokens"])
