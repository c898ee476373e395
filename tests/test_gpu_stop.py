"""GPU parity of the stop-token and output-budget variants (spec_verify_chain_stop,
spec_verify_greedy_stop) against the oracle.

[M7.1] §0x05B / §0x06 and [Tiny] "Normative greedy pseudocode" / "Normative stochastic
pseudocode": an accepted draft that is a stop token, or that uses up the remaining
budget, ends the round after itself; a budget of 0 runs no round.  Statuses exact;
accepted lengths, emitted tokens and finish codes exact outside requests the oracle
flags; chain statistics within the tolerances of tests/gpu_util.py.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import exact_rejection_sampling_amd as sv
from gpu_util import DEV, say, compare_chain, compare_exact, t_logits, t_f32, t_i32, to_np

pytestmark = pytest.mark.gpu

NO_LIMIT = 1 << 30


def run_chain_stop(x, stop, budget, workspace_tensor=None):
    out = sv.spec_verify_chain(t_logits(x.logits, x.logit_dtype), t_f32(x.q), t_i32(x.tokens), t_f32(x.u),
                               float(x.temperature), with_stats=True, stop_tokens=t_i32(stop),
                               budget=None if budget is None else t_i32(budget),
                               workspace_tensor=workspace_tensor)
    return to_np(out)


def oracle_chain_stop(x, stop, budget):
    return oracle.verify_chain(x.logits, x.q, x.tokens, x.u, x.temperature, x.logit_dtype,
                               stop_tokens=stop.tolist(), budget=budget)


def check_chain(x, stop, budget):
    got = run_chain_stop(x, stop, budget)
    exp = oracle_chain_stop(x, stop, budget)
    s = compare_chain(got, exp)
    keep = ~exp["flagged"]
    np.testing.assert_array_equal(got["finish"][keep], exp["finish"][keep], err_msg="finish")
    s["finish"] = np.bincount(exp["finish"][keep & (exp["status"] == 0)], minlength=3).tolist()
    return got, exp, s


def test_chain_headline_shape_with_stops_and_budgets():
    """B=64, gamma=5, V=128256 bf16, T=0.8; 64 stop tokens (48 taken from the drafts),
    budgets uniform on [0, 7]."""
    x = synth.make_config(3, 0)
    stop, budget = synth.make_stop(x.tokens, x.V, seed=301, n_stop=64, from_drafts=48)
    say("chain_stop config3 n_stop=64 budgets 0..7")
    got, exp, s = check_chain(x, stop, budget)
    print(s)
    assert s["finish"][1] > 0 and s["finish"][2] > 0      # both kinds of ending occur


@pytest.mark.parametrize("V,dt,gamma", [(1, "f32", 3), (7, "bf16", 4), (2049, "f32", 8), (20003, "bf16", 5),
                                        (32000, "bf16", 63)])
def test_chain_ragged_with_max_stop_list(V, dt, gamma):
    x = synth.make_chain(16, gamma, V, seed=400 + V, logit_dtype=dt, sigma=2.0, noise=0.3, temperature=0.9)
    stop, budget = synth.make_stop(x.tokens, V, seed=401 + V, n_stop=256, from_drafts=12)
    say(f"chain_stop ragged V={V} {dt} gamma={gamma}")
    print(check_chain(x, stop, budget)[2])


def test_chain_empty_stop_list_matches_the_plain_call():
    x = synth.make_config(2, 1)
    say("chain_stop empty list vs spec_verify_chain")
    got = run_chain_stop(x, np.zeros(0, np.int32), None)
    plain = to_np(sv.spec_verify_chain(t_logits(x.logits, x.logit_dtype), t_f32(x.q), t_i32(x.tokens),
                                       t_f32(x.u), float(x.temperature), with_stats=True))
    for k in ("accepted_len", "out_tokens", "req_status", "stats"):
        np.testing.assert_array_equal(got[k], plain[k], err_msg=k)
    assert (got["finish"] == 0).all()


def _accept_all(V, drafts, bonus, B):
    """Rows where p = q puts all mass on the drafts (acceptance certain), one-hot bonus."""
    G = len(drafts)
    P = np.zeros((G + 1, V))
    for i, d in enumerate(drafts):
        P[i, d] = 1.0
    P[G, bonus] = 1.0
    with np.errstate(divide="ignore"):
        L = np.log(P).astype(np.float32)
    return synth.ChainInputs(B, G, V, 1.0, "f32", np.tile(L, (B, 1, 1)),
                             np.tile(P[:G].astype(np.float32), (B, 1, 1)),
                             np.tile(np.array(drafts, np.int32), (B, 1)),
                             np.tile(np.array([0.3, 0.6, 0.9, 0.5], np.float32), (B, 1)))


def test_chain_pages_examples():
    """[M7.1] §0x06: full acceptance -> [d1, d2, d3, b]; a length cap after d3 -> [d1, d2,
    d3]; an EOS at d2 -> [d1, d2]; and a zero budget runs no round."""
    x = _accept_all(6, [1, 2, 3], 4, 4)
    say("chain_stop pages examples")
    got = run_chain_stop(x, np.zeros(0, np.int32), np.array([NO_LIMIT, 3, 4, 0], np.int32))
    assert got["out_tokens"].tolist() == [[1, 2, 3, 4], [1, 2, 3, -1], [1, 2, 3, 4], [-1] * 4]
    assert got["finish"].tolist() == [0, 2, 2, 2] and got["accepted_len"].tolist() == [3, 3, 3, 0]
    got = run_chain_stop(x, np.array([2], np.int32), np.array([NO_LIMIT, 2, 1, 0], np.int32))
    assert got["out_tokens"][:, :2].tolist() == [[1, 2], [1, 2], [1, -1], [-1, -1]]
    assert got["finish"].tolist() == [1, 1, 2, 2] and (got["req_status"] == 0).all()
    got = run_chain_stop(x, np.array([4, 77, -3], np.int32), None)
    assert got["out_tokens"].tolist() == [[1, 2, 3, 4]] * 4 and (got["finish"] == 1).all()


def test_chain_nothing_checked_after_the_end():
    """Rows, tokens and uniforms past the end of the round are never checked."""
    x = _accept_all(6, [1, 2, 3], 4, 4)
    x.logits = x.logits.copy()
    x.u = x.u.copy()
    x.logits[:, 2, 0] = np.nan              # row 2 invalid ...
    x.u[:, 3] = 1.5                         # ... and the terminal uniform too
    x.logits[3, 0, 0] = np.nan              # request 3: row 0 invalid, but no budget left
    stop = np.array([2], np.int32)
    budget = np.array([NO_LIMIT, 2, 5, 0], np.int32)
    say("chain_stop nothing checked after the end")
    got = run_chain_stop(x, stop, budget)
    exp = oracle_chain_stop(x, stop, budget)
    assert exp["status"].tolist() == [0, 0, 0, 0]
    compare_chain(got, exp)
    np.testing.assert_array_equal(got["finish"], exp["finish"])
    got = run_chain_stop(x, np.zeros(0, np.int32), budget)      # no stop token: row 2 is reached
    exp = oracle_chain_stop(x, np.zeros(0, np.int32), budget)
    assert exp["status"].tolist() == [oracle.NONFINITE, 0, oracle.NONFINITE, 0]
    compare_chain(got, exp)
    np.testing.assert_array_equal(got["finish"], exp["finish"])


def test_chain_errors_before_the_stop_are_reported():
    x = synth.make_chain(12, 4, 3000, seed=88, logit_dtype="f32", sigma=2.0, noise=0.2)
    stop = x.tokens[:, 1].copy()             # the second draft of every request is a stop token
    x.logits[0, 0, 5] = np.nan               # before it: reported
    x.q[1, 0, x.tokens[1, 0]] = 0.0
    x.u[2, 0] = 1.0
    x.tokens[3, 0] = -1
    x.logits[4, 3, 0] = np.nan               # after it: reported only if the stop is not accepted
    say("chain_stop errors before the stop")
    got = run_chain_stop(x, stop, None)
    exp = oracle_chain_stop(x, stop, None)
    assert exp["status"][:4].tolist() == [oracle.NONFINITE, oracle.QZERO, oracle.BADUNIFORM, oracle.BADTOKEN]
    compare_chain(got, exp)
    keep = ~exp["flagged"]
    np.testing.assert_array_equal(got["finish"][keep], exp["finish"][keep])


def test_chain_workspace_returns_to_zero():
    x = synth.make_config(2, 2)
    stop, budget = synth.make_stop(x.tokens, x.V, seed=55, n_stop=32, from_drafts=32)
    ws = torch.zeros(sv.load_library().spec_chain_workspace_bytes(x.B, x.gamma, x.V) + 512,
                     dtype=torch.uint8, device=DEV)
    say("chain_stop workspace reuse")
    a = run_chain_stop(x, stop, budget, workspace_tensor=ws)
    b = run_chain_stop(x, stop, budget, workspace_tensor=ws)
    torch.cuda.synchronize()
    assert int(ws.count_nonzero()) == 0
    for k in a:
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)


def run_greedy_stop(x, stop, budget):
    return to_np(sv.spec_verify_greedy(t_logits(x.logits, x.logit_dtype), t_i32(x.tokens),
                                       stop_tokens=t_i32(stop), budget=None if budget is None else t_i32(budget)))


def oracle_greedy_stop(x, stop, budget):
    return oracle.verify_greedy(x.logits, x.tokens, x.logit_dtype, stop_tokens=stop.tolist(), budget=budget)


def test_greedy_workload_with_stops_and_budgets():
    """B=256, gamma=8, V=128256 bf16; 64 stop tokens (48 from the drafts), budgets 0..10."""
    x = synth.make_config(4, 0)
    stop, budget = synth.make_stop(x.tokens, x.V, seed=402, n_stop=64, from_drafts=48)
    say("greedy_stop config4 n_stop=64 budgets 0..10")
    got = run_greedy_stop(x, stop, budget)
    exp = oracle_greedy_stop(x, stop, budget)
    compare_exact(got, exp, ["accepted_len", "out_tokens", "finish"])
    fin = np.bincount(exp["finish"], minlength=3)
    print("finish", fin.tolist())
    assert fin[1] > 0 and fin[2] > 0


@pytest.mark.parametrize("V,dt,gamma", [(1, "bf16", 3), (7, "f32", 2), (8193, "bf16", 8), (5000, "bf16", 63)])
def test_greedy_ragged_with_stops(V, dt, gamma):
    x = synth.make_greedy(24, gamma, V, seed=V + 3 * gamma, logit_dtype=dt, match_prob=0.85)
    stop, budget = synth.make_stop(x.tokens, V, seed=V + 7, n_stop=256, from_drafts=16)
    # a NaN that is reached or not, depending on the stops
    x.logits[5, min(2, gamma), 0] = 0x7FC0 if dt == "bf16" else np.nan
    say(f"greedy_stop ragged V={V} {dt} gamma={gamma}")
    compare_exact(run_greedy_stop(x, stop, budget), oracle_greedy_stop(x, stop, budget),
                  ["accepted_len", "out_tokens", "finish"])
