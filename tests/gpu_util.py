"""Helpers for the GPU parity tests: move synth inputs to the device, call the library
through the Python binding (which calls the C ABI), bring results back, compare with
the oracle."""
from __future__ import annotations

import numpy as np
import torch

import exact_rejection_sampling_amd as sv
import oracle

DEV = "cuda:0"


def say(msg: str) -> None:
    """Name the case before each GPU step (and flush) so a failing run identifies it."""
    print(f"[gpu] {msg}", flush=True)


def t_logits(arr: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(DEV)


def t_i32(arr) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.int32)).to(DEV)


def t_f32(arr) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(DEV)


def to_np(out: dict) -> dict:
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def run_chain(x, with_stats=True, q_bf16=False) -> dict:
    q = t_f32(x.q)
    if q_bf16:
        q = q.to(torch.bfloat16)
    out = sv.spec_verify_chain(t_logits(x.logits, x.logit_dtype), q, t_i32(x.tokens), t_f32(x.u),
                               float(x.temperature), with_stats=with_stats)
    return to_np(out)


def run_greedy(x) -> dict:
    return to_np(sv.spec_verify_greedy(t_logits(x.logits, x.logit_dtype), t_i32(x.tokens)))


def run_tree(x) -> dict:
    return to_np(sv.spec_verify_tree(t_logits(x.logits, x.logit_dtype), t_i32(x.node_tokens),
                                     t_i32(x.parents), t_f32(x.u), float(x.temperature)))


# Tolerances for the floating-point statistics (absolute unless noted).  The pages fix
# 1e-5 for probabilities from fp32 inputs and 2e-3 for bf16 inputs; both inputs are
# decoded exactly on both sides, so the tighter bound is asserted for every dtype.
PROB_ATOL = 1e-5
M_RTOL = 1e-6
LOGZ_ATOL = 1e-5


# Flags are for rare near-ties only, and a comparison that leaves out more requests than its
# flag rule implies would no longer test the tokens.  For a chain request the rule implies
# an exact probability: a terminal draw u uniform on [0, 1) is flagged when it lies within
# 1e-6 of a boundary of the normalized CDF, which has probability sum_k min(w_k / W, 2e-6)
# over the draw's weights w (the gaps between boundaries are the weights), plus 2e-6 per
# acceptance test.  check_flag_count allows that expectation plus a Poisson margin.
FLAG_WINDOW = 1e-6


def expected_chain_flags(exp) -> float:
    """Expected number of flagged requests under the oracle's flag rule, from the oracle's
    per-request results (terminal weights and acceptance tests)."""
    e = 0.0
    for r in exp.get("results", []):
        e += 2 * FLAG_WINDOW * len(r.a)
        if r.weights is not None and np.isfinite(r.W) and r.W > 0:
            e += float(np.minimum(np.asarray(r.weights) / r.W, 2 * FLAG_WINDOW).sum())
    return e


def check_flag_count(flagged, expected: float) -> int:
    flagged = np.asarray(flagged, bool)
    k = int(flagged.sum())
    limit = expected + 4.0 * np.sqrt(expected) + 2.0
    assert k <= limit, f"{k} of {flagged.size} requests flagged; the flag rule implies {expected:.2f} (limit {limit:.1f})"
    return k


# Where no per-request expectation is at hand (trees, processors), a fixed allowance.
MAX_FLAG_FRAC = 0.05


def check_flag_fraction(flagged, max_frac=MAX_FLAG_FRAC) -> int:
    """Asserts that at most max(3, max_frac * n) of n requests are flagged; returns the count."""
    flagged = np.asarray(flagged, bool)
    n, k = flagged.size, int(flagged.sum())
    assert k <= max(3, int(max_frac * n)), f"{k} of {n} requests flagged (limit {max_frac:.0%}, at least 3)"
    return k


def compare_chain(got: dict, exp: dict, requests=None, check_stats=True, max_flag_frac=None) -> dict:
    """Exact comparison of statuses; exact tokens / lengths outside flagged requests, which
    must be no more than the flag rule implies (check_flag_count; with max_flag_frac, a fixed
    allowance instead, for flags the chain's rule does not account for); statistics within
    tolerance.  Returns a summary dict."""
    idx = np.arange(len(got["accepted_len"])) if requests is None else np.asarray(requests)
    g_acc, g_out, g_st = got["accepted_len"][idx], got["out_tokens"][idx], got["req_status"][idx]
    np.testing.assert_array_equal(g_st, exp["status"], err_msg="request status")
    keep = ~exp["flagged"]
    bad = np.nonzero(keep & ((g_acc != exp["accepted_len"]) |
                             (g_out != exp["out_tokens"]).any(axis=1)))[0]
    assert bad.size == 0, (f"token mismatch in unflagged requests {idx[bad][:10].tolist()}: "
                           f"gpu {g_acc[bad][:5].tolist()} {g_out[bad][:5].tolist()} vs "
                           f"oracle {exp['accepted_len'][bad][:5].tolist()} {exp['out_tokens'][bad][:5].tolist()}")
    if max_flag_frac is None:
        check_flag_count(exp["flagged"], expected_chain_flags(exp))
    else:
        check_flag_fraction(exp["flagged"], max_flag_frac)
    summary = dict(n=len(idx), flagged=int((~keep).sum()), expected_flags=round(expected_chain_flags(exp), 2))
    if check_stats and "stats" in got:
        gs = got["stats"][idx].astype(np.float64)
        es = exp["stats"]
        sel = keep & (exp["status"] == 0)
        gs, es = gs[sel], es[sel]
        np.testing.assert_array_equal(np.isnan(gs), np.isnan(es), err_msg="stats NaN pattern")
        fin = ~np.isnan(es)
        err_m = np.abs(gs[..., 0] - es[..., 0])[fin[..., 0]]
        lim_m = (M_RTOL * np.abs(es[..., 0]) + 1e-6)[fin[..., 0]]
        assert (err_m <= lim_m).all(), f"m error {err_m.max()}"
        err_z = np.abs(gs[..., 1] - es[..., 1])[fin[..., 1]]
        assert (err_z <= LOGZ_ATOL).all(), f"log Z error {err_z.max()}"
        err_p = np.abs(gs[..., 2:4] - es[..., 2:4])[fin[..., 2:4]]
        assert (err_p <= PROB_ATOL).all(), f"probability error {err_p.max()}"
        summary.update(max_err_m=float(err_m.max(initial=0)), max_err_logz=float(err_z.max(initial=0)),
                       max_err_prob=float(err_p.max(initial=0)))
    return summary


def compare_exact(got: dict, exp: dict, keys, requests=None, flagged=None, max_flag_frac=MAX_FLAG_FRAC):
    idx = np.arange(len(got["accepted_len"])) if requests is None else np.asarray(requests)
    np.testing.assert_array_equal(got["req_status"][idx], exp["status"], err_msg="request status")
    keep = np.ones(len(idx), bool) if flagged is None else ~flagged
    for k in keys:
        g = got[k][idx][keep]
        e = exp[k][keep]
        bad = np.nonzero((g != e).reshape(len(g), -1).any(axis=1))[0]
        assert bad.size == 0, f"{k} mismatch at requests {idx[keep][bad][:10].tolist()}"
    if flagged is not None:
        check_flag_fraction(flagged, max_flag_frac)
