"""GPU parity where the residual mass is small.

At high acceptance the draft distribution q is close to the target p, and the mass
W = sum max(p - q, 0) of the residual a rejection samples from ([M7.1] §0x03C) is small
(below 0.01 at drafter noise 0.02).  The draw inverts the residual's CDF normalized by W,
so every rounding error of the weights reaches it multiplied by 1/W ([M7.1] §0x03D asks
for a stable accumulation and a residual that is renormalized only when its mass is
materially positive).  These cases check that tokens still match the oracle exactly
outside the 1e-6 flag window in that regime, and that the reported W matches.

The drafter recipe is the chain recipe at temperature 1 (the drafter's logits are the
target's plus N(0, noise^2), and no temperature separates them), so q approaches p as the
noise shrinks.  At such noise a round almost never rejects on its own, so every draft is
tested against the uniform 0.999: a draft is rejected exactly when p(x)/q(x) < 0.999,
about half the time, which yields hundreds of rejections per batch; the terminal uniform
stays random.  Uniforms are caller inputs, and any value in [0, 1) is a valid one.
"""
import functools

import numpy as np
import pytest

import oracle
import synth
from gpu_util import say, run_chain, compare_chain, compare_exact, to_np, t_logits, t_f32, t_i32
from test_gpu_sparse_q import run_sparse, oracle_sparse
import exact_rejection_sampling_amd as sv

pytestmark = pytest.mark.gpu

U_DRAFT = np.float32(0.999)


def forced_rejections(x):
    x.u[:, :x.gamma] = U_DRAFT
    return x


def rejecting(exp, gamma):
    return (exp["status"] == 0) & (exp["accepted_len"] >= 0) & (exp["accepted_len"] < gamma)


@functools.lru_cache(maxsize=2)
def small_w_inputs(noise, dtype, B=320, gamma=2, V=128256):
    """Read-only inputs, shared by the tests that use the same noise and dtype."""
    x = synth.make_chain(B, gamma, V, seed=4100 + int(noise * 1000) + (7 if dtype == "f32" else 0),
                         logit_dtype=dtype, sigma=3.0, boost_frac=0.01, boost=8.0, noise=noise,
                         temperature=1.0)
    return forced_rejections(x)


def report(exp, gamma, label):
    rej = rejecting(exp, gamma)
    W = exp["stats"][rej, gamma, 2]
    print(f"{label}: {int(rej.sum())} rejections, W median {np.median(W):.5f} min {W.min():.6f}, "
          f"flagged {int(exp['flagged'].sum())}")
    return rej, W


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_chain_small_residual_lazy(dtype):
    """The same regime through lazy rows (rows past a rejection are never read): outputs
    equal the oracle's and the every-row call's."""
    x = small_w_inputs(0.02, dtype)
    say(f"chain small residual lazy rows noise=0.02 {dtype}")
    got = to_np(sv.spec_verify_chain(t_logits(x.logits, x.logit_dtype), t_f32(x.q), t_i32(x.tokens), t_f32(x.u),
                                     float(x.temperature), with_stats=True, lazy_rows=1))
    exp = oracle.verify_chain(x.logits, x.q, x.tokens, x.u, x.temperature, x.logit_dtype)
    print(compare_chain(got, exp))
    rej, _ = report(exp, x.gamma, f"lazy {dtype}")
    assert rej.sum() >= 200
    dense = run_chain(x)
    for k in ("accepted_len", "out_tokens", "req_status"):
        np.testing.assert_array_equal(got[k], dense[k], err_msg=k)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("noise", [0.02, 0.05, 0.1])
def test_chain_small_residual(noise, dtype):
    """V = 128256, 320 requests, gamma = 2: at least 200 rejections; at noise 0.02 the median
    residual mass is below 0.02."""
    x = small_w_inputs(noise, dtype)
    say(f"chain small residual noise={noise} {dtype} B={x.B} gamma={x.gamma} V={x.V}")
    got = run_chain(x)
    exp = oracle.verify_chain(x.logits, x.q, x.tokens, x.u, x.temperature, x.logit_dtype)
    s = compare_chain(got, exp)
    rej, W = report(exp, x.gamma, f"noise {noise} {dtype}")
    assert rej.sum() >= 200
    if noise <= 0.02:
        assert np.median(W) < 0.02
    print(s)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_chain_small_residual_sparse(dtype):
    """A top-4096 drafter at noise 0.02: the residual holds little more than the target mass
    outside the drafter's support (a few percent)."""
    x, idx, vals = synth.make_chain_sparse(320, 2, 128256, 4096, seed=4300 + (7 if dtype == "f32" else 0),
                                           logit_dtype=dtype, sigma=3.0, boost_frac=0.01, boost=8.0, noise=0.02,
                                           temperature=1.0)
    forced_rejections(x)
    say(f"chain small residual sparse K=4096 noise=0.02 {dtype}")
    got = run_sparse(x, idx, vals)
    exp = oracle_sparse(x, idx, vals)
    print(compare_chain(got, exp))
    rej, W = report(exp, x.gamma, f"sparse {dtype}")
    assert rej.sum() >= 200
    assert np.median(W) < 0.1


def test_tree_residual_small_residual():
    """The residual-update tree ([M7.7] §0x09A) at drafter noise 0.02 and T = 1: every child
    is tested against 0.999, so rejections, residual updates and draws of small residuals
    are common."""
    x = synth.make_tree_residual(64, 31, 32000, seed=4400, noise=0.02, temperature=1.0)
    x.u_acc[:] = U_DRAFT
    say(f"tree residual small residual noise=0.02 B={x.B} N={x.N} V={x.V}")
    got = to_np(sv.spec_verify_tree_residual(t_logits(x.logits, x.logit_dtype), t_f32(x.q), t_i32(x.node_tokens),
                                             t_i32(x.parents), t_f32(x.u_acc), t_f32(x.u_draw),
                                             float(x.temperature)))
    exp = oracle.verify_tree_residual(x.logits, x.q, x.parents, x.node_tokens, x.u_acc, x.u_draw,
                                      x.temperature, x.logit_dtype)
    compare_exact(got, exp, ["accepted_len", "out_tokens", "out_nodes"], flagged=exp["flagged"])
    print("accepted", np.bincount(got["accepted_len"][got["req_status"] == 0]).tolist(),
          "flagged", int(exp["flagged"].sum()))
