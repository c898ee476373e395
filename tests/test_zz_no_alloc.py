"""spec_verify_chain_static (no allocation: the library's per-GPU static scratch stands in
for the workspace) against spec_verify_chain on the same inputs, through the C ABI: two
calls in a row, the second with a smaller problem, each equal to the workspace entry
point's results (the same kernels run on the same inputs, so tokens, statuses and
statistics are identical)."""
import numpy as np
import pytest
import torch

import synth
import exact_rejection_sampling_amd as sv
from gpu_util import say, to_np, t_logits, t_i32, t_f32

pytestmark = pytest.mark.gpu


def inputs(x):
    return (t_logits(x.logits, x.logit_dtype), t_f32(x.q), t_i32(x.tokens), t_f32(x.u), float(x.temperature))


def same(a, b, what):
    for k in ("accepted_len", "out_tokens", "req_status"):
        np.testing.assert_array_equal(a[k], b[k], err_msg=f"{what}: {k}")
    np.testing.assert_array_equal(np.isnan(a["stats"]), np.isnan(b["stats"]), err_msg=f"{what}: stats NaN")
    ok = ~np.isnan(a["stats"])
    np.testing.assert_array_equal(a["stats"][ok], b["stats"][ok], err_msg=f"{what}: stats")


def test_static_scratch_entry_matches_the_workspace_entry():
    cases = [("B=64 gamma=5 V=128256 bf16", synth.make_config(3, 0)),
             ("B=12 gamma=3 V=32000 fp32 T=1", synth.make_chain(12, 3, 32000, seed=903, logit_dtype="f32",
                                                                 temperature=1.0))]
    for name, x in cases:
        args = inputs(x)
        say(f"workspace entry point, {name}")
        ref = to_np(sv.spec_verify_chain(*args, with_stats=True))
        say(f"static-scratch entry point, {name}")
        got = to_np(sv.spec_verify_chain_static(*args, with_stats=True))
        assert (ref["req_status"] == 0).all()
        same(got, ref, name)
