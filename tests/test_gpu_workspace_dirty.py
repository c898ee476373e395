"""A workspace marked dirty fails closed, and zero-filling it recovers.

A wait between blocks that gives up (SPEC_REQ_INTERNAL) may leave a published word behind
in the workspace.  A greedy or tree call that gives up marks the workspace dirty (word 0
of its header); every later call on it then reports SPEC_REQ_INTERNAL for all requests,
until the workspace is zero-filled (reset_workspaces() for the binding's cached ones).  A
chain call repairs its own give-ups, and also fails closed on a dirty workspace.

No wait is made to give up here: the dirty word is set from the host, which is the state
a give-up leaves, and every kernel runs its normal path.
"""
import numpy as np
import pytest
import torch

import synth
import exact_rejection_sampling_amd as sv
from exact_rejection_sampling_amd import _binding
from gpu_util import say, to_np, t_logits, t_i32, t_f32

pytestmark = pytest.mark.gpu

INTERNAL = 7


def mark_dirty(ws: torch.Tensor) -> None:
    """Sets the dirty word at the 256-byte aligned base the binding passes to the library."""
    off = (-ws.data_ptr()) % 256
    ws[off:off + 4] = torch.tensor([1, 0, 0, 0], dtype=torch.uint8, device=ws.device)
    torch.cuda.synchronize()


def workloads():
    c = synth.make_chain(8, 3, 4096, seed=71)
    g = synth.make_greedy(8, 4, 4096, seed=72)
    t = synth.make_tree(4, 15, 4096, seed=73)
    r = synth.make_tree_residual(4, 15, 4096, seed=74)
    return [
        ("chain", sv.chain_workspace_bytes(c.B, c.gamma, c.V),
         lambda ws: sv.prepare_chain(t_logits(c.logits, c.logit_dtype), t_f32(c.q), t_i32(c.tokens), t_f32(c.u),
                                     float(c.temperature), workspace_tensor=ws)),
        ("greedy", sv.greedy_workspace_bytes(g.B, g.gamma, g.V),
         lambda ws: sv.prepare_greedy(t_logits(g.logits, g.logit_dtype), t_i32(g.tokens), workspace_tensor=ws)),
        ("tree", sv.tree_workspace_bytes(t.B, t.N, t.V),
         lambda ws: sv.prepare_tree(t_logits(t.logits, t.logit_dtype), t_i32(t.node_tokens), t_i32(t.parents),
                                    t_f32(t.u), float(t.temperature), workspace_tensor=ws)),
        ("tree_residual", sv.tree_residual_workspace_bytes(r.B, r.N, r.V),
         lambda ws: sv.prepare_tree_residual(t_logits(r.logits, r.logit_dtype), t_f32(r.q), t_i32(r.node_tokens),
                                             t_i32(r.parents), t_f32(r.u_acc), t_f32(r.u_draw),
                                             float(r.temperature), workspace_tensor=ws)),
    ]


@pytest.mark.parametrize("kind", ["chain", "greedy", "tree", "tree_residual"])
def test_dirty_workspace_fails_closed_until_zeroed(kind):
    name, nbytes, prep = next(w for w in workloads() if w[0] == kind)
    ws = torch.zeros(nbytes + 512, dtype=torch.uint8, device="cuda:0")
    call = prep(ws)
    say(f"{kind}: clean call")
    clean = to_np(call())
    assert (clean["req_status"] == 0).all()
    mark_dirty(ws)
    for rep in range(2):     # it stays failed: nothing but a zero-fill clears the mark
        say(f"{kind}: call {rep} on a dirty workspace")
        got = to_np(call())
        assert (got["req_status"] == INTERNAL).all(), got["req_status"]
        assert (got["accepted_len"] == -1).all()
        assert (got["out_tokens"] == -1).all()
    ws.zero_()
    say(f"{kind}: call after the zero-fill")
    again = to_np(call())
    for k in clean:
        np.testing.assert_array_equal(again[k], clean[k], err_msg=k)


def test_reset_workspaces_clears_the_cached_ones():
    g = synth.make_greedy(8, 4, 4096, seed=75)
    lt, tt = t_logits(g.logits, g.logit_dtype), t_i32(g.tokens)
    say("greedy through the cached workspace")
    clean = to_np(sv.spec_verify_greedy(lt, tt))
    stream = torch.cuda.current_stream()
    ws, _ = _binding._WS_CACHE[("greedy", 0, stream.cuda_stream)]
    mark_dirty(ws)
    got = to_np(sv.spec_verify_greedy(lt, tt))
    assert (got["req_status"] == INTERNAL).all()
    assert sv.reset_workspaces() >= 1
    again = to_np(sv.spec_verify_greedy(lt, tt))
    for k in clean:
        np.testing.assert_array_equal(again[k], clean[k], err_msg=k)
