"""GPU parity with every row input starting one element past a 16-byte boundary (a
contiguous view into a larger buffer): V is a multiple of 8, but the rows are not 16-byte
aligned, so the kernels read them as whole 16-byte granules shifted by the same offset in
every lane.  bf16 rows start 2 bytes past the boundary, fp32 rows 4 bytes.  Same comparisons
with the oracle as the aligned tests."""
import numpy as np
import pytest
import torch

import oracle
import synth
import exact_rejection_sampling_amd as sv
from gpu_util import DEV, say, compare_chain, compare_exact, t_logits, t_f32, t_i32, to_np

pytestmark = pytest.mark.gpu

TREE_KEYS = ["accepted_len", "out_tokens", "out_nodes"]


def offset(t: torch.Tensor) -> torch.Tensor:
    """A copy of t whose first element sits one element past a 16-byte boundary."""
    flat = torch.empty(t.numel() + 16 // t.element_size(), dtype=t.dtype, device=t.device)
    v = flat[1:1 + t.numel()].view(t.shape)
    v.copy_(t)
    assert v.data_ptr() % 16 == t.element_size() and v.is_contiguous()
    return v


@pytest.mark.parametrize("dt,V", [("bf16", 32000), ("f32", 4096), ("bf16", 2048)])
def test_chain(dt, V):
    x = synth.make_chain(16, 4, V, seed=900 + V, logit_dtype=dt, sigma=2.5, boost_frac=0.01, noise=1.0,
                         temperature=0.9)
    say(f"chain offset rows B=16 gamma=4 V={V} {dt}")
    out = sv.spec_verify_chain(offset(t_logits(x.logits, dt)), offset(t_f32(x.q)), t_i32(x.tokens), t_f32(x.u),
                               float(x.temperature), with_stats=True)
    exp = oracle.verify_chain(x.logits, x.q, x.tokens, x.u, x.temperature, dt)
    print(compare_chain(to_np(out), exp))


def test_chain_processors():
    """bias offset as well (the bias row is shared by every request)."""
    B, G, V = 16, 4, 32000
    x = synth.make_chain(B, G, V, seed=910, logit_dtype="bf16", sigma=2.5, boost_frac=0.01, noise=1.0,
                         temperature=0.8)
    bias, words, k, p = synth.make_processors(B, G + 1, V, seed=911)
    say("chain offset rows with bias, masks, top-k, top-p")
    out = sv.spec_verify_chain(offset(t_logits(x.logits, "bf16")), offset(t_f32(x.q)), t_i32(x.tokens),
                               t_f32(x.u), float(x.temperature), with_stats=True, bias=offset(t_f32(bias)),
                               allowed=torch.from_numpy(words.view(np.int32)).to(DEV), top_k=t_i32(k),
                               top_p=t_f32(p))
    L, pflag = oracle.process_rows(x.logits, "bf16", x.temperature, bias, words, k, p)
    exp = oracle.verify_chain(L, x.q, x.tokens, x.u, x.temperature, "f64")
    exp["flagged"] = exp["flagged"] | pflag
    print(compare_chain(to_np(out), exp, max_flag_frac=0.5))   # top-p windows: see test_gpu_processors


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_greedy(dt):
    x = synth.make_greedy(32, 6, 32000, seed=920, logit_dtype=dt, match_prob=0.7)
    say(f"greedy offset rows V=32000 {dt}")
    got = to_np(sv.spec_verify_greedy(offset(t_logits(x.logits, dt)), t_i32(x.tokens)))
    compare_exact(got, oracle.verify_greedy(x.logits, x.tokens, dt), ["accepted_len", "out_tokens"])


def test_trees():
    x = synth.make_tree(8, 31, 32000, seed=930, logit_dtype="bf16", max_depth=4, max_children=3, boost=6.0)
    say("tree offset rows B=8 N=31 V=32000")
    got = to_np(sv.spec_verify_tree(offset(t_logits(x.logits, "bf16")), t_i32(x.node_tokens), t_i32(x.parents),
                                    t_f32(x.u), float(x.temperature)))
    exp = oracle.verify_tree(x.logits, x.parents, x.node_tokens, x.u, x.temperature, "bf16")
    compare_exact(got, exp, TREE_KEYS, flagged=exp["flagged"])
    say("tree_greedy offset rows")
    got = to_np(sv.spec_verify_tree_greedy(offset(t_logits(x.logits, "bf16")), t_i32(x.node_tokens),
                                           t_i32(x.parents)))
    compare_exact(got, oracle.verify_tree_greedy(x.logits, x.parents, x.node_tokens, "bf16"), TREE_KEYS)


def test_residual_tree():
    x = synth.make_tree_residual(8, 17, 32000, seed=940, sigma=2.0, noise=1.5, max_depth=3, max_children=3)
    say("tree_residual offset rows B=8 N=17 V=32000")
    got = to_np(sv.spec_verify_tree_residual(offset(t_logits(x.logits, x.logit_dtype)), offset(t_f32(x.q)),
                                             t_i32(x.node_tokens), t_i32(x.parents), t_f32(x.u_acc),
                                             t_f32(x.u_draw), float(x.temperature)))
    exp = oracle.verify_tree_residual(x.logits, x.q, x.parents, x.node_tokens, x.u_acc, x.u_draw, x.temperature,
                                      x.logit_dtype)
    compare_exact(got, exp, TREE_KEYS, flagged=exp["flagged"])
