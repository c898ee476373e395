"""HIP graph capture of the verification calls.  A call is captured once and replayed; every
replay must give, bit for bit, the outputs of an eager call on the inputs that the captured
buffers hold at replay time, and must leave the workspace zeroed.  The library's launches
need no allocation and no memset (the kernels return their workspace words to zero
themselves), so a captured call is self-contained.  Replays alternate two input sets copied
into the captured buffers, with eager calls and synchronizations between them; the first
input set is also checked against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import synth
import exact_rejection_sampling_amd as sv
from gpu_util import DEV, say, compare_chain, compare_exact, t_logits, t_f32, t_i32, to_np

pytestmark = pytest.mark.gpu

REPLAYS = 6


def replay_check(prepare, eager, sets, ws):
    """prepare(statics) -> PreparedCall bound to the static buffers `statics` (a copy of
    sets[0]) on the current stream; eager(inputs) -> dict of numpy outputs."""
    statics = [t.clone() for t in sets[0]]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call = prepare(statics)
        call()                                   # eager warm-up on the capture stream
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call()
    torch.cuda.synchronize()
    expected = [eager(inp) for inp in sets]
    keys = sorted(call.out)
    for i in range(REPLAYS):
        k = i % len(sets)
        for dst, src in zip(statics, sets[k]):
            dst.copy_(src)
        g.replay()
        torch.cuda.synchronize()
        for key in keys:
            np.testing.assert_array_equal(call.out[key].cpu().numpy(), expected[k][key], err_msg=f"replay {i} {key}")
        assert int(ws.count_nonzero()) == 0, f"replay {i} left workspace words set"
        eager(sets[(k + 1) % len(sets)])         # the program's own eager work between replays
        torch.cuda.synchronize()
    return expected


def chain_sets(B, G, V, seeds):
    xs = [synth.make_chain(B, G, V, seed=s, logit_dtype="bf16", sigma=2.5, boost_frac=0.01, noise=1.0,
                           temperature=0.8) for s in seeds]
    return xs, [[t_logits(x.logits, "bf16"), t_f32(x.q), t_i32(x.tokens), t_f32(x.u)] for x in xs]


def test_chain_replays():
    B, G, V = 32, 5, 32000
    xs, sets = chain_sets(B, G, V, (1000, 1001))
    T = float(xs[0].temperature)
    ws = torch.zeros(sv.chain_workspace_bytes(B, G, V) + 512, dtype=torch.uint8, device=DEV)
    say("graph: chain B=32 gamma=5 V=32000, 6 replays")
    exp = replay_check(lambda st: sv.prepare_chain(*st, T, with_stats=True, workspace_tensor=ws),
                       lambda inp: to_np(sv.spec_verify_chain(*inp, T, with_stats=True)), sets, ws)
    x = xs[0]
    compare_chain(exp[0], oracle.verify_chain(x.logits, x.q, x.tokens, x.u, x.temperature, "bf16"))


def test_chain_processors_replays():
    """Two launches per call: the threshold pass and the processed chain kernel."""
    B, G, V = 16, 4, 32000
    xs, sets = chain_sets(B, G, V, (1010, 1011))
    T = float(xs[0].temperature)
    for i, x in enumerate(xs):
        bias, words, k, p = synth.make_processors(B, G + 1, V, seed=1020 + i)
        sets[i] += [t_f32(bias), torch.from_numpy(words.view(np.int32)).to(DEV), t_i32(k), t_f32(p)]
    ws = torch.zeros(sv.chain_workspace_bytes(B, G, V) + 512, dtype=torch.uint8, device=DEV)

    def prep(st):
        return sv.prepare_chain(*st[:4], T, with_stats=True, workspace_tensor=ws, bias=st[4], allowed=st[5],
                                top_k=st[6], top_p=st[7])

    def eager(inp):
        return to_np(sv.spec_verify_chain(*inp[:4], T, with_stats=True, bias=inp[4], allowed=inp[5],
                                          top_k=inp[6], top_p=inp[7]))

    say("graph: chain with bias, masks, top-k, top-p, 6 replays")
    replay_check(prep, eager, sets, ws)


def test_greedy_replays():
    B, G, V = 64, 6, 32000
    xs = [synth.make_greedy(B, G, V, seed=s, logit_dtype="bf16", match_prob=0.7) for s in (1030, 1031)]
    sets = [[t_logits(x.logits, "bf16"), t_i32(x.tokens)] for x in xs]
    ws = torch.zeros(sv.greedy_workspace_bytes(B, G, V) + 512, dtype=torch.uint8, device=DEV)
    say("graph: greedy B=64 gamma=6 V=32000, 6 replays")
    exp = replay_check(lambda st: sv.prepare_greedy(*st, workspace_tensor=ws),
                       lambda inp: to_np(sv.spec_verify_greedy(*inp)), sets, ws)
    compare_exact(exp[0], oracle.verify_greedy(xs[0].logits, xs[0].tokens, "bf16"), ["accepted_len", "out_tokens"])


def test_tree_replays():
    B, N, V = 8, 31, 32000
    xs = [synth.make_tree(B, N, V, seed=s, logit_dtype="bf16", max_depth=4, max_children=3, boost=6.0)
          for s in (1040, 1041)]
    sets = [[t_logits(x.logits, "bf16"), t_i32(x.node_tokens), t_i32(x.parents), t_f32(x.u)] for x in xs]
    T = float(xs[0].temperature)
    ws = torch.zeros(sv.tree_workspace_bytes(B, N, V) + 512, dtype=torch.uint8, device=DEV)
    say("graph: tree B=8 N=31 V=32000, 6 replays")
    exp = replay_check(lambda st: sv.prepare_tree(*st, T, workspace_tensor=ws),
                       lambda inp: to_np(sv.spec_verify_tree(*inp, T)), sets, ws)
    x = xs[0]
    e = oracle.verify_tree(x.logits, x.parents, x.node_tokens, x.u, x.temperature, "bf16")
    compare_exact(exp[0], e, ["accepted_len", "out_tokens", "out_nodes"], flagged=e["flagged"])


def test_tree_residual_replays():
    B, N, V = 8, 17, 32000
    xs = [synth.make_tree_residual(B, N, V, seed=s, sigma=2.0, noise=1.5, max_depth=3, max_children=3)
          for s in (1050, 1051)]
    sets = [[t_logits(x.logits, x.logit_dtype), t_f32(x.q), t_i32(x.node_tokens), t_i32(x.parents),
             t_f32(x.u_acc), t_f32(x.u_draw)] for x in xs]
    T = float(xs[0].temperature)
    ws = torch.zeros(sv.tree_residual_workspace_bytes(B, N, V) + 512, dtype=torch.uint8, device=DEV)
    say("graph: tree_residual B=8 N=17 V=32000, 6 replays")
    replay_check(lambda st: sv.prepare_tree_residual(*st, T, workspace_tensor=ws),
                 lambda inp: to_np(sv.spec_verify_tree_residual(*inp, T)), sets, ws)
