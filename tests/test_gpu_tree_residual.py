"""GPU parity of spec_verify_tree_residual against the oracle: statuses, accepted lengths,
path nodes and emitted tokens exact, except requests the oracle flags (a draw within 1e-6
of an acceptance threshold or a CDF boundary); and the emitted law of the pages' example
([M7.7] §0x09A: p = (0.5, 0.3, 0.2), two i.i.d. proposals from q = (0.4, 0.4, 0.2)) over
10^6 independent requests."""
import numpy as np
import pytest
import torch
from scipy import stats as sst

import oracle
import synth
import exact_rejection_sampling_amd as sv
from gpu_util import say, t_logits, t_i32, t_f32, to_np, compare_exact

pytestmark = pytest.mark.gpu

KEYS = ["accepted_len", "out_tokens", "out_nodes"]


def run(x, q_bf16=False, workspace_tensor=None):
    q = (t_logits(synth.f32_to_bf16_bits(x.q), "bf16") if q_bf16 else t_f32(x.q))
    return to_np(sv.spec_verify_tree_residual(t_logits(x.logits, x.logit_dtype), q, t_i32(x.node_tokens),
                                              t_i32(x.parents), t_f32(x.u_acc), t_f32(x.u_draw),
                                              float(x.temperature), workspace_tensor=workspace_tensor))


def expected(x, q_bf16=False):
    q = synth.f32_to_bf16_bits(x.q) if q_bf16 else x.q
    return oracle.verify_tree_residual(x.logits, q, x.parents, x.node_tokens, x.u_acc, x.u_draw,
                                       x.temperature, x.logit_dtype, "bf16" if q_bf16 else "f32")


def check(x, q_bf16=False):
    got = run(x, q_bf16)
    exp = expected(x, q_bf16)
    compare_exact(got, exp, KEYS, flagged=exp["flagged"])
    return got, exp


def test_config6_full():
    """B=32 requests, 31-node trees of depth <= 3, children drawn i.i.d. from a noisy
    drafter, V=32000 bf16, fp32 q, T=1."""
    x = synth.make_config(6, 0)
    say("tree_residual config6 B=32 N=31 V=32000")
    got, exp = check(x)
    print("accepted", got["accepted_len"].tolist(), "flagged", int(exp["flagged"].sum()))


def test_per_child_proposals_and_bf16_q():
    x = synth.make_config(6, 1, per_child=True)
    say("tree_residual config6 per-child proposals")
    check(x)
    say("tree_residual config6 per-child proposals, bf16 q")
    check(x, q_bf16=True)


@pytest.mark.parametrize("V,dt", [(1, "f32"), (7, "bf16"), (2049, "f32"), (4097, "bf16"), (20003, "bf16"),
                                  (65536, "f32"),
                                  # 64 chunks, the most the walker's one-wave steps take, and one
                                  # element more
                                  (131072, "bf16"), (131073, "f32")])
def test_ragged(V, dt):
    x = synth.make_tree_residual(12, 17, V, seed=60 + V, logit_dtype=dt, sigma=2.0, noise=1.5,
                                 temperature=0.9, max_depth=3, max_children=3)
    say(f"tree_residual ragged V={V} {dt}")
    check(x)


@pytest.mark.parametrize("noise", [0.05, 4.0])
def test_acceptance_extremes(noise):
    """noise 0.05: proposals close to the target (long walks, few residual passes);
    noise 4.0: most children rejected (several residual passes per node)."""
    x = synth.make_tree_residual(24, 31, 5000, seed=70 + int(noise * 10), sigma=2.0, noise=noise,
                                 max_depth=4, max_children=4)
    say(f"tree_residual noise={noise}")
    got, exp = check(x)
    print("accepted", np.bincount(got["accepted_len"][got["req_status"] == 0]).tolist())


def test_path_trees_match_the_chain_oracle():
    rng = np.random.default_rng(8)
    B, G, V = 16, 4, 3000
    c = synth.make_chain(B, G, V, seed=81, logit_dtype="f32", sigma=2.0, noise=0.7, temperature=1.0)
    # node i + 1 is draft i (child of node i); node rows are the chain rows
    parents = np.tile(np.arange(-1, G, dtype=np.int32), (B, 1))
    tokens = np.concatenate([np.zeros((B, 1), np.int32), c.tokens], axis=1)
    q = np.concatenate([np.zeros((B, 1, V), np.float32), c.q], axis=1)
    u_acc = np.concatenate([np.full((B, 1), 0.5, np.float32), c.u[:, :G]], axis=1)
    u_draw = np.repeat(c.u[:, G:], G + 1, axis=1)
    x = synth.TreeResidualInputs(B, G + 1, V, c.temperature, "f32", c.logits, q, tokens, parents, u_acc, u_draw)
    say("tree_residual path trees vs chain oracle")
    got = run(x)
    ch = oracle.verify_chain(c.logits, c.q, c.tokens, c.u, c.temperature, "f32")
    keep = ~ch["flagged"]
    np.testing.assert_array_equal(got["req_status"], ch["status"])
    np.testing.assert_array_equal(got["accepted_len"][keep], ch["accepted_len"][keep])
    np.testing.assert_array_equal(got["out_tokens"][keep][:, :G + 1], ch["out_tokens"][keep])


def test_error_statuses():
    B, N, V = 8, 7, 3000
    x = synth.make_tree_residual(B, N, V, seed=90, logit_dtype="f32", sigma=2.0, noise=3.0, max_depth=2,
                                 max_children=3)
    L = x.logits
    kids0 = [np.nonzero(x.parents[b] == 0)[0] for b in range(B)]
    L[0, 0, 5] = np.nan                                   # 0: root row NaN
    x.parents[1, 2] = 5                                   # 1: parent index not below the node
    x.q[2, kids0[2][0], x.node_tokens[2, kids0[2][0]]] = 0.0   # 2: q(x) of the first child is 0
    x.u_acc[3, kids0[3][0]] = 1.0                         # 3: accept uniform out of range
    x.u_draw[4, :] = 1.5                                  # 4: terminal uniform out of range
    x.node_tokens[5, N - 1] = V                           # 5: node token out of range
    # 6: first child certainly rejected (p(x) = 0), its q row has a negative entry
    c6 = kids0[6][0]
    L[6, 0, x.node_tokens[6, c6]] = -np.inf
    x.q[6, c6, 17] = -0.25
    say("tree_residual error statuses")
    got = run(x)
    exp = expected(x)
    compare_exact(got, exp, KEYS, flagged=exp["flagged"])
    st = exp["status"].tolist()
    assert st[0] == oracle.NONFINITE and st[1] == oracle.BADTREE and st[2] == oracle.QZERO
    assert st[3] == oracle.BADUNIFORM and st[5] == oracle.BADTREE and st[6] == oracle.RESIDUAL_EMPTY
    assert (got["out_tokens"][got["req_status"] != 0] == -1).all()


def test_single_node_trees_are_plain_draws():
    x = synth.make_tree_residual(16, 1, 9000, seed=95, sigma=2.0)
    say("tree_residual N=1")
    got, exp = check(x)
    assert (got["accepted_len"] == 0).all()


def test_workspace_returns_to_zero_and_repeats():
    x = synth.make_config(6, 2)
    ws = torch.zeros(sv.tree_residual_workspace_bytes(x.B, x.N, x.V) + 512, dtype=torch.uint8, device="cuda:0")
    say("tree_residual workspace reuse")
    a = run(x, workspace_tensor=ws)
    b = run(x, workspace_tensor=ws)
    torch.cuda.synchronize()
    assert int(ws.count_nonzero()) == 0
    for k in KEYS + ["req_status"]:
        np.testing.assert_array_equal(a[k], b[k])


def test_pages_example_law_million_requests():
    """[M7.7] §0x09A example as 10^6 independent requests: the first emitted token must
    follow p = (0.5, 0.3, 0.2) (Pearson chi-square not rejected at 0.001)."""
    p = np.array([0.5, 0.3, 0.2])
    q = np.array([0.4, 0.4, 0.2], dtype=np.float32)
    B, N, V = 1_000_000, 3, 3
    rng = np.random.default_rng(20240)
    logits = np.tile(np.log(p).astype(np.float32), (B, N, 1))
    qs = np.tile(q, (B, N, 1))
    tokens = np.zeros((B, N), np.int32)
    tokens[:, 1:] = rng.choice(3, size=(B, 2), p=q)
    parents = np.tile(np.array([-1, 0, 0], np.int32), (B, 1))
    u_acc = rng.random((B, N), dtype=np.float32)
    u_draw = rng.random((B, N), dtype=np.float32)
    say("tree_residual law, 10^6 requests")
    out = sv.spec_verify_tree_residual(t_f32(logits), t_f32(qs), t_i32(tokens), t_i32(parents), t_f32(u_acc),
                                       t_f32(u_draw), 1.0)
    got = to_np(out)
    st = got["req_status"]
    bad = np.nonzero(st != 0)[0]
    vals, cnt = np.unique(st, return_counts=True)
    assert bad.size == 0, (f"status histogram {dict(zip(vals.tolist(), cnt.tolist()))}; first failing requests "
                           f"{bad[:5].tolist()}: tokens {tokens[bad[:5]].tolist()} u_acc {u_acc[bad[:5]].tolist()} "
                           f"u_draw {u_draw[bad[:5]].tolist()} out {got['out_tokens'][bad[:5]].tolist()}")
    first = got["out_tokens"][:, 0]
    counts = np.bincount(first, minlength=3)
    chi2, pval = sst.chisquare(counts, p * B)
    print("counts", counts.tolist(), "p-value", pval)
    assert pval > 1e-3


@pytest.mark.parametrize("V,noise", [(32000, 1.0), (3000, 0.1), (50, 0.5)])
def test_without_replacement_siblings(V, noise):
    """[M7.7] §0x0AB (Sequoia): each child drawn from the drafter's row with the earlier
    siblings' tokens removed (uniform over the unsampled tokens once the draft mass is used
    up) and verified against that row; siblings never repeat a token."""
    x = synth.make_tree_residual(32, 31, V, seed=130 + V, sigma=2.0, noise=noise, max_depth=3, max_children=4,
                                 without_replacement=True)
    for b in range(x.B):
        for v in range(x.N):
            kids = np.nonzero(x.parents[b] == v)[0]
            assert len(set(x.node_tokens[b, kids].tolist())) == len(kids)
    say(f"tree_residual without replacement V={V} noise={noise}")
    got, exp = check(x)
    print("accepted", np.bincount(got["accepted_len"][got["req_status"] == 0]).tolist())


@pytest.mark.parametrize("T", [0.01, 100.0])
def test_extreme_temperatures(T):
    x = synth.make_tree_residual(8, 31, 20000, seed=int(T * 10) + 7, sigma=2.0, noise=0.5, temperature=T,
                                 max_depth=3, max_children=4)
    say(f"tree_residual T={T}")
    got, exp = check(x)
    print("accepted", got["accepted_len"].tolist(), "flagged", int(exp["flagged"].sum()))


def _first_child_request(kind, rng, N, V):
    """One request for the helpers' streamed-ahead first root child (node 1, the child the
    walker tests first): 'hit' accepts node 1; 'miss' rejects node 1 and accepts node 2;
    'far' rejects nodes 1, 2 and 3 and accepts node 280.  A rejected child's proposal is a point
    mass at its token, so that its acceptance probability p(x) stays far below its uniform;
    an accepted child has uniform 0.  The walk below the accepted child goes two levels
    deeper, and the filler nodes hang under node 3, which is reached only in 'far', where it
    is rejected before its children are read."""
    par = np.full(N, 3, np.int32)
    par[0], par[1], par[2], par[3] = -1, 0, 0, 0
    tok = rng.integers(0, V, N).astype(np.int32)
    logits = rng.normal(0.0, 1.0, (N, V)).astype(np.float32)
    q = np.exp(rng.normal(0.0, 1.0, (N, V))).astype(np.float32)
    q /= q.sum(axis=1, keepdims=True)
    u_acc = np.full(N, 0.5, np.float32)
    u_draw = rng.random(N).astype(np.float32)

    def reject(c):
        q[c] = 0.0
        q[c, tok[c]] = 1.0
        u_acc[c] = np.float32(0.999999)

    if kind == "far":
        par[280] = 0
    accepted = {"hit": 1, "miss": 2, "far": 280}[kind]
    for c in {"hit": [], "miss": [1], "far": [1, 2, 3]}[kind]:
        reject(c)
    u_acc[accepted] = 0.0
    a, bb = (4, 5) if accepted < 4 else (accepted + 1, accepted + 2)
    par[a], par[bb] = accepted, a
    u_acc[a] = u_acc[bb] = 0.0
    return par, tok, logits, q, u_acc, u_draw


def test_first_root_child_streamed_ahead_hit_and_miss():
    """The residual-update tree's helpers stream the root's first child ahead of the first
    order; a walk that accepts it, one that rejects it, and one that accepts a child past the
    streamed range all match the oracle, and the workspace returns to zero."""
    B, N, V = 6, 300, 3000
    rng = np.random.default_rng(131)
    kinds = ["hit", "miss", "far"] * 2
    parts = [_first_child_request(k, rng, N, V) for k in kinds]
    x = synth.TreeResidualInputs(B, N, V, np.float32(1.0), "f32", np.stack([p[2] for p in parts]),
                                 np.stack([p[3] for p in parts]), np.stack([p[1] for p in parts]),
                                 np.stack([p[0] for p in parts]), np.stack([p[4] for p in parts]),
                                 np.stack([p[5] for p in parts]))
    ws = torch.zeros(sv.tree_residual_workspace_bytes(B, N, V) + 512, dtype=torch.uint8, device="cuda:0")
    say("tree_residual streamed-ahead first child: hit, miss, far")
    got = run(x, workspace_tensor=ws)
    exp = expected(x)
    compare_exact(got, exp, KEYS, flagged=exp["flagged"])
    torch.cuda.synchronize()
    assert int(ws.count_nonzero()) == 0
    assert not exp["flagged"].any()
    assert got["out_nodes"][:, 0].tolist() == [{"hit": 1, "miss": 2, "far": 280}[k] for k in kinds]
