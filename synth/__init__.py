"""Seeded synthetic inputs for the speculative verification step.

This module only *makes inputs*: target logits, the draft distributions q and the
draft tokens a stand-in drafter proposes from them, candidate trees, and the
caller-side uniforms. It contains no part of the verifier (no acceptance test, no
residual, no temperature softmax of the target, no sampling of emitted tokens), so
both the float64 oracle and the GPU path can consume the same arrays without
sharing any of the method's arithmetic.

Recipes (shapes and distributions of the workloads the verifier is measured on):

* chain  -- target logits ~ N(0, sigma^2), optionally with a fraction of entries
  boosted by a constant to give peaked rows, stored as bf16 (round-to-nearest-even)
  or fp32.  The drafter's logits are the *stored* target logits plus N(0, tau^2)
  noise; q = softmax of that (no temperature: the temperature is a target-side
  processor), stored fp32.  Draft token i is drawn from the stored fp32 row q_i by
  the drafter's own inverse-CDF draw, so q_i(x_i) > 0 always holds.
* greedy -- target logits ~ N(0, sigma^2) in bf16; each draft token equals the
  row's first maximal index with probability `match_prob`, otherwise a uniformly
  random *other* id.  (The drafter stand-in needs the row maximum to imitate a
  well-aligned draft; the verifier's own argmax lives elsewhere.)
* tree   -- per request a random ancestor-closed tree: node 0 is the frontier
  root, node i > 0 picks a uniformly random parent among earlier nodes whose depth
  is below `max_depth` and that have fewer than `max_children` children.  The
  children of a node carry distinct tokens drawn without replacement from
  softmax(row + N(0, tau^2)) of that node's own row (a noisy drafter).  The
  optional `boost` adds a constant to the target logit of every child token in
  its parent's row, which makes deep acceptance paths likely (used to exercise
  depth).
* uniforms -- fp32 values k * 2^-24 with k uniform on [0, 2^24), so every
  uniform is exactly representable and strictly below 1.

Every array comes from `numpy.random.Generator(PCG64)` streams spawned from one
`SeedSequence(seed)`, so a (recipe, seed) pair always reproduces the same inputs.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

__all__ = [
    "ChainInputs", "GreedyInputs", "TreeInputs",
    "make_chain", "make_greedy", "make_tree", "make_config",
    "f32_to_bf16_bits", "bf16_bits_to_f32", "uniforms", "CONFIGS",
]

TWO_M24 = np.float64(2.0 ** -24)


# --------------------------------------------------------------------------- bf16
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return raw uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32)
    bias = ((b >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    out = ((b + bias) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen raw bfloat16 bits to float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def uniforms(rng: np.random.Generator, shape) -> np.ndarray:
    """fp32 uniforms on the 2^-24 grid of [0, 1)."""
    k = rng.integers(0, 1 << 24, size=shape, dtype=np.int64)
    return (k.astype(np.float64) * TWO_M24).astype(np.float32)


def _drafter_softmax(z: np.ndarray) -> np.ndarray:
    """The stand-in drafter's distribution: softmax over the last axis in float64."""
    z = z - z.max(axis=-1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=-1, keepdims=True)


def _draw_from_rows(rng: np.random.Generator, q: np.ndarray) -> np.ndarray:
    """The stand-in drafter's sampler: one token per row of `q` (any leading shape)."""
    flat = q.reshape(-1, q.shape[-1]).astype(np.float64)
    c = np.cumsum(flat, axis=1)
    t = rng.random(flat.shape[0]) * c[:, -1]
    idx = np.empty(flat.shape[0], dtype=np.int64)
    for r in range(flat.shape[0]):
        idx[r] = np.searchsorted(c[r], t[r], side="right")
    idx = np.minimum(idx, flat.shape[1] - 1)
    # t can round up to the row total; then fall back to the last positive entry so a
    # proposal never has zero draft probability
    for r in np.nonzero(flat[np.arange(flat.shape[0]), idx] <= 0)[0]:
        idx[r] = np.nonzero(flat[r] > 0)[0][-1]
    return idx.reshape(q.shape[:-1]).astype(np.int32)


def _normal_f32(rng: np.random.Generator, shape, sigma: float) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    x *= np.float32(sigma)
    return x


# --------------------------------------------------------------------------- chain
@dataclass
class ChainInputs:
    B: int
    gamma: int
    V: int
    temperature: np.float32
    logit_dtype: str              # "bf16" (uint16 bits) or "f32"
    logits: np.ndarray            # [B, gamma+1, V] uint16 bits or float32
    q: np.ndarray                 # [B, gamma, V] float32
    tokens: np.ndarray            # [B, gamma] int32
    u: np.ndarray                 # [B, gamma+1] float32
    q_dtype: str = "f32"
    meta: dict = field(default_factory=dict)

    def logits_f32(self) -> np.ndarray:
        return bf16_bits_to_f32(self.logits) if self.logit_dtype == "bf16" else self.logits

    @property
    def nbytes(self) -> int:
        return self.logits.nbytes + self.q.nbytes + self.tokens.nbytes + self.u.nbytes


def make_chain(B: int, gamma: int, V: int, *, seed: int, logit_dtype: str = "bf16",
               sigma: float = 3.0, boost_frac: float = 0.0, boost: float = 8.0,
               noise: float = 1.0, temperature: float = 0.8) -> ChainInputs:
    ss = np.random.SeedSequence(seed)
    s_logit, s_boost, s_noise, s_draft, s_u = (np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(5))
    R = gamma + 1
    lg = _normal_f32(s_logit, (B, R, V), sigma)
    if boost_frac > 0:
        mask = s_boost.random(size=(B, R, V), dtype=np.float32) < np.float32(boost_frac)
        lg[mask] += np.float32(boost)
        del mask
    if logit_dtype == "bf16":
        stored = f32_to_bf16_bits(lg)
        seen = bf16_bits_to_f32(stored)
    elif logit_dtype == "f32":
        stored = lg
        seen = lg
    else:
        raise ValueError(logit_dtype)
    q = np.empty((B, gamma, V), dtype=np.float32)
    for b in range(B):  # per request to bound float64 temporaries
        z = seen[b, :gamma].astype(np.float64) + s_noise.standard_normal(size=(gamma, V)) * noise
        q[b] = _drafter_softmax(z).astype(np.float32)
    tokens = _draw_from_rows(s_draft, q) if gamma > 0 else np.zeros((B, 0), np.int32)
    u = uniforms(s_u, (B, R))
    return ChainInputs(B, gamma, V, np.float32(temperature), logit_dtype, stored, q,
                       tokens.astype(np.int32), u,
                       meta=dict(seed=seed, sigma=sigma, boost_frac=boost_frac, boost=boost,
                                 noise=noise))


# --------------------------------------------------------------------------- greedy
@dataclass
class GreedyInputs:
    B: int
    gamma: int
    V: int
    logit_dtype: str
    logits: np.ndarray            # [B, gamma+1, V]
    tokens: np.ndarray            # [B, gamma] int32
    meta: dict = field(default_factory=dict)

    def logits_f32(self) -> np.ndarray:
        return bf16_bits_to_f32(self.logits) if self.logit_dtype == "bf16" else self.logits


def make_greedy(B: int, gamma: int, V: int, *, seed: int, logit_dtype: str = "bf16",
                sigma: float = 3.0, match_prob: float = 0.7) -> GreedyInputs:
    ss = np.random.SeedSequence(seed)
    s_logit, s_match, s_other = (np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(3))
    R = gamma + 1
    lg = _normal_f32(s_logit, (B, R, V), sigma)
    if logit_dtype == "bf16":
        stored = f32_to_bf16_bits(lg)
        del lg
        seen = bf16_bits_to_f32(stored[:, :gamma])
    else:
        stored = lg
        seen = lg[:, :gamma]
    best = np.argmax(seen, axis=-1) if gamma > 0 else np.zeros((B, 0), np.int64)
    del seen
    match = s_match.random(size=(B, gamma)) < match_prob
    other = s_other.integers(0, max(V - 1, 1), size=(B, gamma))
    other = other + (other >= best)          # uniform over the V-1 ids != best
    if V == 1:
        other = np.zeros_like(best)
    tokens = np.where(match, best, other).astype(np.int32)
    return GreedyInputs(B, gamma, V, logit_dtype, stored, tokens,
                        meta=dict(seed=seed, sigma=sigma, match_prob=match_prob))


# --------------------------------------------------------------------------- tree
@dataclass
class TreeInputs:
    B: int
    N: int
    V: int
    temperature: np.float32
    logit_dtype: str
    logits: np.ndarray            # [B, N, V]
    node_tokens: np.ndarray       # [B, N] int32 (node 0's entry is ignored by the verifier)
    parents: np.ndarray           # [B, N] int32, parents[:, 0] == -1
    u: np.ndarray                 # [B, N] float32
    meta: dict = field(default_factory=dict)

    def logits_f32(self) -> np.ndarray:
        return bf16_bits_to_f32(self.logits) if self.logit_dtype == "bf16" else self.logits


def random_tree(rng: np.random.Generator, N: int, max_depth: int, max_children: int) -> np.ndarray:
    """Parent array of a random ancestor-closed tree with N nodes (node 0 = root)."""
    parents = np.full(N, -1, dtype=np.int32)
    depth = np.zeros(N, dtype=np.int32)
    nchild = np.zeros(N, dtype=np.int32)
    for i in range(1, N):
        ok = np.nonzero((depth[:i] < max_depth) & (nchild[:i] < max_children))[0]
        if ok.size == 0:
            raise ValueError("tree capacity exhausted: raise max_depth or max_children")
        p = int(ok[rng.integers(0, ok.size)])
        parents[i] = p
        depth[i] = depth[p] + 1
        nchild[p] += 1
    return parents


def make_tree(B: int, N: int, V: int, *, seed: int, logit_dtype: str = "bf16", sigma: float = 3.0,
              noise: float = 1.0, temperature: float = 1.0, max_depth: int = 6,
              max_children: int = 4, boost: float = 0.0) -> TreeInputs:
    ss = np.random.SeedSequence(seed)
    s_logit, s_tree, s_noise, s_pick, s_u = (np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(5))
    lg = _normal_f32(s_logit, (B, N, V), sigma)
    parents = np.stack([random_tree(s_tree, N, max_depth, max_children) for _ in range(B)])
    node_tokens = np.zeros((B, N), dtype=np.int32)
    for b in range(B):
        for v in range(N):
            kids = np.nonzero(parents[b] == v)[0]
            if kids.size == 0:
                continue
            z = lg[b, v].astype(np.float64) + s_noise.standard_normal(V) * noise
            w = _drafter_softmax(z)
            n = min(kids.size, V)
            picked = s_pick.choice(V, size=n, replace=False, p=w)
            node_tokens[b, kids[:n]] = picked
            if kids.size > V:     # more children than vocabulary: repeat ids (invalid trie, tests only)
                node_tokens[b, kids[n:]] = picked[0]
            if boost:
                lg[b, v, picked] += np.float32(boost)
    stored = f32_to_bf16_bits(lg) if logit_dtype == "bf16" else lg
    u = uniforms(s_u, (B, N))
    return TreeInputs(B, N, V, np.float32(temperature), logit_dtype, stored, node_tokens,
                      parents.astype(np.int32), u,
                      meta=dict(seed=seed, sigma=sigma, noise=noise, max_depth=max_depth,
                                max_children=max_children, boost=boost))


# ------------------------------------------------------------------ residual tree
@dataclass
class TreeResidualInputs:
    B: int
    N: int
    V: int
    temperature: np.float32
    logit_dtype: str
    logits: np.ndarray            # [B, N, V] target logits (row v scores v's children)
    q: np.ndarray                 # [B, N, V] float32: row c = distribution node c was drawn from
    node_tokens: np.ndarray       # [B, N] int32
    parents: np.ndarray           # [B, N] int32
    u_acc: np.ndarray             # [B, N] float32, entry c for the test of child c
    u_draw: np.ndarray            # [B, N] float32, entry v for the terminal draw at v
    meta: dict = field(default_factory=dict)


def without_replacement_row(q0: np.ndarray, drawn) -> np.ndarray:
    """The proposal after removing the tokens already drawn at a parent: q0 with those
    tokens zeroed and renormalized, or, when no draft mass is left, the uniform distribution
    over the tokens not yet drawn ([M7.7] §0x0AB, Sequoia's proposal process)."""
    r = np.asarray(q0, dtype=np.float64).copy()
    r[list(drawn)] = 0.0
    tot = r.sum()
    if tot > 0.0:
        return r / tot
    u = np.ones_like(r)
    u[list(drawn)] = 0.0
    return u / u.sum()


def make_tree_residual(B: int, N: int, V: int, *, seed: int, logit_dtype: str = "bf16", sigma: float = 3.0,
                       noise: float = 1.0, temperature: float = 1.0, max_depth: int = 3,
                       max_children: int = 4, per_child: bool = False,
                       without_replacement: bool = False) -> TreeResidualInputs:
    """Random candidate trees whose children are proposals of a stand-in drafter: the
    drafter's distribution at node v is softmax(row_v + N(0, noise^2)) (stored fp32), and
    v's children are drawn from it i.i.d. (with replacement, so siblings may repeat a
    token); with per_child every child has a noise draw, a row and a token of its own; with
    without_replacement the children of v are drawn one after another, each from the
    drafter's row with the earlier siblings' tokens removed (without_replacement_row), and
    that row, stored fp32, is the child's proposal row."""
    ss = np.random.SeedSequence(seed)
    s_logit, s_tree, s_noise, s_pick, s_u = (np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(5))
    lg = _normal_f32(s_logit, (B, N, V), sigma)
    parents = np.stack([random_tree(s_tree, N, max_depth, max_children) for _ in range(B)])
    q = np.zeros((B, N, V), dtype=np.float32)
    node_tokens = np.zeros((B, N), dtype=np.int32)
    for b in range(B):
        for v in range(N):
            kids = np.nonzero(parents[b] == v)[0]
            if kids.size == 0:
                continue
            rows = 1 if not per_child else kids.size
            z = lg[b, v].astype(np.float64)[None] + s_noise.standard_normal((rows, V)) * noise
            qr = _drafter_softmax(z).astype(np.float32)
            if without_replacement:
                drawn = []
                for c in kids:
                    q[b, c] = without_replacement_row(qr[0], drawn).astype(np.float32)
                    node_tokens[b, c] = _draw_from_rows(s_pick, q[b, c][None])[0]
                    drawn.append(int(node_tokens[b, c]))
                continue
            q[b, kids] = qr if per_child else qr[0]
            node_tokens[b, kids] = _draw_from_rows(s_pick, q[b, kids])
    stored = f32_to_bf16_bits(lg) if logit_dtype == "bf16" else lg
    u_acc = uniforms(s_u, (B, N))
    u_draw = uniforms(s_u, (B, N))
    return TreeResidualInputs(B, N, V, np.float32(temperature), logit_dtype, stored, q, node_tokens,
                              parents.astype(np.int32), u_acc, u_draw,
                              meta=dict(seed=seed, sigma=sigma, noise=noise, max_depth=max_depth,
                                        max_children=max_children, per_child=per_child))


# --------------------------------------------------------------------------- configs
def make_stop(tokens: np.ndarray, V: int, *, seed: int, n_stop: int = 4, from_drafts: int = 2,
              budget_lo: int = 0, budget_hi: int = None):
    """Stop-token list and per-request output budgets for a batch of draft chains.

    `from_drafts` of the n_stop stop tokens are draft tokens picked at random positions
    (so accepted stop tokens occur), the rest uniform on [0, V).  Budgets are uniform on
    [budget_lo, budget_hi] (default gamma + 2, past the longest round).  Returns
    (stop int32 [n_stop], budget int32 [B]).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    B, G = tokens.shape
    picks = []
    if G > 0 and from_drafts > 0:
        picks = tokens[rng.integers(0, B, from_drafts), rng.integers(0, G, from_drafts)].tolist()
    picks += rng.integers(0, V, max(0, n_stop - len(picks))).tolist()
    hi = G + 2 if budget_hi is None else budget_hi
    budget = rng.integers(budget_lo, hi + 1, B).astype(np.int32)
    return np.asarray(picks[:n_stop], dtype=np.int32), budget


def make_chain_sparse(B: int, gamma: int, V: int, K: int, *, seed: int, **chain_kw):
    """A top-K drafter: the chain recipe's draft rows truncated to their K largest entries
    and renormalized (fp32), the draft tokens drawn again from the truncated rows.  Returns
    (ChainInputs whose q holds the dense truncated rows, index [B, gamma, K] int32,
    values [B, gamma, K] fp32) -- the sparse form lists each row's K tokens in increasing
    index order."""
    x = make_chain(B, gamma, V, seed=seed, **chain_kw)
    rng = np.random.Generator(np.random.PCG64(seed + 7919))
    K = min(K, V)
    idx = np.sort(np.argpartition(-x.q, K - 1, axis=-1)[..., :K], axis=-1).astype(np.int32)
    vals = np.take_along_axis(x.q, idx, -1).astype(np.float64)
    vals = (vals / vals.sum(-1, keepdims=True)).astype(np.float32)
    dense = np.zeros_like(x.q)
    np.put_along_axis(dense, idx, vals, -1)
    x.q = dense
    if gamma > 0:
        x.tokens = _draw_from_rows(rng, dense)
    return x, idx, vals


def make_processors(B: int, R: int, V: int, *, seed: int, bias_sigma: float = 1.0, allowed_frac: float = 0.9,
                    top_k=(0, 1, 20, 1000), top_p=(1.0, 0.5, 0.9, 0.99), with_bias=True, with_mask=True,
                    with_top_k=True, with_top_p=True):
    """Target logit processor inputs: an fp32 bias row [V] ~ N(0, bias_sigma^2); an allowed-token
    bitmask per row [B, R, ceil(V/32)] (uint32 words; each token allowed with probability
    allowed_frac, independently per row); per-request top-k and top-p drawn from the given
    choices.  Disabled parts are None."""
    rng = np.random.Generator(np.random.PCG64(seed))
    bias = rng.normal(0.0, bias_sigma, V).astype(np.float32) if with_bias else None
    words = None
    if with_mask:
        W = (V + 31) // 32
        allowed = rng.random((B, R, W * 32)) < allowed_frac
        allowed[..., V:] = False
        weights = (np.uint64(1) << np.arange(32, dtype=np.uint64))
        words = (allowed.reshape(B, R, W, 32).astype(np.uint64) * weights).sum(-1).astype(np.uint32)
    k = rng.choice(np.asarray(top_k, np.int32), B).astype(np.int32) if with_top_k else None
    p = rng.choice(np.asarray(top_p, np.float32), B).astype(np.float32) if with_top_p else None
    return bias, words, k, p


CONFIGS = {
    # chain, correctness scale: fp32 logits ~ N(0, 2^2), drafter noise 0.5, T = 1
    1: dict(kind="chain", B=4, gamma=4, V=32, logit_dtype="f32", sigma=2.0, boost_frac=0.0,
            noise=0.5, temperature=1.0),
    # chain, bf16, 1% of entries boosted by +8, drafter noise 1, T = 0.8
    2: dict(kind="chain", B=64, gamma=5, V=32000, logit_dtype="bf16", sigma=3.0, boost_frac=0.01,
            boost=8.0, noise=1.0, temperature=0.8),
    # chain headline shape
    3: dict(kind="chain", B=64, gamma=5, V=128256, logit_dtype="bf16", sigma=3.0, boost_frac=0.01,
            boost=8.0, noise=1.0, temperature=0.8),
    # greedy argmax-match
    4: dict(kind="greedy", B=256, gamma=8, V=128256, logit_dtype="bf16", sigma=3.0, match_prob=0.7),
    # tree, membership by target sample
    5: dict(kind="tree", B=32, N=63, V=152064, logit_dtype="bf16", sigma=3.0, noise=1.0,
            temperature=1.0, max_depth=6, max_children=4),
    # multi-candidate tree with residual updates (not one of the pages' workloads): 31 nodes,
    # depth <= 3, up to 4 children drawn i.i.d. from a noisy drafter, 32000-token vocabulary
    6: dict(kind="tree_residual", B=32, N=31, V=32000, logit_dtype="bf16", sigma=3.0, noise=1.0,
            temperature=1.0, max_depth=3, max_children=4),
}


def make_config(k: int, run: int = 0, **override):
    """Inputs for workload k (1..6) with seed 1000*k + run; keyword overrides change the recipe."""
    spec = dict(CONFIGS[k])
    spec.update(override)
    kind = spec.pop("kind")
    seed = spec.pop("seed", 1000 * k + run)
    if kind == "chain":
        return make_chain(seed=seed, **spec)
    if kind == "greedy":
        return make_greedy(seed=seed, **spec)
    if kind == "tree":
        return make_tree(seed=seed, **spec)
    if kind == "tree_residual":
        return make_tree_residual(seed=seed, **spec)
    raise ValueError(kind)
