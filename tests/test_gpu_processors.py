"""GPU parity of the target logit processors (spec_verify_chain_ex, spec_verify_greedy_ex)
against the oracle: the oracle processes every row (bias, mask, top-k, top-p) and runs the
unchanged verifier on the processed rows.  Statuses exact; tokens, lengths and finish codes
exact outside flagged requests (accept/CDF windows, and top-p boundaries within 1e-5 of
the target mass); statistics within the tolerances of tests/gpu_util.py.

[M7.1] §0x06J (p is the processed row), §0x04G (temperature and additive bias); [Tiny]
"Grammar and deterministic opportunities" (q_G) and "Exactness tests" item 6.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import exact_rejection_sampling_amd as sv
from gpu_util import DEV, say, compare_chain, compare_exact, t_logits, t_f32, t_i32, to_np

pytestmark = pytest.mark.gpu


def t_words(w):
    return None if w is None else torch.from_numpy(np.ascontiguousarray(w).view(np.int32)).to(DEV)


def run_chain_proc(x, bias, words, top_k, top_p, stop=None, budget=None, workspace_tensor=None):
    out = sv.spec_verify_chain(t_logits(x.logits, x.logit_dtype), t_f32(x.q), t_i32(x.tokens), t_f32(x.u),
                               float(x.temperature), with_stats=True,
                               bias=None if bias is None else t_f32(bias), allowed=t_words(words),
                               top_k=None if top_k is None else t_i32(top_k),
                               top_p=None if top_p is None else t_f32(top_p),
                               stop_tokens=None if stop is None else t_i32(stop),
                               budget=None if budget is None else t_i32(budget), workspace_tensor=workspace_tensor)
    return to_np(out)


def oracle_chain_proc(x, bias, words, top_k, top_p, stop=(), budget=None):
    L, pflag = oracle.process_rows(x.logits, x.logit_dtype, x.temperature, bias, words, top_k, top_p)
    exp = oracle.verify_chain(L, x.q, x.tokens, x.u, x.temperature, "f64", stop_tokens=list(stop), budget=budget)
    exp["flagged"] = exp["flagged"] | pflag
    return exp


def check(x, bias, words, top_k, top_p, stop=None, budget=None):
    got = run_chain_proc(x, bias, words, top_k, top_p, stop, budget)
    exp = oracle_chain_proc(x, bias, words, top_k, top_p, () if stop is None else stop.tolist(), budget)
    # flags also cover top-p boundaries within TOP_P_FLAG of the target mass, which the
    # chain's flag expectation does not include: a fixed allowance, at most half the batch
    s = compare_chain(got, exp, max_flag_frac=0.5)
    if stop is not None or budget is not None:
        keep = ~exp["flagged"]
        np.testing.assert_array_equal(got["finish"][keep], exp["finish"][keep])
    return got, exp, s


def test_headline_shape_all_processors():
    """B=64, gamma=5, V=128256 bf16, T=0.8; fp32 bias, 90%-allowed masks per row, top-k in
    {0, 1, 20, 1000}, top-p in {1, 0.5, 0.9, 0.99} per request."""
    x = synth.make_config(3, 0)
    bias, words, k, p = synth.make_processors(x.B, x.gamma + 1, x.V, seed=11)
    say("chain_ex config3 bias+mask+top-k+top-p")
    got, exp, s = check(x, bias, words, k, p)
    print(s, "accepted", np.bincount(got["accepted_len"][got["req_status"] == 0], minlength=6).tolist())


@pytest.mark.parametrize("k,tp", [(1000, 0.5), (200, 0.3), (20, 0.9)])
def test_top_k_and_top_p_bins_collected_together(k, tp):
    """Both truncations on every request, on peaked rows (1% of entries boosted by +8): the
    top-p bin usually lies above the top-k bin, and both bins' candidates are then collected
    in one pass over the row; the result must equal the oracle's."""
    x = synth.make_chain(32, 4, 32000, seed=int(k * 10 + tp * 100), logit_dtype="bf16", sigma=2.5,
                         boost_frac=0.01, boost=8.0, noise=1.0, temperature=0.8)
    bias, words, _, _ = synth.make_processors(x.B, x.gamma + 1, x.V, seed=k, with_top_k=False, with_top_p=False)
    kk = np.full(x.B, k, np.int32)
    pp = np.full(x.B, tp, np.float32)
    say(f"chain_ex top-k {k} and top-p {tp} on every request")
    check(x, bias, words, kk, pp)


@pytest.mark.parametrize("V,T", [(40, 0.05), (40, 50.0), (3000, 0.05), (3000, 50.0), (100000, 20.0)])
def test_top_p_weight_scales(V, T):
    """Top-p masses are fixed-point integers with a scale set by the candidate count (up to
    2^51 units per weight when few tokens are candidates).  Small vocabularies and extreme
    temperatures (weights close to 1, or all but the top ones close to 0) reach the widest
    integers and the most rounding; results must equal the oracle's."""
    x = synth.make_chain(24, 3, V, seed=V + int(T * 100), logit_dtype="f32", sigma=2.0, noise=0.8, temperature=T)
    bias, words, k, p = synth.make_processors(x.B, x.gamma + 1, x.V, seed=V, top_k=(0, 5, 30),
                                              top_p=(0.3, 0.7, 0.95))
    say(f"chain_ex top-p weight scales V={V} T={T}")
    check(x, bias, words, k, p)


@pytest.mark.parametrize("which", ["bias", "mask", "top_k", "top_p"])
def test_each_processor_alone(which):
    x = synth.make_chain(24, 4, 20003, seed=300, logit_dtype="bf16", sigma=2.0, noise=0.5, temperature=0.9)
    bias, words, k, p = synth.make_processors(x.B, x.gamma + 1, x.V, seed=12, top_k=(1, 5, 300, 19000),
                                              top_p=(0.3, 0.8, 0.95, 0.999), with_bias=which == "bias",
                                              with_mask=which == "mask", with_top_k=which == "top_k",
                                              with_top_p=which == "top_p")
    say(f"chain_ex {which} alone V=20003")
    print(check(x, bias, words, k, p)[2])


@pytest.mark.parametrize("V,dt,gamma", [(1, "f32", 2), (7, "bf16", 3), (33, "f32", 4), (2049, "bf16", 5),
                                        (8193, "f32", 8), (65536, "bf16", 3)])
def test_ragged_with_every_processor(V, dt, gamma):
    x = synth.make_chain(12, gamma, V, seed=310 + V, logit_dtype=dt, sigma=2.0, noise=0.5, temperature=1.1)
    bias, words, k, p = synth.make_processors(x.B, gamma + 1, V, seed=13 + V, allowed_frac=0.7,
                                              top_k=(0, 1, 3, 100), top_p=(1.0, 0.2, 0.7, 0.97))
    say(f"chain_ex ragged V={V} {dt} gamma={gamma}")
    check(x, bias, words, k, p)


def test_top_k_one_and_ties():
    """top-k = 1 keeps only the maximum (all of its ties): with coarse logits the maximum is
    often shared, and the draw is among the tied tokens."""
    B, G, V = 16, 3, 5000
    rng = np.random.default_rng(14)
    vals = np.round(rng.normal(0, 1, (B, G + 1, V)) * 2) / 2
    x = synth.make_chain(B, G, V, seed=15, logit_dtype="f32", noise=0.5)
    x.logits = vals.astype(np.float32)
    say("chain_ex top-k 1 with ties")
    check(x, None, None, np.ones(B, np.int32), None)


def test_statuses_with_processors():
    B, G, V = 8, 3, 3000
    x = synth.make_chain(B, G, V, seed=16, logit_dtype="f32", sigma=2.0, noise=0.3)
    bias, words, _, _ = synth.make_processors(B, G + 1, V, seed=17, with_top_k=False, with_top_p=False)
    words = words.copy()
    words[0, 0, :] = 0                                    # 0: row 0 entirely masked -> no valid token
    x.logits[1, 0, 5] = np.nan                            # 1: NaN in row 0 ...
    words[1, 0, 0] &= ~np.uint32(1 << 5)                  # ... at a masked position: still invalid
    words[2, 0, x.tokens[2, 0] // 32] &= ~np.uint32(1 << (x.tokens[2, 0] % 32))   # 2: draft 0 masked: rejected
    bias = bias.copy()
    bias[x.tokens[3, 0]] = -np.inf                        # 3: draft 0 banned by the bias
    say("chain_ex statuses")
    got, exp, _ = check(x, bias, words, None, None)
    assert exp["status"].tolist()[:2] == [oracle.NONFINITE, oracle.NONFINITE]
    assert exp["accepted_len"][2] == 0 and exp["accepted_len"][3] == 0


def test_processors_with_stops_and_workspace_reuse():
    x = synth.make_config(2, 3)
    bias, words, k, p = synth.make_processors(x.B, x.gamma + 1, x.V, seed=18)
    stop, budget = synth.make_stop(x.tokens, x.V, seed=19, n_stop=32, from_drafts=32)
    ws = torch.zeros(sv.chain_workspace_bytes(x.B, x.gamma, x.V) + 512, dtype=torch.uint8, device=DEV)
    say("chain_ex processors + stops, workspace reuse")
    a = run_chain_proc(x, bias, words, k, p, stop, budget, workspace_tensor=ws)
    b = run_chain_proc(x, bias, words, k, p, stop, budget, workspace_tensor=ws)
    torch.cuda.synchronize()
    assert int(ws.count_nonzero()) == 0
    for key in a:
        np.testing.assert_array_equal(a[key], b[key], err_msg=key)
    check(x, bias, words, k, p, stop, budget)


def test_no_processor_options_match_the_plain_call():
    x = synth.make_config(2, 4)
    say("chain_ex with disabled processors vs spec_verify_chain")
    got = run_chain_proc(x, None, None, np.zeros(x.B, np.int32), np.ones(x.B, np.float32))
    plain = to_np(sv.spec_verify_chain(t_logits(x.logits, x.logit_dtype), t_f32(x.q), t_i32(x.tokens),
                                       t_f32(x.u), float(x.temperature), with_stats=True))
    for key in ("accepted_len", "out_tokens", "req_status"):
        np.testing.assert_array_equal(got[key], plain[key], err_msg=key)


def test_greedy_with_bias_and_mask():
    x = synth.make_config(4, 1, B=64)
    bias, words, _, _ = synth.make_processors(x.B, x.gamma + 1, x.V, seed=20, bias_sigma=0.5,
                                              with_top_k=False, with_top_p=False)
    say("greedy_ex bias+mask B=64 gamma=8 V=128256")
    got = to_np(sv.spec_verify_greedy(t_logits(x.logits, x.logit_dtype), t_i32(x.tokens), bias=t_f32(bias),
                                      allowed=t_words(words)))
    L, _ = oracle.process_rows(x.logits, x.logit_dtype, 1.0, bias, words)
    exp = oracle.verify_greedy(L, x.tokens, "f64")
    compare_exact(got, exp, ["accepted_len", "out_tokens"])


@pytest.mark.parametrize("V", [5000, 65536])
def test_truncations_on_piled_values(V):
    """Logits on a coarse grid (a few dozen distinct values): with V = 65536 the bin holding
    a threshold has thousands of candidates, so the selection takes its radix fallback; with
    V = 5000 it resolves the bin directly.  Both must give the oracle's thresholds."""
    B, G = 12, 2
    rng = np.random.default_rng(21 + V)
    x = synth.make_chain(B, G, V, seed=22 + V, logit_dtype="f32", noise=0.5)
    x.logits = (np.round(rng.normal(0, 1, (B, G + 1, V)) * 4) / 4).astype(np.float32)
    k = np.array([1, 20, 1000, 0] * 3, np.int32)
    p = np.array([1.0, 0.5, 0.9, 0.99, 0.3, 1.0] * 2, np.float32)
    say(f"chain_ex truncations on piled values V={V}")
    check(x, None, None, k, p)


@pytest.mark.parametrize("dt,V,T", [("f32", 32000, 1.0), ("bf16", 128256, 0.8), ("f32", 4096, 0.25)])
def test_top_p_boundaries_just_outside_the_flag_window(dt, V, T):
    """The oracle flags a top-p decision whose deciding mass lies within 1e-5 of the target
    p * Z.  Here every request's p is placed 2e-5 * Z above or below the mass of its top m
    distinct values (m = 1..32, fewer on very peaked rows), so the boundary is never flagged and the kept set must be
    exactly the oracle's: m or m + 1 values.  gamma = 0 gives one row per request, so p
    decides one boundary; a wrong kept set changes log Z of the bonus row by the boundary
    token's share (far above the 1e-5 tolerance) and usually the token.  The GPU's masses are
    fp64 sums of fp32 weights 2^((s - ref) c2): relative errors near 1e-7 per weight where the
    mass lies, so 2e-5 leaves a wide margin."""
    B = 64
    x = synth.make_chain(B, 0, V, seed=V + int(T * 10), logit_dtype=dt, sigma=3.0, noise=1.0, temperature=T)
    L = oracle.decode(x.logits, x.logit_dtype)[:, 0].astype(np.float32).astype(np.float64)
    Tf = float(np.float32(T))
    p = np.empty(B, np.float32)
    for b in range(B):
        s = L[b]
        w = np.exp((s - s.max()) / Tf)
        Z = w.sum()
        uniq, inv = np.unique(s, return_inverse=True)
        mass = np.bincount(inv, weights=w)[::-1]          # per distinct value, largest first
        # m = 1 + b % 32 values, fewer where the row is so peaked that a value near the
        # boundary holds under 1e-4 of the mass (its own boundary would then be flagged)
        m = 1 + b % 32
        while m > 1 and not (mass[m - 1] > 1e-4 * Z and mass[m] > 1e-4 * Z):
            m -= 1
        top = mass[:m].sum()                              # mass of the top m distinct values
        sign = 1.0 if (b // 32) % 2 == 0 else -1.0
        p[b] = np.float32((top + sign * 2e-5 * Z) / Z)
        if not p[b] < 1.0:                                # p >= 1 turns top-p off: go below instead
            p[b] = np.float32((top - 2e-5 * Z) / Z)
    k = np.zeros(B, np.int32)
    say(f"chain_ex top-p boundaries 2e-5 from the target, {dt} V={V} T={T}")
    got = run_chain_proc(x, None, None, k, p)
    exp = oracle_chain_proc(x, None, None, k, p)
    _, pflag = oracle.process_rows(x.logits, x.logit_dtype, x.temperature, None, None, k, p)
    assert not pflag.any(), "a boundary placed outside the window was flagged"
    s = compare_chain(got, exp, max_flag_frac=0.1)
    print(s)


@pytest.mark.parametrize("sigma,k,tp", [(0.1, 0, 0.9), (3.0, 0, 0.9), (2.0, 1600, 1.0), (2.0, 1700, 1.0),
                                        (0.1, 3000, 0.5)])
def test_threshold_window_and_full_paths(sigma, k, tp):
    """The threshold pass decides most rows from a window of the top candidates collected in
    one pass, and falls back to the full path when the window cannot hold the selection: k
    above about 1600 (k = 1700 here; 1600 still fits), or a top-p nucleus larger than the
    window (near-flat rows, sigma = 0.1, where p = 0.9 keeps most of the row; the window misses
    and the row takes the full path).  Every case must equal the oracle."""
    x = synth.make_chain(16, 2, 50000, seed=int(sigma * 100) + k + int(tp * 10), logit_dtype="bf16", sigma=sigma,
                         noise=0.5, temperature=1.0)
    kk = np.full(x.B, k, np.int32)
    pp = np.full(x.B, tp, np.float32)
    say(f"chain_ex threshold paths sigma={sigma} k={k} p={tp}")
    check(x, None, None, kk, pp)


@pytest.mark.parametrize("tied", [False, True])
def test_top1_kept_set_with_unique_and_tied_maxima(tied):
    """Top-1 on every request keeps each row's largest value with its ties.  With a unique
    maximum the threshold pass hands the statistics pass the row's summary (max, Z); with a
    tied one the row is streamed as usual.  Every row holds one value above all others, once
    or three times; half the requests draft one of its copies.  Tokens, statuses and the
    per-row statistics (max and log Z) must equal the oracle's."""
    x = synth.make_chain(24, 3, 32000, seed=77 if tied else 78, logit_dtype="bf16", temperature=0.8)
    rng = np.random.default_rng(5)
    top = np.uint16(np.float32(30.0).view(np.uint32) >> 16)   # 30.0 in bf16
    for b in range(x.B):
        for r in range(x.gamma + 1):
            pos = rng.choice(x.V, size=3 if tied else 1, replace=False)
            x.logits[b, r, pos] = top
            if r < x.gamma and b % 2 == 0:
                x.tokens[b, r] = pos[0]
    k = np.ones(x.B, np.int32)
    p = np.where(np.arange(x.B) % 3 == 0, 0.5, 1.0).astype(np.float32)
    say(f"chain_ex top-1, {'tied' if tied else 'unique'} maxima")
    got, exp, s = check(x, None, None, k, p)
    assert (got["req_status"] == 0).all()


@pytest.mark.parametrize("k,tp", [(20, 1.0), (0, 0.9), (300, 0.95)])
def test_window_summaries_with_bias_and_masks(k, tp):
    """Rows decided by the threshold pass's window (top-k, top-p alone, both) reach the
    verifier as kept-set summaries rather than through the statistics stream; with bias and
    masks on, the per-row statistics, tokens and statuses must equal the oracle's.  Peaked rows
    (1% of entries boosted by +8) put the nucleus inside the window."""
    x = synth.make_chain(32, 4, 50000, seed=k + int(tp * 100), logit_dtype="bf16", sigma=2.5, boost_frac=0.01,
                         boost=8.0, noise=1.0, temperature=0.8)
    bias, words, _, _ = synth.make_processors(x.B, x.gamma + 1, x.V, seed=k + 1, with_top_k=False,
                                              with_top_p=False)
    kk = np.full(x.B, k, np.int32)
    pp = np.full(x.B, tp, np.float32)
    say(f"chain_ex window summaries k={k} p={tp}")
    check(x, bias, words, kk, pp)


@pytest.mark.parametrize("B,gamma", [(300, 0), (100, 3), (300, 1)])
def test_rows_mapped_heaviest_first(B, gamma):
    """The threshold pass maps blocks to rows by cost class (top-p alone, top-k >= 2, top-1,
    neither) when some CUs hold two rows.  With 300 and 400 rows it takes that order on a
    256-CU device (300 requests: the classes beyond the first 256 are read again); with 600
    rows the rows keep their own order.  Mixed top-k and top-p per request; every row's
    threshold must reach the verifier whatever block computed it, so tokens, statuses and
    statistics must equal the oracle's."""
    x = synth.make_chain(B, gamma, 4096, seed=B + gamma, logit_dtype="bf16", sigma=2.5, boost_frac=0.01,
                         boost=8.0, noise=1.0, temperature=0.8)
    rng = np.random.default_rng(B * 10 + gamma)
    k = rng.choice(np.array([0, 1, 20, 300], np.int32), size=B)
    p = rng.choice(np.array([1.0, 0.5, 0.9], np.float32), size=B)
    say(f"chain_ex rows mapped by cost, B={B} gamma={gamma}")
    check(x, None, None, k, p)
