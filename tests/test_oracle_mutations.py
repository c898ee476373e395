"""The oracle's pins catch plausible mistakes (CPU only).

Each case plants one mistake in a copy of `oracle/`, in a temporary directory, and runs
the CPU pin suites (worked examples, closed forms, exact enumeration, stored regression
outputs) against the copy in a fresh interpreter.  The case passes when the suite
fails.  The real oracle is never modified.  The mistakes are the kind a reader of the
pages could plausibly make: a flipped inequality, a dropped term, a transposed operand,
an off-by-one row, a wrong uniform, a wrong tie rule.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PIN_FILES = ["test_oracle_pins.py", "test_oracle_laws.py", "test_oracle_regression.py",
             "test_oracle_tree_residual.py", "test_oracle_stop.py", "test_oracle_tree_greedy.py",
             "test_oracle_processors.py", "test_oracle_lazy.py"]

# (file under oracle/, text as it stands, the planted mistake)
MUTANTS = {
    # chain: [M7.1] §0x03A-§0x03H, [M16] "The Math: Speculative Sampling"
    "accept_u_le_a": ("chain.py", "if not (u[i] < a):", "if not (u[i] <= a):"),
    "ratio_inverted": ("chain.py", "a = min(1.0, px / qx)", "a = min(1.0, qx / max(px, 1e-300))"),
    "no_clip_at_one": ("chain.py", "a = min(1.0, px / qx)", "a = px / qx if px < qx else 0.999"),
    "residual_q_minus_p": ("chain.py", "w = np.maximum(p - qrow, 0.0)", "w = np.maximum(qrow - p, 0.0)"),
    "residual_dropped": ("chain.py", "w = np.maximum(p - qrow, 0.0)", "w = p"),
    "residual_unclipped": ("chain.py", "w = np.maximum(p - qrow, 0.0)", "w = np.abs(p - qrow)"),
    "residual_next_row": ("chain.py", "p, _, _ = target_probs(L[A], temperature, check_backends=False)",
                          "p, _, _ = target_probs(L[min(A + 1, gamma)], temperature, check_backends=False)"),
    "residual_from_draft_row_0": ("chain.py", "qrow = Q[A]", "qrow = Q[0]"),
    "bonus_from_row_0": ("chain.py", "p, m, Z = target_probs(L[gamma], temperature)",
                         "p, m, Z = target_probs(L[0], temperature)"),
    "no_stop_at_first_rejection": ("chain.py", "            A = i\n            break\n", "            A = i\n"),
    # rows past the first rejection read as if they mattered ([M7.1] §0x03G)
    "chain_validates_every_row": ("chain.py", "    A = gamma\n    end = None",
                                  "    if not all(row_is_valid(L[j]) for j in range(gamma + 1)):\n"
                                  "        return fail(NONFINITE)\n    A = gamma\n    end = None"),
    "greedy_validates_every_row": ("greedy.py", "    for i in range(gamma):\n        if not row_is_valid(L[i]):",
                                   "    if not all(row_is_valid(L[j]) for j in range(gamma + 1)):\n"
                                   "        return NONFINITE, -1, [], 0\n"
                                   "    for i in range(gamma):\n        if not row_is_valid(L[i]):"),
    "terminal_uses_rejecting_uniform": ("chain.py", "k, W, lo, hi = inverse_cdf(w, float(u[gamma]))",
                                        "k, W, lo, hi = inverse_cdf(w, float(u[min(A, gamma)]))"),
    "correction_not_emitted": ("chain.py", "res.tokens = [int(t) for t in x[:A]] + [k]",
                               "res.tokens = [int(t) for t in x[:A]] + ([k] if A == gamma else [])"),
    "uniform_checked_before_q": ("chain.py",
                                 "        if not (np.isfinite(qx) and qx > 0.0):\n            return fail(QZERO)\n"
                                 "        if not (0.0 <= u[i] < 1.0):\n            return fail(BADUNIFORM)\n",
                                 "        if not (0.0 <= u[i] < 1.0):\n            return fail(BADUNIFORM)\n"
                                 "        if not (np.isfinite(qx) and qx > 0.0):\n            return fail(QZERO)\n"),
    "cdf_left_side": ("chain.py", 'k = int(np.searchsorted(c, u * W, side="right"))',
                      'k = int(np.searchsorted(c, u * W, side="left"))'),
    # numerics: decoding, temperature, softmax ([M7.1] §0x04F, §0x04J)
    "temperature_multiplies": ("numerics.py", "s = logits_row / T", "s = logits_row * T"),
    "softmax_drops_a_term": ("numerics.py", "    Z = float(np.sum(e))\n    return e / Z, m, Z",
                             "    Z = float(np.sum(e[1:]))\n    return e / Z, m, Z"),
    "bf16_wrong_shift": ("numerics.py", "* np.uint32(65536)", "* np.uint32(32768)"),
    "posinf_row_valid": ("numerics.py", "if np.isnan(row).any() or np.isposinf(row).any():",
                         "if np.isnan(row).any():"),
    # greedy ([M7.1] §0x02D, [Tiny] "Normative greedy pseudocode")
    "greedy_last_tie": ("greedy.py", "return int(np.flatnonzero(row == row.max())[0])",
                        "return int(np.flatnonzero(row == row.max())[-1])"),
    "greedy_no_correction": ("greedy.py", "return OK, i, [int(v) for v in x[:i]] + [t], (",
                             "return OK, i, [int(v) for v in x[:i]], ("),
    "greedy_bonus_row_off_by_one": ("greedy.py", "t = first_argmax(L[gamma])", "t = first_argmax(L[gamma - 1])"),
    # tree ([M7.7] §0x07E, §0x09, §0x0F, §0x0AA)
    "tree_any_node_with_token": ("tree.py", "if int(parents[c]) == v and int(node_tokens[c]) == y:",
                                 "if int(node_tokens[c]) == y:"),
    "tree_root_uniform_everywhere": ("tree.py", "uv = float(u[v])", "uv = float(u[0])"),
    "tree_row_of_child": ("tree.py", "p, _, _ = target_probs(L[v], temperature)",
                          "p, _, _ = target_probs(L[min(v + 1, N - 1)], temperature)"),
    "tree_highest_index_child": ("tree.py", "for c in range(v + 1, N):", "for c in range(N - 1, v, -1):"),
    "tree_accepts_self_parent": ("tree.py", "if not (0 <= pv < v):", "if not (0 <= pv <= v):"),
    "tree_expectation_uses_child_row": ("tree.py",
                                        "f[v] = f[int(parents[v])] * probs[int(parents[v]), int(node_tokens[v])]",
                                        "f[v] = f[int(parents[v])] * probs[v, int(node_tokens[v])]"),
    # residual-update tree ([M7.7] §0x08B, §0x09A)
    "tree_residual_not_updated": ("tree_residual.py", "            res = g / W\n", "            res = res\n"),
    "tree_residual_unnormalized": ("tree_residual.py", "            res = g / W\n", "            res = g\n"),
    "tree_residual_unclipped": ("tree_residual.py", "            g = np.maximum(res - q, 0.0)",
                                "            g = np.abs(res - q)"),
    "tree_residual_tests_original_p": ("tree_residual.py", "            a = min(1.0, float(res[x]) / qx)",
                                       "            a = min(1.0, float(target_probs(L[v], temperature)[0][x]) / qx)"),
    "tree_residual_reverse_child_order": ("tree_residual.py", "        for c in range(v + 1, N):            # children",
                                          "        for c in range(N - 1, v, -1):            # children"),
    "tree_residual_draw_with_accept_uniform": ("tree_residual.py", "        ud = float(u_draw[v])",
                                               "        ud = float(u_acc[v]) if v > 0 else float(u_draw[v])"),
    # greedy tree ([M16] "Verify the Tree -- and Why It's Exact")
    "tree_greedy_last_tie": ("tree_greedy.py", "y = first_argmax(L[v])",
                             "y = int(np.flatnonzero(L[v] == L[v].max())[-1])"),
    "tree_greedy_child_row": ("tree_greedy.py", "y = first_argmax(L[v])", "y = first_argmax(L[min(v + 1, N - 1)])"),
    "tree_greedy_no_bonus": ("tree_greedy.py", "tokens=[int(node_tokens[c]) for c in path] + [y])",
                             "tokens=[int(node_tokens[c]) for c in path])"),
    "tree_greedy_any_node": ("tree_greedy.py", "if int(parents[c]) == v and int(node_tokens[c]) == y:",
                             "if int(node_tokens[c]) == y:"),
    "tree_greedy_last_sibling": ("tree_greedy.py", "                nxt = c\n                break\n",
                                 "                nxt = c\n"),
    # target logit processors ([Tiny] grammar mask, exactness tests; [M7.1] §0x04G, §0x06J)
    "topk_drops_boundary_ties": ("processors.py", "keep &= s >= kth", "keep &= s > kth"),
    "topk_off_by_one": ("processors.py", "[::-1][top_k - 1]", "[::-1][min(top_k, len(s) - 1)]"),
    "topp_counts_own_mass": ("processors.py", "np.flatnonzero(excl < target)", "np.flatnonzero(incl < target)"),
    "bias_after_temperature": ("processors.py", "s = (l32 + b32).astype(np.float64)",
                               "s = (l32 + b32 * np.float32(temperature)).astype(np.float64)"),
    "masked_fault_hidden": ("processors.py", "    out[fault] = s[fault]\n", ""),
    "mask_ignored_by_truncation": ("processors.py", "        keep &= np.asarray(allowed, dtype=bool)\n",
                                   "        pass\n"),
    # stop tokens and output budget ([M7.1] §0x05B, §0x06)
    "stop_token_not_ending_round": ("chain.py", "            end = (i + 1, 1)\n", "            pass\n"),
    "stop_token_not_emitted": ("chain.py", "res.tokens = [int(t) for t in x[:end[0]]]",
                               "res.tokens = [int(t) for t in x[:end[0] - 1]]"),
    "budget_off_by_one": ("chain.py", "if H is not None and i + 1 == H:", "if H is not None and i == H:"),
    "zero_budget_runs_a_round": ("chain.py", "if H is not None and H <= 0:", "if H is not None and H < 0:"),
    "stop_checked_before_accept": ("chain.py",
                                   "        if not (u[i] < a):          # first rejection: stop here\n"
                                   "            A = i\n            break\n"
                                   "        if int(x[i]) in stop:       # an accepted stop token ends the round\n"
                                   "            end = (i + 1, 1)\n            break\n",
                                   "        if int(x[i]) in stop:       # an accepted stop token ends the round\n"
                                   "            end = (i + 1, 1)\n            break\n"
                                   "        if not (u[i] < a):          # first rejection: stop here\n"
                                   "            A = i\n            break\n"),
    "budget_finish_off_by_one": ("chain.py", "(2 if H is not None and A + 1 == H else 0)",
                                 "(2 if H is not None and A == H else 0)"),
    "greedy_stop_ignored": ("greedy.py", "        if xi in stop:\n", "        if xi in stop and i + 1 == gamma:\n"),
    "greedy_budget_off_by_one": ("greedy.py", "        if H == i + 1:\n", "        if H == i:\n"),
    # laws ([M7.1] §0x05A-§0x05D, [Atlas] mechanism)
    "expected_tokens_off_by_one": ("laws.py", "return (1.0 - alpha ** (gamma + 1)) / (1.0 - alpha)",
                                   "return (1.0 - alpha ** gamma) / (1.0 - alpha)"),
    "tv_without_half": ("laws.py", "return 0.5 * float(np.sum(np.abs(np.asarray(p) - np.asarray(q))))",
                        "return float(np.sum(np.abs(np.asarray(p) - np.asarray(q))))"),
}


def _copy_tree(dst):
    shutil.copytree(os.path.join(ROOT, "oracle"), os.path.join(dst, "oracle"),
                    ignore=shutil.ignore_patterns("__pycache__"))
    shutil.copytree(os.path.join(ROOT, "synth"), os.path.join(dst, "synth"),
                    ignore=shutil.ignore_patterns("__pycache__"))
    tdst = os.path.join(dst, "tests")
    os.makedirs(tdst)
    for f in PIN_FILES + ["conftest.py", "lawcheck.py"]:
        shutil.copy(os.path.join(ROOT, "tests", f), tdst)
    shutil.copytree(os.path.join(ROOT, "tests", "golden"), os.path.join(tdst, "golden"),
                    ignore=shutil.ignore_patterns("__pycache__"))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    fname, before, after = MUTANTS[name]
    _copy_tree(str(tmp_path))
    path = tmp_path / "oracle" / fname
    src = path.read_text()
    assert src.count(before) == 1, f"mutation site for {name} not found exactly once"
    path.write_text(src.replace(before, after))
    env = dict(os.environ, PYTHONDONTWRITEBYTECODE="1")
    proc = subprocess.run(
        [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
         *[os.path.join("tests", f) for f in PIN_FILES]],
        cwd=str(tmp_path), env=env, capture_output=True, text=True, timeout=600)
    assert proc.returncode != 0, f"planted mistake {name!r} passed every pin:\n{proc.stdout[-2000:]}"
    assert "passed" in proc.stdout or "failed" in proc.stdout, proc.stdout[-2000:] + proc.stderr[-2000:]


def test_unmutated_copy_passes(tmp_path):
    """The copied suite itself is green, so a failure above is the planted mistake's doing."""
    _copy_tree(str(tmp_path))
    proc = subprocess.run(
        [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
         *[os.path.join("tests", f) for f in PIN_FILES]],
        cwd=str(tmp_path), env=dict(os.environ, PYTHONDONTWRITEBYTECODE="1"),
        capture_output=True, text=True, timeout=600)
    assert proc.returncode == 0, proc.stdout[-3000:] + proc.stderr[-2000:]
