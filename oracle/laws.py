"""Closed forms and one-position identities of exact speculative sampling (float64).

Test infrastructure only (see the package docstring).  These are the quantities the
pages derive; tests pin them against the values the pages print and use them to
check the samplers' laws.
"""
from __future__ import annotations

import numpy as np


def acceptance_rate(p: np.ndarray, q: np.ndarray) -> float:
    """alpha = sum_x min(p(x), q(x)): the probability that a draft x ~ q survives.

    [M7.1] §0x03B "Acceptance Is The Shared Mass And Is Maximal";
    [M16] "The Speedup: How Many Tokens per Pass".
    """
    return float(np.sum(np.minimum(p, q)))


def total_variation(p: np.ndarray, q: np.ndarray) -> float:
    """TV(p, q) = (1/2) sum_x |p(x) - q(x)|  ([M7.1] §0x03B)."""
    return 0.5 * float(np.sum(np.abs(np.asarray(p) - np.asarray(q))))


def positive_residual(p: np.ndarray, q: np.ndarray) -> np.ndarray:
    """Unnormalized correction weights [p - q]_+  ([M7.1] §0x03C)."""
    return np.maximum(np.asarray(p, dtype=np.float64) - np.asarray(q, dtype=np.float64), 0.0)


def residual_distribution(p: np.ndarray, q: np.ndarray) -> np.ndarray:
    """Normalized correction law p'(x) = [p(x) - q(x)]_+ / sum_y [p(y) - q(y)]_+.

    [M7.1] §0x03 "Draft And Verify"; [M16] "The Math: Speculative Sampling".
    Undefined (raises) when p == q, where the correction branch is unreachable
    ([M7.1] §0x03D).
    """
    w = positive_residual(p, q)
    Z = w.sum()
    if not Z > 0:
        raise ValueError("residual mass is zero: the correction branch is unreachable")
    return w / Z


def accept_probability(p_x: float, q_x: float) -> float:
    """a(x) = min(1, p(x) / q(x)) for a proposed x with q(x) > 0  ([M7.1] §0x03A)."""
    if not q_x > 0:
        raise ValueError("a token with q(x) = 0 cannot be proposed")
    return min(1.0, p_x / q_x)


def expected_tokens(alpha: float, gamma: int) -> float:
    """E[G] = 1 + alpha + ... + alpha^gamma = (1 - alpha^{gamma+1}) / (1 - alpha),
    with the limit gamma + 1 at alpha = 1.  [M7.1] §0x05D; [M16] "The Speedup"."""
    if alpha == 1.0:
        return float(gamma + 1)
    return (1.0 - alpha ** (gamma + 1)) / (1.0 - alpha)


def speculative_speedup(alpha: float, gamma: int, c: float) -> float:
    """Idealized speedup (1 - alpha^{gamma+1}) / ((1 - alpha)(gamma c + 1)).
    [M7.1] §0x05D; [M16] "The Speedup"."""
    return expected_tokens(alpha, gamma) / (gamma * c + 1.0)


def survival(alphas) -> np.ndarray:
    """s_j = Pr(A >= j) = prod_{i<=j} alpha_i^reach, s_0 = 1  ([M7.1] §0x05A)."""
    a = np.asarray(alphas, dtype=np.float64)
    return np.concatenate([[1.0], np.cumprod(a)])


def accepted_length_law(alphas) -> np.ndarray:
    """Pr(A = a) = s_a - s_{a+1} for a < K, Pr(A = K) = s_K  ([M7.1] §0x05A)."""
    s = survival(alphas)
    law = s[:-1] - s[1:]
    return np.concatenate([law, [s[-1]]])


def expected_progress(alphas) -> float:
    """E[G] = 1 + sum_{j=1..K} s_j, G = A + 1 without a stop event ([M7.1] §0x05B)."""
    return float(survival(alphas).sum())


def chain_of_heads_expected_length(probs) -> float:
    """1 + sum_k prod_{j<=k} p_j: expected tokens per pass when head k is right with
    probability p_k given that heads before it were ([M16] "Self-Drafting: Medusa",
    Exercise 4).  Same survival sum as `expected_progress`."""
    return expected_progress(probs)


def iid_output_count_law(alpha: float, gamma: int) -> np.ndarray:
    """Pr(output count = j + 1) for j = 0..gamma with iid acceptance alpha
    ([Atlas] worked example: gamma = 2, alpha = 0.6 gives 0.4, 0.24, 0.36)."""
    return accepted_length_law([alpha] * gamma)
