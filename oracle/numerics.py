"""Decoding, validity checks and the two softmax backends of the oracle (float64).

Test infrastructure only (see the package docstring).
"""
from __future__ import annotations

import numpy as np

# Per-request status codes. Their meaning is fixed by the verification contract:
# a request whose data break a precondition is aborted without emitting anything
# ([Tiny] "Normative stochastic pseudocode": abort the round on a NaN row or a
# residual that is not positive).
OK = 0
NONFINITE = 1        # a reached logits row holds NaN or +inf, or is entirely -inf
BADTOKEN = 2         # a reached draft token (or tree node token) is outside [0, V)
BADUNIFORM = 3       # a uniform that the round consumes is outside [0, 1)
QZERO = 4            # q_i(x_i) is not a positive finite number at a reached position
RESIDUAL_EMPTY = 5   # terminal weight mass is not positive/finite, or the q row at the
                     # rejected position holds a negative or non-finite entry
BADTREE = 6          # parent array is not a rooted tree with parents[v] < v


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 is the upper 16 bits of an IEEE binary32 value: place the bits there."""
    wide = np.asarray(bits).astype(np.uint16).astype(np.uint32) * np.uint32(65536)
    return wide.view(np.float32).astype(np.float64)


def decode(arr: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of stored logits / probabilities ('bf16' raw bits, 'f32', 'f64')."""
    if dtype == "bf16":
        return bf16_to_f64(arr)
    if dtype == "f32":
        return np.asarray(arr, dtype=np.float32).astype(np.float64)
    if dtype == "f64":
        return np.asarray(arr, dtype=np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def row_is_valid(row: np.ndarray) -> bool:
    """A processed logits row defines a distribution iff it has no NaN / +inf and at
    least one finite entry (-inf marks a masked token).  [Tiny] "Normative stochastic
    pseudocode" aborts on a row with NaN or no valid token."""
    if np.isnan(row).any() or np.isposinf(row).any():
        return False
    return bool(np.isfinite(row).any())


def softmax_maxshift(s: np.ndarray):
    """Conventional max-shift softmax of one row of processed logits.

    [M7.1] §0x04J "Backend, Layout, And State Parity", backend 1.
    Returns (p, m, Z) with p = exp(s - m) / Z, m = max s, Z = sum exp(s - m).
    """
    m = float(np.max(s))
    e = np.exp(s - m)
    Z = float(np.sum(e))
    return e / Z, m, Z


def softmax_online(s: np.ndarray, block: int = 1024):
    """Online (m, l) merge over vocabulary blocks.

    [M7.1] §0x04J "Backend, Layout, And State Parity", backend 2: each block keeps its
    own maximum and its sum of exponentials relative to it; two summaries (m, l) and
    (m', l') merge into (M, l e^{m-M} + l' e^{m'-M}) with M = max(m, m').
    Returns (p, m, Z) like `softmax_maxshift`.
    """
    m = -np.inf
    l = 0.0
    for start in range(0, s.shape[0], block):
        blk = s[start:start + block]
        mb = float(np.max(blk))
        if mb == -np.inf:
            continue
        lb = float(np.sum(np.exp(blk - mb)))
        M = max(m, mb)
        l = (l * np.exp(m - M) if m != -np.inf else 0.0) + lb * np.exp(mb - M)
        m = M
    return np.exp(s - m) / l, m, l


def target_probs(logits_row: np.ndarray, temperature: float, check_backends: bool = True):
    """Target distribution p of one row: temperature, then softmax.

    [M7.1] §0x04F "Numerical And Processor Boundary" and §0x03D: p is the normalized
    distribution *after* the declared processors; temperature is the processor here:
    s = l / T.  The temperature is the fp32 value the caller passes (it is widened
    exactly to float64).  Both softmax backends are evaluated and must agree
    ([M7.1] §0x04J requires backend agreement before the coupling is evaluated).
    Returns (p, m, Z) of s.
    """
    T = float(np.float32(temperature))
    s = logits_row / T
    p, m, Z = softmax_maxshift(s)
    if check_backends:
        p2, m2, Z2 = softmax_online(s)
        if m2 != m or not np.allclose(p2, p, rtol=1e-12, atol=1e-300) or abs(Z2 - Z) > 1e-12 * Z:
            raise AssertionError("softmax backends disagree")
    return p, m, Z
