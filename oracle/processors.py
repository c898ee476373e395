"""Target logit processors applied before verification -- the oracle.

Test infrastructure only (see the package docstring).

The verified target distribution is the one the decoding policy actually samples from,
after its processors, not the raw softmax: [M7.1] "M7.1 - Speculative Decoding: Draft,
Verify, Accept, Reject" §0x01 (p_i = Pi_T(l_i; S) owns temperature, masking, top-k,
top-p, grammar) and §0x06J ("Processed Probability Rows And Stateful Sampling");
[Tiny] "Exact Speculative and Assisted Decoding for TinyRustLM", "Grammar and
deterministic opportunities": a grammar mask turns q into
q_G(x) = q(x) 1[x in A_G] / sum_v q(v) 1[v in A_G].  §0x04G lists ordered temperature
and additive-bias processors.

Processors of one row, in this order (the pages fix the set, not every step of the
order; the readings are listed below):
  1. additive bias:  s_x = l_x + b_x, computed in fp32 (both operands are fp32 values);
  2. temperature:    the distribution is proportional to exp(s_x / T);
  3. mask:           tokens outside the allowed set A are removed (q_G above);
  4. top-k:          with k >= 1, only tokens whose s is at least the k-th largest s among
                     the remaining ones are kept (ties at the boundary are kept);
  5. top-p:          with 0 < p < 1, a remaining token x is kept iff the probability mass
                     (after steps 1-4, renormalized) of the tokens with strictly larger s
                     is less than p -- the smallest set of top tokens, closed under ties,
                     whose mass reaches p;
then p = softmax over the kept tokens.  Readings: bias precedes temperature (a logit-space
adjustment); the mask precedes the truncations, so top-k and top-p act on the valid
tokens; ties are never split.  A NaN or +inf in l + b anywhere in the row makes the row
invalid whatever the mask (the row is a numerical fault), as does a row with no kept
token.  Removed tokens become -inf, so the processed row feeds the unchanged verifiers.
"""
from __future__ import annotations

import numpy as np

from .numerics import decode

# A top-p boundary is flagged when a mass that decides it lies within this fraction of the
# row's total of the target p * Z: fp32 exponentials with an fp32 log2(e)/T factor put
# relative errors of up to about (s_max - s) * 1e-7 on a weight, which may decide it either way.
TOP_P_FLAG = 1e-5


def unpack_mask(words: np.ndarray, V: int) -> np.ndarray:
    """Allowed-token bitmask: bit (x mod 32) of 32-bit word x // 32 set means x is allowed."""
    w = np.asarray(words, dtype=np.uint32)
    bits = (w[..., :, None] >> np.arange(32, dtype=np.uint32)) & np.uint32(1)
    return bits.reshape(*w.shape[:-1], -1)[..., :V].astype(bool)


def process_row(l_row: np.ndarray, temperature: float, bias=None, allowed=None, top_k: int = 0,
                top_p: float = 1.0):
    """One row of raw logits (float64 holding fp32/bf16 values) -> (processed logits, flagged).

    Processed logits are s_x for kept tokens and -inf for removed ones (NaN / +inf are kept
    in place so that the row reads as invalid).
    """
    l32 = np.asarray(l_row, dtype=np.float64).astype(np.float32)
    b32 = np.zeros_like(l32) if bias is None else np.asarray(bias, dtype=np.float32)
    s = (l32 + b32).astype(np.float64)                     # the fp32 sum, widened exactly
    V = s.shape[0]
    fault = np.isnan(s) | np.isposinf(s)
    keep = np.isfinite(s)
    if allowed is not None:
        keep &= np.asarray(allowed, dtype=bool)
    flagged = False
    if top_k and top_k >= 1 and int(keep.sum()) > top_k:
        kth = np.sort(s[keep])[::-1][top_k - 1]            # k-th largest, with multiplicity
        keep &= s >= kth
    if 0.0 < top_p < 1.0 and keep.any():
        T = float(np.float32(temperature))
        vals = s[keep]
        w = np.exp((vals - vals.max()) / T)
        Z = float(w.sum())
        target = top_p * Z
        uniq, inv = np.unique(vals, return_inverse=True)   # distinct values, ascending
        mass_at = np.bincount(inv, weights=w)[::-1]        # their masses, largest value first
        uniq = uniq[::-1]
        incl = np.cumsum(mass_at)                          # mass of tokens with s >= v
        excl = incl - mass_at                              # mass of tokens with s >  v
        j = int(np.flatnonzero(excl < target).max())       # smallest value still needed
        tau = uniq[j]
        keep &= s >= tau
        if abs(excl[j] - target) < TOP_P_FLAG * Z or (j + 1 < len(uniq) and abs(excl[j + 1] - target) < TOP_P_FLAG * Z):
            flagged = True
    out = np.where(keep, s, -np.inf)
    out[fault] = s[fault]
    return out, flagged


def process_rows(logits, logit_dtype, temperature, bias=None, mask_words=None, top_k=None, top_p=None):
    """Batched: logits [B, R, V] (raw bf16 bits or fp32), bias [V] fp32 or None, mask_words
    [B, R, ceil(V/32)] uint32 or None, top_k [B] int or None, top_p [B] float or None.
    Returns (processed float64 [B, R, V], flagged [B])."""
    B, R, V = logits.shape
    out = np.empty((B, R, V))
    flagged = np.zeros(B, bool)
    allowed = None if mask_words is None else unpack_mask(mask_words, V)
    for b in range(B):
        L = decode(logits[b], logit_dtype)
        k = 0 if top_k is None else int(top_k[b])
        p = 1.0 if top_p is None else float(top_p[b])
        for i in range(R):
            out[b, i], f = process_row(L[i], temperature, bias, None if allowed is None else allowed[b, i], k, p)
            flagged[b] |= f
    return out, flagged


def densify_sparse_q(index: np.ndarray, values: np.ndarray, V: int) -> np.ndarray:
    """Sparse draft rows -> dense rows.  [Tiny] "Logit and residual scratch": a sparse top-k
    representation is exact only when the omitted proposal probabilities are known to be
    zero, so every token not listed gets q = 0; entries that share an index add up.
    index, values: [..., K] (int indices in [0, V), fp32 values)."""
    index = np.asarray(index)
    if ((index < 0) | (index >= V)).any():
        raise ValueError("sparse q index outside [0, V)")
    vals = np.asarray(values, dtype=np.float32).astype(np.float64)
    lead = index.shape[:-1]
    out = np.zeros(lead + (V,))
    flat_out = out.reshape(-1, V)
    flat_idx = index.reshape(-1, index.shape[-1])
    flat_val = vals.reshape(-1, vals.shape[-1])
    for r in range(flat_out.shape[0]):
        np.add.at(flat_out[r], flat_idx[r], flat_val[r])
    return out
