"""Shared fp64 building blocks of the oracle (test infrastructure only).

[P3] "DSpark Speculative Decoding", section "Semi-Autoregressive Generation": the draft
distribution at a position is the softmax of its logits. Sampling from a distribution
with one host uniform is the inverse CDF taken in token-id order (the reading adopted
where the pages do not say how a sample is drawn).
"""
from __future__ import annotations

import numpy as np

U_MAX = 1.0 - 2.0 ** -24


def decode_factor(a: np.ndarray, w_dtype: str) -> np.ndarray:
    """Exact float64 value of a factor tensor: bf16 bit patterns (uint16) or float32."""
    if w_dtype == "bf16":
        if a.dtype != np.uint16:
            raise TypeError("bf16 factors are passed as uint16 bit patterns")
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if w_dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    raise ValueError(w_dtype)


def clamp_uniform(u) -> float:
    """A host uniform widened to float64 and clamped into [0, 1 - 2^-24].

    Values below 0 (and -0.0) give +0.0, values at or above 1 - 2^-24 give 1 - 2^-24, and a
    NaN uniform counts as 0 (the reading for a uniform that is not a number).
    """
    u = float(np.float32(u))
    if not u > 0.0:                 # negative, zero of either sign, or NaN
        return 0.0
    return min(u, U_MAX)


def softmax_row(l: np.ndarray):
    """(p, lse) of one logit row in float64, or None when every logit is -inf."""
    l = np.asarray(l, dtype=np.float64)
    m = l.max()
    if m == -np.inf:
        return None
    e = np.exp(l - m)
    z = e.sum()
    return e / z, m + np.log(z)


def inverse_cdf(p: np.ndarray, u: float) -> int:
    """Smallest token v with F(v) > u, F the running sum of p in id order.

    When rounding leaves u at or above the final F, the last token with p > 0 is taken.
    """
    f = np.cumsum(p)
    v = int(np.searchsorted(f, u, side="right"))
    if v >= p.shape[0]:
        nz = np.nonzero(p > 0)[0]
        return int(nz[-1]) if nz.size else -1
    return v
