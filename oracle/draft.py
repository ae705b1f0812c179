"""Markov-head sequential draft, fp64 oracle (test infrastructure only).

[P3] "DSpark Speculative Decoding", section "Semi-Autoregressive Generation": position k
is sampled from p_k(v) proportional to exp(U_k(v) + B_k(v)), where the Markov head's bias
depends only on the previous token through the rank-r factors, B = W1[x_{k-1}] W2.
[P1] section "DSpark 架构设计：半自回归生成与马尔可夫修正": the head runs left to right and
looks only at the token drafted just before, so position k+1 conditions on x_k.

Readings taken where the pages are open: position 1 is biased by the context token x_0;
temperature 1 with no truncation; one host uniform per draw, inverse CDF in id order.
Boundary sentinels: a previous token outside [0, V) or a row whose logits are all -inf
gives token -1 (q = 0, lse = -inf), and every later position of that request is -1 too.
"""
from __future__ import annotations

import numpy as np

from .numerics import clamp_uniform, decode_factor, inverse_cdf, softmax_row


def markov_draft(U, W1, W2, x0, u, w_dtype: str = "f32", requests=None, want_logits=False,
                 forced=None):
    """Draft gamma tokens for each request.

    U  [B][gamma][V] float32 base logits; W1 [V][r], W2 [r][V] (float32, or uint16 bf16
    bits when w_dtype == "bf16"); x0 [B] context tokens; u [B][gamma] uniforms.
    ``requests`` restricts the work to a subset of b (outputs keep the full B shape,
    other rows are left at their fill values). Returns a dict with
    x [B][gamma] int64, q [B][gamma] = p_k(x_k), lse [B][gamma], and when asked,
    L [B][gamma][V] float64 logits U_k + B_k.

    ``forced`` [B][gamma] (optional) evaluates the conditional laws along a given block
    instead of the drawn one: position k + 1 conditions on forced[b, k] rather than on the
    token drawn at position k (p_k is a law given the prefix, so this is the same
    definition at another prefix). x still holds the draws each position makes; with
    forced equal to those draws the result is the unforced one.
    """
    U = np.asarray(U)
    B, G, V = U.shape
    w1 = decode_factor(np.asarray(W1), w_dtype)
    w2 = decode_factor(np.asarray(W2), w_dtype)
    if w1.shape[0] != V or w2.shape[1] != V or w1.shape[1] != w2.shape[0]:
        raise ValueError("factor shapes do not match U")
    x = np.full((B, G), -1, dtype=np.int64)
    q = np.zeros((B, G), dtype=np.float64)
    lse = np.full((B, G), -np.inf, dtype=np.float64)
    L = np.zeros((B, G, V), dtype=np.float64) if want_logits else None
    todo = range(B) if requests is None else requests
    for b in todo:
        prev = int(x0[b])
        for k in range(G):
            if not (0 <= prev < V):
                prev = -1
                continue
            h = w1[prev]                                    # gather the previous token's row
            logits = U[b, k].astype(np.float64) + h @ w2    # base logits plus Markov bias
            if L is not None:
                L[b, k] = logits
            st = softmax_row(logits)
            if st is None:
                prev = -1
                continue
            p, row_lse = st
            tok = inverse_cdf(p, clamp_uniform(u[b, k]))
            x[b, k] = tok
            q[b, k] = p[tok] if tok >= 0 else 0.0
            lse[b, k] = row_lse
            prev = tok if forced is None else int(forced[b, k])
    out = dict(x=x, q=q, lse=lse)
    if L is not None:
        out["L"] = L
    return out
