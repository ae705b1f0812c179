"""RNN-head sequential draft, fp64 oracle (test infrastructure only).

[P3] "DSpark Speculative Decoding", section "Semi-Autoregressive Generation": the sequential
stage samples x_k from p_k(v) proportional to exp(U_k(v) + B_k(x_<k, v)), and besides the
default Markov head (B = W1[x_{k-1}] W2) it names an RNN head that keeps a recurrent state
inside the block. [P1] section "DSpark 架构设计：半自回归生成与马尔可夫修正" (the RNN head
paragraph): an optional head that maintains and updates a hidden state along the block, so
that the bias depends on the whole drafted prefix rather than on the last token only.

The pages give no update rule. Reading adopted (the plainest recurrence that keeps the
Markov head as its special case): a linear state of the head's rank r,

    h_1 = W1[x_0],   h_k = A h_{k-1} + W1[x_{k-1}]  (k = 2..gamma),   B_k = h_k W2,

with A an r x r matrix in the factors' dtype. A = 0 gives the Markov head exactly. The draw,
the sentinels and the readings of the Markov draft carry over: one uniform per draw, inverse
CDF in token-id order; a previous token outside [0, V) or an all -inf row ends the request
(token -1 from there on).
"""
from __future__ import annotations

import numpy as np

from .numerics import clamp_uniform, decode_factor, inverse_cdf, softmax_row


def rnn_draft(U, W1, W2, A, x0, u, w_dtype: str = "f32", requests=None, want_logits=False,
              want_state=False, forced=None):
    """Draft gamma tokens per request with the RNN head.

    U [B][gamma][V] float32; W1 [V][r], W2 [r][V], A [r][r] (float32, or uint16 bf16 bits
    when w_dtype == "bf16"); x0 [B]; u [B][gamma]. Returns x [B][gamma], q, lse, and when
    asked L [B][gamma][V] (logits) and h [B][gamma][r] (the state h_k of each position, the
    one its bias is formed from). ``forced`` [B][gamma]: position k + 1's state takes
    forced[b, k] as the previous token instead of the draw (the law given that prefix).
    """
    U = np.asarray(U)
    B, G, V = U.shape
    w1 = decode_factor(np.asarray(W1), w_dtype)
    w2 = decode_factor(np.asarray(W2), w_dtype)
    a = decode_factor(np.asarray(A), w_dtype)
    r = w1.shape[1]
    if w1.shape[0] != V or w2.shape != (r, V) or a.shape != (r, r):
        raise ValueError("factor shapes do not match U")
    x = np.full((B, G), -1, dtype=np.int64)
    q = np.zeros((B, G), dtype=np.float64)
    lse = np.full((B, G), -np.inf, dtype=np.float64)
    L = np.zeros((B, G, V), dtype=np.float64) if want_logits else None
    H = np.zeros((B, G, r), dtype=np.float64) if want_state else None
    todo = range(B) if requests is None else requests
    for b in todo:
        h = np.zeros(r)                             # the state before the block
        prev = int(x0[b])
        for k in range(G):
            if not (0 <= prev < V):
                prev = -1
                continue
            h = a @ h + w1[prev]                    # recurrent update with the previous token
            if H is not None:
                H[b, k] = h
            logits = U[b, k].astype(np.float64) + h @ w2
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
    if H is not None:
        out["h"] = H
    return out
