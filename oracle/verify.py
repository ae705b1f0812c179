"""Lossless rejection-sampling verification, fp64 oracle (test infrastructure only).

[P1] section "大模型推理的显存瓶颈与推测解码的演进逻辑": the target checks the draft tokens left
to right, keeps the longest prefix that passes, resamples one token at the first failure
and drops everything after it, so the output law equals the target's. [P3] intro: the
accepted prefix is followed by a bonus token. [P2] section "为什么推测解码很重要" points to
the speculative sampling papers whose rule this is: token x at a position is kept when
u < p_t(x) / p_d(x); at the first rejection the new token is drawn from
max(0, p_t - p_d) renormalised; when every verified token is kept the bonus token is drawn
from the target distribution at the next position.

Readings: the acceptance test is u * p_d(x) < p_t(x) (strict; p_d(x) = 0 accepts iff
p_t(x) > 0); one final uniform serves the residual or the bonus draw; when the residual
mass is zero (only reachable by rounding) the draw falls back to p_t; a draft row that is
all -inf counts as p_d = 0. Target rows are flattened: request b owns rows
t_off[b] .. t_off[b] + len[b]; row t_off[b] + i is the target law at position i + 1.
Sentinels: a draft token outside [0, V) among the verified ones gives n = -1 and an
all -1 output row; a target row that is all -inf at the final draw gives token -1.
"""
from __future__ import annotations

import numpy as np

from .numerics import clamp_uniform, inverse_cdf, softmax_row


def accept_test(u: float, pd_x: float, pt_x: float) -> bool:
    if pd_x > 0.0:
        return u * pd_x < pt_x
    return pt_x > 0.0


def _probs(row, V):
    st = softmax_row(row)
    if st is None:
        return np.zeros(V), -np.inf
    return st


def verify(Ld, Lt, x, u_acc, u_fin, t_off=None, length=None, requests=None, n_forced=None):
    """Verify each request's draft block.

    Ld [B][gamma][V] draft logits; Lt [rows][V] flattened target logits; x [B][gamma]
    draft tokens; u_acc [B][gamma]; u_fin [B]; t_off [B+1] or None (b*(gamma+1));
    length [B] or None (gamma). Returns dict n [B] int64, y [B][gamma+1] int64 (-1 pad),
    ratio [B][gamma] = min(1, p_t(x_k) / p_d(x_k)) at each verified position (the value the
    acceptance uniform is compared with; NaN beyond the length) and law [B] (the
    distribution the final token was drawn from; None where no draw was made).

    ``n_forced`` [B] (optional) takes the accepted count as given instead of scanning
    (each n in [0, len]), and draws the final token and forms y for that count: the same
    residual or bonus rule, evaluated after another acceptance path.
    """
    Ld = np.asarray(Ld)
    B, G, V = Ld.shape
    n_out = np.zeros(B, dtype=np.int64)
    y_out = np.full((B, G + 1), -1, dtype=np.int64)
    ratio = np.full((B, G), np.nan)
    laws = [None] * B
    todo = range(B) if requests is None else requests
    for b in todo:
        ell = G if length is None else int(length[b])
        off = b * (G + 1) if t_off is None else int(t_off[b])
        xs = [int(v) for v in x[b, :ell]]
        if any(not (0 <= v < V) for v in xs):
            n_out[b] = -1
            continue
        pd = [_probs(Ld[b, k], V)[0] for k in range(ell)]      # draft law at position k+1
        pt = [_probs(Lt[off + k], V)[0] for k in range(ell)]   # target law at position k+1
        for k in range(ell):
            a, t = pd[k][xs[k]], pt[k][xs[k]]
            ratio[b, k] = min(1.0, t / a) if a > 0 else (1.0 if t > 0 else 0.0)
        n = 0
        while n < ell and accept_test(clamp_uniform(u_acc[b, n]), pd[n][xs[n]], pt[n][xs[n]]):
            n += 1
        if n_forced is not None:
            n = int(n_forced[b])
            if not 0 <= n <= ell:
                raise ValueError(f"n_forced[{b}] = {n} outside [0, {ell}]")
        uf = clamp_uniform(u_fin[b])
        if n < ell:
            res = np.maximum(pt[n] - pd[n], 0.0)
            mass = res.sum()
            law = res / mass if mass > 0 else pt[n]
            z = inverse_cdf(law, uf)
        else:
            bonus, _ = _probs(Lt[off + ell], V)
            law = bonus if bonus.sum() > 0 else None
            z = inverse_cdf(bonus, uf) if law is not None else -1
        laws[b] = law
        n_out[b] = n
        y_out[b, :n] = xs[:n]
        y_out[b, n] = z
    return dict(n=n_out, y=y_out, ratio=ratio, law=laws)
