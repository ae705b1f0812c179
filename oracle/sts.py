"""Sequential temperature scaling (STS) fit and expected calibration error, fp64 oracle.

TEST INFRASTRUCTURE ONLY (see the package header).

[P1] section "硬件感知与置信度自适应调度机制": the confidence head's raw scores are
over-confident; STS post-processes them with one temperature per candidate position, each
found independently by a one-dimensional grid search on validation data, which brings the
expected calibration error (ECE) down to about 1 %; temperature scaling keeps the order of
the scores. [P3] "DSpark Speculative Decoding", section "Confidence-Scheduled Verification":
c_k estimates P(position k accepted | its prefix accepted).

Readings taken here (the pages leave them open):
  * validation pairs come from verify: for request i with accepted count n_i and verify
    length len_i, positions k < n_i were accepted (outcome 1), position n_i was rejected
    (outcome 0) when n_i < len_i, and later positions were not observed (-1);
  * the calibrated score is c' = sigmoid(logit(c) / T) = 1 / (1 + ((1 - c)/c)^(1/T)), the
    scheduler's temperature scaling (c <= 0 or NaN -> 0, c >= 1 -> 1, T <= 0 counts as 1);
  * the grid search minimises either the binary negative log-likelihood of the observed
    outcomes (NLL, the usual temperature-scaling objective) or the ECE itself; ties go to
    the first grid value. Probabilities inside the log are floored at 1e-12;
  * ECE uses `bins` equal-width bins on [0, 1] (bin = min(floor(c' * bins), bins - 1)):
    sum over bins of (count / N) * |mean outcome - mean score| over the N observed pairs
    (0 when nothing was observed).
"""
from __future__ import annotations

import numpy as np

NLL = 0
ECE = 1
EPS = 1e-12


def outcomes(n_acc, length, gamma: int) -> np.ndarray:
    """[N][gamma] int: 1 accepted, 0 the first rejection, -1 not observed.

    A request with a negative accepted count (a faulty request) has no observations; a
    length of None means every request was verified over all gamma positions.
    """
    n_acc = np.asarray(n_acc).astype(np.int64)
    N = n_acc.shape[0]
    ln = np.full(N, gamma, np.int64) if length is None else np.asarray(length).astype(np.int64)
    out = np.full((N, gamma), -1, np.int64)
    for i in range(N):
        n, ell = int(n_acc[i]), int(ln[i])
        if n < 0 or ell < 0:
            continue
        for k in range(min(n, gamma)):
            out[i, k] = 1
        if n < ell and n < gamma:
            out[i, n] = 0
    return out


def scale(c, T: float) -> np.ndarray:
    """sigmoid(logit(c) / T) elementwise in fp64 (fp32 inputs widened exactly)."""
    c = np.asarray(c, dtype=np.float32).astype(np.float64)
    t = float(np.float32(T))
    if not t > 0.0:
        t = 1.0
    out = np.zeros_like(c)
    hi = c >= 1.0
    mid = (c > 0.0) & ~hi
    out[hi] = 1.0
    cm = c[mid]
    out[mid] = 1.0 / (1.0 + ((1.0 - cm) / cm) ** (1.0 / t))
    return out


def nll(cs: np.ndarray, o: np.ndarray) -> float:
    """Sum over observed pairs of -log p(outcome) under scores cs (fp64)."""
    obs = o >= 0
    p = np.where(o[obs] == 1, cs[obs], 1.0 - cs[obs])
    return float(-np.sum(np.log(np.maximum(p, EPS))))


def ece(cs: np.ndarray, o: np.ndarray, bins: int) -> float:
    """Expected calibration error of the observed pairs over equal-width bins."""
    obs = o >= 0
    c = cs[obs]
    y = o[obs].astype(np.float64)
    N = c.shape[0]
    if N == 0:
        return 0.0
    b = np.minimum(np.floor(c * bins).astype(np.int64), bins - 1)
    total = 0.0
    for m in range(bins):
        sel = b == m
        cnt = int(sel.sum())
        if cnt:
            total += cnt / N * abs(y[sel].mean() - c[sel].mean())
    return total


def sts_fit(conf, n_acc, length, grid, bins: int = 15, objective: int = NLL) -> dict:
    """Per-position temperature by grid search.

    conf [N][gamma] raw scores, n_acc [N] and length [N] (None: gamma) from verify, grid [nT]
    candidate temperatures. Returns dict T [gamma], idx [gamma], obj [gamma][nT] (the
    objective at every grid value), ece_before [gamma] (T = 1), ece_after [gamma].
    """
    conf = np.asarray(conf, dtype=np.float32)
    N, G = conf.shape
    grid = np.asarray(grid, dtype=np.float32)
    o = outcomes(n_acc, length, G)
    obj = np.empty((G, grid.shape[0]))
    idx = np.zeros(G, np.int64)
    for k in range(G):
        for t in range(grid.shape[0]):
            cs = scale(conf[:, k], grid[t])
            obj[k, t] = nll(cs, o[:, k]) if objective == NLL else ece(cs, o[:, k], bins)
        idx[k] = int(np.argmin(obj[k]))                 # first minimum
    T = grid[idx].astype(np.float64)
    before = np.array([ece(scale(conf[:, k], 1.0), o[:, k], bins) for k in range(G)])
    after = np.array([ece(scale(conf[:, k], T[k]), o[:, k], bins) for k in range(G)])
    return dict(T=T, idx=idx, obj=obj, ece_before=before, ece_after=after, outcomes=o)
