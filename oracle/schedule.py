"""Hardware-aware prefix scheduler, fp64 oracle (test infrastructure only).

[P1] section "硬件感知与置信度自适应调度机制": confidences are calibrated by a per-position
temperature (order preserving); the candidate tokens of all requests are ranked by their
survival probability, added to the verify batch one by one, and the expected throughput
(expected accepted tokens times the engine speed at that batch size, profiled ahead of
time) decides where to cut; a strictly causal variant stops at the first drop, the global
variant searches the whole curve because a step-shaped speed curve traps early stopping.
[P3] "DSpark Speculative Decoding", section "Confidence-Scheduled Verification":
a_{r,j} = prod_{i<=j} c_{r,i} and the objective Theta = tau * SPS(B).

Readings: temperatures act on each conditional c_k as sigmoid(logit(c)/T_k) before the
product; tau counts the always-emitted correction / bonus token, tau = R + sum of the
selected a; B is the total number of verify tokens, R + n (each request feeds its last
token); the rank order is a descending, then position j ascending, then request r
ascending; GLOBAL takes the smallest n maximising Theta over n = 0 .. min(R*gamma, Bmax-R),
EARLY_STOP takes the first n with Theta(n+1) <= Theta(n).
"""
from __future__ import annotations

import itertools

import numpy as np

GLOBAL = 0
EARLY_STOP = 1


def temperature_scale(c, T=None) -> np.ndarray:
    """c' = 1 / (1 + ((1 - c)/c)^(1/T_k)) per position; c = 0 -> 0, c = 1 -> 1.

    Inputs outside the confidence range are clamped into [0, 1] (NaN counts as 0) and a
    temperature that is not positive counts as 1; T = None leaves c unscaled.
    """
    c = np.asarray(c, dtype=np.float32).astype(np.float64)
    R, G = c.shape
    Tk = None if T is None else np.asarray(T, dtype=np.float32).astype(np.float64)
    out = np.empty_like(c)
    for r in range(R):
        for k in range(G):
            ck = c[r, k]
            if not ck > 0.0:
                out[r, k] = 0.0
            elif ck >= 1.0:
                out[r, k] = 1.0
            elif Tk is None:
                out[r, k] = ck
            else:
                t = Tk[k] if Tk[k] > 0.0 else 1.0
                out[r, k] = 1.0 / (1.0 + ((1.0 - ck) / ck) ** (1.0 / t))
    return out


def prefix_survival(cp: np.ndarray) -> np.ndarray:
    """a_{r,j} = prod_{i<=j} c'_{r,i}, multiplied left to right."""
    R, G = cp.shape
    a = np.empty_like(cp)
    for r in range(R):
        acc = 1.0
        for j in range(G):
            acc *= cp[r, j]
            a[r, j] = acc
    return a


def _ranked(a: np.ndarray):
    R, G = a.shape
    cand = [(-a[r, j], j, r) for r in range(R) for j in range(G)]
    cand.sort()
    return cand


def theta_curve(a: np.ndarray, sps, Bmax: int):
    """Theta(n) for n = 0..nmax over the ranked candidates; also returns the ranking."""
    R, G = a.shape
    sps = np.asarray(sps, dtype=np.float32).astype(np.float64)
    nmax = min(R * G, Bmax - R)
    ranked = _ranked(a)
    theta = np.empty(nmax + 1)
    s = 0.0
    for n in range(nmax + 1):
        if n > 0:
            s += -ranked[n - 1][0]
        theta[n] = (R + s) * sps[R + n]
    return theta, ranked


def schedule(conf, temp, sps, Bmax: int, mode: int = GLOBAL) -> dict:
    """Verify lengths for R requests. Returns dict len [R], t_off [R+1], K, theta, n, a."""
    conf = np.asarray(conf)
    R, G = conf.shape
    if R > Bmax:
        raise ValueError("more requests than the engine's batch limit")
    a = prefix_survival(temperature_scale(conf, temp))
    theta, ranked = theta_curve(a, sps, Bmax)
    nmax = theta.shape[0] - 1
    if mode == GLOBAL:
        n_star = int(np.argmax(theta))              # first index of the maximum
    elif mode == EARLY_STOP:
        n_star = nmax
        for n in range(nmax):
            if theta[n + 1] <= theta[n]:
                n_star = n
                break
    else:
        raise ValueError(mode)
    length = np.zeros(R, dtype=np.int64)
    for _, j, r in ranked[:n_star]:
        length[r] += 1
    t_off = np.zeros(R + 1, dtype=np.int64)
    t_off[1:] = np.cumsum(length + 1)
    return dict(len=length, t_off=t_off, K=R + n_star, theta=float(theta[n_star]), n=n_star,
                a=a, theta_curve=theta, ranked=ranked)


def lagged_confidences(history, t: int, R: int, gamma: int) -> np.ndarray:
    """The confidences the scheduler of round t reads under the two-step lag.

    [P1] same section (the asynchronous adaptation): the verify length of step t is decided
    from the confidence predictions made at step t - 2, so the decision cannot depend on the
    tokens being generated now. [P3] same section: the batch capacity is predicted from the
    confidences of two steps earlier. history[i] is the [R][gamma] array recorded at round i.
    Reading: before two rounds have been recorded there is no history, and every position is
    taken to survive (all ones).
    """
    if t >= 2:
        return np.asarray(history[t - 2], dtype=np.float64)
    return np.ones((R, gamma))


def lagged_schedule(history, t: int, temp, sps, Bmax: int, mode: int = GLOBAL) -> dict:
    """The schedule of round t from the confidences recorded at round t - 2."""
    h0 = np.asarray(history[0])
    return schedule(lagged_confidences(history, t, h0.shape[0], h0.shape[1]), temp, sps, Bmax, mode)


def brute_force_schedule(conf, temp, sps, Bmax: int):
    """Maximum of Theta over every length vector l in {0..gamma}^R with R + sum(l) <= Bmax.

    Returns (best_theta, list of maximising length vectors). Exponential: tiny R, gamma only.
    """
    conf = np.asarray(conf)
    R, G = conf.shape
    a = prefix_survival(temperature_scale(conf, temp))
    sps = np.asarray(sps, dtype=np.float32).astype(np.float64)
    scored = []
    for ell in itertools.product(range(G + 1), repeat=R):
        tokens = R + sum(ell)
        if tokens > Bmax:
            continue
        tau = R + sum(a[r, :ell[r]].sum() for r in range(R))
        scored.append((tau * sps[tokens], ell))
    best = max(th for th, _ in scored)
    arg = [ell for th, ell in scored if abs(th - best) <= 1e-12 * max(abs(best), 1e-300)]
    return best, arg
