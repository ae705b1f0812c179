"""Parity checks of GPU results against the fp64 oracle (test infrastructure).

The oracle always runs on the seeded inputs (never on a GPU result's numbers). Every
decision the GPU made is checked on the GPU's own path (teacher forcing), so a sampling tie
never hides the positions after it:

* draft: position k's law is the oracle's law given the GPU's tokens before k
  (``oracle.markov_draft(..., forced=gpu tokens)``); the GPU token must be the oracle's
  inverse-CDF draw for the same uniform, or lie within TIE of a boundary of that draw's cell
  (a tie);
* verify: at each position the GPU accepted, the acceptance uniform must lie below the
  oracle's ratio min(1, p_t/p_d) (or within TIE of it); at the position it rejected, at or
  above it (or within TIE); the final token must be the oracle's draw from the residual or
  bonus law at the GPU's accepted count (``oracle.verify(..., n_forced=...)``), or a CDF tie.

Probabilities, lse and c* are compared to PROB_TOL absolute. Each check returns a report of
what it compared, its ties and a histogram of decision margins (the distance of the uniform to
the nearest boundary of the decision, in the oracle's fp64 arithmetic); ``record`` appends it
as a JSON line to the file named by DSPARK_PARITY_REPORT when that is set.
"""
from __future__ import annotations

import json
import os

import numpy as np
import torch

import oracle

TIE = 1e-5          # CDF / acceptance-ratio margin that counts as a tie
PROB_TOL = 1e-4     # absolute tolerance of probabilities, lse and c*
LOGIT_TOL = 5e-4    # absolute tolerance of logits (fp32 sums of bf16 products and fp32 U)

# decade edges of the margin histogram: [0, 1e-9), [1e-9, 1e-8), ..., [1e-3, 1e-2), [1e-2, inf)
MARGIN_EDGES = [0.0] + [10.0 ** e for e in range(-9, -1)] + [np.inf]


def dev(a: np.ndarray, device="cuda"):
    """numpy -> torch on the GPU; uint16 arrays are bf16 bit patterns."""
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def host(t) -> np.ndarray:
    return t.detach().cpu().numpy()


def tie_bound(rep) -> int:
    """Largest number of ties a check accepts: 2 plus 5 % of its decisions. At V ~ 1.5e5 the
    tail cells of a peaked law are a few 1e-6 wide, so fp32 rounding of the CDF (about 1e-7)
    moves a few per cent of the draws across a boundary; every tie is still asserted to lie
    within TIE of the oracle's cell."""
    return 2 + rep.compared // 20


def cdf_margin(p: np.ndarray, u: float, g: int) -> float:
    """Signed distance of u to the cell of token g under law p: >= 0 when u lies in
    [F(g-1), F(g)) (the distance to the nearer edge), < 0 outside (minus the distance to it)."""
    if not (0 <= g < p.shape[0]) or p[g] <= 0:
        return -np.inf
    F = np.cumsum(p)
    lo = F[g - 1] if g > 0 else 0.0
    hi = F[g]
    if g == p.shape[0] - 1 or not np.any(p[g + 1:] > 0):
        hi = np.inf                   # the last positive token also owns u past the final F
    if lo <= u < hi:
        return float(min(u - lo, hi - u))
    return float(-(lo - u) if u < lo else -(u - hi))


def is_cdf_tie(p: np.ndarray, u: float, g: int, tie: float = TIE) -> bool:
    """GPU token g is an acceptable inverse-CDF draw for u from law p within the margin."""
    return cdf_margin(p, u, g) > -tie


class Report:
    """What a check compared: decisions, ties, margins and the largest value errors."""

    def __init__(self, name: str = ""):
        self.name = name
        self.compared = 0            # decisions compared (draws, accept tests, final draws)
        self.ties = 0                # decisions that differ from the oracle's, within TIE
        self.accept_ties = 0
        self.final_ties = 0
        self.requests = 0
        self.hist = np.zeros(len(MARGIN_EDGES) - 1, dtype=np.int64)
        self.max_prob_err = 0.0
        self.max_lse_err = 0.0
        self.max_logit_err = 0.0
        self.max_cstar_err = 0.0

    # back-compatible name used by older assertions
    @property
    def skipped(self) -> int:
        return 0

    def margin(self, m: float):
        m = abs(m)
        i = int(np.searchsorted(MARGIN_EDGES, m, side="right")) - 1
        self.hist[min(max(i, 0), len(self.hist) - 1)] += 1

    def as_dict(self) -> dict:
        return dict(name=self.name, requests=self.requests, compared=self.compared,
                    ties=self.ties, accept_ties=self.accept_ties, final_ties=self.final_ties,
                    tie_rate=self.ties / max(self.compared, 1),
                    margin_hist={f"<{MARGIN_EDGES[i + 1]:.0e}": int(c)
                                 for i, c in enumerate(self.hist)},
                    max_prob_err=self.max_prob_err, max_lse_err=self.max_lse_err,
                    max_logit_err=self.max_logit_err, max_cstar_err=self.max_cstar_err)

    def record(self):
        d = self.as_dict()
        print("parity", json.dumps(d))
        path = os.environ.get("DSPARK_PARITY_REPORT")
        if path:
            with open(path, "a") as f:
                f.write(json.dumps(d) + "\n")
        return d


# backward-compatible names
DraftReport = Report
VerifyReport = Report


def check_draft(U, W1, W2, x0, u, w_dtype, gx, gq, glse, requests, gL=None, rep=None,
                group: int = 8, keep_logits=None, oracle_fn=None):
    """Compare GPU draft outputs (numpy) with the oracle on the GPU's own prefix.

    Every position of every listed request is compared: the oracle evaluates position k's
    law given the GPU's tokens before it. Returns the report. ``keep_logits`` (a dict) receives
    the oracle's fp64 logits [1][gamma][V] of each request along the GPU's block, by b.
    ``oracle_fn(U, W1, W2, x0, u, w_dtype, forced)`` replaces the Markov draft (e.g. the RNN
    head's oracle with its recurrence bound); it returns the oracle's dict with logits."""
    rep = rep or Report("draft")
    B, G, V = U.shape
    reqs = list(requests)
    for i in range(0, len(reqs), group):
        bs = reqs[i:i + group]
        if oracle_fn is None:
            ref = oracle.markov_draft(U[bs], W1, W2, x0[bs], u[bs], w_dtype, want_logits=True,
                                      forced=gx[bs])
        else:
            ref = oracle_fn(U[bs], W1, W2, x0[bs], u[bs], w_dtype, gx[bs])
        for j, b in enumerate(bs):
            rep.requests += 1
            if keep_logits is not None:
                keep_logits[b] = ref["L"][j:j + 1]
            for k in range(G):
                o, g = int(ref["x"][j, k]), int(gx[b, k])
                if o < 0:
                    assert g == -1, f"b={b} k={k}: oracle gives no token, gpu {g}"
                    rep.compared += 1
                    continue
                if gL is not None:
                    err = float(np.max(np.abs(gL[b, k].astype(np.float64) - ref["L"][j, k])))
                    rep.max_logit_err = max(rep.max_logit_err, err)
                    assert err < LOGIT_TOL, f"logits b={b} k={k} err={err}"
                p, _ = oracle.softmax_row(ref["L"][j, k])
                uu = oracle.clamp_uniform(u[b, k])
                m = cdf_margin(p, uu, g)
                rep.compared += 1
                rep.margin(m)
                if o != g:
                    F = np.cumsum(p)
                    assert m > -TIE, (
                        f"draft token mismatch b={b} k={k}: gpu {g} oracle {o} u={uu} "
                        f"F(o-1..o)={F[max(o - 1, 0)]:.8f},{F[o]:.8f} margin {m:.3e}")
                    rep.ties += 1
                if gq is not None:
                    e = abs(float(gq[b, k]) - p[g])
                    rep.max_prob_err = max(rep.max_prob_err, e)
                    assert e < PROB_TOL, f"q b={b} k={k}: {gq[b, k]} vs {p[g]}"
                if glse is not None:
                    e = abs(float(glse[b, k]) - ref["lse"][j, k])
                    rep.max_lse_err = max(rep.max_lse_err, e)
                    assert e < PROB_TOL, f"lse b={b} k={k}: {glse[b, k]} vs {ref['lse'][j, k]}"
    return rep


def forced_draft_logits(U, W1, W2, x0, u, w_dtype, gx, b):
    """The oracle's fp64 draft logits [1][gamma][V] of request b along the GPU's block."""
    ref = oracle.markov_draft(U[b:b + 1], W1, W2, x0[b:b + 1], u[b:b + 1], w_dtype,
                              want_logits=True, forced=gx[b:b + 1])
    return ref["L"]


def check_verify(Ld, Lt, x, u_acc, u_fin, t_off, length, gn, gy, requests, rep=None):
    """Compare GPU verify outputs (numpy) with the oracle on the GPU's acceptance path.

    Ld [B][gamma][V] are the draft logits both sides verify (the oracle's own, fp64, when
    they come from a draft); gn, gy the GPU's accepted counts and emitted tokens."""
    rep = rep or Report("verify")
    B, G, V = Ld.shape
    for b in requests:
        rep.requests += 1
        ell = G if length is None else int(length[b])
        off = b * (G + 1) if t_off is None else int(t_off[b])
        g_n = int(gn[b])
        args = (Ld[b:b + 1], Lt, x[b:b + 1], u_acc[b:b + 1], u_fin[b:b + 1])
        kw = dict(t_off=np.array([off, off + ell + 1]), length=np.array([ell]))
        assert -1 <= g_n <= ell, f"b={b}: n gpu {g_n} outside [-1, {ell}]"
        ref = oracle.verify(*args, **kw, n_forced=np.array([max(g_n, 0)]))
        if int(ref["n"][0]) < 0 or g_n < 0:     # an invalid draft token: the -1 sentinel
            assert int(ref["n"][0]) == g_n, f"b={b}: n gpu {g_n} oracle {int(ref['n'][0])}"
            assert np.all(gy[b] == -1)
            rep.compared += 1
            continue
        ratio = ref["ratio"][0]
        # acceptance decisions along the GPU's path: accepted below n, rejected at n
        for k in range(min(g_n + 1, ell)):
            uu = oracle.clamp_uniform(u_acc[b, k])
            m = ratio[k] - uu                 # > 0: the oracle accepts
            rep.compared += 1
            rep.margin(m)
            gpu_accepts = k < g_n
            if (m > 0) != gpu_accepts:
                assert abs(m) < TIE, (f"b={b} k={k}: gpu {'accepts' if gpu_accepts else 'rejects'}"
                                      f" u={uu} ratio={ratio[k]}")
                rep.ties += 1
                rep.accept_ties += 1
        assert np.array_equal(gy[b, :g_n], x[b, :g_n]), f"b={b} accepted prefix"
        assert np.all(gy[b, g_n + 1:] == -1), f"b={b} padding"
        gz, oz = int(gy[b, g_n]), int(ref["y"][0, g_n])
        law = ref["law"][0]
        rep.compared += 1
        if law is None:
            assert gz == -1, f"b={b}: no law to draw from, gpu {gz}"
            continue
        m = cdf_margin(law, oracle.clamp_uniform(u_fin[b]), gz)
        rep.margin(m)
        if gz != oz:
            assert m > -TIE, f"b={b}: final token gpu {gz} oracle {oz} (n={g_n}, len={ell})"
            rep.ties += 1
            rep.final_ties += 1
    return rep


def check_cstar(Ld, Lt, t_off, length, gc, requests, rep=None, tol=PROB_TOL):
    """c* of the listed requests against the oracle's labels (NaN pattern exact)."""
    B, G, V = Ld.shape
    for b in requests:
        ell = G if length is None else int(length[b])
        off = b * (G + 1) if t_off is None else int(t_off[b])
        ref = oracle.tv_labels(Ld[b:b + 1], Lt, t_off=np.array([off, off + ell + 1]),
                               length=np.array([ell]))[0]
        fin = np.isfinite(ref)
        assert np.array_equal(fin, np.isfinite(gc[b])), f"b={b} NaN pattern"
        err = float(np.max(np.abs(gc[b][fin] - ref[fin]))) if fin.any() else 0.0
        if rep is not None:
            rep.max_cstar_err = max(rep.max_cstar_err, err)
        assert err < tol, f"b={b} c* err {err}"


def check_schedule(conf, temp, sps, Bmax, mode, glen, gK, gtheta, ga=None):
    """Compare GPU schedule outputs with the oracle; ties at the cut are allowed."""
    ref = oracle.schedule(conf, temp, sps, Bmax, mode)
    R, G = conf.shape
    if ga is not None:
        np.testing.assert_allclose(ga.astype(np.float64), ref["a"], rtol=1e-6, atol=1e-7)
    curve = ref["theta_curve"]
    n_g = int(gK) - R
    assert int(glen.sum()) == n_g, "K must equal R + sum(len)"
    assert 0 <= n_g < curve.shape[0]
    if n_g != ref["n"]:
        if mode == oracle.GLOBAL:
            assert curve[n_g] >= (1 - 1e-6) * curve[ref["n"]], "GPU n is not a near-argmax"
        else:
            lo = min(n_g, ref["n"])
            assert abs(curve[lo + 1] - curve[lo]) <= 1e-6 * abs(curve[lo]), "early-stop tie"
    assert abs(float(gtheta) - curve[n_g]) <= 1e-5 * max(1.0, abs(curve[n_g]))
    # lengths: prefix-closed by construction; the selected set must be a top-n_g set of the
    # oracle's a-values (every selected a at least every unselected a, up to 1e-6 relative),
    # whether or not n_g equals the oracle's n
    a = ref["a"]
    sel = np.zeros((R, G), bool)
    for r in range(R):
        assert 0 <= glen[r] <= G
        sel[r, : glen[r]] = True
    if sel.any() and (~sel).any():
        lo_sel, hi_uns = a[sel].min(), a[~sel].max()
        assert lo_sel >= hi_uns - 1e-6 * max(hi_uns, 1e-300), (
            f"lengths are not a top-{n_g} set: min selected {lo_sel} < max unselected {hi_uns}")
    if n_g == ref["n"] and not np.array_equal(glen, ref["len"]):
        ranked = ref["ranked"]
        cut_hi = -ranked[n_g - 1][0] if n_g > 0 else np.inf
        cut_lo = -ranked[n_g][0] if n_g < len(ranked) else -np.inf
        differ = sel != (np.arange(G)[None, :] < ref["len"][:, None])
        vals = a[differ]
        assert np.all(np.abs(vals - cut_hi) <= 1e-6 * cut_hi) or np.all(
            np.abs(vals - cut_lo) <= 1e-6 * max(cut_lo, 1e-300)), "length mismatch beyond ties"
    return ref
