"""Parity checks of GPU results against the fp64 oracle (test infrastructure).

The oracle always runs on the seeded inputs only (never on a GPU result). Token decisions
must match exactly except at sampling ties: a draw whose uniform lies within TIE of a CDF
boundary of the oracle's own distribution, or an acceptance test with |u - min(1, p_t/p_d)|
below TIE. A request's positions after its first tie are not compared (both sides then
condition on different tokens), and the number of such ties is bounded by the caller.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle

TIE = 1e-5          # CDF / acceptance-ratio margin that counts as a tie
PROB_TOL = 1e-4     # absolute tolerance of probabilities, lse and c*


def dev(a: np.ndarray, device="cuda"):
    """numpy -> torch on the GPU; uint16 arrays are bf16 bit patterns."""
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def host(t) -> np.ndarray:
    return t.detach().cpu().numpy()


def is_cdf_tie(p: np.ndarray, u: float, g: int, tie: float = TIE) -> bool:
    """GPU token g is an acceptable inverse-CDF draw for u from law p within the margin."""
    if not (0 <= g < p.shape[0]) or p[g] <= 0:
        return False
    F = np.cumsum(p)
    lo = F[g - 1] if g > 0 else 0.0
    return lo - tie <= u < F[g] + tie


class DraftReport:
    def __init__(self):
        self.compared = 0
        self.ties = 0
        self.skipped = 0
        self.max_prob_err = 0.0
        self.max_lse_err = 0.0
        self.max_logit_err = 0.0


def check_draft(U, W1, W2, x0, u, w_dtype, gx, gq, glse, requests, gL=None, rep=None):
    """Compare GPU draft outputs (numpy) with the oracle request by request."""
    rep = rep or DraftReport()
    B, G, V = U.shape
    for b in requests:
        ref = oracle.markov_draft(U[b:b + 1], W1, W2, x0[b:b + 1], u[b:b + 1], w_dtype,
                                  want_logits=True)
        for k in range(G):
            o, g = int(ref["x"][0, k]), int(gx[b, k])
            if gL is not None and o >= 0:
                err = np.max(np.abs(gL[b, k].astype(np.float64) - ref["L"][0, k]))
                rep.max_logit_err = max(rep.max_logit_err, float(err))
                assert err < 5e-4, f"logits b={b} k={k} err={err}"
            if o == g:
                rep.compared += 1
                if o >= 0:
                    if gq is not None:
                        e = abs(float(gq[b, k]) - ref["q"][0, k])
                        rep.max_prob_err = max(rep.max_prob_err, e)
                        assert e < PROB_TOL, f"q b={b} k={k}: {gq[b, k]} vs {ref['q'][0, k]}"
                    if glse is not None:
                        e = abs(float(glse[b, k]) - ref["lse"][0, k])
                        rep.max_lse_err = max(rep.max_lse_err, e)
                        assert e < PROB_TOL * max(1.0, abs(ref["lse"][0, k])), \
                            f"lse b={b} k={k}: {glse[b, k]} vs {ref['lse'][0, k]}"
                continue
            p, _ = oracle.softmax_row(ref["L"][0, k])
            uu = oracle.clamp_uniform(u[b, k])
            assert is_cdf_tie(p, uu, g), (
                f"draft token mismatch b={b} k={k}: gpu {g} oracle {o} u={uu} "
                f"F(o-1..o)={np.cumsum(p)[max(o - 1, 0)]:.8f},{np.cumsum(p)[o]:.8f}")
            rep.ties += 1
            rep.skipped += G - k - 1
            break
    return rep


def oracle_final_law(Ld, Lt, b, off, n, ell):
    """The law the final token is drawn from, after n accepted of ell verified positions."""
    if n < ell:
        pd = oracle.softmax_row(Ld[b, n])
        pt = oracle.softmax_row(Lt[off + n])
        pd = pd[0] if pd is not None else np.zeros(Ld.shape[-1])
        pt = pt[0] if pt is not None else np.zeros(Ld.shape[-1])
        res = np.maximum(pt - pd, 0.0)
        return res / res.sum() if res.sum() > 0 else pt
    st = oracle.softmax_row(Lt[off + ell])
    return st[0] if st is not None else None


class VerifyReport:
    def __init__(self):
        self.compared = 0
        self.accept_ties = 0
        self.final_ties = 0


def check_verify(Ld, Lt, x, u_acc, u_fin, t_off, length, gn, gy, requests, rep=None):
    """Compare GPU verify outputs (numpy) with the oracle, request by request."""
    rep = rep or VerifyReport()
    B, G, V = Ld.shape
    for b in requests:
        ell = G if length is None else int(length[b])
        off = b * (G + 1) if t_off is None else int(t_off[b])
        ref = oracle.verify(Ld[b:b + 1], Lt, x[b:b + 1], u_acc[b:b + 1], u_fin[b:b + 1],
                            t_off=np.array([off, off + ell + 1]), length=np.array([ell]))
        on, g_n = int(ref["n"][0]), int(gn[b])
        if on != g_n:
            m = min(on, g_n)
            assert m >= 0, f"b={b}: n gpu {g_n} oracle {on}"
            pd = oracle.softmax_row(Ld[b, m])[0]
            pt = oracle.softmax_row(Lt[off + m])[0]
            xm = int(x[b, m])
            ratio = min(1.0, pt[xm] / pd[xm]) if pd[xm] > 0 else 1.0
            uu = oracle.clamp_uniform(u_acc[b, m])
            assert abs(uu - ratio) < TIE, f"b={b} k={m}: accept mismatch u={uu} ratio={ratio}"
            assert np.array_equal(gy[b, :m], ref["y"][0, :m])
            rep.accept_ties += 1
            continue
        rep.compared += 1
        if on < 0:
            assert np.all(gy[b] == -1)
            continue
        assert np.array_equal(gy[b, :on], ref["y"][0, :on]), f"b={b} accepted prefix"
        assert np.all(gy[b, on + 1:] == -1), f"b={b} padding"
        gz, oz = int(gy[b, on]), int(ref["y"][0, on])
        if gz != oz:
            law = oracle_final_law(Ld, Lt, b, off, on, ell)
            assert law is not None and is_cdf_tie(law, oracle.clamp_uniform(u_fin[b]), gz), (
                f"b={b}: final token gpu {gz} oracle {oz} (n={on}, len={ell})")
            rep.final_ties += 1
    return rep


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
    # lengths: the selected set must be a top-n set of the oracle's ranking up to ties
    a = ref["a"]
    sel = np.zeros((R, G), bool)
    for r in range(R):
        assert 0 <= glen[r] <= G
        sel[r, : glen[r]] = True
    if n_g == ref["n"] and not np.array_equal(glen, ref["len"]):
        ranked = ref["ranked"]
        cut_hi = -ranked[n_g - 1][0] if n_g > 0 else np.inf
        cut_lo = -ranked[n_g][0] if n_g < len(ranked) else -np.inf
        differ = sel != (np.arange(G)[None, :] < ref["len"][:, None])
        vals = a[differ]
        assert np.all(np.abs(vals - cut_hi) <= 1e-6 * cut_hi) or np.all(
            np.abs(vals - cut_lo) <= 1e-6 * max(cut_lo, 1e-300)), "length mismatch beyond ties"
    return ref
