"""CPU checks of the parity harness itself: it passes the oracle's own results, counts a
decision within the tie margin as a tie and keeps comparing after it (teacher forcing), and
fails on planted mistakes (a wrong token, a wrong accepted count, a wrong final token, a
wrong probability)."""
import numpy as np
import pytest

import oracle
import synth
from parity import TIE, Report, check_draft, check_verify, cdf_margin


def _tiny():
    c = synth.config(synth.TINY)
    d = synth.draft_inputs(c)
    ref = oracle.markov_draft(d["U"], d["W1"], d["W2"], d["x0"], d["u"], want_logits=True)
    return c, d, ref


def test_draft_harness_passes_the_oracle_itself():
    c, d, ref = _tiny()
    rep = check_draft(d["U"], d["W1"], d["W2"], d["x0"], d["u"], "f32", ref["x"],
                      ref["q"].astype(np.float32), ref["lse"].astype(np.float32), range(c.B),
                      gL=ref["L"].astype(np.float32))
    assert rep.compared == c.B * c.gamma and rep.ties == 0


def test_draft_harness_rejects_a_wrong_token_and_a_wrong_probability():
    c, d, ref = _tiny()
    x = ref["x"].copy()
    x[1, 2] = (x[1, 2] + 1) % c.V
    with pytest.raises(AssertionError):
        check_draft(d["U"], d["W1"], d["W2"], d["x0"], d["u"], "f32", x, None, None, range(c.B))
    q = ref["q"].astype(np.float32).copy()
    q[2, 1] += 3e-4
    with pytest.raises(AssertionError):
        check_draft(d["U"], d["W1"], d["W2"], d["x0"], d["u"], "f32", ref["x"], q, None,
                    range(c.B))
    lse = ref["lse"].astype(np.float32).copy()
    lse[0, 0] += 2e-4                       # absolute, not relative to |lse|
    with pytest.raises(AssertionError):
        check_draft(d["U"], d["W1"], d["W2"], d["x0"], d["u"], "f32", ref["x"], None, lse,
                    range(c.B))


def test_draft_harness_teacher_forces_after_a_tie():
    """Place u within TIE/2 above a cell boundary and take the token left of it: a tie. The
    positions after it are still compared, on the tied token's prefix."""
    c, d, ref = _tiny()
    b, k = 2, 1
    p, _ = oracle.softmax_row(ref["L"][b, k])
    F = np.cumsum(p)
    o = int(ref["x"][b, k])
    assert o > 0
    u = d["u"].copy()
    u[b, k] = np.float32(F[o - 1] + TIE / 4)
    if not (F[o - 1] <= float(u[b, k]) < F[o]):
        pytest.skip("fp32 rounding moved the uniform out of the cell")
    plain = oracle.markov_draft(d["U"], d["W1"], d["W2"], d["x0"], u)
    gx = plain["x"].copy()
    gx[b, k] = o - 1                        # the neighbouring cell: within the margin
    # the GPU's later positions follow its own prefix
    forced = oracle.markov_draft(d["U"], d["W1"], d["W2"], d["x0"], u, forced=gx)
    gx[b, k + 1:] = forced["x"][b, k + 1:]
    rep = check_draft(d["U"], d["W1"], d["W2"], d["x0"], u, "f32", gx, None, None, range(c.B))
    assert rep.ties == 1 and rep.compared == c.B * c.gamma
    # a token two cells away is no tie
    gx2 = gx.copy()
    gx2[b, k] = o + 1 if o + 1 < c.V else o - 2
    with pytest.raises(AssertionError):
        check_draft(d["U"], d["W1"], d["W2"], d["x0"], u, "f32", gx2, None, None, range(c.B))


def test_cdf_margin_signs():
    p = np.array([0.25, 0.25, 0.5, 0.0])
    assert cdf_margin(p, 0.3, 1) == pytest.approx(0.05)
    assert cdf_margin(p, 0.3, 0) == pytest.approx(-0.05)
    assert cdf_margin(p, 0.999, 2) > 0           # the last positive token owns the tail
    assert cdf_margin(p, 0.5, 3) == -np.inf      # a zero-mass token is never a draw


def _verify_case():
    c = synth.custom(950, B=6, V=300, r=1, gamma=5, w_dtype="f32", tnoise=0.8)
    Ld = synth.draft_logits_all(c).astype(np.float64)
    Lt = synth.target_padded_all(c).reshape(-1, c.V).astype(np.float64)
    ux = synth.token_uniforms(c)
    x = np.array([[oracle.inverse_cdf(oracle.softmax_row(Ld[b, k])[0], oracle.clamp_uniform(ux[b, k]))
                   for k in range(c.gamma)] for b in range(c.B)], np.int32)
    u_acc, u_fin = synth.verify_uniforms(c)
    ref = oracle.verify(Ld, Lt, x, u_acc, u_fin)
    return c, Ld, Lt, x, u_acc, u_fin, ref


def test_verify_harness_passes_the_oracle_and_catches_mistakes():
    c, Ld, Lt, x, u_acc, u_fin, ref = _verify_case()
    rep = check_verify(Ld, Lt, x, u_acc, u_fin, None, None, ref["n"], ref["y"], range(c.B),
                       rep=Report("harness"))
    assert rep.ties == 0 and rep.requests == c.B
    # a wrong accepted count (far from a tie) fails
    b = int(np.argmax(ref["n"] < c.gamma))
    n = ref["n"].copy()
    n[b] += 1
    y = oracle.verify(Ld, Lt, x, u_acc, u_fin, n_forced=n)["y"]
    ratio = ref["ratio"][b, ref["n"][b]]
    if abs(oracle.clamp_uniform(u_acc[b, ref["n"][b]]) - ratio) > TIE:
        with pytest.raises(AssertionError):
            check_verify(Ld, Lt, x, u_acc, u_fin, None, None, n, y, range(c.B))
    # a wrong final token fails; wrong padding fails
    y2 = ref["y"].copy()
    y2[0, ref["n"][0]] = (y2[0, ref["n"][0]] + 7) % c.V
    with pytest.raises(AssertionError):
        check_verify(Ld, Lt, x, u_acc, u_fin, None, None, ref["n"], y2, range(c.B))
    y3 = ref["y"].copy()
    if ref["n"][0] < c.gamma:
        y3[0, c.gamma] = 3
        with pytest.raises(AssertionError):
            check_verify(Ld, Lt, x, u_acc, u_fin, None, None, ref["n"], y3, range(c.B))


def test_verify_harness_teacher_forces_an_accept_tie():
    """Set an acceptance uniform just below the oracle's ratio (an accept) and let the 'GPU'
    reject there: a tie, after which the final draw is checked at the GPU's count."""
    c, Ld, Lt, x, u_acc, u_fin, ref = _verify_case()
    k = 0
    cand = [b for b in range(c.B) if ref["ratio"][b, k] < 0.999]
    assert cand, "no request with a first-position ratio below 1"
    b = cand[0]
    r = ref["ratio"][b, k]
    u2 = u_acc.copy()
    u2[b, k] = np.float32(r - TIE / 4)
    assert r - TIE < float(u2[b, k]) < r
    n = oracle.verify(Ld, Lt, x, u2, u_fin)["n"].copy()
    n[b] = 0                                  # the GPU rejects at the tie
    y = oracle.verify(Ld, Lt, x, u2, u_fin, n_forced=n)["y"]
    rep = check_verify(Ld, Lt, x, u2, u_fin, None, None, n, y, range(c.B))
    assert rep.accept_ties == 1
