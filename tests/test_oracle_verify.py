"""Pins of the oracle's rejection-sampling verifier.

Closed forms come from rational rows (logits = log of integer weights) whose laws are
exact; losslessness is checked by chi-squared tests of the emitted tokens against the
target law, which holds for the speculative-sampling rule and fails for plausible
mistakes (one is planted below to show the test has power).
"""
import importlib

import numpy as np
import pytest
import scipy.stats

import oracle
import synth

oracle_verify = importlib.import_module("oracle.verify")


def _rows_from_weights(w):
    w = np.asarray(w, dtype=np.float64)
    with np.errstate(divide="ignore"):
        return np.log(w).astype(np.float32)


def test_identical_laws_accept_everything():
    c = synth.custom(910, B=5, V=64, r=4, gamma=6, w_dtype="f32")
    g = np.random.default_rng(1)
    Ld = np.stack([synth.base_rows(c, b)[: c.gamma] for b in range(c.B)])
    bonus_w = g.integers(1, 9, size=(c.B, c.V))
    Lt = np.concatenate([np.concatenate([Ld[b], _rows_from_weights(bonus_w[b])[None]])
                         for b in range(c.B)])
    x = g.integers(0, c.V, size=(c.B, c.gamma))
    u_acc = synth.uniforms(g, (c.B, c.gamma))
    cells = np.array([g.integers(0, bonus_w[b].sum()) for b in range(c.B)])
    u_fin = np.array([(cells[b] + 0.5) / bonus_w[b].sum() for b in range(c.B)], np.float32)
    out = oracle.verify(Ld, Lt, x, u_acc, u_fin)
    for b in range(c.B):
        assert out["n"][b] == c.gamma
        assert np.array_equal(out["y"][b, : c.gamma], x[b])
        z = int(np.searchsorted(np.cumsum(bonus_w[b]), cells[b], side="right"))
        assert out["y"][b, c.gamma] == z


def test_zero_target_mass_rejects_and_residual_is_exact():
    # p_d = (1/2, 1/4, 1/8, 1/8), p_t = (0, 1/2, 1/4, 1/4); draft token 0 has p_t = 0.
    Ld = _rows_from_weights([[4, 2, 1, 1]])[None]
    Lt = np.concatenate([_rows_from_weights([[0, 2, 1, 1]]), _rows_from_weights([[1, 1, 1, 1]])])
    # residual max(0, p_t - p_d) = (0, 1/4, 1/8, 1/8) -> normalised (0, 1/2, 1/4, 1/4)
    for u_fin, z in [(0.1, 1), (0.49, 1), (0.6, 2), (0.74, 2), (0.8, 3), (0.999, 3)]:
        out = oracle.verify(Ld, Lt, np.array([[0]]), np.array([[0.0]], np.float32),
                            np.array([u_fin], np.float32))
        assert out["n"][0] == 0
        assert list(out["y"][0]) == [z, -1]


def test_accept_test_boundaries():
    # ratio p_t/p_d = 0.5: accept iff u < 0.5
    Ld = _rows_from_weights([[2, 1, 1]])[None]          # p_d(0) = 1/2
    Lt = np.concatenate([_rows_from_weights([[1, 1, 2]]), _rows_from_weights([[1, 0, 0]])])  # p_t(0) = 1/4
    for u, n in [(0.49, 1), (0.51, 0)]:
        out = oracle.verify(Ld, Lt, np.array([[0]]), np.array([[u]], np.float32),
                            np.array([0.3], np.float32))
        assert out["n"][0] == n
    # accepted -> bonus from row 2, which is a point mass on token 0
    out = oracle.verify(Ld, Lt, np.array([[0]]), np.array([[0.2]], np.float32),
                        np.array([0.9], np.float32))
    assert list(out["y"][0]) == [0, 0]


def test_zero_length_samples_first_target_row():
    w = np.array([3, 1, 4, 1, 5, 9, 2, 6])
    Ld = np.zeros((1, 3, 8), np.float32)
    Lt = _rows_from_weights(w)[None]
    for cell in range(w.sum()):
        u = np.float32((cell + 0.5) / w.sum())
        out = oracle.verify(Ld, Lt, np.zeros((1, 3), np.int64), np.zeros((1, 3), np.float32),
                            np.array([u]), t_off=np.array([0, 1]), length=np.array([0]))
        assert out["n"][0] == 0
        assert out["y"][0, 0] == np.searchsorted(np.cumsum(w), cell, side="right")
        assert list(out["y"][0, 1:]) == [-1, -1, -1]


def test_flattened_layout_matches_padded():
    c = synth.custom(911, B=6, V=96, r=4, gamma=5, w_dtype="f32", tnoise=0.7)
    g = np.random.default_rng(2)
    Ld = np.stack([synth.base_rows(c, b)[: c.gamma] for b in range(c.B)])
    Lt_pad = np.stack([synth.target_rows(c, b) for b in range(c.B)])
    length = np.array([0, 5, 2, 3, 1, 4])
    t_off = np.zeros(c.B + 1, np.int64)
    t_off[1:] = np.cumsum(length + 1)
    Lt_flat = np.concatenate([Lt_pad[b, : length[b] + 1] for b in range(c.B)])
    x = g.integers(0, c.V, size=(c.B, c.gamma))
    u_acc, u_fin = synth.uniforms(g, (c.B, c.gamma)), synth.uniforms(g, (c.B,))
    a = oracle.verify(Ld, Lt_pad.reshape(-1, c.V), x, u_acc, u_fin, length=length)
    b = oracle.verify(Ld, Lt_flat, x, u_acc, u_fin, t_off=t_off, length=length)
    assert np.array_equal(a["n"], b["n"]) and np.array_equal(a["y"], b["y"])
    assert np.all(a["n"] <= length)


def test_bad_draft_token_sentinel():
    Ld = np.zeros((2, 2, 4), np.float32)
    Lt = np.zeros((6, 4), np.float32)
    out = oracle.verify(Ld, Lt, np.array([[0, 9], [1, 2]]), np.zeros((2, 2), np.float32),
                        np.zeros(2, np.float32))
    assert out["n"][0] == -1 and list(out["y"][0]) == [-1, -1, -1]
    assert out["n"][1] == 2


# ---------------------------------------------------------------- losslessness
def _markov_tables(V, seed):
    g = np.random.default_rng(seed)
    P = g.integers(1, 12, size=(V, V)).astype(np.float64)
    P[g.random((V, V)) < 0.2] = 0.0                # some impossible target transitions
    P[np.arange(V), g.integers(0, V, V)] += 1.0    # keep every row non-empty
    P /= P.sum(1, keepdims=True)
    Q = g.integers(1, 12, size=(V, V)).astype(np.float64)
    Q /= Q.sum(1, keepdims=True)
    return P, Q


def _draft_markov(Q, x0, u):
    """Draft with the oracle's Markov head: W1 = identity, W2 = log Q, U = 0."""
    V = Q.shape[0]
    N, G = u.shape
    out = oracle.markov_draft(np.zeros((N, G, V), np.float32), np.eye(V, dtype=np.float32),
                              np.log(Q).astype(np.float32), x0, u)
    return out["x"], np.log(Q).astype(np.float32)


def _one_round(P, Q, prev, G, seed):
    """One draft + verify round from context tokens prev; returns emitted tokens per request."""
    V = P.shape[0]
    N = prev.shape[0]
    gu = np.random.default_rng(seed)
    x, logQ = _draft_markov(Q, prev, synth.uniforms(gu, (N, G)))
    Ld = np.empty((N, G, V), np.float32)
    Lt = np.empty((N * (G + 1), V), np.float32)
    logP = _rows_from_weights(P)
    ctx = np.concatenate([prev[:, None], x], axis=1)      # token before each position
    for k in range(G):
        Ld[:, k] = logQ[ctx[:, k]]
    for k in range(G + 1):
        Lt[np.arange(N) * (G + 1) + k] = logP[ctx[:, k]]
    u_acc, u_fin = synth.uniforms(gu, (N, G)), synth.uniforms(gu, (N,))
    res = oracle.verify(Ld, Lt, x, u_acc, u_fin)
    return [list(res["y"][i, : res["n"][i] + 1]) for i in range(N)]


def _chi2_pvalue(counts, probs, N):
    expected = N * probs
    keep = expected >= 5
    obs = np.append(counts[keep], counts[~keep].sum())
    exp = np.append(expected[keep], expected[~keep].sum())
    if exp[-1] == 0:
        obs, exp = obs[:-1], exp[:-1]
    return scipy.stats.chisquare(obs, exp).pvalue


def _first_token_law_pvalue(N=30000, G=1, seed=0):
    V = 8
    P, Q = _markov_tables(V, 123)
    prev = np.full(N, 3)
    ys = _one_round(P, Q, prev, G, seed)
    first = np.array([y[0] for y in ys])
    return _chi2_pvalue(np.bincount(first, minlength=V).astype(float), P[3], N)


def test_lossless_single_position():
    assert _first_token_law_pvalue() > 1e-3


def test_lossless_test_has_power(monkeypatch):
    """Planted mistake: accept with u < p_t(x), ignoring p_d. The law of the first emitted
    token then differs from the target's and the chi-squared test must reject it."""
    monkeypatch.setattr(oracle_verify, "accept_test", lambda u, pd, pt: u < pt)
    assert _first_token_law_pvalue() < 1e-3


@pytest.mark.slow
def test_lossless_multi_round_joint():
    """First three emitted tokens over repeated rounds follow the target chain's joint law."""
    V, G, N = 8, 3, 20000
    P, Q = _markov_tables(V, 321)
    x0 = 5
    seqs = [[] for _ in range(N)]
    prev = np.full(N, x0)
    active = np.arange(N)
    rnd = 0
    while active.size:
        ys = _one_round(P, Q, prev[active], G, seed=1000 + rnd)
        for i, y in zip(active, ys):
            seqs[i].extend(y)
        prev[active] = [seqs[i][-1] for i in active]
        active = np.array([i for i in active if len(seqs[i]) < 3], dtype=np.int64)
        rnd += 1
    idx = np.array([s[0] * V * V + s[1] * V + s[2] for s in seqs])
    counts = np.bincount(idx, minlength=V ** 3).astype(float)
    joint = (P[x0][:, None, None] * P[:, :, None] * P[None, :, :]).reshape(-1)
    assert _chi2_pvalue(counts, joint, N) > 1e-3


def test_accept_rate_matches_tv_label():
    """Monte-Carlo acceptance at position 1 equals c*_1 = sum_v min(p_d, p_t)."""
    V, N = 6, 40000
    wd = np.array([5, 1, 3, 2, 6, 3])
    wt = np.array([1, 4, 3, 0, 6, 2])
    Ld1 = _rows_from_weights(wd)
    x, _ = _draft_markov(np.broadcast_to(wd / wd.sum(), (V, V)).copy(), np.zeros(N, np.int64),
                         synth.uniforms(synth.rng(912, 0), (N, 1)))
    Ld = np.broadcast_to(Ld1, (N, 1, V))
    Lt = np.tile(np.stack([_rows_from_weights(wt), Ld1]), (N, 1))
    u_acc, u_fin = synth.uniforms(synth.rng(912, 1), (N, 1)), synth.uniforms(synth.rng(912, 2), (N,))
    res = oracle.verify(Ld, Lt, x, u_acc, u_fin)
    rate = (res["n"] == 1).mean()
    cstar = oracle.tv_labels(Ld[:1], Lt[:2])[0, 0]
    exact = np.minimum(wd / wd.sum(), wt / wt.sum()).sum()
    assert cstar == pytest.approx(exact, abs=1e-6)      # fp32 logits of exact weights
    assert abs(rate - exact) < 4 * np.sqrt(exact * (1 - exact) / N)
