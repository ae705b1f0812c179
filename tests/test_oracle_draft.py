"""Pins of the oracle's Markov-head draft against values fixed by construction.

Each test builds inputs whose answer is known without the softmax the oracle uses:
rational weight rows (U = log w) have the exact law w / sum(w), so the inverse-CDF
token for a uniform placed inside an integer cell is known by integer arithmetic.
"""
import numpy as np
import pytest
import scipy.special
import scipy.stats

import oracle
import synth


def _int_cell_token(w, c):
    """Token whose integer CDF cell [W(v-1), W(v)) contains integer c."""
    cw = np.cumsum(w)
    return int(np.searchsorted(cw, c, side="right"))


def _midpoint_uniform(w, c):
    return np.float32((c + 0.5) / float(np.sum(w)))


def test_rational_rows_integer_cdf():
    g = np.random.default_rng(11)
    B, G, V, r = 3, 5, 12, 4
    w = g.integers(1, 50, size=(B, G, V))
    U = np.log(w).astype(np.float32)
    W1 = np.zeros((V, r), np.float32)
    W2 = g.standard_normal((r, V)).astype(np.float32)   # irrelevant: W1 = 0
    cells = g.integers(0, w.sum(-1))
    u = np.empty((B, G), np.float32)
    for b in range(B):
        for k in range(G):
            u[b, k] = _midpoint_uniform(w[b, k], cells[b, k])
    out = oracle.markov_draft(U, W1, W2, x0=np.arange(B), u=u)
    for b in range(B):
        for k in range(G):
            tok = _int_cell_token(w[b, k], cells[b, k])
            assert out["x"][b, k] == tok
            W = w[b, k].sum()
            assert out["q"][b, k] == pytest.approx(w[b, k, tok] / W, rel=1e-6)
            assert out["lse"][b, k] == pytest.approx(np.log(W), abs=1e-6)


def test_w1_zero_ignores_previous_token():
    c = synth.custom(900, B=3, V=256, r=8, gamma=5, w_dtype="f32")
    d = synth.draft_inputs(c)
    W1 = np.zeros_like(d["W1"])
    a = oracle.markov_draft(d["U"], W1, d["W2"], d["x0"], d["u"])
    b = oracle.markov_draft(d["U"], W1, d["W2"] * 7.0, (d["x0"] + 17) % c.V, d["u"])
    assert np.array_equal(a["x"], b["x"])


def test_one_hot_markov_bias_chain():
    """W1[x] = e_{x mod r} and W2 rows = log of integer weights, U = 0: position k follows
    the integer law of row (x_{k-1} mod r). Pins the gathered row, the orientation
    W1[x] @ W2 and the dependence on the previous token (x_0 for position 1)."""
    g = np.random.default_rng(5)
    B, G, V, r = 6, 7, 10, 4
    wrow = g.integers(1, 30, size=(r, V))
    W1 = np.zeros((V, r), np.float32)
    W1[np.arange(V), np.arange(V) % r] = 1.0
    W2 = np.log(wrow).astype(np.float32)
    U = np.zeros((B, G, V), np.float32)
    x0 = g.integers(0, V, size=B)
    u = np.empty((B, G), np.float32)
    expect = np.empty((B, G), np.int64)
    for b in range(B):
        prev = x0[b]
        for k in range(G):
            w = wrow[prev % r]
            cell = g.integers(0, w.sum())
            u[b, k] = _midpoint_uniform(w, cell)
            expect[b, k] = _int_cell_token(w, cell)
            prev = expect[b, k]
    out = oracle.markov_draft(U, W1, W2, x0, u)
    assert np.array_equal(out["x"], expect)


def test_permutation_chain():
    """A +50 bias on token g(x mod r) forces x_k = g(x_{k-1} mod r) for every uniform."""
    g = np.random.default_rng(7)
    B, G, V, r = 8, 6, 64, 16
    perm = g.permutation(V)[:r]
    W1 = np.zeros((V, r), np.float32)
    W1[np.arange(V), np.arange(V) % r] = 50.0
    W2 = np.zeros((r, V), np.float32)
    W2[np.arange(r), perm] = 1.0
    U = (0.1 * g.standard_normal((B, G, V))).astype(np.float32)
    x0 = g.integers(0, V, size=B)
    u = g.uniform(1e-3, 1 - 2 ** -24, size=(B, G)).astype(np.float32)
    out = oracle.markov_draft(U, W1, W2, x0, u)
    for b in range(B):
        prev = x0[b]
        for k in range(G):
            prev = perm[prev % r]
            assert out["x"][b, k] == prev


def test_dominant_logit_wins_every_uniform():
    g = np.random.default_rng(3)
    V = 300
    U = g.standard_normal((1, 40, V)).astype(np.float32)
    hot = g.integers(0, V, size=40)
    U[0, np.arange(40), hot] += 50.0
    u = np.linspace(1e-3, 1 - 2 ** -24, 40, dtype=np.float32)[None, :]
    out = oracle.markov_draft(U, np.zeros((V, 2), np.float32), np.zeros((2, V), np.float32),
                              np.array([0]), u)
    assert np.array_equal(out["x"][0], hot)


def test_lse_matches_scipy_and_q_is_a_probability():
    c = synth.config(synth.TINY)
    d = synth.draft_inputs(c)
    out = oracle.markov_draft(d["U"], d["W1"], d["W2"], d["x0"], d["u"], want_logits=True)
    L = out["L"]
    ref = scipy.special.logsumexp(L, axis=-1)
    np.testing.assert_allclose(out["lse"], ref, rtol=0, atol=1e-12)
    B, G, V = L.shape
    for b in range(B):
        for k in range(G):
            x = out["x"][b, k]
            assert 0 <= x < V
            assert out["q"][b, k] == pytest.approx(np.exp(L[b, k, x] - ref[b, k]), rel=1e-12)


def test_bf16_factors_decode_exactly():
    bits = np.array([0x3F80, 0xC000, 0x3F81, 0x0000, 0x8000, 0x7F80], np.uint16)
    val = oracle.decode_factor(bits, "bf16")
    assert list(val[:5]) == [1.0, -2.0, 1.0078125, 0.0, -0.0]
    assert val[5] == np.inf
    # the generator's round-to-nearest-even
    f = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -3.0, 1.0 + 2 ** -9], np.float32)
    assert list(synth.f32_to_bf16_bits(f)) == [0x3F80, 0x3F82, 0xC040, 0x3F80]


def test_sampler_chi_squared():
    g = np.random.default_rng(21)
    V, N = 16, 40000
    w = g.integers(1, 20, size=V)
    U = np.broadcast_to(np.log(w).astype(np.float32), (N, 1, V))
    u = synth.uniforms(synth.rng(901, synth.T_UDRAFT), (N, 1))
    out = oracle.markov_draft(U, np.zeros((V, 1), np.float32), np.zeros((1, V), np.float32),
                              np.zeros(N, np.int64), u)
    counts = np.bincount(out["x"][:, 0], minlength=V)
    expected = N * w / w.sum()
    assert scipy.stats.chisquare(counts, expected).pvalue > 1e-3


def test_sentinels():
    V = 32
    U = np.zeros((2, 3, V), np.float32)
    U[1, 1, :] = -np.inf
    u = np.full((2, 3), 0.5, np.float32)
    out = oracle.markov_draft(U, np.zeros((V, 2), np.float32), np.zeros((2, V), np.float32),
                              np.array([V + 3, 1]), u)
    assert list(out["x"][0]) == [-1, -1, -1]            # context token out of range
    assert out["x"][1, 0] == 16                           # uniform row, u = 0.5
    assert list(out["x"][1, 1:]) == [-1, -1]             # all -inf row, then nothing
    assert out["lse"][1, 1] == -np.inf and out["q"][1, 1] == 0.0
