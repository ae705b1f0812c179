"""Pins of the oracle's RNN-head draft against values fixed by construction.

The recurrence read from the pages ([P3] "Semi-Autoregressive Generation", the RNN head;
[P1] "DSpark 架构设计：半自回归生成与马尔可夫修正"): h_1 = W1[x_0], h_k = A h_{k-1} + W1[x_{k-1}],
B_k = h_k W2. Each pin fixes the answer without the oracle's own softmax:

* A = 0 is the Markov head: the oracle's Markov draft bit for bit;
* A a permutation matrix P (e_i -> e_{sigma(i)}), W1[x] = e_{x mod r}, U = 0 and W2 = log of
  integer weights: h_k = sum_j e_{sigma^{k-1-j}(x_j mod r)}, so p_k(v) is proportional to the
  integer prod_j w[sigma^{k-1-j}(x_j mod r)][v], and the token of a uniform placed inside an
  integer CDF cell is known by integer arithmetic (a transposed A, a missing or extra
  application of A, or a state that forgets the context token all change the law);
* A = 2I, W1[x] = 40 e_{x mod r}, W2 a +1 on token g(i) for rank i: the context token keeps
  the largest weight, so every position drafts g(x_0 mod r), whatever the uniforms (the Markov
  head would follow the previous token instead).
"""
import numpy as np
import pytest

import oracle
import synth


def _perm_matrix(sigma):
    r = len(sigma)
    A = np.zeros((r, r), np.float32)
    A[sigma, np.arange(r)] = 1.0            # A e_i = e_{sigma(i)}
    return A


def test_zero_recurrence_is_the_markov_head():
    c = synth.custom(1500, B=3, V=700, r=16, gamma=6, w_dtype="bf16", w_sigma=0.3)
    d = synth.draft_inputs(c)
    A = np.zeros((c.r, c.r), np.uint16)
    m = oracle.markov_draft(d["U"], d["W1"], d["W2"], d["x0"], d["u"], "bf16", want_logits=True)
    h = oracle.rnn_draft(d["U"], d["W1"], d["W2"], A, d["x0"], d["u"], "bf16", want_logits=True,
                         want_state=True)
    for k in ("x", "q", "lse", "L"):
        assert np.array_equal(m[k], h[k]), k
    w1 = oracle.decode_factor(d["W1"], "bf16")
    for b in range(c.B):
        prev = [d["x0"][b]] + list(m["x"][b, :-1])
        for k in range(c.gamma):
            assert np.array_equal(h["h"][b, k], w1[prev[k]])


def _integer_chain_case(seed, B=4, G=6, V=11, r=5):
    g = np.random.default_rng(seed)
    sigma = g.permutation(r)
    while np.array_equal(sigma[sigma], np.arange(r)):       # not an involution: P != P^T
        sigma = g.permutation(r)
    w = g.integers(1, 6, size=(r, V))
    W1 = np.zeros((V, r), np.float32)
    W1[np.arange(V), np.arange(V) % r] = 1.0
    W2 = np.log(w).astype(np.float64)
    A = _perm_matrix(sigma)
    x0 = g.integers(0, V, size=B)
    return g, sigma, w, W1, W2, A, x0


def _expected_integer_chain(g, sigma, w, x0, G, V, r):
    """Tokens and states of the permutation chain by integer arithmetic, with a uniform at the
    midpoint of a random integer CDF cell at every position."""
    B = len(x0)
    u = np.empty((B, G), np.float32)
    x = np.empty((B, G), np.int64)
    H = np.zeros((B, G, r))
    for b in range(B):
        toks = [int(x0[b])]
        for k in range(G):
            weight = np.ones(V, dtype=object)
            state = np.zeros(r, np.int64)
            for j, t in enumerate(toks):                    # j = 0..k, the prefix x_0..x_k-1
                i = t % r
                for _ in range(k - j):                      # sigma^(k - j)
                    i = sigma[i]
                state[i] += 1
                weight = weight * w[i].astype(object)
            H[b, k] = state
            tot = int(sum(weight))
            cw = np.cumsum(np.array([int(v) for v in weight]))
            cell = int(g.integers(0, tot))
            u[b, k] = np.float32((cell + 0.5) / tot)
            tok = int(np.searchsorted(cw, cell, side="right"))
            x[b, k] = tok
            toks.append(tok)
    return u, x, H


def test_permutation_recurrence_integer_law():
    G, V, r = 6, 11, 5
    g, sigma, w, W1, W2, A, x0 = _integer_chain_case(3, G=G, V=V, r=r)
    u, x_exp, H_exp = _expected_integer_chain(g, sigma, w, x0, G, V, r)
    U = np.zeros((len(x0), G, V), np.float32)
    out = oracle.rnn_draft(U, W1, W2.astype(np.float32), A, x0, u, "f32", want_state=True)
    assert np.array_equal(out["x"], x_exp)
    assert np.array_equal(out["h"], H_exp)
    # the same recurrence with A transposed is a different law: the pin sees the orientation
    bad = oracle.rnn_draft(U, W1, W2.astype(np.float32), A.T.copy(), x0, u, "f32")
    assert not np.array_equal(bad["x"], x_exp)


def test_doubling_recurrence_keeps_the_context_token():
    g = np.random.default_rng(9)
    B, G, V, r = 6, 12, 64, 16
    perm = g.permutation(V)[:r]
    W1 = np.zeros((V, r), np.float32)
    W1[np.arange(V), np.arange(V) % r] = 40.0
    W2 = np.zeros((r, V), np.float32)
    W2[np.arange(r), perm] = 1.0
    A = (2.0 * np.eye(r)).astype(np.float32)
    U = (0.1 * g.standard_normal((B, G, V))).astype(np.float32)
    x0 = g.integers(0, V, size=B)
    u = g.uniform(1e-3, 1 - 2 ** -24, size=(B, G)).astype(np.float32)
    out = oracle.rnn_draft(U, W1, W2, A, x0, u)
    for b in range(B):
        assert np.all(out["x"][b] == perm[x0[b] % r])
    # the Markov head on the same factors follows the previous token instead
    m = oracle.markov_draft(U, W1, W2, x0, u)
    assert not np.array_equal(m["x"], out["x"])


def test_forced_block_and_sentinels():
    c = synth.custom(1501, B=3, V=500, r=8, gamma=5, w_dtype="f32", w_sigma=0.3)
    d = synth.draft_inputs(c)
    A = synth.rnn_factor(c)
    a = oracle.rnn_draft(d["U"], d["W1"], d["W2"], A, d["x0"], d["u"], want_logits=True)
    f = oracle.rnn_draft(d["U"], d["W1"], d["W2"], A, d["x0"], d["u"], want_logits=True,
                         forced=a["x"])
    for k in ("x", "q", "lse", "L"):
        assert np.array_equal(a[k], f[k]), k
    x0 = d["x0"].copy()
    x0[1] = c.V + 2
    s = oracle.rnn_draft(d["U"], d["W1"], d["W2"], A, x0, d["u"])
    assert np.all(s["x"][1] == -1) and np.all(s["lse"][1] == -np.inf)
    assert np.array_equal(s["x"][0], a["x"][0])
