"""GPU parity of dspark_rnn_draft (the RNN head) against the fp64 oracle, through the C ABI.

The recurrence read from the pages ([P3] "Semi-Autoregressive Generation", the RNN head):
h_1 = W1[x_0], h_k = A h_{k-1} + W1[x_{k-1}], B_k = h_k W2. Every position of every checked
request is compared with the oracle's law given the GPU's own prefix (teacher forcing), the
states h_k with the oracle's, and closed forms run through both kernel paths."""
import numpy as np
import pytest
import torch

import oracle
import synth
import draft_sampling_verification_head_amd as dspark
from parity import Report, check_draft, dev, host, tie_bound

pytestmark = pytest.mark.gpu


def _inputs(c, A=None):
    d = synth.draft_inputs(c)
    d["A"] = synth.rnn_factor(c) if A is None else A
    return d


def _run(d, want_logits=True):
    out = dspark.rnn_draft(dev(d["U"]), dev(d["W1"]), dev(d["W2"]), dev(d["A"]), dev(d["x0"]),
                           dev(d["u"]), want_logits=want_logits, want_state=True)
    torch.cuda.synchronize()
    return {k: (host(v) if v is not None else None) for k, v in out.items()}


def _rnn_oracle(A, states):
    """check_draft's oracle: the RNN draft along the GPU's block; keeps the states."""
    def fn(U, W1, W2, x0, u, w_dtype, forced):
        ref = oracle.rnn_draft(U, W1, W2, A, x0, u, w_dtype, want_logits=True, want_state=True,
                               forced=forced)
        states.append(ref["h"])
        return ref
    return fn


def _check(d, g, requests, name, wdt="bf16"):
    states = []
    rep = check_draft(d["U"], d["W1"], d["W2"], d["x0"], d["u"], wdt, g["x"], g["q"], g["lse"],
                      requests, gL=g["L"], rep=Report(name), oracle_fn=_rnn_oracle(d["A"], states))
    H = np.concatenate(states)
    err = np.max(np.abs(g["h"][list(requests)].astype(np.float64) - H))
    assert err < 1e-5, f"state error {err}"
    assert rep.ties <= tie_bound(rep)
    return rep, err


@pytest.mark.parametrize("B,V,r,G", [
    (1, 151936, 256, 7),      # the single-request shape: one launch, W2 in registers, A in LDS
    (1, 20000, 64, 16),
    (1, 1288, 248, 5),        # ragged tiles, rank not a multiple of 16
    (3, 1000, 8, 4),          # per-position launches from here on
    (9, 4104, 32, 3),
    (70, 20000, 248, 5),      # two request groups of the MFMA step, the second ragged
])
def test_rnn_shapes(gpu, B, V, r, G):
    c = synth.custom(1600 + B + G, B=B, V=V, r=r, gamma=G, w_dtype="bf16", w_sigma=0.3)
    d = _inputs(c)
    path = dspark.rnn_draft_path(B, dev(d["W1"]), dev(d["W2"]), dev(d["A"]))
    assert path == ("resident" if B == 1 else "mfma")
    g = _run(d)
    _check(d, g, range(B), f"rnn B={B} V={V}")


def test_rnn_batched_workload_all_requests(gpu):
    """The batched shape (B=64, gamma=16, V=151936, r=256) with the seeded recurrence."""
    c = synth.config(synth.BATCHED)
    d = _inputs(c)
    g = _run(d)
    rep, err = _check(d, g, range(c.B), "rnn batched draft")
    assert rep.compared == c.B * c.gamma
    rep.record()


def test_rnn_single_request_workload(gpu):
    c = synth.config(synth.SINGLE)
    d = _inputs(c)
    g = _run(d)
    rep, err = _check(d, g, [0], "rnn single-request draft")
    assert rep.compared == c.gamma
    rep.record()


@pytest.mark.parametrize("B", [1, 9])
def test_rnn_doubling_chain_keeps_the_context_token(gpu, B):
    """A = 2I, W1[x] = 40 e_{x mod r}, W2 a +1 on token g(i): every position drafts
    g(x_0 mod r), on both paths (all values exact in bf16)."""
    g_ = np.random.default_rng(31 + B)
    G, V, r = 10, 4096, 16
    perm = g_.permutation(V)[:r]
    W1 = np.zeros((V, r), np.float32)
    W1[np.arange(V), np.arange(V) % r] = 40.0
    W2 = np.zeros((r, V), np.float32)
    W2[np.arange(r), perm] = 1.0
    A = (2.0 * np.eye(r)).astype(np.float32)
    d = dict(U=(0.1 * g_.standard_normal((B, G, V))).astype(np.float32),
             W1=synth.f32_to_bf16_bits(W1), W2=synth.f32_to_bf16_bits(W2), A=synth.f32_to_bf16_bits(A),
             x0=g_.integers(0, V, size=B).astype(np.int32),
             u=g_.uniform(1e-3, 1 - 2 ** -24, size=(B, G)).astype(np.float32))
    g = _run(d, want_logits=False)
    for b in range(B):
        assert np.all(g["x"][b] == perm[d["x0"][b] % r])


def test_rnn_zero_recurrence_is_the_markov_draft(gpu):
    """A = 0 on the single-request path: the hi parts are the W1 rows and the lo parts zero, so
    the tokens, probabilities, normalisers and logits equal the Markov draft's bit for bit."""
    c = synth.custom(1650, B=1, V=151936, r=256, gamma=7, w_dtype="bf16", w_sigma=0.3)
    d = _inputs(c, A=np.zeros((256, 256), np.uint16))
    g = _run(d)
    m = dspark.markov_draft(dev(d["U"]), dev(d["W1"]), dev(d["W2"]), dev(d["x0"]), dev(d["u"]),
                            want_logits=True)
    torch.cuda.synchronize()
    for k in ("x", "q", "lse", "L"):
        assert np.array_equal(g[k].view(np.uint8), host(m[k]).view(np.uint8)), k


def test_rnn_sentinels_and_rejects(gpu):
    c = synth.custom(1660, B=12, V=3000, r=16, gamma=4, w_dtype="bf16", w_sigma=0.3)
    d = _inputs(c)
    d["x0"][3] = c.V + 5
    d["x0"][7] = -2
    g = _run(d)
    for b in (3, 7):
        assert np.all(g["x"][b] == -1) and np.all(g["lse"][b] == -np.inf)
    _check(d, g, [0, 1, 11], "rnn sentinels")
    f = synth.custom(1661, B=2, V=3000, r=16, gamma=2, w_dtype="f32")
    e = _inputs(f)
    with pytest.raises(TypeError):
        dspark.rnn_draft(dev(e["U"]), dev(e["W1"]), dev(e["W2"]), dev(e["A"]), dev(e["x0"]), dev(e["u"]))


def test_rnn_joint_law_chi_squared(gpu):
    """2^18 requests from one context, two positions (the batched kernels): the pairs
    (x_1, x_2) follow p_1(x_1) p_2(x_2 | x_1), where p_2's bias comes from the state
    h_2 = A W1[x_0] + W1[x_1]; chi-squared over the 256 cells, small cells pooled. The law is
    the oracle's, with x_1 forced to each value in turn."""
    import scipy.stats
    N, V, r, G = 1 << 18, 16, 8, 2
    g = np.random.default_rng(45)
    U2 = (0.7 * g.standard_normal((G, V))).astype(np.float32)
    W1 = synth.f32_to_bf16_bits((0.8 * g.standard_normal((V, r))).astype(np.float32))
    W2 = synth.f32_to_bf16_bits((0.8 * g.standard_normal((r, V))).astype(np.float32))
    A = synth.f32_to_bf16_bits((0.5 * g.standard_normal((r, r))).astype(np.float32))
    x0 = 5
    P = np.zeros((V, V))
    for x1 in range(V):
        ref = oracle.rnn_draft(U2[None], W1, W2, A, np.array([x0]), np.full((1, G), 0.5, np.float32),
                               "bf16", want_logits=True, forced=np.array([[x1, 0]]))
        P[x1] = oracle.softmax_row(ref["L"][0, 0])[0][x1] * oracle.softmax_row(ref["L"][0, 1])[0]
    assert abs(P.sum() - 1.0) < 1e-12
    U = torch.from_numpy(U2).cuda().expand(N, G, V).contiguous()
    u = torch.from_numpy(synth.uniforms(synth.rng(935, 0), (N, G))).cuda()
    assert dspark.rnn_draft_path(N, dev(W1), dev(W2), dev(A)) == "mfma"
    out = dspark.rnn_draft(U, dev(W1), dev(W2), dev(A), torch.full((N,), x0, dtype=torch.int32,
                                                                  device="cuda"), u,
                           want_q=False, want_lse=False)
    x = host(out["x"]).astype(np.int64)
    assert x.min() >= 0 and x.max() < V
    counts = np.bincount(x[:, 0] * V + x[:, 1], minlength=V * V).astype(float)
    expected = N * P.ravel()
    keep = expected >= 5
    obs = np.append(counts[keep], counts[~keep].sum())
    exp = np.append(expected[keep], expected[~keep].sum())
    assert scipy.stats.chisquare(obs, exp).pvalue > 1e-3
    # the Markov head's law differs: without A h_1 the same counts are far from it
    Pm = np.zeros((V, V))
    for x1 in range(V):
        ref = oracle.markov_draft(U2[None], W1, W2, np.array([x0]), np.full((1, G), 0.5, np.float32),
                                  "bf16", want_logits=True, forced=np.array([[x1, 0]]))
        Pm[x1] = oracle.softmax_row(ref["L"][0, 0])[0][x1] * oracle.softmax_row(ref["L"][0, 1])[0]
    em = N * Pm.ravel()
    km = em >= 5
    assert scipy.stats.chisquare(np.append(counts[km], counts[~km].sum()),
                                 np.append(em[km], em[~km].sum())).pvalue < 1e-6
