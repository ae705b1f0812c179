"""GPU parity of dspark_verify_markov (verify + TV labels with the draft logits rebuilt from
the Markov factors) against the materialised verify on the draft's own logits and against the
fp64 oracle, called through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
import synth
import draft_sampling_verification_head_amd as dspark
from parity import (tie_bound, PROB_TOL, Report, check_cstar, check_draft, check_verify, dev,
                    forced_draft_logits, host, is_cdf_tie)
from test_gpu_verify import _chi2_pvalue, _markov_tables

pytestmark = pytest.mark.gpu


def _inputs(c, lengths, flat):
    d = synth.draft_inputs(c)
    Lt_pad = synth.target_padded_all(c)
    u_acc, u_fin = synth.verify_uniforms(c)
    t_off = None
    if flat:
        t_off = np.zeros(c.B + 1, np.int32)
        t_off[1:] = np.cumsum(lengths + 1)
        Lt = np.concatenate([Lt_pad[b, : lengths[b] + 1] for b in range(c.B)])
    else:
        Lt = Lt_pad.reshape(-1, c.V)
    d.update(Lt=Lt, u_acc=u_acc, u_fin=u_fin, t_off=t_off,
             length=None if lengths is None else lengths.astype(np.int32))
    return d


def _run(inp, x=None, x0=None):
    """Draft on the GPU (keeping its logits), then both verifies on the same tokens."""
    t = {k: (dev(v) if isinstance(v, np.ndarray) else v) for k, v in inp.items()}
    D = dspark.markov_draft(t["U"], t["W1"], t["W2"], t["x0"], t["u"], want_logits=True)
    xs = D["x"] if x is None else dev(x)
    x0s = t["x0"] if x0 is None else dev(x0)
    A = dspark.verify(D["L"], t["Lt"], xs, t["u_acc"], t["u_fin"], t_off=t["t_off"],
                      length=t["length"], ld_lse=D["lse"], want_lse=True, with_tv=True)
    M = dspark.verify_markov(t["U"], t["W1"], t["W2"], x0s, xs, D["lse"], t["Lt"], t["u_acc"],
                             t["u_fin"], t_off=t["t_off"], length=t["length"])
    torch.cuda.synchronize()
    h = lambda o: {k: (host(v) if v is not None else None) for k, v in o.items()}  # noqa: E731
    return h(D), h(A), h(M)


def _final_law(L, Lt, b, off, n, ell):
    """The law of the final token from the GPU's own draft logits (fp64)."""
    if n < ell:
        pd = oracle.softmax_row(L[b, n])[0]
        pt = oracle.softmax_row(Lt[off + n])[0]
        res = np.maximum(pt - pd, 0.0)
        return res / res.sum() if res.sum() > 0 else pt
    return oracle.softmax_row(Lt[off + ell])[0]


def _compare(inp, D, A, M, B, G):
    """Identical acceptance decisions and normalisers; final tokens equal up to CDF ties;
    labels equal up to summation order. The two paths form the final-draw weights from
    different exponentials (per 8192-logit chunk from the read rows, per slab tile from the
    rebuilt logits), so a final draw may fall on either side of a cell edge: each such
    difference must be a CDF tie of the token the rebuilt path drew, and their number stays
    within the harness's tie bound over the B final draws."""
    assert np.array_equal(A["n"], M["n"])
    assert np.array_equal(A["lse_t"].view(np.uint8), M["lse_t"].view(np.uint8))
    ties = 0
    for b in range(B):
        n = int(A["n"][b])
        if n < 0:
            assert np.all(M["y"][b] == -1)
            continue
        assert np.array_equal(A["y"][b, :n], M["y"][b, :n])
        assert np.all(M["y"][b, n + 1:] == -1)
        if A["y"][b, n] != M["y"][b, n]:
            ell = G if inp["length"] is None else int(inp["length"][b])
            off = b * (G + 1) if inp["t_off"] is None else int(inp["t_off"][b])
            law = _final_law(D["L"], inp["Lt"], b, off, n, ell)
            assert is_cdf_tie(law, oracle.clamp_uniform(inp["u_fin"][b]), int(M["y"][b, n]))
            ties += 1
    assert ties <= 2 + B // 20
    fin = np.isfinite(A["cstar"])
    assert np.array_equal(fin, np.isfinite(M["cstar"]))
    if fin.any():
        assert np.max(np.abs(A["cstar"][fin] - M["cstar"][fin])) < 1e-5


def _oracle_check(inp, D, M, requests, G, rep=None):
    """Requests against the oracle: the GPU's draft tokens are oracle draws (or CDF ties) on
    the GPU's own prefix, and the verify and labels are checked on the oracle's fp64 logits
    of that same block (teacher forcing), so no request is skipped."""
    rep = rep or Report("verify_markov")
    check_draft(inp["U"], inp["W1"], inp["W2"], inp["x0"], inp["u"], "bf16", D["x"], D["q"],
                D["lse"], requests, rep=Report("draft of the verified block"),
                keep_logits=(kept := {}))
    for b in requests:
        L = kept.pop(b)
        ell = G if inp["length"] is None else int(inp["length"][b])
        off = b * (G + 1) if inp["t_off"] is None else int(inp["t_off"][b])
        t_off = np.array([off, off + ell + 1], np.int32)
        check_verify(L, inp["Lt"], D["x"][b:b + 1], inp["u_acc"][b:b + 1], inp["u_fin"][b:b + 1],
                     t_off, np.array([ell], np.int32), M["n"][b:b + 1], M["y"][b:b + 1], [0],
                     rep=rep)
        check_cstar(L, inp["Lt"], t_off, np.array([ell]), M["cstar"][b:b + 1], [0], rep=rep)
    return rep


@pytest.mark.parametrize("B,V,r,G,flat", [
    (12, 2056, 248, 4, True),      # one 16-column tile per wave; two 8-row groups, one ragged
    (20, 40000, 64, 6, True),      # two tiles per wave, two rank chunks
    (9, 70000, 128, 3, False),     # three tiles, padded target layout
    (33, 129280, 256, 5, True),    # four tiles
    (10, 151936, 256, 7, True),    # five tiles, the full vocabulary
])
def test_matches_materialised_verify(gpu, B, V, r, G, flat):
    c = synth.custom(970 + B, B=B, V=V, r=r, gamma=G, w_dtype="bf16", w_sigma=0.3, tnoise=0.7)
    g = np.random.default_rng(V + B)
    lengths = g.integers(0, G + 1, size=B) if flat else None
    if flat:
        lengths[0], lengths[-1] = 0, G
    inp = _inputs(c, lengths, flat)
    D, A, M = _run(inp)
    _compare(inp, D, A, M, B, G)
    _oracle_check(inp, D, M, sorted({1, B // 2, B - 1}), G)


def test_faulty_requests(gpu):
    """Out-of-range length, a token outside [0, V), an invalid context token with len > 0:
    n = -1, y all -1, NaN labels. A zero length with an invalid context token is fine (the
    bonus row needs no draft logits)."""
    B, V, r, G = 10, 3000, 32, 4
    c = synth.custom(981, B=B, V=V, r=r, gamma=G, w_dtype="bf16", w_sigma=0.3)
    lengths = np.full(B, G)
    lengths[8] = 0
    inp = _inputs(c, lengths, True)
    t = {k: (dev(v) if isinstance(v, np.ndarray) else v) for k, v in inp.items()}
    D = dspark.markov_draft(t["U"], t["W1"], t["W2"], t["x0"], t["u"])
    x = host(D["x"]).copy()
    x[5, 1] = V + 3
    x0 = inp["x0"].copy()
    x0[7] = -1
    x0[8] = V + 1
    ln = lengths.astype(np.int32).copy()
    ln[2] = G + 3
    M = dspark.verify_markov(t["U"], t["W1"], t["W2"], dev(x0), dev(x), D["lse"], t["Lt"],
                             t["u_acc"], t["u_fin"], t_off=t["t_off"], length=dev(ln))
    torch.cuda.synchronize()
    n, y, cs = host(M["n"]), host(M["y"]), host(M["cstar"])
    for b in (2, 5, 7):
        assert n[b] == -1 and np.all(y[b] == -1) and np.all(np.isnan(cs[b]))
    assert n[8] == 0 and 0 <= y[8, 0] < V and np.all(y[8, 1:] == -1) and np.all(np.isnan(cs[8]))
    for b in (0, 1, 3, 4, 6, 9):
        assert 0 <= n[b] <= G and np.all(np.isfinite(cs[b]))


def test_round_rebuilt_logits(gpu):
    """The full round workload (B=512, V=129280, gamma=16) with the draft's logits never written: draft -> schedule ->
    verify_markov, against the same round verified on materialised logits, and sampled
    requests against the oracle."""
    c = synth.config(synth.ROUND)
    base = [synth.base_rows(c, b) for b in range(c.B)]
    U = np.stack([r_[: c.gamma] for r_ in base])
    Lt_pad = np.stack([synth.target_rows(c, b, base[b]) for b in range(c.B)])
    w1, w2 = synth.factors(c)
    u_acc, u_fin = synth.verify_uniforms(c)
    inp = dict(U=U, W1=w1, W2=w2, x0=synth.x0(c), u=synth.draft_uniforms(c))
    t = {k: dev(v) for k, v in inp.items()}
    s = dspark.schedule(dev(synth.confidences(c)), dev(synth.sps_table(4096)), 4096,
                        temp=dev(synth.temperatures(c.gamma)))
    length = host(s["len"])
    Lt = np.concatenate([Lt_pad[b, : length[b] + 1] for b in range(c.B)])
    inp.update(Lt=Lt, u_acc=u_acc, u_fin=u_fin, t_off=host(s["t_off"]), length=length)
    D, A, M = _run(inp)
    assert dspark.markov_draft_path(c.B, t["W1"], t["W2"]) == "slab"
    _compare(inp, D, A, M, c.B, c.gamma)
    rep = _oracle_check(inp, D, M, list(range(0, c.B, 8)), c.gamma,
                        rep=Report("round verify_markov (64 of 512 requests)"))
    assert rep.ties <= tie_bound(rep)
    rep.record()
    # the same draft without its logits output gives the same tokens
    D2 = dspark.markov_draft(t["U"], t["W1"], t["W2"], t["x0"], t["u"])
    torch.cuda.synchronize()
    assert np.array_equal(host(D2["x"]), D["x"])


def test_lossless_first_token_chi2(gpu):
    """2^18 requests, gamma = 3, bf16 factors (W1 = I, W2 = the draft table's logs): the first
    emitted token follows the target law."""
    V, G, N = 8, 3, 1 << 18
    P, Q = _markov_tables(V, 124)
    with np.errstate(divide="ignore"):
        logP = torch.from_numpy(np.log(P).astype(np.float32)).cuda()
    W1 = torch.eye(V, dtype=torch.bfloat16, device="cuda")
    W2 = torch.from_numpy(np.log(Q).astype(np.float32)).cuda().to(torch.bfloat16)
    prev = torch.full((N,), 3, dtype=torch.int32, device="cuda")
    gen = synth.rng(982, 0)
    U = torch.zeros((N, G, V), dtype=torch.float32, device="cuda")
    u = torch.from_numpy(synth.uniforms(gen, (N, G))).cuda()
    d = dspark.markov_draft(U, W1, W2, prev, u)
    ctx = torch.cat([prev[:, None], d["x"]], dim=1).long()
    Lt = logP[ctx].reshape(N * (G + 1), V).contiguous()
    u_acc = torch.from_numpy(synth.uniforms(gen, (N, G))).cuda()
    u_fin = torch.from_numpy(synth.uniforms(gen, (N,))).cuda()
    res = dspark.verify_markov(U, W1, W2, prev, d["x"], d["lse"], Lt, u_acc, u_fin)
    y = host(res["y"])
    assert np.all(host(res["n"]) >= 0)
    counts = np.bincount(y[:, 0], minlength=V).astype(float)
    assert _chi2_pvalue(counts, P[3], N) > 1e-3


def _random_shapes(n, seed):
    """Verify shapes drawn from a fixed seed within the entry point's caps: B 9..96 (the slab
    draft, whose logits the rebuild reproduces bit for bit), V a multiple of 8 from 1024 to
    163840, r a multiple of 8 up to 256, gamma 1..20, flattened or padded target rows."""
    g = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        B = int(g.integers(9, 97))
        V = int(g.integers(128, 20481)) * 8
        r = int(g.integers(1, 33)) * 8
        G = int(g.integers(1, 21))
        out.append((B, V, r, G, bool(g.random() < 0.7)))
    return out


@pytest.mark.parametrize("B,V,r,G,flat", _random_shapes(8, 2027))
def test_random_shapes(gpu, B, V, r, G, flat):
    """Seeded random shapes and verify lengths: the rebuilt-logit verify against the verify
    on the draft's own logits, and sampled requests against the oracle."""
    c = synth.custom(1100 + B + G, B=B, V=V, r=r, gamma=G, w_dtype="bf16", w_sigma=0.3,
                     tnoise=0.7)
    g = np.random.default_rng(V + r)
    lengths = g.integers(0, G + 1, size=B) if flat else None
    if flat:
        lengths[0], lengths[-1] = 0, G
    inp = _inputs(c, lengths, flat)
    D, A, M = _run(inp)
    _compare(inp, D, A, M, B, G)
    _oracle_check(inp, D, M, sorted({1, B // 2, B - 1}), G)
