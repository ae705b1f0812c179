"""GPU parity of dspark_verify and dspark_tv_labels against the fp64 oracle."""
import numpy as np
import pytest
import scipy.stats
import torch

import oracle
import synth
import draft_sampling_verification_head_amd as dspark
from parity import tie_bound, PROB_TOL, Report, check_cstar, check_verify, dev, host

pytestmark = pytest.mark.gpu


def tokens_from_logits(Ld, u):
    """Draft tokens x ~ p_d drawn by the oracle's inverse CDF (an input for both sides)."""
    B, G, V = Ld.shape
    x = np.empty((B, G), np.int32)
    for b in range(B):
        for k in range(G):
            x[b, k] = oracle.inverse_cdf(oracle.softmax_row(Ld[b, k])[0], oracle.clamp_uniform(u[b, k]))
    return x


def verify_inputs(c, lengths=None, flat=False):
    Ld = synth.draft_logits_all(c)
    Lt_pad = synth.target_padded_all(c)
    x = tokens_from_logits(Ld, synth.token_uniforms(c))
    u_acc, u_fin = synth.verify_uniforms(c)
    t_off = None
    if flat:
        t_off = np.zeros(c.B + 1, np.int32)
        t_off[1:] = np.cumsum(lengths + 1)
        Lt = np.concatenate([Lt_pad[b, : lengths[b] + 1] for b in range(c.B)])
    else:
        Lt = Lt_pad.reshape(-1, c.V)
    return dict(Ld=Ld, Lt=Lt, x=x, u_acc=u_acc, u_fin=u_fin, t_off=t_off,
                length=None if lengths is None else lengths.astype(np.int32))


def run_verify(inp, want_lse=False, ld_lse=None):
    t = {k: (dev(v) if isinstance(v, np.ndarray) else v) for k, v in inp.items()}
    out = dspark.verify(t["Ld"], t["Lt"], t["x"], t["u_acc"], t["u_fin"], t_off=t["t_off"],
                        length=t["length"], ld_lse=ld_lse, want_lse=want_lse)
    torch.cuda.synchronize()
    return {k: (host(v) if v is not None else None) for k, v in out.items()}


def run_tv(inp, lse_d=None, lse_t=None):
    t = {k: (dev(v) if isinstance(v, np.ndarray) else v) for k, v in inp.items()}
    c = dspark.tv_labels(t["Ld"], t["Lt"], t_off=t["t_off"], length=t["length"],
                         lse_d=lse_d, lse_t=lse_t)
    torch.cuda.synchronize()
    return host(c)


def check_tv(inp, gc, requests):
    ref = oracle.tv_labels(inp["Ld"], inp["Lt"], t_off=inp["t_off"], length=inp["length"],
                           requests=requests)
    for b in requests:
        fin = np.isfinite(ref[b])
        assert np.array_equal(fin, np.isfinite(gc[b])), f"b={b} NaN pattern"
        err = np.max(np.abs(gc[b][fin] - ref[b][fin])) if fin.any() else 0.0
        assert err < PROB_TOL, f"b={b} c* err {err}"


@pytest.mark.parametrize("B,V,G,flat", [
    (4, 1024, 4, False),
    (7, 1000, 5, True),        # V % 4 != 0: scalar loads
    (5, 9000, 3, True),        # several 4096-element chunks + ragged tail
    (3, 5, 6, False),          # tiny vocabulary
])
def test_small_shapes(gpu, B, V, G, flat):
    c = synth.custom(940 + V % 89, B=B, V=V, r=1, gamma=G, w_dtype="f32", tnoise=0.8)
    g = np.random.default_rng(V)
    lengths = g.integers(0, G + 1, size=B) if flat else None
    if flat:
        lengths[0], lengths[-1] = 0, G
    inp = verify_inputs(c, lengths, flat)
    out = run_verify(inp)
    rep = check_verify(inp["Ld"], inp["Lt"], inp["x"], inp["u_acc"], inp["u_fin"], inp["t_off"],
                       inp["length"], out["n"], out["y"], range(B))
    assert rep.ties <= tie_bound(rep)
    check_tv(inp, run_tv(inp), range(B))


def test_identical_laws_accept_all(gpu):
    c = synth.custom(945, B=6, V=5000, r=1, gamma=7, w_dtype="f32")
    Ld = synth.draft_logits_all(c)
    extra = np.stack([synth.base_rows(c, b)[c.gamma] for b in range(c.B)])
    Lt = np.concatenate([np.concatenate([Ld[b], extra[b][None]]) for b in range(c.B)])
    x = tokens_from_logits(Ld, synth.token_uniforms(c))
    u_acc, u_fin = synth.verify_uniforms(c)
    inp = dict(Ld=Ld, Lt=Lt, x=x, u_acc=u_acc, u_fin=u_fin, t_off=None, length=None)
    out = run_verify(inp)
    assert np.all(out["n"] == c.gamma)
    assert np.array_equal(out["y"][:, : c.gamma], x)
    check_verify(Ld, Lt, x, u_acc, u_fin, None, None, out["n"], out["y"], range(c.B))
    cs = run_tv(inp)
    assert np.all(np.abs(cs - 1.0) < 1e-5)


def test_ld_lse_input_matches_computed(gpu):
    c = synth.custom(946, B=5, V=3333, r=1, gamma=4, w_dtype="f32", tnoise=1.0)
    inp = verify_inputs(c)
    a = run_verify(inp, want_lse=True)
    b = run_verify(inp, ld_lse=dev(a["lse_d"]), want_lse=True)
    assert np.array_equal(a["n"], b["n"]) and np.array_equal(a["y"], b["y"])
    assert np.array_equal(a["lse_d"], b["lse_d"])
    ref = np.array([[oracle.softmax_row(inp["Ld"][i, k])[1] for k in range(c.gamma)]
                    for i in range(c.B)])
    assert np.max(np.abs(a["lse_d"] - ref)) < 1e-4
    # the TV kernel gives the same labels from supplied or computed normalisers
    c1 = run_tv(inp)
    c2 = run_tv(inp, lse_d=dev(a["lse_d"]), lse_t=dev(a["lse_t"]))
    assert np.max(np.abs(c1 - c2)) < 1e-6


def run_verify_tv(inp, ld_lse=None):
    t = {k: (dev(v) if isinstance(v, np.ndarray) else v) for k, v in inp.items()}
    out = dspark.verify(t["Ld"], t["Lt"], t["x"], t["u_acc"], t["u_fin"], t_off=t["t_off"],
                        length=t["length"], ld_lse=ld_lse, want_lse=True, with_tv=True)
    torch.cuda.synchronize()
    return {k: (host(v) if v is not None else None) for k, v in out.items()}


@pytest.mark.parametrize("B,V,G,flat,given", [
    (4, 1024, 4, False, False),
    (7, 1000, 5, True, False),      # V % 4 != 0
    (5, 9000, 3, True, True),       # several chunks, draft normalisers supplied
    (1, 151936, 7, True, True),     # one request at the full vocabulary
])
def test_verify_tv_matches_separate_calls(gpu, B, V, G, flat, given):
    """dspark_verify_tv gives bit-identical tokens, normalisers and c* to dspark_verify
    followed by dspark_tv_labels on that verify's normalisers, and c* within tolerance of the
    oracle."""
    c = synth.custom(950 + V % 83, B=B, V=V, r=1, gamma=G, w_dtype="f32", tnoise=0.8)
    g = np.random.default_rng(V + B)
    lengths = g.integers(0, G + 1, size=B) if flat else None
    if flat:
        lengths[0] = G
    inp = verify_inputs(c, lengths, flat)
    ld_lse = None
    if given:
        ld_lse = dev(np.array([[oracle.softmax_row(inp["Ld"][i, k])[1] for k in range(G)]
                               for i in range(B)], np.float32))
    a = run_verify(inp, want_lse=True, ld_lse=ld_lse)
    tv = run_tv(inp, lse_d=dev(a["lse_d"]) if not given else ld_lse, lse_t=dev(a["lse_t"]))
    f = run_verify_tv(inp, ld_lse=ld_lse)
    for k in ("n", "y", "lse_d", "lse_t"):
        assert np.array_equal(a[k].view(np.uint8), f[k].view(np.uint8)), k
    assert np.array_equal(np.isnan(tv), np.isnan(f["cstar"]))
    fin = ~np.isnan(tv)
    assert np.array_equal(tv[fin], f["cstar"][fin])
    rep = check_verify(inp["Ld"], inp["Lt"], inp["x"], inp["u_acc"], inp["u_fin"], inp["t_off"],
                       inp["length"], f["n"], f["y"], range(B))
    assert rep.ties <= tie_bound(rep)
    check_tv(inp, f["cstar"], range(B))


@pytest.mark.parametrize("B,V,G,flat,given", [
    (2, 600000, 2, True, False),    # 74 chunks per row: past the one-sweep form, the chunked kernels
    (3, 524288, 2, False, True),    # exactly 64 chunks: the persistent sweep (576 tasks)
    (64, 40000, 5, True, False),    # 1920 tasks: the persistent sweep
    (2, 40000, 5, False, True),     # 60 tasks: the one-launch form
])
def test_verify_tv_at_the_sweep_cap(gpu, B, V, G, flat, given):
    """Both implementations of dspark_verify_tv (one sweep up to 64 chunks per row, the chunked
    kernels beyond) match the separate calls bit for bit and the oracle."""
    test_verify_tv_matches_separate_calls(gpu, B, V, G, flat, given)


def test_verify_tv_sweep_over_verified_rows_only(gpu):
    """With lengths given, the persistent sweep's tasks run over the verified rows only: empty
    requests (length 0: one target row), full ones, ragged ones and requests with an invalid
    length (no rows at all) in the padded layout. The results equal the separate calls bit for
    bit, the invalid requests come back as faults, and the others match the oracle."""
    B, V, G = 40, 40000, 5
    c = synth.custom(977, B=B, V=V, r=1, gamma=G, w_dtype="f32", tnoise=0.8)
    g = np.random.default_rng(977)
    lengths = g.integers(0, G + 1, size=B)
    lengths[:4] = [0, G, 0, G]
    bad = [7, 21]
    inp = verify_inputs(c, lengths, flat=False)
    inp["length"][bad[0]] = G + 3
    inp["length"][bad[1]] = -2
    a = run_verify(inp, want_lse=True)
    tv = run_tv(inp, lse_d=dev(a["lse_d"]), lse_t=dev(a["lse_t"]))
    f = run_verify_tv(inp)
    for k in ("n", "y", "lse_d", "lse_t"):
        assert np.array_equal(a[k].view(np.uint8), f[k].view(np.uint8)), k
    assert np.array_equal(np.isnan(tv), np.isnan(f["cstar"]))
    fin = ~np.isnan(tv)
    assert np.array_equal(tv[fin], f["cstar"][fin])
    assert all(f["n"][b] == -1 and np.all(f["y"][b] == -1) for b in bad)
    good = [b for b in range(B) if b not in bad]
    rep = check_verify(inp["Ld"], inp["Lt"], inp["x"], inp["u_acc"], inp["u_fin"], inp["t_off"],
                       inp["length"], f["n"], f["y"], good)
    assert rep.ties <= tie_bound(rep)
    check_tv(inp, f["cstar"], good)


@pytest.mark.parametrize("fill", ["zeros", "ones", "random"])
def test_verify_tv_sweep_workspace_and_graph_replays(gpu, fill):
    """The one-sweep form tags its chunk slots with a key derived from a call counter in the
    workspace: a workspace of zeros, of all-one bytes or of random bytes, calls in a row, and
    replays of a captured call all give the separate calls' results bit for bit."""
    from draft_sampling_verification_head_amd import binding
    c = synth.custom(960, B=6, V=40000, r=1, gamma=5, w_dtype="f32", tnoise=0.8)
    g = np.random.default_rng(960)
    lengths = g.integers(0, c.gamma + 1, size=c.B)
    lengths[0] = c.gamma
    inp = verify_inputs(c, lengths, True)
    a = run_verify(inp, want_lse=True)
    tv = run_tv(inp, lse_d=dev(a["lse_d"]), lse_t=dev(a["lse_t"]))
    lib = binding.load()
    ws = torch.empty(lib.dspark_verify_tv_workspace_bytes(c.B, c.V, c.gamma), dtype=torch.uint8,
                     device="cuda")
    if fill == "zeros":
        ws.zero_()
    elif fill == "ones":
        ws.fill_(255)
    else:
        ws.copy_(torch.randint(0, 256, ws.shape, dtype=torch.uint8, device="cuda",
                               generator=torch.Generator(device="cuda").manual_seed(7)))
    t = {k: (dev(v) if isinstance(v, np.ndarray) else v) for k, v in inp.items()}
    out = {k: torch.empty_like(dev(a[k])) for k in ("n", "y", "lse_d", "lse_t")}
    out["cstar"] = torch.empty((c.B, c.gamma), dtype=torch.float32, device="cuda")

    def call():
        dspark.verify(t["Ld"], t["Lt"], t["x"], t["u_acc"], t["u_fin"], t_off=t["t_off"],
                      length=t["length"], want_lse=True, with_tv=True, out=out, ws=ws)

    def check():
        torch.cuda.synchronize()
        for k in ("n", "y", "lse_d", "lse_t"):
            assert np.array_equal(host(out[k]).view(np.uint8), a[k].view(np.uint8)), k
        cs = host(out["cstar"])
        assert np.array_equal(np.isnan(cs), np.isnan(tv))
        fin = ~np.isnan(tv)
        assert np.array_equal(cs[fin], tv[fin])
        for v in out.values():
            v.fill_(-3)
        torch.cuda.synchronize()

    for _ in range(3):
        call()
        check()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        call()                                      # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    check()
    with torch.cuda.graph(graph, stream=s):
        call()
    for _ in range(4):
        graph.replay()
        check()
        call()                                      # eager calls between the replays
        check()


def test_device_data_faults(gpu):
    c = synth.custom(947, B=4, V=700, r=1, gamma=3, w_dtype="f32")
    lengths = np.array([3, 2, 1, 3])
    inp = verify_inputs(c, lengths, flat=True)
    inp["x"][1, 0] = c.V + 1                    # invalid verified token
    inp["x"][2, 2] = -7                         # invalid but beyond len: ignored
    inp["t_off"][3] = inp["Lt"].shape[0] - 2    # rows past the end of Lt
    out = run_verify(inp)
    assert out["n"][1] == -1 and np.all(out["y"][1] == -1)
    assert out["n"][3] == -1 and np.all(out["y"][3] == -1)
    assert out["n"][2] >= 0
    check_verify(inp["Ld"], inp["Lt"], inp["x"], inp["u_acc"], inp["u_fin"], inp["t_off"],
                 inp["length"], out["n"], out["y"], [0, 2])
    cs = run_tv(inp)
    assert np.all(np.isnan(cs[3]))
    bad = dict(inp, length=np.array([3, 2, 9, -1], np.int32))
    out = run_verify(bad)
    assert out["n"][2] == -1 and out["n"][3] == -1


def test_batched_verify_all_requests(gpu):
    """Every request of the batched verify workload (B=256, gamma=16, V=151936): each
    acceptance decision on the GPU's path, the final draw and every c* against the oracle."""
    c = synth.config(synth.VERIFY)
    inp = verify_inputs(c)
    out = run_verify(inp, want_lse=True)
    rep = check_verify(inp["Ld"], inp["Lt"], inp["x"], inp["u_acc"], inp["u_fin"], None, None,
                       out["n"], out["y"], range(c.B), rep=Report("batched verify"))
    assert rep.ties <= tie_bound(rep)
    cs = run_tv(inp, lse_d=dev(out["lse_d"]), lse_t=dev(out["lse_t"]))
    check_cstar(inp["Ld"], inp["Lt"], None, None, cs, range(c.B), rep=rep)
    rep.record()
    # acceptance falls along the block as the target noise grows
    mean_c = np.nanmean(cs, axis=0)
    assert mean_c[0] > 0.8 and mean_c[-1] < 0.6
    n = out["n"]
    assert np.all((n >= 0) & (n <= c.gamma))


def _markov_tables(V, seed):
    g = np.random.default_rng(seed)
    P = g.integers(1, 12, size=(V, V)).astype(np.float64)
    P[g.random((V, V)) < 0.2] = 0.0
    P[np.arange(V), g.integers(0, V, V)] += 1.0
    P /= P.sum(1, keepdims=True)
    Q = g.integers(1, 12, size=(V, V)).astype(np.float64)
    Q /= Q.sum(1, keepdims=True)
    return P, Q


def _gpu_round(logP, logQ, prev, G, seed):
    """One GPU draft + verify round; the target model is the table logP indexed by context."""
    N, V = prev.shape[0], logP.shape[0]
    gen = synth.rng(950, seed)
    u = torch.from_numpy(synth.uniforms(gen, (N, G))).cuda()
    d = dspark.markov_draft(torch.zeros((N, G, V), dtype=torch.float32, device="cuda"),
                            torch.eye(V, dtype=torch.float32, device="cuda"), logQ, prev, u,
                            want_logits=True)
    ctx = torch.cat([prev[:, None], d["x"]], dim=1).long()
    Lt = logP[ctx].reshape(N * (G + 1), V).contiguous()
    u_acc = torch.from_numpy(synth.uniforms(gen, (N, G))).cuda()
    u_fin = torch.from_numpy(synth.uniforms(gen, (N,))).cuda()
    return dspark.verify(d["L"], Lt, d["x"], u_acc, u_fin, ld_lse=d["lse"])


def _chi2_pvalue(counts, probs, N):
    expected = N * probs
    keep = expected >= 5
    obs = np.append(counts[keep], counts[~keep].sum())
    exp = np.append(expected[keep], expected[~keep].sum())
    if exp[-1] == 0:
        obs, exp = obs[:-1], exp[:-1]
    return scipy.stats.chisquare(obs, exp).pvalue


def test_lossless_first_token_chi2(gpu):
    """2^20 requests, gamma = 3: the first emitted token follows the target law exactly."""
    V, G, N = 8, 3, 1 << 20
    P, Q = _markov_tables(V, 123)
    with np.errstate(divide="ignore"):
        logP = torch.from_numpy(np.log(P).astype(np.float32)).cuda()
    logQ = torch.from_numpy(np.log(Q).astype(np.float32)).cuda()
    prev = torch.full((N,), 3, dtype=torch.int32, device="cuda")
    res = _gpu_round(logP, logQ, prev, G, 0)
    y = host(res["y"])
    assert np.all(host(res["n"]) >= 0)
    counts = np.bincount(y[:, 0], minlength=V).astype(float)
    assert _chi2_pvalue(counts, P[3], N) > 1e-3


def test_lossless_multi_round_joint_chi2(gpu):
    """First three emitted tokens over repeated rounds follow the target chain's joint law."""
    V, G, N, x0 = 8, 3, 1 << 20, 5
    P, Q = _markov_tables(V, 321)
    with np.errstate(divide="ignore"):
        logP = torch.from_numpy(np.log(P).astype(np.float32)).cuda()
    logQ = torch.from_numpy(np.log(Q).astype(np.float32)).cuda()
    seq = np.full((N, 3), -1, np.int64)
    filled = np.zeros(N, np.int64)
    prev = np.full(N, x0, np.int32)
    rnd = 0
    while (filled < 3).any():
        act = np.nonzero(filled < 3)[0]
        res = _gpu_round(logP, logQ, torch.from_numpy(prev[act]).cuda(), G, 1 + rnd)
        y, n = host(res["y"]), host(res["n"]).astype(np.int64)
        assert np.all(n >= 0)
        f = filled[act]
        for t in range(G + 1):
            m = (t <= n) & (f + t < 3)
            seq[act[m], (f + t)[m]] = y[m, t]
        filled[act] = np.minimum(3, f + n + 1)
        prev[act] = y[np.arange(act.shape[0]), n]
        rnd += 1
    idx = seq[:, 0] * V * V + seq[:, 1] * V + seq[:, 2]
    counts = np.bincount(idx, minlength=V ** 3).astype(float)
    joint = (P[x0][:, None, None] * P[:, :, None] * P[None, :, :]).reshape(-1)
    assert _chi2_pvalue(counts, joint, N) > 1e-3


def test_accept_rate_matches_tv(gpu):
    """Monte-Carlo acceptance at position 1 equals the GPU's own c*_1 within 4 sigma."""
    V, N = 50, 1 << 18
    g = np.random.default_rng(9)
    ld = (1.5 * g.standard_normal(V)).astype(np.float32)
    lt = (ld + 0.9 * g.standard_normal(V)).astype(np.float32)
    Ld = torch.from_numpy(ld).cuda().expand(N, 1, V).contiguous()
    Lt = torch.from_numpy(np.stack([lt, ld])).cuda().repeat(N, 1).contiguous()
    x = dspark.markov_draft(Ld, torch.zeros((V, 1), device="cuda"), torch.zeros((1, V), device="cuda"),
                            torch.zeros(N, dtype=torch.int32, device="cuda"),
                            torch.from_numpy(synth.uniforms(synth.rng(951, 0), (N, 1))).cuda())["x"]
    u_acc = torch.from_numpy(synth.uniforms(synth.rng(951, 1), (N, 1))).cuda()
    u_fin = torch.from_numpy(synth.uniforms(synth.rng(951, 2), (N,))).cuda()
    res = dspark.verify(Ld, Lt, x, u_acc, u_fin)
    rate = float((host(res["n"]) == 1).mean())
    c1 = float(host(dspark.tv_labels(Ld[:1], Lt[:2]))[0, 0])
    ref = oracle.tv_row_pair(ld, lt)
    assert abs(c1 - ref) < PROB_TOL
    assert abs(rate - ref) < 4 * np.sqrt(ref * (1 - ref) / N)


def test_tv_two_point_closed_form(gpu):
    qs = np.array([0.3, 0.5, 0.01, 0.9], np.float64)
    ss = np.array([0.7, 0.5, 0.99, 0.2], np.float64)
    B = len(qs)
    Ld = np.log(np.stack([qs, 1 - qs], -1)).astype(np.float32)[:, None, :]
    Lt = np.concatenate([np.log(np.stack([ss, 1 - ss], -1)).astype(np.float32)[:, None, :],
                         np.zeros((B, 1, 2), np.float32)], 1).reshape(-1, 2)
    inp = dict(Ld=Ld, Lt=Lt, t_off=None, length=None)
    cs = run_tv(inp)
    np.testing.assert_allclose(cs[:, 0], 1 - np.abs(qs - ss), atol=1e-6)


def _random_shapes(n, seed):
    """Verify shapes drawn from a fixed seed: V from 2 to 200000 (any residue mod 4), gamma
    1..20, B up to 64 with B * gamma * V kept under 4e7 logits, flattened or padded target
    rows, draft normalisers supplied or computed."""
    g = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        V = int(np.exp(g.uniform(np.log(2), np.log(200000))))
        G = int(g.integers(1, 21))
        B = int(g.integers(1, max(2, min(64, 40_000_000 // (G * V)) + 1)))
        out.append((B, V, G, bool(g.random() < 0.7), bool(g.random() < 0.5)))
    return out


@pytest.mark.parametrize("B,V,G,flat,given", _random_shapes(10, 2028))
def test_random_shapes(gpu, B, V, G, flat, given):
    """Seeded random shapes and verify lengths: dspark_verify_tv bit for bit against
    dspark_verify then dspark_tv_labels, and sampled requests against the oracle."""
    c = synth.custom(1200 + V % 97, B=B, V=V, r=1, gamma=G, w_dtype="f32", tnoise=0.8)
    g = np.random.default_rng(V + G)
    lengths = g.integers(0, G + 1, size=B) if flat else None
    if flat:
        lengths[0] = G
    inp = verify_inputs(c, lengths, flat)
    ld_lse = None
    if given:
        ld_lse = dev(np.array([[oracle.softmax_row(inp["Ld"][i, k])[1] for k in range(G)]
                               for i in range(B)], np.float32))
    a = run_verify(inp, want_lse=True, ld_lse=ld_lse)
    tv = run_tv(inp, lse_d=ld_lse if given else dev(a["lse_d"]), lse_t=dev(a["lse_t"]))
    f = run_verify_tv(inp, ld_lse=ld_lse)
    for k in ("n", "y", "lse_d", "lse_t"):
        assert np.array_equal(a[k].view(np.uint8), f[k].view(np.uint8)), k
    assert np.array_equal(np.isnan(tv), np.isnan(f["cstar"]))
    fin = ~np.isnan(tv)
    assert np.array_equal(tv[fin].view(np.uint8), f["cstar"][fin].view(np.uint8))
    reqs = sorted({0, B // 2, B - 1})
    rep = check_verify(inp["Ld"], inp["Lt"], inp["x"], inp["u_acc"], inp["u_fin"], inp["t_off"],
                       inp["length"], f["n"], f["y"], reqs)
    assert rep.ties <= tie_bound(rep)
    check_tv(inp, f["cstar"], reqs)
