"""GPU parity of dspark_markov_draft against the fp64 oracle (called through the C ABI)."""
import numpy as np
import pytest
import scipy.stats
import torch

import oracle
import synth
import draft_sampling_verification_head_amd as dspark
from parity import tie_bound, Report, check_draft, dev, host

pytestmark = pytest.mark.gpu


def run_draft(d, want_logits=True, per_position=False):
    out = dspark.markov_draft(dev(d["U"]), dev(d["W1"]), dev(d["W2"]), dev(d["x0"]),
                              dev(d["u"]), want_logits=want_logits, per_position=per_position)
    torch.cuda.synchronize()
    return {k: (host(v) if v is not None else None) for k, v in out.items()}


def test_tiny_fp32_exact(gpu):
    c = synth.config(synth.TINY)
    d = synth.draft_inputs(c)
    g = run_draft(d)
    rep = check_draft(d["U"], d["W1"], d["W2"], d["x0"], d["u"], c.w_dtype, g["x"], g["q"],
                      g["lse"], range(c.B), gL=g["L"])
    assert rep.ties == 0 and rep.compared == c.B * c.gamma


@pytest.mark.parametrize("B,V,r,G,wdt", [
    (3, 1000, 17, 5, "f32"),      # V % 8 != 0: guarded loads, ragged last tile
    (5, 4099, 64, 3, "bf16"),
    (1, 513, 8, 9, "bf16"),       # one column into the second tile
    (2, 2056, 256, 4, "bf16"),
    (9, 3000, 32, 2, "f32"),      # two request groups, the second ragged
    (4, 1, 3, 3, "f32"),          # a single-token vocabulary
    (2, 4096, 1024, 2, "bf16"),   # rank at its cap
    (1, 777, 5, 64, "f32"),       # gamma at its cap
])
def test_ragged_shapes(gpu, B, V, r, G, wdt):
    c = synth.custom(920 + B + V % 97, B=B, V=V, r=r, gamma=G, w_dtype=wdt, w_sigma=0.3)
    d = synth.draft_inputs(c)
    assert dspark.markov_draft_path(B, dev(d["W1"]), dev(d["W2"])) == "sweep"
    g = run_draft(d)
    rep = check_draft(d["U"], d["W1"], d["W2"], d["x0"], d["u"], wdt, g["x"], g["q"], g["lse"],
                      range(B), gL=g["L"])
    assert rep.ties <= tie_bound(rep)


@pytest.mark.parametrize("B,V,r,G", [
    (9, 163848, 16, 3),     # one ragged request group, V past the slab path's cap
    (65, 164000, 248, 2),   # two request groups; rank padded to the 16-row chunk
])
def test_batched_mfma_shapes(gpu, B, V, r, G):
    c = synth.custom(935 + B, B=B, V=V, r=r, gamma=G, w_dtype="bf16", w_sigma=0.3)
    d = synth.draft_inputs(c)
    assert dspark.markov_draft_path(B, dev(d["W1"]), dev(d["W2"])) == "mfma"
    g = run_draft(d)
    rep = check_draft(d["U"], d["W1"], d["W2"], d["x0"], d["u"], "bf16", g["x"], g["q"], g["lse"],
                      range(B), gL=g["L"])
    assert rep.ties <= tie_bound(rep)
    assert np.all((g["x"] >= 0) & (g["x"] < V))


@pytest.mark.parametrize("B,V,r,G", [
    (9, 4104, 16, 3),       # one ragged request group of 16, one slab tile past V
    (65, 2056, 248, 2),     # five groups, the last ragged; rank padded to the 32-rank chunk
    (130, 3000, 64, 3),     # two MFMA rank chunks
    (64, 8192, 256, 2),     # exact slabs
    (20, 40000, 256, 2),    # two 16-column tiles per wave
    (33, 70000, 128, 3),    # three
    (17, 129280, 256, 2),   # four
    (40, 151936, 256, 2),   # five, the full vocabulary
])
def test_batched_slab_shapes(gpu, B, V, r, G):
    """bf16 batches: W2 slabs in registers, draws that recompute the chosen tile. One
    persistent launch draws every position, with or without the logits output; the
    per-position form (a stream and a draw launch per position) gives the same tokens,
    probabilities, normalisers and logits bit for bit."""
    c = synth.custom(955 + B, B=B, V=V, r=r, gamma=G, w_dtype="bf16", w_sigma=0.3)
    d = synth.draft_inputs(c)
    W1, W2 = dev(d["W1"]), dev(d["W2"])
    assert dspark.markov_draft_path(B, W1, W2) == "slab"
    assert dspark.markov_draft_one_launch(B, W1, W2)
    assert dspark.markov_draft_one_launch(B, W1, W2, want_logits=True)
    g = run_draft(d)
    rep = check_draft(d["U"], d["W1"], d["W2"], d["x0"], d["u"], "bf16", g["x"], g["q"], g["lse"],
                      range(B), gL=g["L"])
    assert rep.ties <= tie_bound(rep)
    assert np.all((g["x"] >= 0) & (g["x"] < V))
    per = run_draft(d, per_position=True)
    for k in ("x", "q", "lse", "L"):
        assert np.array_equal(g[k].view(np.uint8), per[k].view(np.uint8)), k
    one = run_draft(d, want_logits=False)
    for k in ("x", "q", "lse"):
        assert np.array_equal(g[k].view(np.uint8), one[k].view(np.uint8)), k


@pytest.mark.parametrize("V,r,G", [
    (8, 8, 3),              # one 16-byte chunk: one workgroup, one live lane
    (640, 256, 5),          # exactly one 640-column workgroup tile
    (1288, 64, 7),          # two full tiles and a ragged third
    (20000, 248, 16),       # rank not a multiple of the 32-rank lane group
    (151936, 256, 64),      # full vocabulary, gamma at its cap
])
def test_single_request_bf16_shapes(gpu, V, r, G):
    """One bf16 request: the single-launch path with W2 held in registers."""
    c = synth.custom(940 + V % 89, B=1, V=V, r=r, gamma=G, w_dtype="bf16", w_sigma=0.3)
    d = synth.draft_inputs(c)
    assert dspark.markov_draft_path(1, dev(d["W1"]), dev(d["W2"])) == "resident"
    g = run_draft(d)
    rep = check_draft(d["U"], d["W1"], d["W2"], d["x0"], d["u"], "bf16", g["x"], g["q"],
                      g["lse"], [0], gL=g["L"])
    assert rep.ties <= tie_bound(rep)
    assert rep.compared == G
    # per-position launches instead (the vocabulary sweep): the same function to within fp32
    # rounding order, so checked against the oracle rather than bit for bit
    p = run_draft(d, per_position=True)
    rep = check_draft(d["U"], d["W1"], d["W2"], d["x0"], d["u"], "bf16", p["x"], p["q"],
                      p["lse"], [0], gL=p["L"])
    assert rep.ties <= tie_bound(rep)


def test_slab_logits_output_is_optional(gpu):
    """The slab path's draws do not read the logits: the same tokens, probabilities and
    normalisers with and without the logits output, in both launch forms, and the stored
    logits match the oracle's."""
    c = synth.custom(961, B=24, V=30000, r=256, gamma=4, w_dtype="bf16", w_sigma=0.3)
    d = synth.draft_inputs(c)
    assert dspark.markov_draft_one_launch(c.B, dev(d["W1"]), dev(d["W2"]))
    a = run_draft(d, want_logits=True)
    b = run_draft(d, want_logits=False)
    pa = run_draft(d, want_logits=True, per_position=True)
    pb = run_draft(d, want_logits=False, per_position=True)
    for k in ("x", "q", "lse"):
        for o in (b, pa, pb):
            assert np.array_equal(a[k].view(np.uint8), o[k].view(np.uint8)), k
    assert np.array_equal(a["L"].view(np.uint8), pa["L"].view(np.uint8))
    check_draft(d["U"], d["W1"], d["W2"], d["x0"], d["u"], "bf16", a["x"], a["q"], a["lse"],
                [0, 11, 23], gL=a["L"])


def test_slab_permutation_chain_and_sentinels(gpu):
    """Closed form through the slab path (W1[x] = 50 e_{x mod r}, W2 a partial permutation:
    x_k = perm[x_{k-1} mod r]), with dead requests: an out-of-range context token gives -1
    everywhere, a row of -inf from its position on."""
    g = np.random.default_rng(9)
    B, G, V, r = 21, 6, 9000, 16
    perm = g.permutation(V)[:r]
    W1 = np.zeros((V, r), np.float32)
    W1[np.arange(V), np.arange(V) % r] = 50.0
    W2 = np.zeros((r, V), np.float32)
    W2[np.arange(r), perm] = 1.0
    x0 = g.integers(0, V, size=B).astype(np.int32)
    x0[3] = V + 2
    x0[17] = -1
    U = (0.1 * g.standard_normal((B, G, V))).astype(np.float32)
    U[8, 2, :] = -np.inf
    d = dict(U=U, W1=synth.f32_to_bf16_bits(W1), W2=synth.f32_to_bf16_bits(W2), x0=x0,
             u=g.uniform(1e-3, 1 - 2 ** -24, size=(B, G)).astype(np.float32))
    assert dspark.markov_draft_path(B, dev(d["W1"]), dev(d["W2"])) == "slab"
    out = run_draft(d, want_logits=False)
    for b in range(B):
        if b in (3, 17):
            assert np.all(out["x"][b] == -1)
            assert np.all(out["lse"][b] == -np.inf) and np.all(out["q"][b] == 0.0)
            continue
        prev = x0[b]
        for k in range(G):
            if b == 8 and k >= 2:
                assert out["x"][b, k] == -1
                continue
            prev = perm[prev % r]
            assert out["x"][b, k] == prev
            assert 0.99 < out["q"][b, k] <= 1.0


@pytest.mark.parametrize("B,one_launch", [
    (2044, True),     # the largest batch whose persistent launch fits in LDS at V = 151936
    (2048, False),    # the slab path's cap: per-position launches
])
def test_slab_max_batch(gpu, B, one_launch):
    """The slab path at its LDS limits on the full vocabulary (V = 151936), one position;
    sampled requests against the oracle. U is generated on the device (seeded) and the
    sampled rows are copied back for the oracle."""
    V, r = 151936, 256
    c = synth.custom(962, B=2, V=V, r=r, gamma=1, w_dtype="bf16", w_sigma=0.3)
    d = synth.draft_inputs(c)
    gen = torch.Generator(device="cuda").manual_seed(962)
    U = torch.randn((B, 1, V), generator=gen, device="cuda") * 3.0
    x0 = torch.randint(0, V, (B,), generator=gen, device="cuda", dtype=torch.int32)
    u = torch.rand((B, 1), generator=gen, device="cuda").clamp_(max=1 - 2 ** -24)
    W1, W2 = dev(d["W1"]), dev(d["W2"])
    assert dspark.markov_draft_path(B, W1, W2) == "slab"
    assert dspark.markov_draft_one_launch(B, W1, W2) == one_launch
    out = dspark.markov_draft(U, W1, W2, x0, u)
    torch.cuda.synchronize()
    reqs = [0, 1, 1023, B - 2, B - 1]
    idx = torch.tensor(reqs, device="cuda")
    rep = check_draft(host(U[idx]), d["W1"], d["W2"], host(x0[idx]), host(u[idx]), "bf16",
                      host(out["x"][idx]), host(out["q"][idx]), host(out["lse"][idx]),
                      range(len(reqs)))
    assert rep.ties <= tie_bound(rep)
    assert bool(((out["x"] >= 0) & (out["x"] < V)).all())


def test_single_request_bf16_permutation_chain(gpu):
    """Closed form through the single-request path: W1[x] = 50 e_{x mod r}, W2 a partial
    permutation, so x_k = perm[x_{k-1} mod r] whatever the uniforms."""
    g = np.random.default_rng(8)
    G, V, r = 12, 6000, 16
    perm = g.permutation(V)[:r]
    W1 = np.zeros((V, r), np.float32)
    W1[np.arange(V), np.arange(V) % r] = 50.0
    W2 = np.zeros((r, V), np.float32)
    W2[np.arange(r), perm] = 1.0
    d = dict(U=(0.1 * g.standard_normal((1, G, V))).astype(np.float32),
             W1=synth.f32_to_bf16_bits(W1), W2=synth.f32_to_bf16_bits(W2),
             x0=np.array([4321], np.int32),
             u=g.uniform(1e-3, 1 - 2 ** -24, size=(1, G)).astype(np.float32))
    out = run_draft(d, want_logits=False)
    prev = 4321
    for k in range(G):
        prev = perm[prev % r]
        assert out["x"][0, k] == prev


def test_single_request_pick_in_first_and_last_tile(gpu):
    """The single-request draft's draw when the picked tile is workgroup 0's own (the
    workgroup that gathers the tile partials then also rescans) and when it is the last,
    ragged tile: a +20 boost puts almost all of a position's mass on token 5 (tile 0) or on
    token V - 1 (the third tile of V = 1288), alternately."""
    c = synth.custom(947, B=1, V=1288, r=64, gamma=8, w_dtype="bf16", w_sigma=0.02)
    d = synth.draft_inputs(c)
    d["U"] = (0.1 * np.random.default_rng(947).standard_normal(d["U"].shape)).astype(np.float32)
    want = [5 if k % 2 == 0 else c.V - 1 for k in range(c.gamma)]
    for k, tok in enumerate(want):
        d["U"][0, k, tok] += 20.0
    assert dspark.markov_draft_path(1, dev(d["W1"]), dev(d["W2"])) == "resident"
    g = run_draft(d)
    assert g["x"][0].tolist() == want
    rep = check_draft(d["U"], d["W1"], d["W2"], d["x0"], d["u"], "bf16", g["x"], g["q"],
                      g["lse"], [0], gL=g["L"])
    assert rep.ties == 0 and rep.compared == c.gamma


def test_single_request_bf16_sentinels(gpu):
    c = synth.custom(936, B=1, V=3000, r=32, gamma=5)
    d = synth.draft_inputs(c)
    d["U"][0, 2, :] = -np.inf                  # position 3 has no mass: -1 from there on
    g = run_draft(d)
    ref = oracle.markov_draft(d["U"], d["W1"], d["W2"], d["x0"], d["u"], "bf16")
    assert np.array_equal(ref["x"], g["x"])
    assert np.all(g["x"][0, 2:] == -1) and g["lse"][0, 2] == -np.inf and g["q"][0, 2] == 0.0
    d["x0"][0] = c.V + 7                       # out-of-range context token: all -1
    g = run_draft(d)
    assert np.all(g["x"] == -1)


def test_w1_zero_is_independent_sampling(gpu):
    c = synth.custom(930, B=6, V=3001, r=16, gamma=5, w_dtype="bf16")
    d = synth.draft_inputs(c)
    d["W1"] = np.zeros_like(d["W1"])
    a = run_draft(d)
    d2 = dict(d, x0=((d["x0"] + 11) % c.V).astype(np.int32))
    b = run_draft(d2)
    assert np.array_equal(a["x"], b["x"])
    check_draft(d["U"], d["W1"], d["W2"], d["x0"], d["u"], "bf16", a["x"], a["q"], a["lse"],
                range(c.B))


def test_permutation_chain_closed_form(gpu):
    g = np.random.default_rng(7)
    B, G, V, r = 8, 6, 5000, 16
    perm = g.permutation(V)[:r]
    W1 = np.zeros((V, r), np.float32)
    W1[np.arange(V), np.arange(V) % r] = 50.0
    W2 = np.zeros((r, V), np.float32)
    W2[np.arange(r), perm] = 1.0
    d = dict(U=(0.1 * g.standard_normal((B, G, V))).astype(np.float32), W1=W1, W2=W2,
             x0=g.integers(0, V, size=B).astype(np.int32),
             u=g.uniform(1e-3, 1 - 2 ** -24, size=(B, G)).astype(np.float32))
    out = run_draft(d, want_logits=False)
    for b in range(B):
        prev = d["x0"][b]
        for k in range(G):
            prev = perm[prev % r]
            assert out["x"][b, k] == prev


def test_single_request_full(gpu):
    c = synth.config(synth.SINGLE)
    d = synth.draft_inputs(c)
    g = run_draft(d)
    rep = check_draft(d["U"], d["W1"], d["W2"], d["x0"], d["u"], c.w_dtype, g["x"], g["q"],
                      g["lse"], range(c.B), gL=g["L"])
    assert rep.compared == c.gamma
    assert rep.ties <= tie_bound(rep)
    rep.record()


def test_batched_draft_all_requests(gpu):
    """Every request and position of the batched workload (B=64, gamma=16, V=151936) against
    the oracle on the GPU's own prefix; ties stay within the shared bound (5 % plus 2)."""
    c = synth.config(synth.BATCHED)
    d = synth.draft_inputs(c)
    g = run_draft(d)
    rep = check_draft(d["U"], d["W1"], d["W2"], d["x0"], d["u"], c.w_dtype, g["x"], g["q"],
                      g["lse"], range(c.B), gL=g["L"], rep=Report("batched draft"))
    assert rep.compared == c.B * c.gamma
    assert rep.ties <= tie_bound(rep)
    rep.record()
    assert np.all((g["x"] >= 0) & (g["x"] < c.V))
    assert np.all((g["q"] > 0) & (g["q"] <= 1))


def test_determinism_bitwise(gpu):
    c = synth.custom(931, B=16, V=20000, r=256, gamma=4)
    d = synth.draft_inputs(c)
    a = run_draft(d)
    b = run_draft(d)
    for k in ("x", "q", "lse", "L"):
        assert np.array_equal(a[k].view(np.uint8), b[k].view(np.uint8)), k


def test_sentinels(gpu):
    c = synth.custom(932, B=3, V=600, r=8, gamma=4, w_dtype="f32")
    d = synth.draft_inputs(c)
    d["x0"][0] = c.V + 5
    d["x0"][1] = -3
    d["U"][2, 2, :] = -np.inf
    g = run_draft(d)
    assert np.all(g["x"][0] == -1) and np.all(g["x"][1] == -1)
    assert g["x"][2, 0] >= 0 and g["x"][2, 1] >= 0
    assert np.all(g["x"][2, 2:] == -1)
    assert g["lse"][2, 2] == -np.inf and g["q"][2, 2] == 0.0
    ref = oracle.markov_draft(d["U"], d["W1"], d["W2"], d["x0"], d["u"], "f32")
    assert np.array_equal(ref["x"], g["x"])


def test_uniform_edges(gpu):
    c = synth.custom(933, B=4, V=2500, r=8, gamma=3, w_dtype="f32")
    d = synth.draft_inputs(c)
    d["u"][0, :] = 0.0
    d["u"][1, :] = 1.0            # clamped to 1 - 2^-24
    d["u"][2, :] = np.nextafter(np.float32(1.0), np.float32(0.0))
    g = run_draft(d)
    check_draft(d["U"], d["W1"], d["W2"], d["x0"], d["u"], "f32", g["x"], g["q"], g["lse"],
                range(c.B))


def test_sampler_chi_squared(gpu):
    """2^18 requests drafting one token from the same context: the law of x_1 is
    softmax(U_1 + W1[x0] W2), compared by a chi-squared test."""
    N, V, r = 1 << 18, 12, 3
    g = np.random.default_rng(44)
    U1 = (0.7 * g.standard_normal(V)).astype(np.float32)
    W1 = (0.5 * g.standard_normal((V, r))).astype(np.float32)
    W2 = (0.5 * g.standard_normal((r, V))).astype(np.float32)
    x0 = np.full(N, 5, np.int32)
    U = torch.from_numpy(U1).cuda().expand(N, 1, V).contiguous()
    u = torch.from_numpy(synth.uniforms(synth.rng(934, 0), (N, 1))).cuda()
    out = dspark.markov_draft(U, dev(W1), dev(W2), dev(x0), u, want_q=False, want_lse=False)
    counts = np.bincount(host(out["x"])[:, 0], minlength=V).astype(float)
    p = oracle.softmax_row(U1.astype(np.float64) + W1[5].astype(np.float64) @ W2.astype(np.float64))[0]
    assert scipy.stats.chisquare(counts, N * p).pvalue > 1e-3


@pytest.mark.parametrize("B,V,r,G,wdt,want_logits", [
    (4, 3000, 32, 7, "f32", True),          # vocabulary sweep
    (1, 20000, 256, 9, "bf16", False),      # single-request resident launch
    (40, 40000, 256, 6, "bf16", False),     # slab path, persistent launch
    (40, 40000, 256, 6, "bf16", True),      # slab path, per-position launches
])
def test_resume_split_generation(gpu, B, V, r, G, wdt, want_logits):
    """Resuming a generation: a gamma-position draft equals a g1-position draft followed by a
    (gamma - g1)-position draft started from the last drafted token with the remaining U rows
    and uniforms, bit for bit (position k depends only on U_k, x_{k-1}, u_k and the factors)."""
    c = synth.custom(990 + B + G, B=B, V=V, r=r, gamma=G, w_dtype=wdt, w_sigma=0.3)
    d = synth.draft_inputs(c)
    full = run_draft(d, want_logits=want_logits)
    for g1 in (1, G // 2, G - 1):
        a = dict(d, U=np.ascontiguousarray(d["U"][:, :g1]), u=np.ascontiguousarray(d["u"][:, :g1]))
        first = run_draft(a, want_logits=want_logits)
        b = dict(d, U=np.ascontiguousarray(d["U"][:, g1:]), u=np.ascontiguousarray(d["u"][:, g1:]),
                 x0=np.ascontiguousarray(first["x"][:, -1]).astype(np.int32))
        second = run_draft(b, want_logits=want_logits)
        for k in ("x", "q", "lse"):
            joined = np.concatenate([first[k], second[k]], axis=1)
            assert np.array_equal(joined.view(np.uint8), full[k].view(np.uint8)), (g1, k)
        if want_logits:
            joined = np.concatenate([first["L"], second["L"]], axis=1)
            assert np.array_equal(joined.view(np.uint8), full["L"].view(np.uint8)), g1


def test_single_request_graph_replays(gpu):
    """The single-request resident draft captured once and replayed: the launch resets its
    own position slots (keyed by a call counter in the workspace), so every replay, with
    eager calls of other shapes on the same workspace between them, equals the eager call."""
    c = synth.custom(977, B=1, V=20000, r=64, gamma=6, w_dtype="bf16", w_sigma=0.3)
    d = synth.draft_inputs(c)
    U, W1, W2, x0, u = (dev(d[k]) for k in ("U", "W1", "W2", "x0", "u"))
    assert dspark.markov_draft_path(1, W1, W2) == "resident"
    out = dict(x=torch.empty((1, c.gamma), dtype=torch.int32, device="cuda"),
               q=torch.empty((1, c.gamma), dtype=torch.float32, device="cuda"),
               lse=torch.empty((1, c.gamma), dtype=torch.float32, device="cuda"),
               L=torch.empty((1, c.gamma, c.V), dtype=torch.float32, device="cuda"))
    ref = run_draft(d)
    other = synth.custom(978, B=1, V=9000, r=64, gamma=3, w_dtype="bf16", w_sigma=0.3)
    od = synth.draft_inputs(other)
    dspark.markov_draft(U, W1, W2, x0, u, out=out)          # workspace sized before capture
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            dspark.markov_draft(U, W1, W2, x0, u, out=out)
    torch.cuda.synchronize()
    for rep in range(4):
        for k in out.values():
            k.fill_(-7)
        graph.replay()
        torch.cuda.synchronize()
        for k in ("x", "q", "lse", "L"):
            assert np.array_equal(host(out[k]).view(np.uint8), ref[k].view(np.uint8)), (rep, k)
        run_draft(od)                                        # another shape between replays


def _random_shapes(n, seed):
    """Draft shapes drawn from a fixed seed within the slab and resident paths' caps: B = 1
    (resident) or 9..96 (slab), V a multiple of 8 from 1024 to 163840, r a multiple of 8 up
    to 256, gamma 1..20; the batch kept small enough for the oracle."""
    g = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        B = 1 if g.random() < 0.3 else int(g.integers(9, 97))
        V = int(g.integers(128, 20481)) * 8
        r = int(g.integers(1, 33)) * 8
        G = int(g.integers(1, 21))
        out.append((B, V, r, G))
    return out


@pytest.mark.parametrize("B,V,r,G", _random_shapes(10, 2026))
def test_random_shapes_all_forms(gpu, B, V, r, G):
    """Seeded random shapes: the default form (one launch where it fits) with and without
    the logits, and the per-position form, each against the oracle on sampled requests;
    on the slab path the forms agree bit for bit."""
    c = synth.custom(1000 + B + G, B=B, V=V, r=r, gamma=G, w_dtype="bf16", w_sigma=0.3)
    d = synth.draft_inputs(c)
    W1, W2 = dev(d["W1"]), dev(d["W2"])
    path = dspark.markov_draft_path(B, W1, W2)
    assert path == ("resident" if B == 1 else "slab")
    a = run_draft(d, want_logits=True)
    b = run_draft(d, want_logits=False)
    p = run_draft(d, want_logits=True, per_position=True)
    reqs = sorted({0, B // 2, B - 1})
    for o in (a, p):
        rep = check_draft(d["U"], d["W1"], d["W2"], d["x0"], d["u"], "bf16", o["x"], o["q"], o["lse"],
                          reqs, gL=o["L"])
        assert rep.ties <= tie_bound(rep)
    for k in ("x", "q", "lse"):
        assert np.array_equal(a[k].view(np.uint8), b[k].view(np.uint8)), k
        if path == "slab":
            assert np.array_equal(a[k].view(np.uint8), p[k].view(np.uint8)), k
    if path == "slab":
        assert np.array_equal(a["L"].view(np.uint8), p["L"].view(np.uint8))
